"""fp64 CPU oracle for exact softmax attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never loads it and the
two share no code.  The arithmetic lives in ``oracle.c`` (plain C, fp64); this
module only marshals numpy arrays in and out and adds the central-difference
gradient, which is a loop of calls to the dense forward.

Conventions: arrays are float64, contiguous, shaped [B, H, N, d].  Scores are
``scale * Q @ K^T``; with ``causal`` key j is visible to query i iff
``j <= q_start + i``.  L is the natural-log log-sum-exp.

Pages followed (named in each function): attention_kernels.py (CMU 15-779
lecture 5), lab.py (hs-black FlashAttention post), model.py (tensorviz
flash-attention), flash_attention_numpy.py (first_principles).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_LIB = None

_i64 = ctypes.c_int64
_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp, "-lm"],
            check=True,
        )
        os.replace(tmp, _SO)
    return _SO


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        lib.oracle_dense_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64, _i64,
                                         _i64, ctypes.c_double, ctypes.c_int, _i64, _ip, _i64,
                                         ctypes.c_int]
        lib.oracle_online_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64, _i64,
                                          _i64, ctypes.c_double, ctypes.c_int, _i64, _i64, _ip,
                                          _i64, ctypes.c_int]
        lib.oracle_dense_bwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _i64,
                                         _i64, _i64, _i64, _i64, _i64, ctypes.c_double,
                                         ctypes.c_int, _i64, _ip, _i64, ctypes.c_int]
        lib.oracle_bwd_query_rows.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _i64,
                                              _i64, _i64, _i64, _i64, _i64, ctypes.c_double,
                                              ctypes.c_int, _i64, _ip, _i64, ctypes.c_int]
        lib.oracle_bwd_key_rows.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _i64, _i64,
                                            _i64, _i64, _i64, _i64, ctypes.c_double,
                                            ctypes.c_int, _i64, _ip, _i64, ctypes.c_int]
        lib.oracle_state.argtypes = [_dp, _dp, _i64, _i64, _dp, _dp, _dp]
        lib.oracle_state.restype = None
        lib.oracle_merge.argtypes = [ctypes.c_double, ctypes.c_double, _dp, ctypes.c_double,
                                     ctypes.c_double, _dp, _i64, _dp, _dp, _dp]
        lib.oracle_merge.restype = None
        lib.oracle_split_decode.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _i64, _i64,
                                            _i64, _i64, _i64, _i64, _i64, ctypes.c_double, _ip,
                                            _i64, ctypes.c_int]
        for f in ("oracle_dense_fwd", "oracle_online_fwd", "oracle_dense_bwd",
                  "oracle_bwd_query_rows", "oracle_bwd_key_rows", "oracle_split_decode"):
            getattr(lib, f).restype = ctypes.c_int
        _LIB = lib
    return _LIB


def default_threads() -> int:
    """Host threads the oracle uses: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _f64(a) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    return a


def _p(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def _check4(*arrs):
    for a in arrs:
        if a.ndim != 4:
            raise ValueError("oracle arrays are [B, H, N, d]")


def dense_fwd(Q, K, V, scale: float, causal: bool = False, q_start: int = 0, rows=None,
              nthreads: int | None = None):
    """The definition of softmax attention (standard_attention in
    attention_kernels.py; dense in lab.py): whole score row, max, exp, sum,
    one division.  Returns (O [B,H,Nq,dv], L [B,H,Nq]); with ``rows`` (flat
    ids ``(b*H + h)*Nq + i``) returns (O [n,dv], L [n]) for those rows only."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    _check4(Q, K, V)
    B, H, Nq, d = Q.shape
    Nk, dv = K.shape[2], V.shape[3]
    nt = nthreads or default_threads()
    if rows is None:
        O = np.empty((B, H, Nq, dv))
        L = np.empty((B, H, Nq))
        rp, nr = None, 0
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        O = np.empty((rows.size, dv))
        L = np.empty(rows.size)
        rp, nr = rows.ctypes.data_as(_ip), rows.size
    st = _lib().oracle_dense_fwd(_p(Q), _p(K), _p(V), _p(O), _p(L), B, H, Nq, Nk, d, dv,
                                 float(scale), int(bool(causal)), int(q_start), rp, nr, nt)
    if st != 0:
        raise ValueError("a query row sees no key")
    return O, L


def online_fwd(Q, K, V, scale: float, causal: bool = False, block: int = 64, q_start: int = 0,
               rows=None, nthreads: int | None = None):
    """Per-row online softmax over key blocks of ``block`` (tiled in lab.py;
    TiledAttention in model.py; flash_forward in attention_kernels.py).
    Returns (O, L) like dense_fwd, ``rows`` included."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    _check4(Q, K, V)
    B, H, Nq, d = Q.shape
    Nk, dv = K.shape[2], V.shape[3]
    if rows is None:
        O = np.empty((B, H, Nq, dv))
        L = np.empty((B, H, Nq))
        rp, nr = None, 0
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        O = np.empty((rows.size, dv))
        L = np.empty(rows.size)
        rp, nr = rows.ctypes.data_as(_ip), rows.size
    st = _lib().oracle_online_fwd(_p(Q), _p(K), _p(V), _p(O), _p(L), B, H, Nq, Nk, d, dv,
                                  float(scale), int(bool(causal)), int(q_start), int(block),
                                  rp, nr, nthreads or default_threads())
    if st == 2:
        raise ValueError("block must be >= 1")
    if st != 0:
        raise ValueError("a query row sees no key")
    return O, L


def dense_bwd(Q, K, V, dO, scale: float, causal: bool = False, q_start: int = 0, heads=None,
              nthreads: int | None = None):
    """Gradients of <O, dO> (flash_backward in attention_kernels.py; backward in
    lab.py), from this oracle's own fp64 forward.  Returns a dict with dQ, dK,
    dV, O, L, D; with ``heads`` (flat ids b*H + h) arrays are [n_heads, N, d]."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    _check4(Q, K, V, dO)
    B, H, Nq, d = Q.shape
    Nk, dv = K.shape[2], V.shape[3]
    if heads is None:
        nh, hp, lead = B * H, None, (B, H)
    else:
        heads = np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
        nh, hp, lead = heads.size, heads.ctypes.data_as(_ip), (heads.size,)
    out = {
        "dQ": np.empty(lead + (Nq, d)), "dK": np.empty(lead + (Nk, d)),
        "dV": np.empty(lead + (Nk, dv)), "O": np.empty(lead + (Nq, dv)),
        "L": np.empty(lead + (Nq,)), "D": np.empty(lead + (Nq,)),
    }
    st = _lib().oracle_dense_bwd(_p(Q), _p(K), _p(V), _p(dO), _p(out["dQ"]), _p(out["dK"]),
                                 _p(out["dV"]), _p(out["O"]), _p(out["L"]), _p(out["D"]), B, H,
                                 Nq, Nk, d, dv, float(scale), int(bool(causal)), int(q_start),
                                 hp, nh, nthreads or default_threads())
    if st != 0:
        raise ValueError("a query row sees no key")
    return out


def _central_difference(f, theta: np.ndarray, h: float) -> np.ndarray:
    """Gradient of the scalar function f at the parameter vector theta by
    central differences, (f(theta + h e_n) - f(theta - h e_n)) / 2h for every
    coordinate n, with theta restored after each pair of evaluations."""
    grad = np.empty_like(theta)
    for n in range(theta.size):
        x0 = theta[n]
        theta[n] = x0 + h
        up = f(theta)
        theta[n] = x0 - h
        down = f(theta)
        theta[n] = x0
        grad[n] = (up - down) / (2.0 * h)
    return grad


def fd_grad(Q, K, V, dO, scale: float, causal: bool = False, h: float = 1e-5):
    """Central-difference gradients (dQ, dK, dV) of f = sum(O * dO), O the
    dense definition, with step h (the numerical check of lab.py,
    finite_difference, with the same h).  Q, K and V are packed into one
    parameter vector.  Tiny inputs only."""
    arrays = [np.asarray(x, dtype=np.float64) for x in (Q, K, V)]
    dO = np.asarray(dO, dtype=np.float64)
    shapes = [a.shape for a in arrays]
    cuts = np.cumsum([a.size for a in arrays])[:-1]
    theta = np.concatenate([a.ravel() for a in arrays])

    def f(t):
        q, k, v = (p.reshape(shp) for p, shp in zip(np.split(t, cuts), shapes))
        return float(np.sum(dense_fwd(q, k, v, scale, causal, nthreads=1)[0] * dO))

    grad = _central_difference(f, theta, h)
    return tuple(p.reshape(shp) for p, shp in zip(np.split(grad, cuts), shapes))


def bwd_rows(Q, K, V, dO, scale: float, causal: bool = False, q_start: int = 0,
             query_rows=None, key_rows=None, nthreads: int | None = None):
    """The backward (dense_bwd's formulas) restricted to chosen rows, for
    checks where the whole backward is too slow.  ``query_rows`` are flat ids
    (b*H + h)*Nq + i and give dQ [n, d] (with O, L and D of those rows);
    ``key_rows`` are flat ids (b*H + h)*Nk + j and give dK [n, d], dV [n, dv],
    summed over every query that sees the key, with L and D of those queries
    from this oracle's own forward."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    _check4(Q, K, V, dO)
    B, H, Nq, d = Q.shape
    Nk, dv = K.shape[2], V.shape[3]
    nt = nthreads or default_threads()
    out = {}
    if query_rows is not None:
        rows = np.ascontiguousarray(np.asarray(query_rows, dtype=np.int64))
        out.update(dQ=np.empty((rows.size, d)), O=np.empty((rows.size, dv)),
                   L=np.empty(rows.size), D=np.empty(rows.size))
        st = _lib().oracle_bwd_query_rows(_p(Q), _p(K), _p(V), _p(dO), _p(out["dQ"]),
                                          _p(out["O"]), _p(out["L"]), _p(out["D"]), B, H, Nq,
                                          Nk, d, dv, float(scale), int(bool(causal)),
                                          int(q_start), rows.ctypes.data_as(_ip), rows.size, nt)
        if st != 0:
            raise ValueError("a query row sees no key")
    if key_rows is not None:
        keys = np.ascontiguousarray(np.asarray(key_rows, dtype=np.int64))
        # L and D of every query of the heads involved (other heads stay NaN)
        heads = np.unique(keys // Nk)
        L = np.full(B * H * Nq, np.nan)
        D = np.full(B * H * Nq, np.nan)
        qrows = (heads[:, None] * Nq + np.arange(Nq)[None, :]).ravel()
        O_r, L_r = dense_fwd(Q, K, V, scale, causal, q_start, rows=qrows, nthreads=nt)
        L[qrows] = L_r
        D[qrows] = np.sum(dO.reshape(-1, dv)[qrows] * O_r, axis=1)
        out.update(dK=np.empty((keys.size, d)), dV=np.empty((keys.size, dv)))
        _lib().oracle_bwd_key_rows(_p(Q), _p(K), _p(V), _p(dO), _p(L), _p(D), _p(out["dK"]),
                                   _p(out["dV"]), B, H, Nq, Nk, d, dv, float(scale),
                                   int(bool(causal)), int(q_start), keys.ctypes.data_as(_ip),
                                   keys.size, nt)
    return out


def state(s, v):
    """(m, l, o) summary of one score segment s [n] with values v [n, dv]
    (state_of_scores in attention_kernels.py); empty -> (-inf, 0, 0)."""
    s = _f64(np.reshape(s, (-1,)))
    v = _f64(v)
    n = s.size
    dv = v.shape[-1] if v.ndim == 2 else 0
    if n == 0:
        v = np.zeros((1, dv))
    m, l = ctypes.c_double(), ctypes.c_double()
    o = np.empty(dv)
    _lib().oracle_state(_p(s) if n else _p(np.zeros(1)), _p(v), n, dv, ctypes.byref(m),
                        ctypes.byref(l), _p(o))
    return m.value, l.value, o


def merge(a, b):
    """a (+) b for states (m, l, o) (merge_states in attention_kernels.py)."""
    oa, ob = _f64(a[2]), _f64(b[2])
    dv = oa.size
    m, l = ctypes.c_double(), ctypes.c_double()
    o = np.empty(dv)
    _lib().oracle_merge(float(a[0]), float(a[1]), _p(oa), float(b[0]), float(b[1]), _p(ob), dv,
                        ctypes.byref(m), ctypes.byref(l), _p(o))
    return m.value, l.value, o


def split_decode(Q, K, V, n_split: int, scale: float, heads=None, nthreads: int | None = None):
    """Split-KV decoding (flash_decode in attention_kernels.py) with floor split
    bounds.  Returns (O, L, part_m, part_l, part_o) shaped [nh, Nq, ...] where nh
    is B*H or len(heads) (flat ids b*H + h)."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    _check4(Q, K, V)
    B, H, Nq, d = Q.shape
    Nk, dv = K.shape[2], V.shape[3]
    if heads is None:
        nh, hp = B * H, None
    else:
        heads = np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
        nh, hp = heads.size, heads.ctypes.data_as(_ip)
    n = int(n_split)
    O = np.empty((nh, Nq, dv))
    L = np.empty((nh, Nq))
    pm = np.empty((nh, Nq, max(n, 1)))
    pl = np.empty((nh, Nq, max(n, 1)))
    po = np.empty((nh, Nq, max(n, 1), dv))
    st = _lib().oracle_split_decode(_p(Q), _p(K), _p(V), _p(O), _p(L), _p(pm), _p(pl), _p(po), B,
                                    H, Nq, Nk, d, dv, n, float(scale), hp, nh,
                                    nthreads or default_threads())
    if st != 0:
        raise ValueError("n_split must be >= 1")
    return O, L, pm, pl, po
