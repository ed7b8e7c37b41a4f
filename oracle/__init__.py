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
                                          _i64, ctypes.c_double, ctypes.c_int, _i64, _i64,
                                          ctypes.c_int]
        lib.oracle_dense_bwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _i64,
                                         _i64, _i64, _i64, _i64, _i64, ctypes.c_double,
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
                  "oracle_split_decode"):
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
               nthreads: int | None = None):
    """Per-row online softmax over key blocks of ``block`` (tiled in lab.py;
    TiledAttention in model.py; flash_forward in attention_kernels.py).
    Returns (O, L) like dense_fwd."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    _check4(Q, K, V)
    B, H, Nq, d = Q.shape
    Nk, dv = K.shape[2], V.shape[3]
    O = np.empty((B, H, Nq, dv))
    L = np.empty((B, H, Nq))
    st = _lib().oracle_online_fwd(_p(Q), _p(K), _p(V), _p(O), _p(L), B, H, Nq, Nk, d, dv,
                                  float(scale), int(bool(causal)), int(q_start), int(block),
                                  nthreads or default_threads())
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


def fd_grad(Q, K, V, dO, scale: float, causal: bool = False, h: float = 1e-5):
    """Central differences of f = sum(dense_fwd(Q, K, V) * dO) with step h, one
    element at a time (finite_difference in lab.py).  Tiny inputs only."""
    Q, K, V, dO = (np.array(x, dtype=np.float64, copy=True) for x in (Q, K, V, dO))
    grads = []
    for arr in (Q, K, V):
        g = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            plus = float(np.sum(dense_fwd(Q, K, V, scale, causal, nthreads=1)[0] * dO))
            arr[idx] = old - h
            minus = float(np.sum(dense_fwd(Q, K, V, scale, causal, nthreads=1)[0] * dO))
            arr[idx] = old
            g[idx] = (plus - minus) / (2.0 * h)
        grads.append(g)
    return tuple(grads)


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
