"""The fp32 backward and decoding paths, and decoding of several new tokens
with a causal offset, against the oracle.

fp32 (vector ALUs): gradients per-tensor max-rel 1e-5 against the oracle's
fp64 backward and against central finite differences of the oracle's fp64
forward (tiny inputs); decode states and merged O, L within 1e-5.
Causal decoding (fa_decode_split_offset, bf16 and fp32): row i of the Nq new
tokens sees keys 0 .. q_start + i.  The merged O, L are compared with the
oracle's dense forward at the same offset; every split state with the
oracle's state of the split's visible keys (an empty set gives
(-inf, 0, 0)).  bf16 tolerances as the other decode tests."""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_inputs
from tests.gpu_helpers import host, max_abs, max_rel, say

pytestmark = pytest.mark.gpu
TOL32 = 1e-5


@pytest.fixture(scope="module")
def fa():
    import flashattention_online_softmax_fa_amd as m
    return m


BWD_CASES = [  # (B, H, Nq, Nk, d, causal, q_start)
    (1, 2, 37, 53, 16, False, None),
    (1, 1, 70, 70, 64, True, None),
    (2, 1, 33, 90, 128, True, 57),
    (1, 1, 20, 20, 7, True, None),
    (1, 1, 64, 200, 33, True, 20),     # keys past the last position: zero gradient
]


@pytest.mark.parametrize("case", BWD_CASES)
def test_bwd_f32_vs_oracle(fa, case):
    B, H, Nq, Nk, d, causal, q_start = case
    x = make_inputs(B, H, Nq, Nk, d, "f32", seed=Nq + Nk + d, device="cuda", backward=True)
    scale = 1 / math.sqrt(d)
    say(f"bwd f32 {case}")
    o, lse = fa.forward(x.q, x.k, x.v, scale, causal, q_start=q_start)
    dq, dk, dv = fa.backward(x.q, x.k, x.v, o, lse, x.do, scale, causal, q_start=q_start)
    torch.cuda.synchronize()
    g = oracle.dense_bwd(host(x.q), host(x.k), host(x.v), host(x.do), scale,
                         causal=causal or q_start is not None, q_start=q_start or 0)
    assert max_rel(dq, g["dQ"]) <= TOL32, "dQ"
    assert max_rel(dk, g["dK"]) <= TOL32, "dK"
    assert max_rel(dv, g["dV"]) <= TOL32, "dV"


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_f32_vs_finite_differences(fa, causal):
    B, H, Nq, Nk, d = 1, 1, 4, 5, 3
    x = make_inputs(B, H, Nq, Nk, d, "f32", seed=7 + causal, device="cuda", backward=True)
    scale = 0.8
    say(f"bwd f32 finite differences causal={causal}")
    o, lse = fa.forward(x.q, x.k, x.v, scale, causal)
    dq, dk, dv = fa.backward(x.q, x.k, x.v, o, lse, x.do, scale, causal)
    torch.cuda.synchronize()
    gq, gk, gv = oracle.fd_grad(host(x.q), host(x.k), host(x.v), host(x.do), scale, causal)
    assert max_rel(dq, gq) <= TOL32
    assert max_rel(dk, gk) <= TOL32
    assert max_rel(dv, gv) <= TOL32


def _check_states_exact(pm, pl, po, rm, rl, ro, m_tol, rel):
    pm, pl, po = host(pm).reshape(rm.shape), host(pl).reshape(rl.shape), host(po).reshape(ro.shape)
    empty = np.isneginf(rm)
    assert np.array_equal(np.isneginf(pm), empty)
    assert np.all(pl[empty] == 0) and np.all(po[empty] == 0)
    full = ~empty
    assert np.abs(pm[full] - rm[full]).max() <= m_tol
    w = np.exp(pm[full] - rm[full])
    assert max_rel(pl[full] * w, rl[full]) <= rel
    assert max_rel(po[full] * w[:, None], ro[full]) <= rel


@pytest.mark.parametrize("n_split", [1, 7, 64, 600])
def test_decode_f32(fa, n_split):
    B, H, Nq, Nk, d = 2, 2, 3, 500, 64
    x = make_inputs(B, H, Nq, Nk, d, "f32", seed=n_split, device="cuda")
    scale = 1 / math.sqrt(d)
    say(f"decode f32 n_split={n_split}")
    o, lse, (pm, pl, po) = fa.decode(x.q, x.k, x.v, n_split, scale)
    torch.cuda.synchronize()
    Q, K, V = host(x.q), host(x.k), host(x.v)
    O_ref, L_ref, rm, rl, ro = oracle.split_decode(Q, K, V, n_split, scale)
    assert max_abs(o, O_ref.reshape(B, H, Nq, d)) <= TOL32
    assert max_abs(lse, L_ref.reshape(B, H, Nq)) <= TOL32
    _check_states_exact(pm, pl, po, rm, rl, ro, TOL32, TOL32)


def _causal_split_states(Q, K, V, n_split, scale, q_start):
    """Oracle states of each split's visible keys: [B*H, Nq, n] and [.., d]."""
    B, H, Nq, d = Q.shape
    Nk = K.shape[2]
    rm = np.empty((B * H, Nq, n_split))
    rl = np.empty_like(rm)
    ro = np.empty((B * H, Nq, n_split, d))
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                s_all = scale * (K[b, h] @ Q[b, h, i])
                last = min(Nk, q_start + i + 1)
                for s in range(n_split):
                    j0, j1 = Nk * s // n_split, min(Nk * (s + 1) // n_split, last)
                    j1 = max(j0, j1)
                    m, l, o = oracle.state(s_all[j0:j1], V[b, h, j0:j1])
                    rm[b * H + h, i, s], rl[b * H + h, i, s] = m, l
                    ro[b * H + h, i, s] = o
    return rm, rl, ro


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("d,Nk,Nq,q_start,n_split", [
    (128, 300, 6, 294, 5),      # the last 6 keys are the new tokens
    (64, 300, 6, 294, 64),
    (128, 257, 4, 100, 7),      # keys after each row's position are invisible
    (64, 90, 3, 10, 30),        # many splits empty for every row
])
def test_decode_causal_offset(fa, dt, d, Nk, Nq, q_start, n_split):
    B, H = 1, 2
    x = make_inputs(B, H, Nq, Nk, d, dt, seed=Nk + q_start + d, device="cuda")
    scale = 1 / math.sqrt(d)
    say(f"decode causal {dt} d={d} Nk={Nk} Nq={Nq} q_start={q_start} n_split={n_split}")
    o, lse, (pm, pl, po) = fa.decode(x.q, x.k, x.v, n_split, scale, q_start=q_start)
    torch.cuda.synchronize()
    Q, K, V = host(x.q), host(x.k), host(x.v)
    O_ref, L_ref = oracle.dense_fwd(Q, K, V, scale, causal=True, q_start=q_start)
    o_tol, l_tol = (TOL32, TOL32) if dt == "f32" else (2e-2, 1e-3)
    assert max_abs(o, O_ref) <= o_tol
    assert max_abs(lse, L_ref) <= l_tol
    rm, rl, ro = _causal_split_states(Q, K, V, n_split, scale, q_start)
    if dt == "f32":
        _check_states_exact(pm, pl, po, rm, rl, ro, TOL32, TOL32)
    else:
        _check_states_exact(pm, pl, po, rm, rl, ro, 1e-3, 1e-2)
