"""fp32 forward (vector-ALU kernel) against the oracle: the 64x64 d=16
workload with online-softmax steps of 1..16 keys, the hand anchor, uniform
scores, large logits and ragged shapes.  Tolerance: max-abs 1e-5 on O and L."""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_inputs
from tests.gpu_helpers import host, max_abs, say

pytestmark = pytest.mark.gpu
TOL = 1e-5


@pytest.fixture(scope="module")
def fa():
    import flashattention_online_softmax_fa_amd as m
    return m


def _dev(a):
    return torch.tensor(np.asarray(a), dtype=torch.float32, device="cuda")


@pytest.mark.parametrize("causal", [False, True])
def test_tiny_workload_block_sweep(fa, causal):
    x = make_inputs(1, 1, 64, 64, 16, "f32", seed=1, device="cuda")
    O_ref, L_ref = oracle.dense_fwd(host(x.q), host(x.k), host(x.v), 0.25, causal)
    for kv_block in list(range(1, 17)) + [None]:
        say(f"tiny f32 causal={causal} kv_block={kv_block}")
        o, lse = fa.forward(x.q, x.k, x.v, 0.25, causal, kv_block=kv_block)
        torch.cuda.synchronize()
        assert max_abs(o, O_ref) <= TOL, kv_block
        assert max_abs(lse, L_ref) <= TOL, kv_block


@pytest.mark.parametrize("causal", [False, True])
def test_anchor(fa, golden, causal):
    g = golden("anchor_n3_d2.txt")
    Q = np.array(g["Q"]).reshape(1, 1, 3, 2)
    K = np.array(g["K"]).reshape(1, 1, 3, 2)
    V = np.array(g["V"]).reshape(1, 1, 3, 2)
    say(f"anchor causal={causal}")
    o, lse = fa.forward(_dev(Q), _dev(K), _dev(V), scale=1.0, causal=causal, kv_block=2)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.dense_fwd(Q, K, V, 1.0, causal)
    assert max_abs(o, O_ref) <= TOL and max_abs(lse, L_ref) <= TOL
    if not causal:
        np.testing.assert_array_equal(np.round(host(o)[0, 0, 0], 3), g["O_row0_3dp"])


def test_uniform_scores(fa):
    """q = k = 0 make every score equal: O is the mean of V, L = ln 3."""
    v = np.array([[1.0, 0.25], [4.0, -2.0], [7.0, 0.5]]).reshape(1, 1, 3, 2)
    say("uniform scores")
    o, lse = fa.forward(_dev(np.zeros((1, 1, 1, 2))), _dev(np.zeros((1, 1, 3, 2))), _dev(v),
                        scale=1 / math.sqrt(2))
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(o).reshape(-1), [4.0, (0.25 - 2.0 + 0.5) / 3], atol=TOL)
    np.testing.assert_allclose(host(lse).reshape(-1), [math.log(3)], atol=TOL)


def test_large_logits(fa):
    """Q*100, K*100: scores reach ~1e4, where fp32 scores carry absolute error
    ~|s| * 2^-24 * d ~ 1e-2, so O is compared at 2e-2 and L relative 1e-6."""
    x = make_inputs(1, 1, 64, 64, 16, "f32", seed=1, device="cuda", q_scale=100.0,
                    k_scale=100.0)
    say("large logits")
    o, lse = fa.forward(x.q, x.k, x.v, 0.25, kv_block=2)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    O_ref, L_ref = oracle.dense_fwd(host(x.q), host(x.k), host(x.v), 0.25)
    assert max_abs(o, O_ref) <= 2e-2
    assert float(np.abs(host(lse) - L_ref).max() / np.abs(L_ref).max()) <= 1e-6


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 3, 37, 53, 24), (1, 2, 130, 70, 128), (1, 1, 1, 1, 1),
                                   (3, 1, 300, 300, 7)])
def test_ragged(fa, shape, causal):
    B, H, Nq, Nk, d = shape
    x = make_inputs(B, H, Nq, Nk, d, "f32", seed=sum(shape), device="cuda")
    scale = 1 / math.sqrt(d)
    say(f"f32 ragged {shape} causal={causal}")
    o, lse = fa.forward(x.q, x.k, x.v, scale, causal)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.dense_fwd(host(x.q), host(x.k), host(x.v), scale, causal)
    assert max_abs(o, O_ref) <= TOL and max_abs(lse, L_ref) <= TOL
