"""Every element at mid sizes whose head count splits evenly over the eight
XCDs, so that the matrix-core launches take the XCD-remapped tile order (each
XCD a contiguous range of heads, their tiles dealt rank-major in groups):
the forward (d = 64 and 128, with and without the causal mask, and at a causal
offset) and the backward (both passes), against the oracle.  Tolerances as in
the other bf16 tests: O max-abs 2e-2, L max-abs 1e-3, gradients max-rel 5e-2
per tensor and per head."""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_inputs
from tests.gpu_helpers import host, max_abs, max_rel, say

pytestmark = pytest.mark.gpu
O_TOL, L_TOL, REL = 2e-2, 1e-3, 5e-2


@pytest.fixture(scope="module")
def fa():
    import flashattention_online_softmax_fa_amd as m
    return m


FWD_CASES = [
    # B, H, Nq, Nk, d, causal (False / True / q_start)
    (2, 8, 640, 640, 64, False),
    (2, 8, 640, 640, 64, True),
    (1, 16, 1100, 1100, 128, True),
    (1, 16, 1100, 1100, 128, False),
    (4, 2, 700, 700, 128, True),
    (2, 8, 300, 640, 64, 340),     # bottom-right: the queries are the last 300 keys
    (1, 16, 500, 1100, 128, 250),  # queries in the middle of the keys
]


@pytest.mark.parametrize("case", FWD_CASES)
def test_forward(fa, case):
    B, H, Nq, Nk, d, causal = case
    assert (B * H) % 8 == 0
    x = make_inputs(B, H, Nq, Nk, d, "bf16", seed=Nq + Nk + d + B * H, device="cuda")
    scale = 1 / math.sqrt(d)
    say(f"xcd fwd {case}")
    if causal is True or causal is False:
        o, lse = fa.forward(x.q, x.k, x.v, scale, causal)
        q_start, c = 0, causal
    else:
        o, lse = fa.forward(x.q, x.k, x.v, scale, q_start=causal)
        q_start, c = causal, True
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.dense_fwd(host(x.q), host(x.k), host(x.v), scale, c, q_start)
    assert max_abs(o, O_ref) <= O_TOL
    assert max_abs(lse, L_ref) <= L_TOL


BWD_CASES = [
    (2, 8, 640, 640, 64, True),
    (2, 8, 640, 640, 64, False),
    (1, 16, 1100, 1100, 128, True),
    (4, 2, 700, 700, 128, False),
    (2, 8, 300, 640, 64, 340),
]


@pytest.mark.parametrize("case", BWD_CASES)
def test_backward(fa, case):
    B, H, Nq, Nk, d, causal = case
    assert (B * H) % 8 == 0
    x = make_inputs(B, H, Nq, Nk, d, "bf16", seed=7 * Nq + Nk + d, device="cuda",
                    backward=True)
    scale = 1 / math.sqrt(d)
    say(f"xcd bwd {case}")
    if causal is True or causal is False:
        o, lse = fa.forward(x.q, x.k, x.v, scale, causal)
        dq, dk, dv = fa.backward(x.q, x.k, x.v, o, lse, x.do, scale, causal)
        q_start, c = 0, causal
    else:
        o, lse = fa.forward(x.q, x.k, x.v, scale, q_start=causal)
        dq, dk, dv = fa.backward(x.q, x.k, x.v, o, lse, x.do, scale, q_start=causal)
        q_start, c = causal, True
    torch.cuda.synchronize()
    g = oracle.dense_bwd(host(x.q), host(x.k), host(x.v), host(x.do), scale, c, q_start)
    for got, key in ((dq, "dQ"), (dk, "dK"), (dv, "dV")):
        h = host(got)
        assert max_rel(h, g[key]) <= REL, key
        n = g[key].shape[2]
        ref = g[key].reshape(B * H, n, d)
        for bh in range(B * H):
            if np.abs(ref[bh]).max() > 0:
                assert max_rel(h.reshape(B * H, n, d)[bh], ref[bh]) <= REL, f"{key} head {bh}"
