"""Causal attention with a query offset (fa_fwd_offset, fa_bwd_offset)
against the oracle: query row i sits at key position q_start + i.

Cases: bottom-right alignment (q_start = Nk - Nq, a chunk of new tokens at
the end of the keys), an offset in the middle of the keys (key tiles after
the last query's position are never visible; their dK, dV must be exactly
zero), q_start = 0 (must equal fa_fwd with causal = 1, bit for bit),
Nq > Nk with an offset, and an offset past the last key (every key visible:
the non-causal result).  Tolerances as the other parity tests: bf16 O
max-abs 2e-2, L 1e-3, gradients per-tensor max-rel 5e-2; fp32 1e-5."""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_inputs
from tests.gpu_helpers import host, max_abs, max_rel, say

pytestmark = pytest.mark.gpu
O_TOL, L_TOL, REL, F32_TOL = 2e-2, 1e-3, 5e-2, 1e-5


@pytest.fixture(scope="module")
def fa():
    import flashattention_online_softmax_fa_amd as m
    return m


CASES = [  # (B, H, Nq, Nk, d, q_start)
    (1, 2, 100, 300, 64, 200),     # bottom-right
    (2, 1, 77, 333, 128, 256),     # bottom-right, ragged
    (1, 2, 130, 400, 64, 70),      # middle: keys >= 200 invisible
    (1, 1, 96, 700, 128, 33),      # middle, most key tiles invisible
    (1, 2, 200, 150, 64, 10),      # Nq > Nk
    (1, 1, 50, 120, 64, 1000),     # past the last key: unmasked
    (1, 1, 1, 513, 128, 512),      # one new token at the end
]


@pytest.mark.parametrize("case", CASES)
def test_forward_bf16(fa, case):
    B, H, Nq, Nk, d, q_start = case
    x = make_inputs(B, H, Nq, Nk, d, "bf16", seed=sum(case), device="cuda")
    scale = 1 / math.sqrt(d)
    say(f"offset fwd bf16 {case}")
    o, lse = fa.forward(x.q, x.k, x.v, scale, q_start=q_start)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.dense_fwd(host(x.q), host(x.k), host(x.v), scale, causal=True,
                                    q_start=q_start)
    assert max_abs(o, O_ref) <= O_TOL
    assert max_abs(lse, L_ref) <= L_TOL


@pytest.mark.parametrize("case", [(1, 2, 40, 90, 16, 50), (1, 1, 33, 20, 128, 3),
                                  (2, 1, 5, 300, 64, 295)])
def test_forward_f32(fa, case):
    B, H, Nq, Nk, d, q_start = case
    x = make_inputs(B, H, Nq, Nk, d, "f32", seed=sum(case), device="cuda")
    say(f"offset fwd f32 {case}")
    o, lse = fa.forward(x.q, x.k, x.v, 0.3, q_start=q_start)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.dense_fwd(host(x.q), host(x.k), host(x.v), 0.3, causal=True,
                                    q_start=q_start)
    assert max_abs(o, O_ref) <= F32_TOL
    assert max_abs(lse, L_ref) <= F32_TOL


@pytest.mark.parametrize("d", [64, 128])
def test_zero_offset_is_causal(fa, d):
    x = make_inputs(1, 2, 260, 260, d, "bf16", seed=d, device="cuda", backward=True)
    scale = 1 / math.sqrt(d)
    say(f"offset 0 vs causal d={d}")
    o0, l0 = fa.forward(x.q, x.k, x.v, scale, causal=True)
    o1, l1 = fa.forward(x.q, x.k, x.v, scale, q_start=0)
    g0 = fa.backward(x.q, x.k, x.v, o0, l0, x.do, scale, causal=True)
    g1 = fa.backward(x.q, x.k, x.v, o1, l1, x.do, scale, q_start=0)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)


@pytest.mark.parametrize("case", CASES)
def test_backward(fa, case):
    B, H, Nq, Nk, d, q_start = case
    x = make_inputs(B, H, Nq, Nk, d, "bf16", seed=sum(case) + 1, device="cuda", backward=True)
    scale = 1 / math.sqrt(d)
    say(f"offset bwd {case}")
    o, lse = fa.forward(x.q, x.k, x.v, scale, q_start=q_start)
    dq, dk, dv = fa.backward(x.q, x.k, x.v, o, lse, x.do, scale, q_start=q_start)
    torch.cuda.synchronize()
    g = oracle.dense_bwd(host(x.q), host(x.k), host(x.v), host(x.do), scale, causal=True,
                         q_start=q_start)
    assert max_rel(dq, g["dQ"]) <= REL, "dQ"
    assert max_rel(dk, g["dK"]) <= REL, "dK"
    assert max_rel(dv, g["dV"]) <= REL, "dV"
    # keys after the last query's position: exactly zero
    last = q_start + Nq - 1
    if last + 1 < Nk:
        assert not torch.any(dk[:, :, last + 1:]) and not torch.any(dv[:, :, last + 1:])
