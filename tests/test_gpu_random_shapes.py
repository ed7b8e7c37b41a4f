"""Seeded random shapes through the bf16 forward and backward, against the
oracle on every element.

The shapes are drawn so that the kernels' block structure is crossed in
every way at once: query counts that leave whole wavefronts (and whole
workgroups of eight wavefronts) without rows, key counts that are not a
multiple of the 32-key tile nor of the groups of tiles one LDS barrier
publishes (4 at d = 64, 2 at d = 128), Nq != Nk, top-left causal, and the
causal mask at a query offset (query row i at key position q_start + i).
Tolerances as in the other bf16 tests: O max-abs 2e-2, L max-abs 1e-3,
gradients max-rel 5e-2 per tensor."""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_inputs
from tests.gpu_helpers import host, max_abs, max_rel, say

pytestmark = pytest.mark.gpu
O_TOL, L_TOL, REL = 2e-2, 1e-3, 5e-2


def _shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = 64 if i % 2 == 0 else 128
        Nq = int(rng.integers(1, 700))
        Nk = int(rng.integers(1, 700))
        mode = ("full", "causal", "offset")[i % 3]
        if mode == "causal":
            Nk = Nq  # top-left causal at equal lengths, as the workloads use it
        q_start = int(rng.integers(0, 400)) if mode == "offset" else None
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        out.append((B, H, Nq, Nk, d, mode, q_start))
    return out


SHAPES = _shapes(18, 2026)


@pytest.fixture(scope="module")
def fa():
    import flashattention_online_softmax_fa_amd as m
    return m


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}x{s[1]}x{s[2]}x{s[3]}d{s[4]}{s[5]}"
                                                for s in SHAPES])
def test_random_shape_fwd_bwd(fa, shape):
    B, H, Nq, Nk, d, mode, q_start = shape
    x = make_inputs(B, H, Nq, Nk, d, "bf16", seed=Nq * 1000 + Nk, device="cuda", backward=True)
    scale = 1 / math.sqrt(d)
    causal = mode != "full"
    qs = q_start if mode == "offset" else 0
    say(f"random shape fwd {shape}")
    if mode == "offset":
        o, lse = fa.forward(x.q, x.k, x.v, scale, q_start=q_start)
    else:
        o, lse = fa.forward(x.q, x.k, x.v, scale, causal)
    torch.cuda.synchronize()
    Q, K, V, dO = (host(t) for t in (x.q, x.k, x.v, x.do))
    O_ref, L_ref = oracle.dense_fwd(Q, K, V, scale, causal, q_start=qs)
    assert max_abs(o, O_ref) <= O_TOL
    assert max_abs(lse, L_ref) <= L_TOL

    say(f"random shape bwd {shape}")
    if mode == "offset":
        dq, dk, dv = fa.backward(x.q, x.k, x.v, o, lse, x.do, scale, q_start=q_start)
    else:
        dq, dk, dv = fa.backward(x.q, x.k, x.v, o, lse, x.do, scale, causal)
    torch.cuda.synchronize()
    g = oracle.dense_bwd(Q, K, V, dO, scale, causal, q_start=qs)
    for name, got in (("dQ", dq), ("dK", dk), ("dV", dv)):
        err = max_rel(got, g[name])
        assert err <= REL, f"{name} max-rel {err:.3e}"
