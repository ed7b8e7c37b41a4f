"""Event counters of the debug build libfa_stats.so (include/fa_stats.h).

Tiles computed and skipped are checked exactly against the page's tile loop
(flash_forward / flash_backward in attention_kernels.py: a key tile is
skipped under causal when it starts after the last query position of the
block), run on the host at the block shape the kernels report.  Rescales are
checked exactly where the page's count is known in closed form: zero when
every score is equal, and one per row and tile after the first when every
key tile raises each row's maximum by more than the kernels' threshold.
dQ is never added atomically, so that counter stays zero.  The outputs of
the counting build are also compared with the release build, bit for bit."""
import math

import numpy as np
import pytest
import torch

from fa_inputs import make_inputs
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    import flashattention_online_softmax_fa_amd as fa
    from flashattention_online_softmax_fa_amd import stats
    return fa, stats.load()


def page_fwd_counts(Nq, Nk, Br, Bc, causal, q_start):
    tiles = skipped = 0
    for i0 in range(0, Nq, Br):
        i1 = min(i0 + Br, Nq)
        for j0 in range(0, Nk, Bc):
            if causal and j0 > q_start + i1 - 1:
                skipped += 1
            else:
                tiles += 1
    return tiles, skipped


def page_bwd_kv_tiles(Nq, Nk, Bk, Bq, causal, q_start):
    """Key-major pass: (key block, query tile) pairs with a visible pair."""
    n = 0
    for j0 in range(0, Nk, Bk):
        for i0 in range(0, Nq, Bq):
            i1 = min(i0 + Bq, Nq)
            n += int(not causal or q_start + i1 - 1 >= j0)
    return n


@pytest.mark.parametrize("d,B,H,Nq,Nk,causal,q_start", [
    (64, 1, 2, 300, 300, True, 0),
    (64, 2, 1, 333, 333, False, 0),
    (128, 1, 2, 200, 450, True, 250),
    (128, 1, 1, 129, 700, True, 37),
    (64, 1, 1, 90, 64, True, 5),
])
def test_tile_counts(libs, d, B, H, Nq, Nk, causal, q_start):
    fa, st = libs
    x = make_inputs(B, H, Nq, Nk, d, "bf16", seed=Nq + Nk, device="cuda", backward=True)
    scale = 1 / math.sqrt(d)
    qs = q_start if causal else None
    say(f"stats d={d} {(B, H, Nq, Nk)} causal={causal} q_start={q_start}")
    st.reset()
    o, lse = st.forward(x.q, x.k, x.v, scale, causal, q_start=qs)
    dq, dk, dv = st.backward(x.q, x.k, x.v, o, lse, x.do, scale, causal, q_start=qs)
    got = st.read()
    # the counting build computes exactly what the release build computes
    o2, l2 = fa.forward(x.q, x.k, x.v, scale, causal, q_start=qs)
    g2 = fa.backward(x.q, x.k, x.v, o2, l2, x.do, scale, causal, q_start=qs)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)
    for a, b in zip((dq, dk, dv), g2):
        assert torch.equal(a, b)
    br, bc = st.tile(0, d, causal)
    tiles, skipped = page_fwd_counts(Nq, Nk, br, bc, causal, q_start)
    assert got["fwd_tiles"] == B * H * tiles
    assert got["fwd_skipped"] == B * H * skipped
    kr, kc = st.tile(1, d, causal)
    assert got["bwd_kv_tiles"] == B * H * page_bwd_kv_tiles(Nq, Nk, kr, kc, causal, q_start)
    qr, qc = st.tile(2, d, causal)
    q_tiles, _ = page_fwd_counts(Nq, Nk, qr, qc, causal, q_start)
    assert got["bwd_q_tiles"] == B * H * q_tiles
    assert got["dq_atomic_adds"] == 0


@pytest.mark.parametrize("d", [64, 128])
def test_rescales_closed_form(libs, d):
    fa, st = libs
    B, H, Nq, Nk = 1, 2, 100, 256
    br, bc = st.tile(0, d, False)
    scale = 0.125
    # every score equal: the maximum never grows after the first tile
    z = torch.zeros((B, H, Nq, d), dtype=torch.bfloat16, device="cuda")
    zk = torch.zeros((B, H, Nk, d), dtype=torch.bfloat16, device="cuda")
    v = make_inputs(B, H, Nq, Nk, d, "bf16", seed=d, device="cuda").v
    say(f"stats rescales uniform d={d}")
    st.reset()
    st.forward(z, zk, v, scale, False)
    assert st.read()["fwd_rescales"] == 0
    # s_ij = scale * a * j: each key tile raises every row's maximum by
    # scale * a * bc * log2(e) = 40 in base 2, more than the rescale margin (8)
    # and more than a mask-free step lets through (a probability sum above 2^24
    # in a lane's half row), so every tile after the first raises it
    a = 40.0 / (scale * bc * math.log2(math.e))
    q = torch.zeros((B, H, Nq, d), dtype=torch.float32, device="cuda")
    q[..., 0] = 1.0
    k = torch.zeros((B, H, Nk, d), dtype=torch.float32, device="cuda")
    k[..., 0] = a * torch.arange(Nk, dtype=torch.float32, device="cuda")
    kb = k.to(torch.bfloat16)
    # the bf16 rounding of k keeps the rise of the tile maxima above the threshold
    rise = (kb[0, 0, bc - 1::bc, 0].float()[1:] - kb[0, 0, bc - 1::bc, 0].float()[:-1]).min()
    assert float(rise) * scale * math.log2(math.e) > 28.5
    say(f"stats rescales monotone d={d}")
    st.reset()
    st.forward(q.to(torch.bfloat16), kb, v, scale, False)
    ntiles = -(-Nk // bc)
    assert st.read()["fwd_rescales"] == B * H * Nq * (ntiles - 1)
