"""bf16 matrix-core backward against the oracle.

The GPU backward consumes the GPU forward's O and L; the oracle backward
computes its own fp64 O and L from Q, K, V.  Error measure per tensor:
max |g - g_ref| / max |g_ref| <= 5e-2 for dQ, dK and dV.  Mid sizes are
compared on every element (several 128-key and 64-query tiles, ragged
tails), and so is the full workload (2 x 16 heads, 4096 tokens, d = 64,
causal), which is also checked on every head through two identities of the
exact gradient: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i."""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_inputs, workload_inputs
from tests.gpu_helpers import host, max_rel, say

pytestmark = pytest.mark.gpu
REL = 5e-2


@pytest.fixture(scope="module")
def fa():
    import flashattention_online_softmax_fa_amd as m
    return m


def _fwd_bwd(fa, x, scale, causal):
    o, lse = fa.forward(x.q, x.k, x.v, scale, causal)
    dq, dk, dv = fa.backward(x.q, x.k, x.v, o, lse, x.do, scale, causal)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [
    (1, 2, 200, 200, 64),
    (2, 1, 300, 300, 64),
    (1, 2, 333, 333, 128),
    (1, 1, 64, 64, 64),
    (1, 1, 1, 1, 64),
    (1, 2, 130, 77, 64),     # Nq != Nk
    (1, 1, 70, 260, 128),    # Nq < Nk
])
def test_full_compare(fa, shape, causal):
    B, H, Nq, Nk, d = shape
    x = make_inputs(B, H, Nq, Nk, d, "bf16", seed=sum(shape) + 2 * causal, device="cuda",
                    backward=True)
    scale = 1 / math.sqrt(d)
    say(f"bwd {shape} causal={causal}")
    dq, dk, dv = _fwd_bwd(fa, x, scale, causal)
    g = oracle.dense_bwd(host(x.q), host(x.k), host(x.v), host(x.do), scale, causal)
    assert max_rel(dq, g["dQ"]) <= REL, "dQ"
    assert max_rel(dk, g["dK"]) <= REL, "dK"
    assert max_rel(dv, g["dV"]) <= REL, "dV"


def test_hot_rows(fa):
    x = make_inputs(1, 2, 300, 300, 64, "bf16", seed=41, device="cuda", backward=True,
                    hot_row_factor=30.0)
    say("bwd hot rows")
    dq, dk, dv = _fwd_bwd(fa, x, 0.125, True)
    g = oracle.dense_bwd(host(x.q), host(x.k), host(x.v), host(x.do), 0.125, True)
    for got, key in ((dq, "dQ"), (dk, "dK"), (dv, "dV")):
        assert max_rel(got, g[key]) <= REL, key


def test_repeat_calls_bitwise_equal(fa):
    """No atomics: two calls on the same inputs give identical bits."""
    x = make_inputs(1, 2, 256, 256, 64, "bf16", seed=3, device="cuda", backward=True)
    say("bwd repeat")
    a = _fwd_bwd(fa, x, 0.125, True)
    b = _fwd_bwd(fa, x, 0.125, True)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def _identities(x, dk, dv):
    """On every head: sum_j dK_j = 0 (each row of dS sums to zero), with dK
    itself far from zero, and sum_j dV_j = sum_i dO_i (each row of P sums to
    one)."""
    dkf = dk.float()
    mag = dkf.abs().sum(2)
    assert (mag > 0).all() and float(mag.min()) > 1e-3 * float(mag.max()), "dK vanishes"
    assert (dkf.sum(2).abs() <= 2e-2 * mag + 1e-3).all(), "sum_j dK_j"
    sum_dv, sum_do = dv.float().sum(2), x.do.float().sum(2)
    assert ((sum_dv - sum_do).abs().max() / sum_do.abs().max()).item() <= 2e-2, "sum_j dV_j"


def test_full_workload(fa):
    """The causal backward workload (2 x 16 heads x 4096, d = 64; the XCD
    tile order of both passes) on every element of dQ, dK and dV."""
    say("bwd full workload: generating")
    x = workload_inputs("bwd_causal_d64", device="cuda")
    B, H, N, d = x.q.shape
    scale = 1 / math.sqrt(d)
    say("bwd full workload: running")
    dq, dk, dv = _fwd_bwd(fa, x, scale, True)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    _identities(x, dk, dv)
    say("bwd full workload: oracle on every head")
    g = oracle.dense_bwd(host(x.q), host(x.k), host(x.v), host(x.do), scale, True)
    for got, key in ((dq, "dQ"), (dk, "dK"), (dv, "dV")):
        assert max_rel(got, g[key]) <= REL, key
        # and per head, so that no head's error hides under another's scale
        ref = g[key].reshape(B * H, N, d)
        h = host(got).reshape(B * H, N, d)
        for bh in range(B * H):
            assert max_rel(h[bh], ref[bh]) <= REL, f"{key} head {bh}"


@pytest.mark.parametrize("d", [64, 128])
def test_long_sequence(fa, d):
    """Two heads of 32768 tokens, causal (up to 512 query tiles of 64 per key
    block at d = 64).  On every head the two identities that hold at any size;
    against the oracle, dQ on sampled query rows of both heads (each row needs
    only its own scores) and dK, dV on sampled key rows of the second head
    (each key needs L and D of every query that sees it: the oracle's forward
    of all 32768 rows of that head).  Max-rel per tensor over the rows drawn,
    relative to the largest reference value among them."""
    N = 32768
    say(f"bwd long sequence N={N} d={d}")
    x = make_inputs(1, 2, N, N, d, "bf16", seed=32 + d, device="cuda", backward=True)
    scale = 1 / math.sqrt(d)
    dq, dk, dv = _fwd_bwd(fa, x, scale, True)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    _identities(x, dk, dv)
    rng = np.random.default_rng(d)
    edge = [0, 1, 31, 32, 63, 64, 4095, 4096, N - 65, N - 64, N - 2, N - 1]
    qrows = np.unique(np.concatenate([[h * N + i for h in (0, 1) for i in edge],
                                      rng.integers(0, 2 * N, 40)])).astype(np.int64)
    krows = np.unique(np.concatenate([[N + j for j in edge],
                                      N + rng.integers(0, N, 40)])).astype(np.int64)
    Q, K, V, dO = (host(t) for t in (x.q, x.k, x.v, x.do))
    say(f"bwd long sequence d={d}: oracle on {qrows.size} query and {krows.size} key rows")
    r = oracle.bwd_rows(Q, K, V, dO, scale, True, query_rows=qrows, key_rows=krows)
    assert max_rel(host(dq).reshape(-1, d)[qrows], r["dQ"]) <= REL, "dQ"
    assert max_rel(host(dk).reshape(-1, d)[krows], r["dK"]) <= REL, "dK"
    assert max_rel(host(dv).reshape(-1, d)[krows], r["dV"]) <= REL, "dV"
