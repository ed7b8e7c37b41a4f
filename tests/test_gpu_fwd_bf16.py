"""bf16 matrix-core forward against the oracle.

Tolerances: O max-abs 2e-2 and L max-abs 1e-3 (bf16 inputs are exact in the
oracle; the GPU rounds P to bf16 before the PV product and O on output).
Mid sizes are compared on every element and span several 128-query and
64-key tiles with ragged tails; the full workloads (4 x 16 heads x 2048, d=64;
32 heads x 8192 causal, d=128, with one K row per head scaled by 30) are
compared on every element too, in the launch configuration the benchmark
times."""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_inputs, workload_inputs
from tests.gpu_helpers import head_block, host, max_abs, say

pytestmark = pytest.mark.gpu
O_TOL, L_TOL = 2e-2, 1e-3


@pytest.fixture(scope="module")
def fa():
    import flashattention_online_softmax_fa_amd as m
    return m


def _run(fa, x, scale, causal):
    o, lse = fa.forward(x.q, x.k, x.v, scale, causal)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [
    (1, 2, 200, 200, 64),
    (2, 2, 333, 333, 128),
    (1, 3, 129, 129, 128),
    (1, 1, 64, 64, 64),
    (1, 1, 1, 1, 64),
    (2, 1, 130, 77, 64),     # Nq != Nk
    (1, 2, 50, 300, 128),    # Nq < Nk
])
def test_full_compare(fa, shape, causal):
    B, H, Nq, Nk, d = shape
    x = make_inputs(B, H, Nq, Nk, d, "bf16", seed=sum(shape) + causal, device="cuda")
    scale = 1 / math.sqrt(d)
    say(f"bf16 fwd {shape} causal={causal}")
    o, lse = _run(fa, x, scale, causal)
    O_ref, L_ref = oracle.dense_fwd(host(x.q), host(x.k), host(x.v), scale, causal)
    assert max_abs(o, O_ref) <= O_TOL
    assert max_abs(lse, L_ref) <= L_TOL


@pytest.mark.parametrize("scale", [0.0, -0.1, 1.0])
def test_other_scales(fa, scale):
    """scale = 0 (every score equal: O is the mean of the visible V rows),
    a negative scale, and the unscaled case."""
    x = make_inputs(1, 2, 150, 150, 64, "bf16", seed=5, device="cuda")
    for causal in (False, True):
        say(f"bf16 fwd scale={scale} causal={causal}")
        o, lse = _run(fa, x, scale, causal)
        O_ref, L_ref = oracle.dense_fwd(host(x.q), host(x.k), host(x.v), scale, causal)
        assert max_abs(o, O_ref) <= O_TOL
        assert max_abs(lse, L_ref) <= L_TOL


def test_hot_rows_mid(fa):
    """One K row per head scaled by 30: the running maximum jumps mid-row."""
    x = make_inputs(1, 4, 700, 700, 128, "bf16", seed=8, device="cuda", hot_row_factor=30.0)
    for causal in (False, True):
        say(f"bf16 fwd hot rows causal={causal}")
        o, lse = _run(fa, x, 1 / math.sqrt(128), causal)
        O_ref, L_ref = oracle.dense_fwd(host(x.q), host(x.k), host(x.v), 1 / math.sqrt(128),
                                        causal)
        assert max_abs(o, O_ref) <= O_TOL
        assert max_abs(lse, L_ref) <= L_TOL


def test_uniform_scores_bf16(fa):
    """q = k = 0 (d = 64): O is the mean of the visible V rows, L = ln(count)."""
    B, H, N, d = 1, 1, 100, 64
    z = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    v = torch.arange(N, dtype=torch.float32, device="cuda").repeat_interleave(d).reshape(
        B, H, N, d).to(torch.bfloat16)
    say("bf16 uniform scores causal")
    o, lse = fa.forward(z, z, v, 0.125, causal=True)
    torch.cuda.synchronize()
    want = np.arange(N) / 2.0  # mean of 0..i
    np.testing.assert_allclose(host(o)[0, 0, :, 0], want, atol=O_TOL * 4, rtol=4e-3)
    np.testing.assert_allclose(host(lse)[0, 0], np.log(np.arange(1, N + 1)), atol=L_TOL)


def test_full_workload_prefill_d64(fa):
    """The non-causal d = 64 workload (4 x 16 heads x 2048, 256 workgroups of
    512 queries dealt to the XCDs by head range), every element of O and L."""
    say("bf16 fwd full workload prefill_d64: generating")
    x = workload_inputs("prefill_d64", device="cuda")
    B, H, Nq, d = x.q.shape
    scale = 1 / math.sqrt(d)
    say("bf16 fwd full workload prefill_d64: running")
    o, lse = _run(fa, x, scale, False)
    say("bf16 fwd full workload prefill_d64: oracle on every row")
    O_ref, L_ref = oracle.dense_fwd(host(x.q), host(x.k), host(x.v), scale, False)
    assert max_abs(o, O_ref) <= O_TOL
    assert max_abs(lse, L_ref) <= L_TOL


def test_full_workload_prefill_causal_d128(fa):
    """The causal d = 128 workload with one K row per head scaled by 30
    (32 heads x 8192, 1024 workgroups of 256 queries), every element of O and
    L, the oracle run over eight heads at a time."""
    say("bf16 fwd full workload prefill_causal_d128: generating")
    x = workload_inputs("prefill_causal_d128", device="cuda")
    B, H, Nq, d = x.q.shape
    scale = 1 / math.sqrt(d)
    say("bf16 fwd full workload prefill_causal_d128: running")
    o, lse = _run(fa, x, scale, True)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    for lo in range(0, B * H, 8):
        say(f"bf16 fwd full workload prefill_causal_d128: oracle on heads {lo}..{lo + 7}")
        Q, K, V = (head_block(t, lo, lo + 8) for t in (x.q, x.k, x.v))
        O_ref, L_ref = oracle.dense_fwd(Q, K, V, scale, True)
        assert max_abs(head_block(o, lo, lo + 8), O_ref) <= O_TOL, f"O, heads {lo}.."
        assert max_abs(head_block(lse[..., None], lo, lo + 8)[..., 0], L_ref) <= L_TOL, \
            f"L, heads {lo}.."


@pytest.mark.parametrize("causal", [False, True, "offset"])
@pytest.mark.parametrize("d", [64, 128])
def test_rising_scores(fa, d, causal):
    """Base-2 scores q.k * scale * log2(e) close to +j for key j in the even
    query rows and -j in the odd ones: from one 32-key tile to the next the
    maximum of an even row rises by 32, far past any reference maximum kept
    so far, while the odd rows in the same wavefront peak on their first key.
    The running maximum, the rescale of O and l, and the logsumexp (about 200
    in natural units) must all follow."""
    B, H, N = 1, 2, 300
    Nq, qs = (200, 90) if causal == "offset" else (N, 0)  # offset: row i at key qs + i
    x = make_inputs(B, H, Nq, N, d, "bf16", seed=77 + d + (causal is True), device="cpu")
    scale = 1 / math.sqrt(d)
    c = scale / math.log(2)
    q = x.q.float() * 0.1
    k = x.k.float() * 0.1
    q[..., 0] = torch.where(torch.arange(Nq) % 2 == 0, 1.0, -1.0)
    k[..., 0] = torch.arange(N, dtype=torch.float32) / c
    qb, kb = q.to(torch.bfloat16), k.to(torch.bfloat16)
    say(f"bf16 fwd rising scores d={d} causal={causal}")
    if causal == "offset":
        o, lse = fa.forward(qb.cuda(), kb.cuda(), x.v.cuda(), scale, q_start=qs)
    else:
        o, lse = fa.forward(qb.cuda(), kb.cuda(), x.v.cuda(), scale, causal)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.dense_fwd(host(qb), host(kb), host(x.v), scale, bool(causal), q_start=qs)
    assert float(np.abs(L_ref).max()) > 150  # the case really has large logits
    assert max_abs(o, O_ref) <= O_TOL
    assert max_abs(lse, L_ref) <= L_TOL


@pytest.mark.parametrize("causal", [False, True])
def test_rising_scores_long_d128(fa, causal):
    """The rising scores of test_rising_scores over 700 keys at d = 128, so
    that the raise happens inside the mask-free stretches (runs of 9 or more
    unmasked key tiles) that the d = 128 kernel steps through in groups of 8,
    under causal as well (every wave of the later query tiles)."""
    d, B, H, N = 128, 1, 2, 700
    x = make_inputs(B, H, N, N, d, "bf16", seed=91 + (causal is True), device="cpu")
    scale = 1 / math.sqrt(d)
    c = scale / math.log(2)
    q = x.q.float() * 0.1
    k = x.k.float() * 0.1
    q[..., 0] = torch.where(torch.arange(N) % 2 == 0, 1.0, -1.0)
    k[..., 0] = torch.arange(N, dtype=torch.float32) / c
    qb, kb = q.to(torch.bfloat16), k.to(torch.bfloat16)
    say(f"bf16 fwd rising scores over {N} keys d={d} causal={causal}")
    o, lse = fa.forward(qb.cuda(), kb.cuda(), x.v.cuda(), scale, causal)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.dense_fwd(host(qb), host(kb), host(x.v), scale, causal)
    assert float(np.abs(L_ref).max()) > 400
    assert max_abs(o, O_ref) <= O_TOL
    assert max_abs(lse, L_ref) <= L_TOL


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_long_sequence_sampled(fa, d, causal):
    """One head of 65536 queries and keys: 2048 key tiles per wave, the K/V
    ring wrapping around 128 (d = 64) or 256 (d = 128) times, and the last
    rows seeing every key.
    Sampled rows (the first, the last, and seeded ones) against the oracle."""
    N = 65536
    say(f"bf16 fwd long sequence N={N} d={d} causal={causal}")
    x = make_inputs(1, 1, N, N, d, "bf16", seed=65 + d + causal, device="cuda")
    scale = 1 / math.sqrt(d)
    o, lse = _run(fa, x, scale, causal)
    rng = np.random.default_rng(d + causal)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, N - 33, N - 2, N - 1],
                                     rng.integers(0, N, 40)])).astype(np.int64)
    O_ref, L_ref = oracle.dense_fwd(host(x.q), host(x.k), host(x.v), scale, causal, rows=rows)
    got_o = host(o).reshape(-1, d)[rows]
    got_l = host(lse).reshape(-1)[rows]
    assert float(np.abs(got_o - O_ref).max()) <= O_TOL
    assert float(np.abs(got_l - L_ref).max()) <= L_TOL
