"""Split-KV decoding and the state merge against the oracle.

O max-abs 2e-2 and L max-abs 1e-3 against the dense definition; per-split
states against the oracle's split summaries (m max-abs 1e-3; l and o rebased
to the oracle's m, max-rel 1e-2); the merge on random states against the
oracle's left fold.  Full-size decode (64 x 32 heads, 32768 keys, d = 128) is
checked on every head at every split count the benchmark uses."""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_inputs, workload_inputs, WORKLOADS
from tests.gpu_helpers import head_block, host, max_abs, max_rel, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import flashattention_online_softmax_fa_amd as m
    return m


def _check_states(pm, pl, po, rm, rl, ro):
    """Compare split states; l and o are rebased onto the oracle's m."""
    pm, pl, po = host(pm).reshape(rm.shape), host(pl).reshape(rl.shape), host(po).reshape(ro.shape)
    empty = np.isneginf(rm)
    assert np.array_equal(np.isneginf(pm), empty)
    assert np.all(pl[empty] == 0) and np.all(po[empty] == 0)
    full = ~empty
    assert np.abs(pm[full] - rm[full]).max() <= 1e-3
    w = np.exp(pm[full] - rm[full])
    assert max_rel(pl[full] * w, rl[full]) <= 1e-2
    assert max_rel(po[full] * w[:, None], ro[full]) <= 1e-2


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("n_split", [1, 7, 16, 64, 1003])
def test_decode_small(fa, d, n_split):
    B, H, Nq, Nk = 2, 3, 1, 1000
    x = make_inputs(B, H, Nq, Nk, d, "bf16", seed=31 + d + n_split, device="cuda")
    scale = 1 / math.sqrt(d)
    say(f"decode small d={d} n_split={n_split}")
    o, lse, (pm, pl, po) = fa.decode(x.q, x.k, x.v, n_split, scale)
    torch.cuda.synchronize()
    Q, K, V = host(x.q), host(x.k), host(x.v)
    O_ref, L_ref = oracle.dense_fwd(Q, K, V, scale)
    assert max_abs(o, O_ref) <= 2e-2
    assert max_abs(lse, L_ref) <= 1e-3
    _, _, rm, rl, ro = oracle.split_decode(Q, K, V, n_split, scale)
    _check_states(pm, pl, po, rm, rl, ro)


def test_decode_multi_query_rows(fa):
    B, H, Nq, Nk, d = 1, 2, 5, 777, 128
    x = make_inputs(B, H, Nq, Nk, d, "bf16", seed=77, device="cuda")
    say("decode Nq=5")
    o, lse, _ = fa.decode(x.q, x.k, x.v, 9, 0.09)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.dense_fwd(host(x.q), host(x.k), host(x.v), 0.09)
    assert max_abs(o, O_ref) <= 2e-2 and max_abs(lse, L_ref) <= 1e-3


def test_decode_one_key(fa):
    x = make_inputs(1, 1, 1, 1, 128, "bf16", seed=3, device="cuda")
    say("decode Nk=1")
    o, lse, _ = fa.decode(x.q, x.k, x.v, 4, 0.1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(o), host(x.v))
    s = 0.1 * float((host(x.q) * host(x.k)).sum())
    assert abs(float(host(lse).reshape(-1)[0]) - s) <= 1e-3


def test_merge_random_states(fa):
    """fa_merge_states on random states, including empty ones, against the
    oracle's left fold of merge."""
    rng = np.random.default_rng(9)
    B, H, Nq, n, d = 2, 2, 3, 6, 40
    m = rng.normal(size=(B, H, Nq, n)) * 3
    m[rng.random(m.shape) < 0.3] = -np.inf
    m[0, 0, 0, :] = -np.inf  # an all-empty row
    l = np.where(np.isneginf(m), 0.0, rng.random(m.shape) * 5 + 0.1)
    o = np.where(np.isneginf(m)[..., None], 0.0, rng.normal(size=(B, H, Nq, n, d)))
    # round to fp32 first so both sides see the same values
    m, l, o = (np.asarray(a, dtype=np.float32).astype(np.float64) for a in (m, l, o))
    t = lambda a: torch.tensor(a, dtype=torch.float32, device="cuda")
    out = torch.empty((B, H, Nq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    say("merge random states")
    fa.fa_merge_states(t(m), t(l), t(o), out, lse)
    torch.cuda.synchronize()
    got_o, got_l = host(out), host(lse)
    for idx in np.ndindex(B, H, Nq):
        acc = (m[idx][0], l[idx][0], o[idx][0])
        for s in range(1, n):
            acc = oracle.merge(acc, (m[idx][s], l[idx][s], o[idx][s]))
        if acc[1] == 0.0:
            assert np.all(np.isnan(got_o[idx])) and got_l[idx] == -np.inf
            continue
        np.testing.assert_allclose(got_o[idx], acc[2] / acc[1], rtol=1e-5, atol=1e-5)
        assert abs(got_l[idx] - (acc[0] + math.log(acc[1]))) <= 1e-5


@pytest.fixture(scope="module")
def decode_full(fa):
    """The decode workload (64 x 32 heads, one query, 32768 keys, d = 128) at
    every split count the benchmark uses: the GPU's O, L and split states on
    the host, and the oracle's, computed one batch index (32 heads, 0.5 GiB of
    bf16 K and V) at a time so that host memory stays bounded."""
    say("decode full: generating 64 x 32 x 32768 x 128 bf16 K/V")
    x = workload_inputs("decode_d128", device="cuda")
    B, H, _, d = x.q.shape
    scale = 1 / math.sqrt(d)
    splits = list(WORKLOADS["decode_d128"]["n_split"])
    got, ref = {}, {n: {"O": [], "L": [], "m": [], "l": [], "o": []} for n in splits}
    for n in splits:
        say(f"decode full: GPU at n_split={n}")
        o, lse, (pm, pl, po) = fa.decode(x.q, x.k, x.v, n, scale)
        torch.cuda.synchronize()
        got[n] = tuple(host(t) for t in (o, lse, pm, pl, po))
        del o, lse, pm, pl, po
    for b in range(B):
        if b % 8 == 0:
            say(f"decode full: oracle on batch index {b}..{b + 7}")
        Q, K, V = (head_block(t, b * H, (b + 1) * H) for t in (x.q, x.k, x.v))
        for n in splits:
            O_r, L_r, rm, rl, ro = oracle.split_decode(Q, K, V, n, scale)
            for key, val in zip(("O", "L", "m", "l", "o"), (O_r, L_r, rm, rl, ro)):
                ref[n][key].append(val)
        del Q, K, V
    del x
    torch.cuda.empty_cache()
    return got, {n: {k: np.concatenate(v) for k, v in r.items()} for n, r in ref.items()}


@pytest.mark.parametrize("n_split", list(WORKLOADS["decode_d128"]["n_split"]))
def test_decode_full_size(decode_full, n_split):
    """Every head of the decode workload: O and L against the split-and-merge
    oracle (equal to the definition), and every split state."""
    got, ref = decode_full
    o, lse, pm, pl, po = got[n_split]
    r = ref[n_split]
    BH = r["O"].shape[0]
    d = r["O"].shape[-1]
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert max_abs(o.reshape(BH, 1, d), r["O"]) <= 2e-2
    assert max_abs(lse.reshape(BH, 1), r["L"]) <= 1e-3
    _check_states(pm.reshape(BH, 1, n_split), pl.reshape(BH, 1, n_split),
                  po.reshape(BH, 1, n_split, d), r["m"], r["l"], r["o"])


@pytest.mark.parametrize("n_split", [16, 64, 1000])
def test_decode_long_cache(fa, n_split):
    """One query row against 2^20 - 5 cached keys (d = 128): long chunks per
    split, uneven split bounds (floor(Nk*s/n)), and the merge of many states."""
    Nk = (1 << 20) - 5
    say(f"decode long cache Nk={Nk} n_split={n_split}")
    x = make_inputs(1, 2, 1, Nk, 128, "bf16", seed=n_split, device="cuda")
    scale = 1 / math.sqrt(128)
    o, lse, _ = fa.decode(x.q, x.k, x.v, n_split, scale)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.dense_fwd(host(x.q), host(x.k), host(x.v), scale)
    assert max_abs(o, O_ref) <= 2e-2
    assert max_abs(lse, L_ref) <= 1e-3
