"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

None of these compares the oracle with itself: each check is a printed value,
a closed form, a library routine for a special case, an invariant, finite
differences, or brute force on a tiny input.  The planted-mistake tests at the
end rebuild the oracle with one step broken and show that a pin fails.
"""
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_inputs, to_f64_numpy

E = math.e


def _anchor(golden):
    g = golden("anchor_n3_d2.txt")
    Q = np.array(g["Q"]).reshape(1, 1, 3, 2)
    K = np.array(g["K"]).reshape(1, 1, 3, 2)
    V = np.array(g["V"]).reshape(1, 1, 3, 2)
    return Q, K, V, np.array(g["O_row0_3dp"])


def _rand(shape, seed):
    return np.random.default_rng(seed).normal(size=shape)


# ---------------------------------------------------------------------------
# R1, the definition
# ---------------------------------------------------------------------------
def test_anchor_printed_row(golden):
    """flash_attention_numpy.py prints the first anchor row to 3 decimals."""
    Q, K, V, row0 = _anchor(golden)
    O, _ = oracle.dense_fwd(Q, K, V, scale=1.0)
    np.testing.assert_array_equal(np.round(O[0, 0, 0], 3), row0)


def test_anchor_closed_form(golden):
    """Scores [[1,0,2],[2,2,0],[2,1,2]]; every row worked out by hand."""
    Q, K, V, _ = _anchor(golden)
    O, L = oracle.dense_fwd(Q, K, V, scale=1.0)
    z0 = 1 + E + E * E
    want_O = np.array([
        [(E + E * E) / z0, (1 + E * E) / z0],
        [(E * E + 1) / (2 * E * E + 1)] * 2,
        [2 * E / (2 * E + 1), (1 + E) / (2 * E + 1)],
    ])
    want_L = np.array([math.log(z0), math.log(2 * E * E + 1), 1 + math.log(2 * E + 1)])
    np.testing.assert_allclose(O[0, 0], want_O, atol=1e-12, rtol=0)
    np.testing.assert_allclose(L[0, 0], want_L, atol=1e-12, rtol=0)
    # the same, digits written out
    np.testing.assert_allclose(O[0, 0, 0], [0.909969426830, 0.755271528945], atol=1e-11)
    np.testing.assert_allclose(L[0, 0], [2.407605964444, 2.758623675680, 2.861994804058],
                               atol=1e-11)


def test_anchor_causal(golden):
    """Top-left causal: row 0 sees key 0 only, row 1 two equal scores."""
    Q, K, V, _ = _anchor(golden)
    O, L = oracle.dense_fwd(Q, K, V, scale=1.0, causal=True)
    On, Ln = oracle.dense_fwd(Q, K, V, scale=1.0, causal=False)
    np.testing.assert_allclose(O[0, 0, 0], [1.0, 0.0], atol=1e-15)
    np.testing.assert_allclose(L[0, 0, 0], 1.0, atol=1e-15)
    np.testing.assert_allclose(O[0, 0, 1], [0.5, 0.5], atol=1e-15)
    np.testing.assert_allclose(L[0, 0, 1], 2 + math.log(2), atol=1e-14)
    np.testing.assert_allclose(O[0, 0, 2], On[0, 0, 2], atol=1e-15)
    np.testing.assert_allclose(L[0, 0, 2], Ln[0, 0, 2], atol=1e-15)


def test_anchor_scaled_differs(golden):
    """At scale 1/sqrt(2) the anchor's first row is [0.860, 0.716] (not the
    printed one): the pages' anchor is unscaled."""
    Q, K, V, row0 = _anchor(golden)
    O, _ = oracle.dense_fwd(Q, K, V, scale=1 / math.sqrt(2))
    np.testing.assert_array_equal(np.round(O[0, 0, 0], 3), [0.860, 0.716])
    assert not np.allclose(np.round(O[0, 0, 0], 3), row0)


def test_uniform_scores(golden):
    """Equal scores average the values (lab.py); L = ln 3 by hand."""
    g = golden("uniform_scores.txt")
    q = np.array(g["q"]).reshape(1, 1, 1, 2)
    k = np.array(g["k"]).reshape(1, 1, 3, 2)
    v = np.array(g["v"]).reshape(1, 1, 3, 1)
    for fn in (lambda: oracle.dense_fwd(q, k, v, 1 / math.sqrt(2)),
               lambda: oracle.online_fwd(q, k, v, 1 / math.sqrt(2), block=2)):
        O, L = fn()
        np.testing.assert_allclose(O.reshape(-1), g["O"], atol=1e-15)
        np.testing.assert_allclose(L.reshape(-1), [math.log(3)], atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 64, 64, 16), (2, 3, 37, 53, 24)])
def test_dense_vs_torch_softmax(shape, causal):
    """Library special case: torch fp64 softmax / logsumexp of the masked scores."""
    B, H, Nq, Nk, d = shape
    Q, K, V = _rand((B, H, Nq, d), 1), _rand((B, H, Nk, d), 2), _rand((B, H, Nk, d), 3)
    scale = 1 / math.sqrt(d)
    O, L = oracle.dense_fwd(Q, K, V, scale, causal)
    S = torch.from_numpy(Q) @ torch.from_numpy(K).transpose(-1, -2) * scale
    if causal:
        mask = torch.arange(Nk)[None, :] > torch.arange(Nq)[:, None]
        S = S.masked_fill(mask, float("-inf"))
    P = torch.softmax(S, dim=-1)
    np.testing.assert_allclose(O, (P @ torch.from_numpy(V)).numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(L, torch.logsumexp(S, dim=-1).numpy(), atol=1e-12, rtol=0)


def test_dense_brute_force_tiny():
    """Brute force with Python floats on a 2x3 case with causal offset."""
    Q, K, V = _rand((1, 1, 2, 2), 5), _rand((1, 1, 3, 2), 6), _rand((1, 1, 3, 2), 7)
    scale = 0.7
    for q_start in (0, 1):
        O, L = oracle.dense_fwd(Q, K, V, scale, causal=True, q_start=q_start)
        for i in range(2):
            vis = [j for j in range(3) if j <= q_start + i]
            s = [scale * sum(Q[0, 0, i, c] * K[0, 0, j, c] for c in range(2)) for j in vis]
            w = [math.exp(x) for x in s]
            z = sum(w)
            o = [sum(w[t] * V[0, 0, j, c] for t, j in enumerate(vis)) / z for c in range(2)]
            assert abs(L[0, 0, i] - math.log(z)) < 1e-14
            np.testing.assert_allclose(O[0, 0, i], o, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_dense_invariants(causal):
    """O_i lies in the box of the visible V rows; max s <= L <= max s + ln|vis|."""
    B, H, N, d = 2, 2, 40, 8
    Q, K, V = _rand((B, H, N, d), 11), _rand((B, H, N, d), 12), _rand((B, H, N, d), 13)
    scale = 0.35
    O, L = oracle.dense_fwd(Q, K, V, scale, causal)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                nv = i + 1 if causal else N
                s = scale * K[b, h, :nv] @ Q[b, h, i]
                assert s.max() - 1e-12 <= L[b, h, i] <= s.max() + math.log(nv) + 1e-12
                assert np.all(O[b, h, i] >= V[b, h, :nv].min(0) - 1e-12)
                assert np.all(O[b, h, i] <= V[b, h, :nv].max(0) + 1e-12)


def test_online_rows_subset():
    """The online routine on listed rows returns exactly those rows of the
    whole computation, in list order."""
    Q, K, V = (_rand((2, 3, 21, 5), 60 + t) for t in range(3))
    O, L = oracle.online_fwd(Q, K, V, 0.4, True, block=4)
    rows = np.array([17, 0, 125, 64, 3])
    Or, Lr = oracle.online_fwd(Q, K, V, 0.4, True, block=4, rows=rows)
    np.testing.assert_array_equal(Or, O.reshape(-1, 5)[rows])
    np.testing.assert_array_equal(Lr, L.reshape(-1)[rows])


def test_dense_rows_subset():
    """The row-sampled entry returns exactly the full rows it names."""
    Q, K, V = _rand((2, 3, 20, 8), 21), _rand((2, 3, 25, 8), 22), _rand((2, 3, 25, 8), 23)
    O, L = oracle.dense_fwd(Q, K, V, 0.3, causal=True)
    rows = np.array([0, 19, 20, 77, 119])
    Os, Ls = oracle.dense_fwd(Q, K, V, 0.3, causal=True, rows=rows)
    np.testing.assert_array_equal(Os, O.reshape(-1, 8)[rows])
    np.testing.assert_array_equal(Ls, L.reshape(-1)[rows])


# ---------------------------------------------------------------------------
# R2, the online recurrence
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_online_block_sweep_tiny_workload(causal):
    """Block sizes 1..16 on the 64x64, d=16 fp32 workload equal the definition."""
    x = make_inputs(1, 1, 64, 64, 16, "f32", seed=1)
    Q, K, V = (to_f64_numpy(t) for t in (x.q, x.k, x.v))
    O, L = oracle.dense_fwd(Q, K, V, 0.25, causal)
    for block in range(1, 17):
        Ob, Lb = oracle.online_fwd(Q, K, V, 0.25, causal, block=block)
        np.testing.assert_allclose(Ob, O, atol=1e-12, rtol=1e-12)
        np.testing.assert_allclose(Lb, L, atol=1e-12, rtol=1e-12)


def test_online_model_py_lengths():
    """model.py's sweep: lengths 5 and 6, d = 4, blocks 1, 2, 3, 4, 8 (uneven tails)."""
    for n in (5, 6):
        Q, K, V = _rand((1, 1, n, 4), 40 + n), _rand((1, 1, n, 4), 50 + n), _rand((1, 1, n, 4), 60 + n)
        O, L = oracle.dense_fwd(Q, K, V, 0.5)
        for block in (1, 2, 3, 4, 8):
            Ob, Lb = oracle.online_fwd(Q, K, V, 0.5, block=block)
            np.testing.assert_allclose(Ob, O, atol=1e-12, rtol=1e-12)
            np.testing.assert_allclose(Lb, L, atol=1e-12, rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_online_lab_py_case(causal):
    """lab.py's default: N = 7, d = 3, block 3."""
    Q, K, V = _rand((1, 1, 7, 3), 7), _rand((1, 1, 7, 3), 8), _rand((1, 1, 7, 3), 9)
    O, L = oracle.dense_fwd(Q, K, V, 1 / math.sqrt(3), causal)
    Ob, Lb = oracle.online_fwd(Q, K, V, 1 / math.sqrt(3), causal, block=3)
    np.testing.assert_allclose(Ob, O, atol=1e-12, rtol=1e-12)
    np.testing.assert_allclose(Lb, L, atol=1e-12, rtol=1e-12)


def test_online_large_logits():
    """Q*100 and K*100 (logits grow 1e4 times): finite and equal to the definition."""
    Q, K, V = _rand((1, 1, 6, 4), 70), _rand((1, 1, 6, 4), 71), _rand((1, 1, 6, 4), 72)
    O, L = oracle.dense_fwd(Q * 100, K * 100, V, 0.5)
    Ob, Lb = oracle.online_fwd(Q * 100, K * 100, V, 0.5, block=2)
    assert np.all(np.isfinite(Ob)) and np.all(np.isfinite(Lb))
    np.testing.assert_allclose(Ob, O, atol=1e-10, rtol=1e-10)
    # with |s| ~ 1e4 the row is one-hot on its argmax (no ties in random data)
    S = 0.5 * (Q * 100)[0, 0] @ (K * 100)[0, 0].T
    np.testing.assert_allclose(Ob[0, 0], V[0, 0][S.argmax(1)], atol=1e-10)


def test_online_fire_test():
    """flash_attention_numpy.py's fire test: Q ~ N(100, 1), K ~ N(0, 1)/8, 64x8,
    scale 1, tiles of 16."""
    rng = np.random.default_rng(0)
    Q = rng.normal(100, 1, (1, 1, 64, 8))
    K = rng.normal(0, 1, (1, 1, 64, 8)) / 8
    V = rng.normal(0, 1, (1, 1, 64, 8))
    O, L = oracle.dense_fwd(Q, K, V, 1.0)
    Ob, Lb = oracle.online_fwd(Q, K, V, 1.0, block=16)
    np.testing.assert_allclose(Ob, O, atol=1e-10)
    np.testing.assert_allclose(Lb, L, atol=1e-10)


def test_online_gpt2_shape_uneven():
    """flash_attention_numpy.py's N = 1024, d = 64 case with 390-key blocks."""
    rng = np.random.default_rng(3)
    Q, K, V = (rng.normal(0, 1, (1, 1, 1024, 64)) for _ in range(3))
    O, L = oracle.dense_fwd(Q, K, V, 1.0)
    Ob, Lb = oracle.online_fwd(Q, K, V, 1.0, block=390)
    np.testing.assert_allclose(Ob, O, atol=1e-9)
    np.testing.assert_allclose(Lb, L, atol=1e-9)


# ---------------------------------------------------------------------------
# R3, the backward
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_vs_finite_differences_lab(causal):
    """lab.py: N = 7, d = 3, central differences with h = 1e-5."""
    rng = np.random.default_rng(7)
    Q, K, V, dO = (rng.normal(size=(1, 1, 7, 3)) for _ in range(4))
    scale = 1 / math.sqrt(3)
    g = oracle.dense_bwd(Q, K, V, dO, scale, causal)
    fd = oracle.fd_grad(Q, K, V, dO, scale, causal)
    for a, b in zip((g["dQ"], g["dK"], g["dV"]), fd):
        np.testing.assert_allclose(a, b, atol=2e-8, rtol=2e-6)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_vs_finite_differences_rect(causal):
    """Nq != Nk, two heads, d = 4, causal offset 2."""
    Q, K, V, dO = _rand((1, 2, 5, 4), 80), _rand((1, 2, 8, 4), 81), _rand((1, 2, 8, 4), 82), \
        _rand((1, 2, 5, 4), 83)
    g = oracle.dense_bwd(Q, K, V, dO, 0.5, causal)
    fd = oracle.fd_grad(Q, K, V, dO, 0.5, causal)
    for a, b in zip((g["dQ"], g["dK"], g["dV"]), fd):
        np.testing.assert_allclose(a, b, atol=2e-8, rtol=2e-6)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_vs_torch_autograd(causal):
    """Library special case: torch fp64 autograd of the dense definition."""
    B, H, N, d = 1, 2, 24, 8
    Q, K, V, dO = (_rand((B, H, N, d), 90 + t) for t in range(4))
    scale = 1 / math.sqrt(d)
    g = oracle.dense_bwd(Q, K, V, dO, scale, causal)
    q, k, v = (torch.from_numpy(x).requires_grad_() for x in (Q, K, V))
    S = q @ k.transpose(-1, -2) * scale
    if causal:
        S = S.masked_fill(torch.arange(N)[None, :] > torch.arange(N)[:, None], float("-inf"))
    O = torch.softmax(S, -1) @ v
    gq, gk, gv = torch.autograd.grad((O * torch.from_numpy(dO)).sum(), (q, k, v))
    np.testing.assert_allclose(g["dQ"], gq.numpy(), atol=1e-11, rtol=1e-11)
    np.testing.assert_allclose(g["dK"], gk.numpy(), atol=1e-11, rtol=1e-11)
    np.testing.assert_allclose(g["dV"], gv.numpy(), atol=1e-11, rtol=1e-11)
    np.testing.assert_allclose(g["O"], O.detach().numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_invariants(causal):
    """Rows of dS sum to zero, so sum_j dK_j = 0; and sum_j dV_j = sum_i dO_i.
    D_i = sum_c dO_ic O_ic (flash_backward's D)."""
    Q, K, V, dO = (_rand((2, 2, 33, 8), 100 + t) for t in range(4))
    g = oracle.dense_bwd(Q, K, V, dO, 0.4, causal)
    np.testing.assert_allclose(g["dK"].sum(2), 0.0, atol=1e-12)
    np.testing.assert_allclose(g["dV"].sum(2), dO.sum(2), atol=1e-12)
    np.testing.assert_allclose(g["D"], (dO * g["O"]).sum(-1), atol=1e-13)


def _torch_grads(Q, K, V, dO, scale, causal, q_start=0):
    """torch fp64 autograd of the dense definition (a library special case)."""
    q, k, v = (torch.from_numpy(x).requires_grad_() for x in (Q, K, V))
    S = q @ k.transpose(-1, -2) * scale
    if causal:
        Nq, Nk = Q.shape[2], K.shape[2]
        hidden = torch.arange(Nk)[None, :] > (q_start + torch.arange(Nq))[:, None]
        S = S.masked_fill(hidden, float("-inf"))
    O = torch.softmax(S, -1) @ v
    L = torch.logsumexp(S, -1)
    gq, gk, gv = torch.autograd.grad((O * torch.from_numpy(dO)).sum(), (q, k, v))
    return gq.numpy(), gk.numpy(), gv.numpy(), O.detach().numpy(), L.detach().numpy()


@pytest.mark.parametrize("causal,q_start,Nq,Nk", [(False, 0, 11, 11), (True, 0, 11, 11),
                                                  (True, 4, 7, 13), (False, 0, 5, 9),
                                                  (True, 20, 6, 10)])
def test_bwd_rows_vs_torch_autograd(causal, q_start, Nq, Nk):
    """The row-restricted backward on every query row and every key row equals
    torch fp64 autograd (dQ, dK, dV) and torch's softmax and logsumexp (O, L),
    causal at several offsets and with Nq != Nk; rows are asked for in a
    shuffled order and come back in that order."""
    B, H, d = 2, 2, 5
    Q, dO = _rand((B, H, Nq, d), 200), _rand((B, H, Nq, d), 201)
    K, V = _rand((B, H, Nk, d), 202), _rand((B, H, Nk, d), 203)
    scale = 0.45
    gq, gk, gv, O, L = _torch_grads(Q, K, V, dO, scale, causal, q_start)
    rng = np.random.default_rng(5)
    qrows = rng.permutation(B * H * Nq)
    krows = rng.permutation(B * H * Nk)
    r = oracle.bwd_rows(Q, K, V, dO, scale, causal, q_start, query_rows=qrows, key_rows=krows)
    np.testing.assert_allclose(r["dQ"], gq.reshape(-1, d)[qrows], atol=1e-12, rtol=1e-11)
    np.testing.assert_allclose(r["O"], O.reshape(-1, d)[qrows], atol=1e-13)
    np.testing.assert_allclose(r["L"], L.reshape(-1)[qrows], atol=1e-13)
    np.testing.assert_allclose(r["D"], (dO * O).sum(-1).reshape(-1)[qrows], atol=1e-12)
    np.testing.assert_allclose(r["dK"], gk.reshape(-1, d)[krows], atol=1e-12, rtol=1e-11)
    np.testing.assert_allclose(r["dV"], gv.reshape(-1, d)[krows], atol=1e-12, rtol=1e-11)


def test_bwd_rows_key_subset_of_one_head():
    """Key rows of one head only: L and D are needed for that head alone."""
    Q, K, V, dO = (_rand((1, 3, 16, 4), 210 + t) for t in range(4))
    gq, gk, gv, _, _ = _torch_grads(Q, K, V, dO, 0.5, True)
    keys = np.array([2 * 16 + 15, 2 * 16 + 0, 2 * 16 + 7])
    r = oracle.bwd_rows(Q, K, V, dO, 0.5, True, key_rows=keys)
    np.testing.assert_allclose(r["dK"], gk.reshape(-1, 4)[keys], atol=1e-12, rtol=1e-11)
    np.testing.assert_allclose(r["dV"], gv.reshape(-1, 4)[keys], atol=1e-12, rtol=1e-11)


def test_bwd_heads_subset():
    Q, K, V, dO = (_rand((2, 3, 9, 4), 110 + t) for t in range(4))
    g = oracle.dense_bwd(Q, K, V, dO, 0.5, True)
    gs = oracle.dense_bwd(Q, K, V, dO, 0.5, True, heads=[4, 1])
    for key in ("dQ", "dK", "dV", "O", "L"):
        full = g[key].reshape((6,) + g[key].shape[2:])
        np.testing.assert_array_equal(gs[key], full[[4, 1]])


# ---------------------------------------------------------------------------
# R5 states and merge, R6 split decoding
# ---------------------------------------------------------------------------
def _random_state(rng, dv, empty=False):
    if empty:
        return (-math.inf, 0.0, np.zeros(dv))
    n = int(rng.integers(1, 6))
    return oracle.state(rng.normal(size=n) * 3, rng.normal(size=(n, dv)))


def test_state_brute_force():
    s = np.array([0.5, -1.0, 2.0])
    v = np.array([[1.0, 2.0], [3.0, -1.0], [0.0, 4.0]])
    m, l, o = oracle.state(s, v)
    assert m == 2.0
    w = np.exp(s - 2.0)
    assert abs(l - w.sum()) < 1e-15
    np.testing.assert_allclose(o, w @ v, atol=1e-15)
    m0, l0, o0 = oracle.state(np.zeros(0), np.zeros((0, 2)))
    assert m0 == -math.inf and l0 == 0.0 and np.all(o0 == 0.0)


def test_merge_algebra():
    """Associative, commutative, identity (-inf, 0, 0); empty + empty is empty,
    never NaN (merge_states in attention_kernels.py)."""
    rng = np.random.default_rng(5)
    dv = 3
    for trial in range(200):
        a, b, c = (_random_state(rng, dv, empty=(rng.random() < 0.2)) for _ in range(3))
        ab_c = oracle.merge(oracle.merge(a, b), c)
        a_bc = oracle.merge(a, oracle.merge(b, c))
        for x, y in zip(ab_c, a_bc):
            np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-300)
        ab, ba = oracle.merge(a, b), oracle.merge(b, a)
        for x, y in zip(ab, ba):
            np.testing.assert_allclose(x, y, rtol=1e-15, atol=0)
        e = (-math.inf, 0.0, np.zeros(dv))
        ae = oracle.merge(a, e)
        assert ae[0] == a[0] and ae[1] == a[1] and np.array_equal(ae[2], a[2])
    ee = oracle.merge((-math.inf, 0.0, np.zeros(dv)), (-math.inf, 0.0, np.zeros(dv)))
    assert ee[0] == -math.inf and ee[1] == 0.0 and np.all(ee[2] == 0.0)


def test_merge_is_concatenation():
    """state(s1 ++ s2) == state(s1) (+) state(s2)."""
    rng = np.random.default_rng(6)
    s, v = rng.normal(size=11) * 4, rng.normal(size=(11, 5))
    whole = oracle.state(s, v)
    parts = oracle.merge(oracle.state(s[:4], v[:4]), oracle.state(s[4:], v[4:]))
    for x, y in zip(whole, parts):
        np.testing.assert_allclose(x, y, rtol=1e-13)


@pytest.mark.parametrize("n_split", [1, 2, 7, 16, 64, 103])
def test_split_decode_equals_definition(n_split):
    """Any split count, including more splits than keys (empty splits)."""
    B, H, Nq, Nk, d = 2, 3, 2, 100, 8
    Q, K, V = _rand((B, H, Nq, d), 120), _rand((B, H, Nk, d), 121), _rand((B, H, Nk, d), 122)
    O, L = oracle.dense_fwd(Q, K, V, 0.3)
    Od, Ld, pm, pl, po = oracle.split_decode(Q, K, V, n_split, 0.3)
    np.testing.assert_allclose(Od, O.reshape(B * H, Nq, d), atol=1e-12, rtol=1e-12)
    np.testing.assert_allclose(Ld, L.reshape(B * H, Nq), atol=1e-12, rtol=1e-12)
    # floor split bounds: split s holds keys [floor(Nk s/n), floor(Nk (s+1)/n))
    sizes = [Nk * (s + 1) // n_split - Nk * s // n_split for s in range(n_split)]
    assert np.all(np.isneginf(pm[..., [i for i, z in enumerate(sizes) if z == 0]]))
    np.testing.assert_array_equal(pl[..., [i for i, z in enumerate(sizes) if z == 0]], 0.0)
    # the first non-empty chunk by brute force
    c = next(i for i, z in enumerate(sizes) if z > 0)
    j0, j1 = Nk * c // n_split, Nk * (c + 1) // n_split
    s = 0.3 * K[0, 0, j0:j1] @ Q[0, 0, 0]
    assert abs(pm[0, 0, c] - s.max()) < 1e-14
    np.testing.assert_allclose(pl[0, 0, c], np.exp(s - s.max()).sum(), rtol=1e-14)
    np.testing.assert_allclose(po[0, 0, c], np.exp(s - s.max()) @ V[0, 0, j0:j1], rtol=1e-13)


def test_split_decode_heads_subset():
    Q, K, V = _rand((2, 2, 1, 4), 130), _rand((2, 2, 50, 4), 131), _rand((2, 2, 50, 4), 132)
    full = oracle.split_decode(Q, K, V, 5, 0.5)
    sub = oracle.split_decode(Q, K, V, 5, 0.5, heads=[3, 0])
    for x, y in zip(full, sub):
        np.testing.assert_array_equal(y, x[[3, 0]])


# ---------------------------------------------------------------------------
# Planted mistakes: rebuild the oracle with one step broken; a pin must fail.
# ---------------------------------------------------------------------------
def _planted(tmp_path, name):
    import ctypes
    src = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")
    so = str(tmp_path / f"liboracle_{name}.so")
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-pthread",
                    f"-DORACLE_PLANT_{name}", src, "-o", so, "-lm"], check=True)
    return ctypes.CDLL(so)


def _with_lib(lib, fn):
    saved = oracle._LIB
    try:
        oracle._LIB = None
        real = oracle._lib()  # set argtypes on a fresh load
        for f in ("oracle_dense_fwd", "oracle_online_fwd", "oracle_dense_bwd", "oracle_state",
                  "oracle_merge", "oracle_split_decode"):
            getattr(lib, f).argtypes = getattr(real, f).argtypes
            getattr(lib, f).restype = getattr(real, f).restype
        oracle._LIB = lib
        return fn()
    finally:
        oracle._LIB = saved


def _pins_pass(golden):
    """A compact run of the pins above; True when all hold."""
    checks = [test_anchor_closed_form, test_anchor_causal, test_uniform_scores]
    try:
        for c in checks:
            c(golden)
        test_online_block_sweep_tiny_workload(True)
        test_online_lab_py_case(True)
        test_bwd_vs_finite_differences_lab(False)
        test_bwd_invariants(True)
        test_merge_algebra()
        test_merge_is_concatenation()
        test_split_decode_equals_definition(7)
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("name", ["NO_RESCALE", "NO_MASK", "NO_SCALE", "BWD_SIGN",
                                  "BWD_OPERAND", "MERGE_NO_REBASE", "SPLIT_OVERLAP"])
def test_planted_mistake_is_caught(tmp_path, golden, name):
    lib = _planted(tmp_path, name)
    assert not _with_lib(lib, lambda: _pins_pass(golden)), f"planted {name} went unnoticed"


def test_unplanted_build_passes(golden):
    assert _pins_pass(golden)


# ---------------------------------------------------------------------------
# Causal offset q_start (standard_attention / flash_forward: query row i sits
# at absolute position q_start + i).  Pinned to the q_start = 0 path, which is
# pinned above, through the chunked-prefill identity: the rows s .. s+m-1 of
# the causal attention over the whole sequence are the offset attention of
# those m queries at q_start = s over the same keys.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("s,m", [(0, 7), (5, 9), (17, 3), (23, 1)])
def test_offset_is_chunked_prefill(s, m):
    B, H, N, d = 1, 2, 24, 8
    Q, K, V = _rand((B, H, N, d), 31), _rand((B, H, N, d), 32), _rand((B, H, N, d), 33)
    scale = 0.3
    O_full, L_full = oracle.dense_fwd(Q, K, V, scale, causal=True)
    O, L = oracle.dense_fwd(Q[:, :, s:s + m], K, V, scale, causal=True, q_start=s)
    np.testing.assert_allclose(O, O_full[:, :, s:s + m], atol=1e-13, rtol=0)
    np.testing.assert_allclose(L, L_full[:, :, s:s + m], atol=1e-13, rtol=0)
    # the online recurrence follows the same mask
    O2, L2 = oracle.online_fwd(Q[:, :, s:s + m], K, V, scale, causal=True, block=5, q_start=s)
    np.testing.assert_allclose(O2, O, atol=1e-12, rtol=0)
    np.testing.assert_allclose(L2, L, atol=1e-12, rtol=0)


def test_offset_past_the_keys_is_unmasked():
    """q_start >= Nk - 1: every row sees every key (non-causal result)."""
    Q, K, V = _rand((1, 1, 6, 4), 41), _rand((1, 1, 10, 4), 42), _rand((1, 1, 10, 4), 43)
    O0, L0 = oracle.dense_fwd(Q, K, V, 0.5, causal=False)
    for q_start in (9, 50):
        O, L = oracle.dense_fwd(Q, K, V, 0.5, causal=True, q_start=q_start)
        np.testing.assert_allclose(O, O0, atol=1e-14, rtol=0)
        np.testing.assert_allclose(L, L0, atol=1e-14, rtol=0)


@pytest.mark.parametrize("s,m", [(4, 8), (13, 11)])
def test_offset_backward_is_chunked_prefill(s, m):
    """Gradient of <O_rows, dO_rows> for the rows s .. s+m-1: the offset
    backward over those rows equals the full causal backward with dO = 0 on
    every other row (dK, dV), and its dQ is those rows of the full dQ."""
    B, H, N, d = 1, 1, 24, 6
    Q, K, V = _rand((B, H, N, d), 51), _rand((B, H, N, d), 52), _rand((B, H, N, d), 53)
    dO = np.zeros((B, H, N, d))
    dO[:, :, s:s + m] = _rand((B, H, m, d), 54)
    scale = 0.4
    full = oracle.dense_bwd(Q, K, V, dO, scale, causal=True)
    part = oracle.dense_bwd(Q[:, :, s:s + m], K, V, dO[:, :, s:s + m], scale, causal=True,
                            q_start=s)
    np.testing.assert_allclose(part["dK"], full["dK"], atol=1e-12, rtol=0)
    np.testing.assert_allclose(part["dV"], full["dV"], atol=1e-12, rtol=0)
    np.testing.assert_allclose(part["dQ"], full["dQ"][:, :, s:s + m], atol=1e-12, rtol=0)
    # keys after the last query's position get no gradient
    last = s + m - 1
    assert np.all(part["dK"][:, :, last + 1:] == 0) and np.all(part["dV"][:, :, last + 1:] == 0)
