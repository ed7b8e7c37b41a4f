"""fa_bwd_noalloc (the backward with its workspace in the library's fixed
device array) against fa_bwd with a caller-allocated workspace: the same
kernels on the same inputs, so the gradients must be bit-identical; and both
within the usual tolerance of the oracle.  Calls follow one another with
shrinking inputs, so the second call runs on the array the first one left
behind."""
import ctypes
import math

import pytest
import torch

import oracle
from fa_inputs import make_inputs
from tests.gpu_helpers import host, max_rel, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import flashattention_online_softmax_fa_amd as m
    return m


CASES = [  # B, H, N, d, dtype, causal; each smaller than the one before
    (2, 8, 1000, 64, "bf16", True),
    (1, 3, 333, 128, "bf16", False),
    (1, 2, 100, 64, "bf16", True),
    (1, 1, 50, 16, "f32", True),
]


def test_noalloc_equals_fa_bwd(fa):
    for B, H, N, d, dt, causal in CASES:
        x = make_inputs(B, H, N, N, d, dt, seed=N + d, device="cuda", backward=True)
        scale = 1 / math.sqrt(d)
        say(f"noalloc bwd B={B} H={H} N={N} d={d} {dt} causal={causal}")
        o, lse = fa.forward(x.q, x.k, x.v, scale, causal)
        ref = fa.backward(x.q, x.k, x.v, o, lse, x.do, scale, causal)
        got = [torch.full_like(t, float("nan")) for t in ref]
        fa.fa_bwd_noalloc(x.q, x.k, x.v, o, lse, x.do, *got, scale, causal)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.equal(a, b), f"{name} differs from fa_bwd"
        g = oracle.dense_bwd(host(x.q), host(x.k), host(x.v), host(x.do), scale, causal)
        tol = 5e-2 if dt == "bf16" else 1e-5
        for name, a in zip(("dQ", "dK", "dV"), got):
            assert max_rel(a, g[name]) <= tol, name


def test_noalloc_rejects_sizes_past_the_array(fa):
    """2^21 + 1 query rows do not fit: the binding raises, and the C call
    itself returns FA_ERR_INVALID_ARG without launching."""
    B, H, N, d = 1, 1, (1 << 21) + 1, 64
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, H, N), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="fixed"):
        fa.fa_bwd_noalloc(q, q, q, q, lse, q, q, q, q)
    p = q.data_ptr()
    st = fa._lib.fa_bwd_noalloc(fa.FA_BF16, p, p, p, p, lse.data_ptr(), p, p, p, p, B, H, N, N,
                                d, 0.125, 1, None)
    assert st == fa.FA_ERR_INVALID_ARG
