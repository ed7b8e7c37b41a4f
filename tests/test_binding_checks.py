"""The Python binding rejects operands whose shape, dtype or device does not
match what the C call will assume from q's sizes, before anything reaches the
library (host only: the library is replaced by an object that fails on any
call, so a test passes only if nothing was called)."""
import pytest
import torch

import flashattention_online_softmax_fa_amd as fa


class _NoCalls:
    def __getattr__(self, name):
        def fail(*args):
            raise AssertionError(f"the library was called ({name}) despite a bad operand")
        return fail


@pytest.fixture
def nolib(monkeypatch):
    monkeypatch.setattr(fa, "_lib", _NoCalls())


def _t(*shape, dtype=torch.bfloat16, device="cpu"):
    return torch.zeros(shape, dtype=dtype, device=device)


B, H, NQ, NK, D, NS = 2, 3, 5, 7, 64, 4


def fwd_ops():
    return dict(q=_t(B, H, NQ, D), k=_t(B, H, NK, D), v=_t(B, H, NK, D), o=_t(B, H, NQ, D),
                lse=_t(B, H, NQ, dtype=torch.float32))


def bwd_ops():
    x = fwd_ops()
    x.update(do=_t(B, H, NQ, D), dq=_t(B, H, NQ, D), dk=_t(B, H, NK, D), dv=_t(B, H, NK, D),
             workspace=_t(4096, dtype=torch.uint8))
    return x


def dec_ops():
    return dict(q=_t(B, H, NQ, D), k=_t(B, H, NK, D), v=_t(B, H, NK, D),
                part_m=_t(B, H, NQ, NS, dtype=torch.float32),
                part_l=_t(B, H, NQ, NS, dtype=torch.float32),
                part_o=_t(B, H, NQ, NS, D, dtype=torch.float32))


def merge_ops():
    return dict(part_m=_t(B, H, NQ, NS, dtype=torch.float32),
                part_l=_t(B, H, NQ, NS, dtype=torch.float32),
                part_o=_t(B, H, NQ, NS, D, dtype=torch.float32), o=_t(B, H, NQ, D),
                lse=_t(B, H, NQ, dtype=torch.float32))


def call_fwd(x):
    fa.fa_fwd(x["q"], x["k"], x["v"], x["o"], x["lse"])


def call_fwd_offset(x):
    fa.fa_fwd_offset(x["q"], x["k"], x["v"], x["o"], x["lse"], 1)


def call_fwd_blocked(x):
    fa.fa_fwd_blocked(x["q"], x["k"], x["v"], x["o"], x["lse"], 4)


def call_bwd(x):
    fa.fa_bwd(x["q"], x["k"], x["v"], x["o"], x["lse"], x["do"], x["dq"], x["dk"], x["dv"],
              x["workspace"])


def call_bwd_offset(x):
    fa.fa_bwd_offset(x["q"], x["k"], x["v"], x["o"], x["lse"], x["do"], x["dq"], x["dk"],
                     x["dv"], x["workspace"], 2)


def call_dec(x):
    fa.fa_decode_split(x["q"], x["k"], x["v"], x["part_m"], x["part_l"], x["part_o"], NS)


def call_dec_offset(x):
    fa.fa_decode_split_offset(x["q"], x["k"], x["v"], x["part_m"], x["part_l"], x["part_o"],
                              NS, 3)


def call_merge(x):
    fa.fa_merge_states(x["part_m"], x["part_l"], x["part_o"], x["o"], x["lse"])


FWD_BAD = [
    ("k", _t(B, H + 1, NK, D)),                    # fewer/more heads than q
    ("k", _t(B, H, NK, D // 2)),                   # other head dimension
    ("v", _t(B, H, NK + 1, D)),                    # V rows != K rows
    ("v", _t(B, H, NK, D, dtype=torch.float32)),   # mixed dtypes
    ("o", _t(B, H, NQ, D, dtype=torch.float32)),
    ("o", _t(B, H, NQ + 1, D)),
    ("lse", _t(B, H, NQ)),                         # bf16 L
    ("lse", _t(B, H, NQ + 2, dtype=torch.float32)),
    ("q", _t(B, H, NQ, D, device="meta")),         # another device
    ("k", "not a tensor"),
]


@pytest.mark.parametrize("call", [call_fwd, call_fwd_offset, call_fwd_blocked])
@pytest.mark.parametrize("name,bad", FWD_BAD)
def test_forward_rejects(nolib, call, name, bad):
    x = fwd_ops()
    x[name] = bad
    with pytest.raises(ValueError):
        call(x)


BWD_BAD = FWD_BAD + [
    ("do", _t(B, H, NQ, D, dtype=torch.float32)),
    ("do", _t(B, H, NK, D)),
    ("dq", _t(B, H, NQ, D // 2)),
    ("dk", _t(B, H, NQ, D)),                       # dK sized like Q (Nq != Nk)
    ("dv", _t(B, H - 1, NK, D)),
    ("dv", _t(B, H, NK, D, dtype=torch.float32)),
    ("workspace", _t(4096, dtype=torch.uint8, device="meta")),
]


@pytest.mark.parametrize("call", [call_bwd, call_bwd_offset])
@pytest.mark.parametrize("name,bad", BWD_BAD)
def test_backward_rejects(nolib, call, name, bad):
    x = bwd_ops()
    x[name] = bad
    with pytest.raises(ValueError):
        call(x)


DEC_BAD = [
    ("k", _t(B, H, NK, 128)),
    ("v", _t(B, H, NK - 1, D)),
    ("part_m", _t(B, H, NQ, NS + 1, dtype=torch.float32)),
    ("part_m", _t(B, H, NQ, NS)),
    ("part_l", _t(B, H, NQ, NS, dtype=torch.float64)),
    ("part_o", _t(B, H, NQ, NS, D // 2, dtype=torch.float32)),
    ("part_o", _t(B, H, NQ, NS - 1, D, dtype=torch.float32)),
]


@pytest.mark.parametrize("call", [call_dec, call_dec_offset])
@pytest.mark.parametrize("name,bad", DEC_BAD)
def test_decode_rejects(nolib, call, name, bad):
    x = dec_ops()
    x[name] = bad
    with pytest.raises(ValueError):
        call(x)


MERGE_BAD = [
    ("part_l", _t(B, H, NQ, NS + 1, dtype=torch.float32)),
    ("part_l", _t(B, H, NQ, NS)),
    ("part_o", _t(B, H, NQ, NS, D + 8, dtype=torch.float32)),
    ("o", _t(B, H, NQ + 1, D)),
    ("o", _t(B, H, NQ, D, dtype=torch.float16)),
    ("lse", _t(B, H, NQ)),
    ("lse", _t(B, H, NQ, 1, dtype=torch.float32)),
    ("part_m", _t(B, H, NQ, dtype=torch.float32)),
]


@pytest.mark.parametrize("name,bad", MERGE_BAD)
def test_merge_rejects(nolib, name, bad):
    x = merge_ops()
    x[name] = bad
    with pytest.raises(ValueError):
        call_merge(x)


@pytest.mark.parametrize("call,ops", [(call_fwd, fwd_ops), (call_fwd_offset, fwd_ops),
                                      (call_fwd_blocked, fwd_ops), (call_bwd, bwd_ops),
                                      (call_bwd_offset, bwd_ops), (call_dec, dec_ops),
                                      (call_dec_offset, dec_ops), (call_merge, merge_ops)])
def test_consistent_host_tensors_still_rejected(nolib, call, ops):
    """Matching shapes pass the operand check; host memory is then refused,
    again before the library is called."""
    with pytest.raises(ValueError, match="GPU"):
        call(ops())
