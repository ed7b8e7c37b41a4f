"""The debug build libfa_stats.so: the same calls as libfa.so, whose bf16
kernels also count tiles computed, tiles skipped under causal, accumulator
rescales and dQ atomic additions (include/fa_stats.h).

Load it with :func:`load`; its ``forward`` and ``backward`` run the counting
kernels, ``read`` returns the counters, ``reset`` zeroes them and ``tile``
reports the block shape the counts refer to.  Like the release binding, this
module only marshals arguments; there is no fallback when the library is
missing.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import (_PKG_DIR, _check, _declare, _dt, _ptr, _scale, _stream, FA_BF16,
               fa_bwd_workspace_size)

STATS_PATH = os.path.join(_PKG_DIR, "libfa_stats.so")
NAMES = ("fwd_tiles", "fwd_skipped", "fwd_rescales", "bwd_kv_tiles", "bwd_q_tiles",
         "dq_atomic_adds")
COUNT = 8


class StatsLib:
    def __init__(self, path: str = STATS_PATH):
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run __graft_entry__.build()")
        self.lib = _declare(ctypes.CDLL(path))
        self.lib.fa_stats_reset.argtypes = []
        self.lib.fa_stats_read.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
        self.lib.fa_stats_tile.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                           ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
                                           ctypes.POINTER(ctypes.c_int64)]
        for f in ("fa_stats_reset", "fa_stats_read", "fa_stats_tile"):
            getattr(self.lib, f).restype = ctypes.c_int

    def reset(self) -> None:
        _check(self.lib.fa_stats_reset(), "fa_stats_reset")

    def read(self) -> dict:
        buf = (ctypes.c_uint64 * COUNT)()
        _check(self.lib.fa_stats_read(buf), "fa_stats_read")
        return {n: int(buf[i]) for i, n in enumerate(NAMES)}

    def tile(self, kind: int, d: int, causal: bool, dtype=FA_BF16) -> tuple[int, int]:
        r, c = ctypes.c_int64(), ctypes.c_int64()
        _check(self.lib.fa_stats_tile(int(kind), int(dtype), int(d), int(bool(causal)),
                                      ctypes.byref(r), ctypes.byref(c)), "fa_stats_tile")
        return r.value, c.value

    def forward(self, q, k, v, scale=None, causal=False, q_start=None, stream=None):
        B, H, Nq, d = q.shape
        Nk = k.shape[2]
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
        args = (_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                _scale(d, scale))
        if q_start is None:
            _check(self.lib.fa_fwd(*args, int(bool(causal)), _stream(stream)), "fa_fwd")
        else:
            _check(self.lib.fa_fwd_offset(*args, int(q_start), _stream(stream)), "fa_fwd_offset")
        return o, lse

    def backward(self, q, k, v, o, lse, do, scale=None, causal=False, q_start=None, stream=None):
        B, H, Nq, d = q.shape
        Nk = k.shape[2]
        ws = torch.empty(fa_bwd_workspace_size(q.dtype, B, H, Nq, d), dtype=torch.uint8,
                         device=q.device)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        args = (_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(), B, H, Nq, Nk, d, _scale(d, scale))
        if q_start is None:
            _check(self.lib.fa_bwd(*args, int(bool(causal)), _stream(stream)), "fa_bwd")
        else:
            _check(self.lib.fa_bwd_offset(*args, int(q_start), _stream(stream)), "fa_bwd_offset")
        return dq, dk, dv


def load(path: str = STATS_PATH) -> StatsLib:
    return StatsLib(path)
