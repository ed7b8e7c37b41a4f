"""MI355X (gfx950) FlashAttention: a thin Python binding over libfa.so.

The functions named like the C entry points (``fa_fwd``, ``fa_fwd_offset``,
``fa_fwd_blocked``, ``fa_bwd``, ``fa_bwd_offset``, ``fa_bwd_noalloc``,
``fa_bwd_workspace_size``, ``fa_decode_split``, ``fa_decode_split_offset``,
``fa_merge_states``, ``fa_status_str``) only check and marshal torch tensors
into the C ABI of ``include/fa.h``; every step of the computation runs in the
library's HIP kernels.  ``forward``, ``backward`` and ``decode`` additionally
allocate the outputs with torch before calling them.

torch provides device memory and streams only.  It is imported before
libfa.so is loaded so that both use the one HIP runtime already in the
process.  There is no fallback: if libfa.so is missing, importing this module
raises ImportError.  FA_LIBRARY, when set, names another build of the same
sources to load instead (``build.py --variant``: other tile constants).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG_DIR = _HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FA_LIBRARY") or os.path.join(_HERE, "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
FA_F32, FA_BF16 = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "(hipcc --offload-arch=gfx950)")

_vp, _i64, _f32, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    """Argument and result types of the include/fa.h entry points of `lib`."""
    lib.fa_fwd.argtypes = [_int, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f32,
                           _int, _vp]
    lib.fa_fwd_offset.argtypes = [_int, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                  _f32, _i64, _vp]
    lib.fa_fwd_blocked.argtypes = [_int, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                   _f32, _int, _i64, _vp]
    lib.fa_bwd_workspace_size.argtypes = [_int, _i64, _i64, _i64, _i64]
    lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                           ctypes.c_size_t, _i64, _i64, _i64, _i64, _i64, _f32, _int, _vp]
    lib.fa_bwd_offset.argtypes = [_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  ctypes.c_size_t, _i64, _i64, _i64, _i64, _i64, _f32, _i64, _vp]
    lib.fa_bwd_noalloc.argtypes = [_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                                   _i64, _i64, _i64, _i64, _f32, _int, _vp]
    lib.fa_decode_split.argtypes = [_int, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                    _i64, _i64, _f32, _vp]
    lib.fa_decode_split_offset.argtypes = [_int, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                           _i64, _i64, _i64, _f32, _i64, _vp]
    lib.fa_merge_states.argtypes = [_int, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                    _vp]
    lib.fa_status_str.argtypes = [_int]
    lib.fa_status_str.restype = ctypes.c_char_p
    for f in ("fa_fwd", "fa_fwd_offset", "fa_fwd_blocked", "fa_bwd", "fa_bwd_offset",
              "fa_bwd_noalloc", "fa_decode_split", "fa_decode_split_offset",
              "fa_merge_states"):
        getattr(lib, f).restype = _int
    return lib


_lib = _declare(ctypes.CDLL(LIB_PATH))

EXPORTS = ("fa_fwd", "fa_fwd_offset", "fa_fwd_blocked", "fa_bwd_workspace_size", "fa_bwd",
           "fa_bwd_offset", "fa_bwd_noalloc", "fa_decode_split", "fa_decode_split_offset",
           "fa_merge_states", "fa_status_str")

# Size of the device array fa_bwd_noalloc keeps its workspace in (include/fa.h).
FA_NOALLOC_SCRATCH_BYTES = 16 << 20


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_str(status)}")


def fa_status_str(status: int) -> str:
    return _lib.fa_status_str(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != FA_OK:
        raise FaError(status, where)


_DT = {torch.float32: FA_F32, torch.bfloat16: FA_BF16}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _scale(d: int, scale) -> float:
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _bhnd(t: torch.Tensor):
    if not isinstance(t, torch.Tensor) or t.dim() != 4:
        raise ValueError("expected a [B, H, N, d] tensor")
    return tuple(t.shape)


def _operands(where: str, dtype, device, **spec) -> None:
    """Check every operand against the shape the C call will assume from the
    sizes it is given, and against one dtype and one device: a mismatch would
    otherwise make a kernel read or write past the end of a buffer.  `spec`
    maps a name to (tensor, shape, dtype); dtype None means the common one.
    Raises ValueError before anything reaches the library."""
    for name, (t, shape, dt) in spec.items():
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{where}: {name} must be a tensor")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{where}: {name} has shape {tuple(t.shape)}, "
                             f"expected {tuple(shape)}")
        want = dtype if dt is None else dt
        if t.dtype != want:
            raise ValueError(f"{where}: {name} is {t.dtype}, expected {want}")
        if t.device != device:
            raise ValueError(f"{where}: {name} is on {t.device}, expected {device}")


def _fwd_operands(where, q, k, v, o, lse):
    B, H, Nq, d = _bhnd(q)
    Nk = _bhnd(k)[2]
    f32 = torch.float32
    _operands(where, q.dtype, q.device, k=(k, (B, H, Nk, d), None), v=(v, (B, H, Nk, d), None),
              o=(o, (B, H, Nq, d), None), lse=(lse, (B, H, Nq), f32))
    return B, H, Nq, Nk, d


def _bwd_operands(where, q, k, v, o, lse, do, dq, dk, dv, workspace):
    B, H, Nq, Nk, d = _fwd_operands(where, q, k, v, o, lse)
    _operands(where, q.dtype, q.device, do=(do, (B, H, Nq, d), None),
              dq=(dq, (B, H, Nq, d), None), dk=(dk, (B, H, Nk, d), None),
              dv=(dv, (B, H, Nk, d), None))
    if not isinstance(workspace, torch.Tensor) or workspace.device != q.device:
        raise ValueError(f"{where}: workspace must be a tensor on {q.device}")
    return B, H, Nq, Nk, d


def _decode_operands(where, q, k, v, part_m, part_l, part_o, n_split):
    B, H, Nq, d = _bhnd(q)
    Nk = _bhnd(k)[2]
    n = int(n_split)
    f32 = torch.float32
    _operands(where, q.dtype, q.device, k=(k, (B, H, Nk, d), None), v=(v, (B, H, Nk, d), None),
              part_m=(part_m, (B, H, Nq, n), f32), part_l=(part_l, (B, H, Nq, n), f32),
              part_o=(part_o, (B, H, Nq, n, d), f32))
    return B, H, Nq, Nk, d


def fa_fwd(q, k, v, o, lse, scale=None, causal=False, stream=None) -> None:
    B, H, Nq, Nk, d = _fwd_operands("fa_fwd", q, k, v, o, lse)
    _check(_lib.fa_fwd(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                       _scale(d, scale), int(bool(causal)), _stream(stream)), "fa_fwd")


def fa_fwd_offset(q, k, v, o, lse, q_start, scale=None, stream=None) -> None:
    B, H, Nq, Nk, d = _fwd_operands("fa_fwd_offset", q, k, v, o, lse)
    _check(_lib.fa_fwd_offset(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq,
                              Nk, d, _scale(d, scale), int(q_start), _stream(stream)),
           "fa_fwd_offset")


def fa_fwd_blocked(q, k, v, o, lse, kv_block, scale=None, causal=False, stream=None) -> None:
    B, H, Nq, Nk, d = _fwd_operands("fa_fwd_blocked", q, k, v, o, lse)
    _check(_lib.fa_fwd_blocked(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq,
                               Nk, d, _scale(d, scale), int(bool(causal)), int(kv_block),
                               _stream(stream)), "fa_fwd_blocked")


def fa_bwd_workspace_size(dtype, B, H, Nq, d) -> int:
    dt = _DT[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.fa_bwd_workspace_size(dt, B, H, Nq, d))


def fa_bwd(q, k, v, o, lse, do, dq, dk, dv, workspace, scale=None, causal=False,
           stream=None) -> None:
    B, H, Nq, Nk, d = _bwd_operands("fa_bwd", q, k, v, o, lse, do, dq, dk, dv, workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.fa_bwd(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                       _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, B, H, Nq, Nk, d,
                       _scale(d, scale), int(bool(causal)), _stream(stream)), "fa_bwd")


def fa_bwd_offset(q, k, v, o, lse, do, dq, dk, dv, workspace, q_start, scale=None,
                  stream=None) -> None:
    B, H, Nq, Nk, d = _bwd_operands("fa_bwd_offset", q, k, v, o, lse, do, dq, dk, dv,
                                    workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.fa_bwd_offset(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, B, H, Nq,
                              Nk, d, _scale(d, scale), int(q_start), _stream(stream)),
           "fa_bwd_offset")


def fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale=None, causal=False,
                   stream=None) -> None:
    """fa_bwd without a workspace: the library keeps it in a fixed device array
    of FA_NOALLOC_SCRATCH_BYTES, shared by every call on the GPU (calls that
    overlap on one GPU race)."""
    B, H, Nq, Nk, d = _fwd_operands("fa_bwd_noalloc", q, k, v, o, lse)
    _operands("fa_bwd_noalloc", q.dtype, q.device, do=(do, (B, H, Nq, d), None),
              dq=(dq, (B, H, Nq, d), None), dk=(dk, (B, H, Nk, d), None),
              dv=(dv, (B, H, Nk, d), None))
    need = fa_bwd_workspace_size(q.dtype, B, H, Nq, d) if q.dtype in _DT else 0
    if need > FA_NOALLOC_SCRATCH_BYTES:
        raise ValueError(f"fa_bwd_noalloc: {B}*{H}*{Nq} query rows need {need} bytes of "
                         f"workspace, more than its fixed {FA_NOALLOC_SCRATCH_BYTES} "
                         "(use fa_bwd with a workspace)")
    _check(_lib.fa_bwd_noalloc(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                               _ptr(dq), _ptr(dk), _ptr(dv), B, H, Nq, Nk, d, _scale(d, scale),
                               int(bool(causal)), _stream(stream)), "fa_bwd_noalloc")


def fa_decode_split(q, k, v, part_m, part_l, part_o, n_split, scale=None, stream=None) -> None:
    B, H, Nq, Nk, d = _decode_operands("fa_decode_split", q, k, v, part_m, part_l, part_o,
                                       n_split)
    _check(_lib.fa_decode_split(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(part_m), _ptr(part_l),
                                _ptr(part_o), B, H, Nq, Nk, d, int(n_split), _scale(d, scale),
                                _stream(stream)), "fa_decode_split")


def fa_decode_split_offset(q, k, v, part_m, part_l, part_o, n_split, q_start, scale=None,
                           stream=None) -> None:
    B, H, Nq, Nk, d = _decode_operands("fa_decode_split_offset", q, k, v, part_m, part_l,
                                       part_o, n_split)
    _check(_lib.fa_decode_split_offset(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(part_m),
                                       _ptr(part_l), _ptr(part_o), B, H, Nq, Nk, d, int(n_split),
                                       _scale(d, scale), int(q_start), _stream(stream)),
           "fa_decode_split_offset")


def fa_merge_states(part_m, part_l, part_o, o, lse, stream=None) -> None:
    if not isinstance(part_m, torch.Tensor) or part_m.dim() != 4:
        raise ValueError("fa_merge_states: part_m must be a [B, H, Nq, n_split] tensor")
    B, H, Nq, n_split = part_m.shape
    d = _bhnd(o)[3]
    if o.dtype not in _DT:
        raise ValueError(f"fa_merge_states: o is {o.dtype}, expected float32 or bfloat16")
    f32 = torch.float32
    _operands("fa_merge_states", f32, part_m.device, part_l=(part_l, (B, H, Nq, n_split), None),
              part_o=(part_o, (B, H, Nq, n_split, d), None), o=(o, (B, H, Nq, d), o.dtype),
              lse=(lse, (B, H, Nq), None))
    _check(_lib.fa_merge_states(_dt(o), _ptr(part_m), _ptr(part_l), _ptr(part_o), _ptr(o),
                                _ptr(lse), B, H, Nq, d, n_split, _stream(stream)),
           "fa_merge_states")


# ---------------------------------------------------------------------------
# Convenience wrappers that allocate outputs with torch.
# ---------------------------------------------------------------------------
def forward(q, k, v, scale=None, causal=False, kv_block=None, stream=None, q_start=None):
    """(O, L) for Q [B,H,Nq,d], K, V [B,H,Nk,d]; L is fp32 [B,H,Nq].

    With ``q_start`` set, the attention is causal with query row i at key
    position q_start + i (``causal`` is then implied)."""
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    if q_start is not None:
        if kv_block is not None:
            raise ValueError("kv_block and q_start cannot be combined")
        fa_fwd_offset(q, k, v, o, lse, q_start, scale, stream)
    elif kv_block is None:
        fa_fwd(q, k, v, o, lse, scale, causal, stream)
    else:
        fa_fwd_blocked(q, k, v, o, lse, kv_block, scale, causal, stream)
    return o, lse


def backward(q, k, v, o, lse, do, scale=None, causal=False, stream=None, q_start=None):
    """(dQ, dK, dV) of <O, dO>; O and L from forward() with the same arguments."""
    B, H, Nq, d = q.shape
    ws = torch.empty(fa_bwd_workspace_size(q.dtype, B, H, Nq, d), dtype=torch.uint8,
                     device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if q_start is not None:
        fa_bwd_offset(q, k, v, o, lse, do, dq, dk, dv, ws, q_start, scale, stream)
    else:
        fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, scale, causal, stream)
    return dq, dk, dv


def decode(q, k, v, n_split, scale=None, stream=None, out_dtype=None, q_start=None):
    """Split-KV decoding: returns (O, L, (part_m, part_l, part_o)).  With
    ``q_start`` the Nq query rows attend causally from key position q_start + i."""
    B, H, Nq, d = q.shape
    dev = q.device
    pm = torch.empty((B, H, Nq, n_split), dtype=torch.float32, device=dev)
    pl = torch.empty_like(pm)
    po = torch.empty((B, H, Nq, n_split, d), dtype=torch.float32, device=dev)
    if q_start is None:
        fa_decode_split(q, k, v, pm, pl, po, n_split, scale, stream)
    else:
        fa_decode_split_offset(q, k, v, pm, pl, po, n_split, q_start, scale, stream)
    o = torch.empty((B, H, Nq, d), dtype=out_dtype or q.dtype, device=dev)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    fa_merge_states(pm, pl, po, o, lse, stream)
    return o, lse, (pm, pl, po)
