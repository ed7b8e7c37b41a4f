"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the GPU tests and the oracle side consume the exact
tensors it returns (the oracle after an exact upcast to fp64), so the choice of
generator never affects parity.

Recipe (every workload):
  * a ``torch.Generator`` seeded with the workload's seed, on the device the
    tensors are made on;
  * draw order Q, K, V, then dO (backward workloads only), then the "hot" key
    rows (see below);
  * values ~ N(0, 1) drawn in fp32, one [H, N, d] batch slice at a time, then
    rounded to the storage dtype (bf16 round-to-nearest-even) once.
Hot rows: for each (b, h) one key index j* is drawn uniformly from [0, Nk) and
that fp32 K row is multiplied by ``hot_row_factor`` before the single rounding.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

# The five workloads.  Seeds are the workload numbers 1..5.
WORKLOADS = {
    "tiny_f32": dict(seed=1, B=1, H=1, Nq=64, Nk=64, d=16, dtype="f32", causal=(False, True)),
    "prefill_d64": dict(seed=2, B=4, H=16, Nq=2048, Nk=2048, d=64, dtype="bf16",
                        causal=(False,)),
    "prefill_causal_d128": dict(seed=3, B=1, H=32, Nq=8192, Nk=8192, d=128, dtype="bf16",
                                causal=(True,), hot_row_factor=30.0),
    "bwd_causal_d64": dict(seed=4, B=2, H=16, Nq=4096, Nk=4096, d=64, dtype="bf16",
                           causal=(True,), backward=True),
    "decode_d128": dict(seed=5, B=64, H=32, Nq=1, Nk=32768, d=128, dtype="bf16",
                        causal=(False,), n_split=(16, 32, 64)),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def default_scale(d: int) -> float:
    """1/sqrt(d), the score scale every workload uses."""
    return 1.0 / math.sqrt(d)


@dataclass
class Inputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    do: torch.Tensor | None = None
    hot_rows: torch.Tensor | None = None  # [B, H] int64, or None
    meta: dict = field(default_factory=dict)


def _randn_slices(gen: torch.Generator, B: int, H: int, N: int, d: int, device, out_dtype,
                  hot=None):
    out = torch.empty((B, H, N, d), dtype=out_dtype, device=device)
    for b in range(B):
        x = torch.randn((H, N, d), generator=gen, dtype=torch.float32, device=device)
        if hot is not None:
            x = hot(b, x)
        out[b].copy_(x)
        del x
    return out


def make_inputs(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str = "bf16", seed: int = 0,
                device="cpu", backward: bool = False, hot_row_factor: float | None = None,
                q_scale: float = 1.0, k_scale: float = 1.0) -> Inputs:
    """Draw Q [B,H,Nq,d], K and V [B,H,Nk,d] (and dO [B,H,Nq,d] when
    ``backward``) ~ N(0, 1) in fp32 and round them once to ``dtype``.
    ``q_scale``/``k_scale`` multiply the fp32 draws before rounding (large-logit
    cases)."""
    tdt = TORCH_DTYPE[dtype]
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    q = _randn_slices(gen, B, H, Nq, d, device, torch.float32 if q_scale != 1.0 else tdt)
    if q_scale != 1.0:
        q = (q * q_scale).to(tdt)
    if hot_row_factor is None:
        k = _randn_slices(gen, B, H, Nk, d, device, torch.float32 if k_scale != 1.0 else tdt)
        if k_scale != 1.0:
            k = (k * k_scale).to(tdt)
        kf = None
    else:
        # keep K in fp32 until the hot rows are drawn, then round once
        kf = _randn_slices(gen, B, H, Nk, d, device, torch.float32)
        if k_scale != 1.0:
            kf.mul_(k_scale)
        k = None
    v = _randn_slices(gen, B, H, Nk, d, device, tdt)
    do = _randn_slices(gen, B, H, Nq, d, device, tdt) if backward else None
    hot_rows = None
    if hot_row_factor is not None:
        hot_rows = torch.randint(0, Nk, (B, H), generator=gen, device=device, dtype=torch.int64)
        bidx = torch.arange(B, device=device)[:, None].expand(B, H)
        hidx = torch.arange(H, device=device)[None, :].expand(B, H)
        kf[bidx, hidx, hot_rows] *= float(hot_row_factor)
        k = kf.to(tdt)
        del kf
    meta = dict(B=B, H=H, Nq=Nq, Nk=Nk, d=d, dtype=dtype, seed=seed,
                hot_row_factor=hot_row_factor, q_scale=q_scale, k_scale=k_scale,
                torch=torch.__version__)
    return Inputs(q, k, v, do, hot_rows, meta)


def workload_inputs(name: str, device="cpu") -> Inputs:
    """Inputs of one named workload at its full size."""
    w = WORKLOADS[name]
    return make_inputs(w["B"], w["H"], w["Nq"], w["Nk"], w["d"], w["dtype"], w["seed"], device,
                       backward=w.get("backward", False),
                       hot_row_factor=w.get("hot_row_factor"))


def to_f64_numpy(t: torch.Tensor):
    """Exact upcast of a float32/bf16 tensor to a float64 numpy array on the host."""
    return t.detach().to("cpu").to(torch.float64).numpy()
