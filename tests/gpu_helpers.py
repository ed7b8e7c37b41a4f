"""Shared helpers of the GPU parity tests (comparison and sampling only)."""
import sys

import numpy as np
import torch

from fa_inputs import to_f64_numpy


def say(*a):
    """Name the case before a GPU step so a failing run still identifies it."""
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    """fp64 numpy copy of a tensor (or an array already on the host)."""
    if isinstance(t, np.ndarray):
        return t.astype(np.float64, copy=False)
    return to_f64_numpy(t)


def max_abs(got, want):
    got = got if isinstance(got, np.ndarray) else host(got)
    return float(np.abs(got - want).max()) if want.size else 0.0


def max_rel(got, want):
    """Per-tensor relative error: max |got - want| / max |want|."""
    got = got if isinstance(got, np.ndarray) else host(got)
    den = float(np.abs(want).max())
    return float(np.abs(got - want).max()) / (den if den > 0 else 1.0)


def heads_slice(t: torch.Tensor, heads):
    """Host fp64 copy [1, len(heads), N, d] of flat heads (b*H + h) of a
    [B, H, N, d] tensor."""
    B, H = t.shape[0], t.shape[1]
    parts = [t[h // H, h % H] for h in heads]
    return host(torch.stack(parts, 0)).reshape((1, len(heads)) + tuple(t.shape[2:]))


def sample_heads(B, H, k, seed):
    rng = np.random.default_rng(seed)
    n = B * H
    picks = {0, n - 1}
    while len(picks) < min(k, n):
        picks.add(int(rng.integers(0, n)))
    return sorted(picks)


def head_block(t: torch.Tensor, lo: int, hi: int):
    """Host fp64 copy [1, hi-lo, N, d] of flat heads lo .. hi-1 (b*H + h) of a
    [B, H, N, d] tensor; the exact upcast runs on the device, then one copy."""
    B, H = t.shape[0], t.shape[1]
    flat = t.reshape((B * H,) + tuple(t.shape[2:]))[lo:hi]
    return flat.to(torch.float64).cpu().numpy()[None]
