"""Host logic of bench.py's oracle leg on small CPU tensors: the sample,
the units and the parity fields, and that a wrong output is flagged (the
"GPU" outputs here are the oracle's own results, rounded like the kernels',
or a copy with one element changed)."""
import importlib.util
import math
import os

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_inputs, to_f64_numpy

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _fwd_run(name, causal, d=64, N=96):
    x = make_inputs(1, 2, N, N, d, "bf16", seed=3)
    scale = 1 / math.sqrt(d)
    O, L = oracle.dense_fwd(*(to_f64_numpy(t) for t in (x.q, x.k, x.v)), scale, causal)
    out = dict(o=torch.from_numpy(O).to(torch.bfloat16), lse=torch.from_numpy(L).float())
    return dict(x=x, out=out, scale=scale, causal=causal, cfg={"workload": name})


@pytest.mark.parametrize("causal", [False, True])
def test_forward_leg(bench, causal):
    run = _fwd_run("prefill_d64", causal)
    cpu, par = bench.oracle_leg(run, budget_s=0.05)
    assert cpu["kind"] == "oracle" and cpu["unit"] == "TFLOP/s" and cpu["cores"] >= 1
    assert set(cpu["routines"]) == {"dense_definition", "online_block64"}
    assert par["ok"] and par["o_max_abs"] <= 1e-2 and par["l_max_abs"] <= 1e-6
    assert par["online_vs_dense_max_abs"] <= 1e-12
    run["out"]["o"].view(-1)[5] += 1.0
    _, par = bench.oracle_leg(run, budget_s=1e9)  # whole tensor: the change is seen
    assert not par["ok"]


def test_backward_leg(bench):
    x = make_inputs(1, 2, 64, 64, 64, "bf16", seed=4, backward=True)
    scale = 0.125
    g = oracle.dense_bwd(*(to_f64_numpy(t) for t in (x.q, x.k, x.v, x.do)), scale, True)
    out = {k.lower(): torch.from_numpy(g[k]).to(torch.bfloat16) for k in ("dQ", "dK", "dV")}
    run = dict(x=x, out=out, scale=scale, causal=True, cfg={"workload": "bwd_causal_d64"})
    cpu, par = bench.oracle_leg(run, budget_s=0.05)
    assert cpu["unit"] == "TFLOP/s" and "dense_jacobian_backward" in cpu["routines"]
    assert par["ok"] and max(par["dQ_max_rel"], par["dK_max_rel"], par["dV_max_rel"]) < 1e-2
    out["dk"].mul_(1.2)
    _, par = bench.oracle_leg(run, budget_s=1e9)
    assert not par["ok"]


def test_decode_leg(bench):
    x = make_inputs(2, 3, 1, 200, 128, "bf16", seed=5)
    scale = 1 / math.sqrt(128)
    O, L = oracle.dense_fwd(*(to_f64_numpy(t) for t in (x.q, x.k, x.v)), scale)
    out = dict(o=torch.from_numpy(O).to(torch.bfloat16), lse=torch.from_numpy(L).float())
    run = dict(x=x, out=out, scale=scale, causal=False, cfg={"workload": "decode_d128"},
               state={"n": 7})
    cpu, par = bench.oracle_leg(run, budget_s=0.05)
    assert cpu["unit"] == "GB/s" and "split_merge_7" in cpu["routines"]
    assert par["ok"] and par["split_vs_dense_max_abs"] <= 1e-12
