"""The generated d = 128 forward step (csrc/fwd128_step.inc), checked on the
host: the committed file is what its generator writes, and an independent
reading of each step's instruction list shows that every LDS read has landed
before its destination is touched, that the matrix-core and vector hazards are
covered by enough wait states, that each step reads its own ring slot, and
that it holds the work of one tile step (16 products, 16 exponentials)."""
import importlib.util
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "flashattention_online_softmax_fa_amd", "csrc")
TILEB, ROWB = 8192, 256


def _steps():
    text = open(os.path.join(CSRC, "fwd128_step.inc")).read()
    out = {}
    for u, body in re.findall(r'#define FA_FWD128_STEP_(\d) "(.*)"', text):
        out[int(u)] = body.split("\\n\\t")
    return out


def _regs(tok):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _parse(line):
    """(mnemonic, destination registers, source registers, LDS offset or None)"""
    parts = line.replace(",", " ").split()
    op, args = parts[0], parts[1:]
    off = None
    if args and args[-1].startswith("offset:"):
        off = int(args.pop()[7:])
    if op.startswith("s_"):
        return op, set(), set(), off
    dst = _regs(args[0])
    src = set().union(*[_regs(a) for a in args[1:]]) if len(args) > 1 else set()
    if op.startswith("v_mfma") and args[-1] != "0":
        src |= _regs(args[-1])
    return op, dst, src, off


def test_generated_file_is_current():
    spec = importlib.util.spec_from_file_location("gen", os.path.join(CSRC, "gen_fwd128_step.py"))
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    assert gen.render() == open(os.path.join(CSRC, "fwd128_step.inc")).read()


@pytest.mark.parametrize("u", range(8))
def test_step_waits_and_hazards(u):
    lines = _steps()[u]
    allowed = ("ds_read_b128", "ds_read_b64_tr_b16", "v_mfma_f32_32x32x16_bf16", "v_fma_f32",
               "v_exp_f32", "v_add_f32", "v_cvt_pk_bf16_f32", "v_max_f32", "v_max3_f32",
               "v_mul_f32", "s_nop", "s_waitcnt")
    inflight = []          # destination sets of LDS reads not yet waited for, oldest first
    clock = 0              # wait states issued so far
    last = {}              # register -> (kind of the instruction that last wrote it, clock)
    for line in lines:
        op, dst, src, off = _parse(line)
        assert op in allowed, line
        if op == "s_waitcnt":
            n = int(re.search(r"lgkmcnt\((\d+)\)", line).group(1))
            while len(inflight) > n:
                inflight.pop(0)
            clock += 1
            continue
        if op == "s_nop":
            clock += int(line.split()[1]) + 1
            continue
        for d in inflight:
            assert not (d & (dst | src)), f"step {u}: {line} touches an LDS read in flight"
        kind = ("lds" if op.startswith("ds_") else "mfma" if op.startswith("v_mfma")
                else "trans" if op == "v_exp_f32" else "valu")
        for r in dst | src:
            if r not in last:
                continue
            wk, at = last[r]
            gap = clock - at - 1
            if wk == "mfma" and kind != "mfma":
                assert gap >= 18, f"step {u}: {line} reads a product {gap} wait states after it"
            if wk == "valu" and kind == "mfma" and r in src:
                assert gap >= 2, f"step {u}: {line} takes a vector result after {gap}"
            if wk == "trans" and kind in ("valu", "trans"):
                assert gap >= 1, f"step {u}: {line} takes an exponential after {gap}"
        if kind == "lds":
            inflight.append(dst)
            assert len(inflight) <= 15
        for r in dst:
            last[r] = ("valu" if kind == "lds" else kind, clock)
        clock += 1
    assert not inflight, f"step {u} leaves LDS reads in flight"


@pytest.mark.parametrize("u", range(8))
def test_step_reads_its_slot(u):
    ops = [_parse(x) for x in _steps()[u]]
    k_offs = sorted(o for op, _, _, o in ops if op == "ds_read_b128")
    v_offs = sorted(o for op, _, _, o in ops if op == "ds_read_b64_tr_b16")
    # K of the next tile (slot u+1: fragments 4-7, the first 4 carried in from
    # the step before) and of the one after (slot u+2: fragments 0-3 for the
    # next step), V of this tile (slot u), each in its half of the ring
    assert k_offs == sorted([((u + 1) % 8) * TILEB] * 4 + [((u + 2) % 8) * TILEB] * 4)
    assert v_offs == sorted([u * TILEB] * 8 + [u * TILEB + 16 * ROWB] * 8)
    assert all(o < 1 << 16 for o in k_offs + v_offs)
    # fragments 0-3 of the next tile are read only after the last product that
    # reads the registers they land in
    lines = [_parse(x) for x in _steps()[u]]
    last_s = max(i for i, (op, d, _, _) in enumerate(lines) if op.startswith("v_mfma") and d == set(range(96 + 16 * (1 - u % 2), 112 + 16 * (1 - u % 2))))
    pre = [i for i, (op, _, _, o) in enumerate(lines) if op == "ds_read_b128" and o == ((u + 2) % 8) * TILEB]
    assert min(pre) > last_s
    mfma = [(d, s) for op, d, s, _ in ops if op.startswith("v_mfma")]
    assert len(mfma) == 16
    cur, nxt = set(range(96 + 16 * (u % 2), 112 + 16 * (u % 2))), set(range(96 + 16 * (1 - u % 2), 112 + 16 * (1 - u % 2)))
    assert sum(d == nxt for d, _ in mfma) == 8           # scores of the next tile
    assert sum(d <= set(range(32, 96)) for d, _ in mfma) == 8   # O accumulators
    exps = [d for op, d, _, _ in ops if op == "v_exp_f32"]
    assert len(exps) == 16 and set().union(*exps) == cur  # each current score once
