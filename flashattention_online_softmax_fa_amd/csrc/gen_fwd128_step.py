"""Writes fwd128_step.inc: the mask-free step of the d = 128 forward (one 32-query
block per wave, 32-key tiles, an 8-slot ring of 16 KiB K+V stages) as inline
assembly with its own instruction order.

Run  python gen_fwd128_step.py  to rewrite fwd128_step.inc beside it (the output is committed).

The step of tile t (ring slot u = t % 8):
  S^T of tile t+1 = K Q^T  (8 v_mfma_f32_32x32x16_bf16 over d, K from slot u+1;
                           its first 4 fragments were read by the previous step),
  P = exp2(S c - m) of tile t, in place, with the row sums and the bf16 packing,
  O^T += V^T P^T           (8 products, V^T from slot u read transposed),
  the lane maximum of tile t+1's scores (times c) for the next step's check,
  the first 4 K fragments of tile t+2 (slot u+2) for the next step, read under
  the PV products so that a step starts with its first product.
The order interleaves the score products with the exponentials and reads each
LDS operand well before its product; s_waitcnt and s_nop are placed by the
rules below (the compiler does not see into inline assembly):
  * an LDS read's destination is waited for (lgkmcnt) before any use;
  * a matrix-core result is read by vector code >= 18 wait states later;
  * a vector result feeds a matrix-core operand >= 2 wait states later;
  * a transcendental result feeds vector code >= 1 wait state later.
(The wait-state counts follow the data-hazard tables of AMD's public CDNA3
instruction-set reference for 16-pass matrix instructions, which gfx950
keeps; the GPU parity tests check the result.)  Products chained on one
accumulator need no waits: the matrix pipe forwards srcC between them.
The ring keeps the K tiles of its 8 slots in the first 64 KiB of LDS and the
V tiles in the second, so that one base register per read and a 16-bit
immediate reach every slot.  Registers are fixed (the kernel binds its
variables to them):
  v[0:31] Q fragments, v[32:95] O accumulators, v[96:111] and v[112:127] the two
  score sets, v[128:143] 4 K fragments (reused; they carry the first 4 of the
  next tile from step to step), v[144:183] temporaries (8 V^T fragments, 2 P^T
  fragments), v184/v185 row sums, v186 = -m, v[187:194] LDS addresses of
  the K reads, v[195:202] of the V^T reads (+64 KiB), v203 scratch, v204 the
  lane maximum.
"""
import re

ROWB, TILEB = 256, 8192


def regs_of(op):
    m = re.match(r"v\[(\d+):(\d+)\]", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", op)
    return {int(m.group(1))} if m else set()


class Ins:
    def __init__(self, kind, text, dst=(), src=()):
        self.kind, self.text = kind, text
        self.dst = set().union(*[regs_of(d) for d in dst]) if dst else set()
        self.src = set().union(*[regs_of(s) for s in src]) if src else set()


QF = lambda k: f"v[{4*k}:{4*k+3}]"
OACC = lambda b: f"v[{32+16*b}:{32+16*b+15}]"
SC = lambda st, i=None: f"v[{96+16*st}:{111+16*st}]" if i is None else f"v{96+16*st+i}"
KF = lambda k: f"v[{128+4*(k%4)}:{131+4*(k%4)}]"
VF = lambda ks, b, h=None: (f"v[{144+16*ks+4*b}:{147+16*ks+4*b}]" if h is None
                            else f"v[{144+16*ks+4*b+2*h}:{145+16*ks+4*b+2*h}]")
PF = lambda ks: f"v[{176+4*ks}:{179+4*ks}]"
PFW = lambda ks, w: f"v{176+4*ks+w}"
L = ("v184", "v185")
NEGM, MX, MT = "v186", "v203", "v204"
KOFF = lambda k: f"v{187+k}"
VOFF = lambda b, h: f"v{195+2*b+h}"


def step_ops(u):
    cur, nxt = u % 2, 1 - u % 2
    kimm = ((u + 1) % 8) * TILEB   # K of tile t+1
    vimm = u * TILEB               # V of tile t (the V registers hold the +64 KiB)
    ops = {}
    kpre = ((u + 2) % 8) * TILEB   # K of tile t+2, the first half read ahead for the next step
    for k in range(8):
        ops[f"rk{k}"] = Ins("ds", f"ds_read_b128 {KF(k)}, {KOFF(k)} offset:{kimm}", [KF(k)], [KOFF(k)])
    for k in range(4):
        ops[f"pk{k}"] = Ins("ds", f"ds_read_b128 {KF(k)}, {KOFF(k)} offset:{kpre}", [KF(k)], [KOFF(k)])
    for ks in range(2):
        for b in range(4):
            for h in range(2):
                ops[f"rv{ks}{b}{h}"] = Ins(
                    "ds", f"ds_read_b64_tr_b16 {VF(ks, b, h)}, {VOFF(b, h)} offset:{vimm + ks * 16 * ROWB}",
                    [VF(ks, b, h)], [VOFF(b, h)])
    for k in range(8):
        c = "0" if k == 0 else SC(nxt)
        ops[f"s{k}"] = Ins("mfma", f"v_mfma_f32_32x32x16_bf16 {SC(nxt)}, {KF(k)}, {QF(k)}, {c}",
                           [SC(nxt)], [KF(k), QF(k)] + ([SC(nxt)] if k else []))
    for i in range(16):
        x = SC(cur, i)
        ops[f"f{i}"] = Ins("valu", f"v_fma_f32 {x}, {x}, %[c], {NEGM}", [x], [x, NEGM])
        ops[f"e{i}"] = Ins("trans", f"v_exp_f32 {x}, {x}", [x], [x])
        ops[f"a{i}"] = Ins("valu", f"v_add_f32 {L[i % 2]}, {L[i % 2]}, {x}", [L[i % 2]], [L[i % 2], x])
    for j in range(8):
        ks, w = divmod(j, 4)
        d = PFW(ks, w)
        ops[f"c{j}"] = Ins("valu", f"v_cvt_pk_bf16_f32 {d}, {SC(cur, 2*j)}, {SC(cur, 2*j+1)}",
                           [d], [SC(cur, 2*j), SC(cur, 2*j+1)])
    for ks in range(2):
        for b in range(4):
            ops[f"p{ks}{b}"] = Ins("mfma", f"v_mfma_f32_32x32x16_bf16 {OACC(b)}, {VF(ks, b)}, {PF(ks)}, {OACC(b)}",
                                   [OACC(b)], [VF(ks, b), PF(ks), OACC(b)])
    # lane maximum of the next tile's scores, in the order of the C++ tile_max
    ops["m0"] = Ins("valu", f"v_max_f32 {MX}, {SC(nxt, 0)}, {SC(nxt, 1)}", [MX], [SC(nxt, 0), SC(nxt, 1)])
    for i in range(2, 16, 2):
        ops[f"m{i//2}"] = Ins("valu", f"v_max3_f32 {MX}, {MX}, {SC(nxt, i)}, {SC(nxt, i+1)}",
                              [MX], [MX, SC(nxt, i), SC(nxt, i + 1)])
    ops["mc"] = Ins("valu", f"v_mul_f32 {MT}, %[c], {MX}", [MT], [MX])
    return ops


def order():
    """S products interleaved with the exponentials of the current tile; every
    exponential before the first PV product; the maximum of the next tile after
    its last score product, under the PV products."""
    vre = [f"rv{ks}{b}{h}" for ks in range(2) for b in range(4) for h in range(2)]
    o = vre[:4]   # K fragments 0-3 of tile t+1 were read by the previous step
    el = iter(range(16))
    for k in range(8):
        o += [f"s{k}"]
        i, j = next(el), next(el)
        o += [f"f{i}", f"f{j}", f"e{i}", f"e{j}"]
        if k < 4:
            o += [f"rk{k+4}"]
        o += [v for v in vre[4 + 2 * k:6 + 2 * k]]
        if k >= 1:
            o += [f"a{2*k-2}", f"a{2*k-1}", f"c{k-1}"]
    o += ["a14", "a15", "c7"]
    pv = [f"p{ks}{b}" for ks in range(2) for b in range(4)]
    mx = ["m0"] + [f"m{i}" for i in range(1, 8)] + ["mc"]
    for n in range(8):
        o += [pv[n]]
        o += mx[n:n + 1] if n < 7 else mx[7:]
        if n < 4:  # K fragment n of tile t+2; its register was last read 4 products ago
            o += [f"pk{n}"]
    return o


def emit(names, ops):
    out = []
    ds = []                   # destination registers of the LDS reads in flight, oldest first
    since = {}                # register -> (kind of last writer, wait states since)

    def advance(n):
        for r in list(since):
            k, d = since[r]
            since[r] = (k, d + n)

    for name in names:
        ins = ops[name]
        if ins.kind == "ds" and len(ds) >= 15:  # the counter holds 15 reads at most
            out.append(f"s_waitcnt lgkmcnt({len(ds) - 1})")
            ds = ds[1:]
            advance(1)
        use = ins.src | ins.dst
        last = max((i for i, d in enumerate(ds) if d & use), default=None)
        if last is not None:
            out.append(f"s_waitcnt lgkmcnt({len(ds) - last - 1})")
            ds = ds[last + 1:]
            advance(1)
        need = 0
        for r in ins.src | ins.dst:
            if r in since:
                k, d = since[r]
                if k == "mfma" and ins.kind in ("valu", "trans", "ds"):
                    need = max(need, 18 - d)
                elif k == "valu" and ins.kind == "mfma" and r in ins.src:
                    need = max(need, 2 - d)
                elif k == "trans" and ins.kind in ("valu", "trans"):
                    need = max(need, 1 - d)
        while need > 0:
            n = min(need, 8)
            out.append(f"s_nop {n - 1}")
            advance(n)
            need -= n
        out.append(ins.text)
        advance(1)
        if ins.kind == "ds":
            ds.append(set(ins.dst))
        for r in ins.dst:
            since[r] = ("valu" if ins.kind == "ds" else ins.kind, 0)
    # leave no LDS read in flight, and no matrix-core result closer than 18
    # wait states to the compiler's code that follows
    out.append("s_waitcnt lgkmcnt(0)")
    return out


HEADER = """// fwd128_step.inc -- written by gen_fwd128_step.py; do not edit by hand.
// The mask-free step of the d = 128 forward for ring slot U (see the generator
// for the instruction order, the wait rules and the fixed registers).
"""


def render():
    """The text of fwd128_step.inc."""
    parts = [HEADER]
    for u in range(8):
        body = "\\n\\t".join(emit(order(), step_ops(u)))
        parts.append(f'#define FA_FWD128_STEP_{u} "{body}"\n')
    temps = ", ".join(f'"v{r}"' for r in range(144, 184))
    parts.append(f"// the step's temporaries: V^T fragments, P^T\n#define FA_ASM_TEMPS {temps},\n")
    return "\n".join(parts)


if __name__ == "__main__":
    import os
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fwd128_step.inc")
    with open(out, "w") as f:
        f.write(render())
