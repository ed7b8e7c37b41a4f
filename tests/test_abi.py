"""The C ABI on the host, without a GPU: the library loads, exports every
function include/fa.h declares, and rejects bad arguments before it touches
the HIP runtime (argument checks come first and launch nothing)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
SO = os.path.join(ROOT, "flashattention_online_softmax_fa_amd", "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
FA_F32, FA_BF16 = 0, 1


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(SO):
        pytest.fail("libfa.so is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(SO)
    vp, i64, f32, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    lib.fa_fwd.argtypes = [i, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i, vp]
    lib.fa_fwd_offset.argtypes = [i, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i64, vp]
    lib.fa_fwd_blocked.argtypes = [i, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i, i64,
                                   vp]
    lib.fa_bwd_workspace_size.argtypes = [i, i64, i64, i64, i64]
    lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64, i64,
                           i64, i64, i64, f32, i, vp]
    lib.fa_bwd_offset.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64,
                                  i64, i64, i64, i64, f32, i64, vp]
    lib.fa_bwd_noalloc.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                   i64, f32, i, vp]
    lib.fa_decode_split.argtypes = [i, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32,
                                    vp]
    lib.fa_decode_split_offset.argtypes = [i, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                           i64, f32, i64, vp]
    lib.fa_merge_states.argtypes = [i, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp]
    lib.fa_status_str.argtypes = [i]
    lib.fa_status_str.restype = ctypes.c_char_p
    return lib


def test_header_declares_the_calls():
    assert _declared() == sorted(["fa_fwd", "fa_fwd_offset", "fa_fwd_blocked",
                                  "fa_bwd_workspace_size", "fa_bwd", "fa_bwd_offset",
                                  "fa_bwd_noalloc", "fa_decode_split", "fa_decode_split_offset",
                                  "fa_merge_states", "fa_status_str"])


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_binding_exposes_the_same_names():
    import flashattention_online_softmax_fa_amd as fa
    for name in _declared():
        assert callable(getattr(fa, name)), name
    assert sorted(fa.EXPORTS) == _declared()


def test_status_strings(lib):
    assert lib.fa_status_str(0) == b"FA_OK"
    assert lib.fa_status_str(1) == b"FA_ERR_INVALID_ARG"
    assert lib.fa_status_str(2) == b"FA_ERR_UNSUPPORTED"
    assert lib.fa_status_str(3) == b"FA_ERR_HIP"


# Fake, well-aligned addresses: every call below must be rejected before any
# pointer is used or any HIP call is made.
P = 0x10000000
NULL = None


def fwd(lib, **kw):
    a = dict(dt=FA_BF16, Q=P, K=P, V=P, O=P, L=P, B=1, H=1, Nq=8, Nk=8, d=64, scale=0.125,
             causal=0)
    a.update(kw)
    return lib.fa_fwd(a["dt"], a["Q"], a["K"], a["V"], a["O"], a["L"], a["B"], a["H"], a["Nq"],
                      a["Nk"], a["d"], a["scale"], a["causal"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(Q=NULL), FA_ERR_INVALID_ARG),
    (dict(L=NULL), FA_ERR_INVALID_ARG),
    (dict(B=0), FA_ERR_INVALID_ARG),
    (dict(H=-1), FA_ERR_INVALID_ARG),
    (dict(Nq=0), FA_ERR_INVALID_ARG),
    (dict(Nk=0), FA_ERR_INVALID_ARG),
    (dict(d=0), FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), FA_ERR_INVALID_ARG),
    (dict(causal=2), FA_ERR_INVALID_ARG),
    (dict(dt=7), FA_ERR_INVALID_ARG),
    (dict(Q=P + 8), FA_ERR_INVALID_ARG),          # bf16 needs 16-byte alignment
    (dict(L=P + 2), FA_ERR_INVALID_ARG),
    (dict(d=96), FA_ERR_UNSUPPORTED),             # bf16 tiles exist for d = 64, 128
    (dict(dt=FA_F32, d=129), FA_ERR_UNSUPPORTED),
    (dict(B=1 << 40, H=1 << 30), FA_ERR_INVALID_ARG),  # element count overflow
])
def test_fwd_rejects(lib, kw, want):
    assert fwd(lib, **kw) == want


def test_offset_rejects(lib):
    args = (P, P, P, P, P, 1, 1, 8, 8, 64, 0.125)
    assert lib.fa_fwd_offset(FA_BF16, *args, -1, None) == FA_ERR_INVALID_ARG
    assert lib.fa_fwd_offset(FA_BF16, *args, (1 << 40) + 1, None) == FA_ERR_INVALID_ARG
    assert lib.fa_fwd_offset(FA_BF16, *args[:-2], 96, 0.125, 3, None) == FA_ERR_UNSUPPORTED
    assert lib.fa_fwd_offset(FA_F32, P, P, P, P, P, 1, 1, 8, 8, 129, 0.125, 3,
                             None) == FA_ERR_UNSUPPORTED
    need = lib.fa_bwd_workspace_size(FA_BF16, 1, 1, 8, 64)
    bargs = (P, P, P, P, P, P, P, P, P, P, need, 1, 1, 8, 8, 64, 0.125)
    assert lib.fa_bwd_offset(FA_BF16, *bargs, -5, None) == FA_ERR_INVALID_ARG
    assert lib.fa_bwd_offset(FA_F32, *bargs[:-2], 129, 0.125, 2, None) == FA_ERR_UNSUPPORTED
    assert lib.fa_bwd_offset(FA_BF16, *bargs[:-1], float("nan"), 2, None) == FA_ERR_INVALID_ARG


def test_fwd_blocked_rejects(lib):
    args = (P, P, P, P, P, 1, 1, 8, 8, 16, 0.25, 0)
    assert lib.fa_fwd_blocked(FA_F32, *args, 0, None) == FA_ERR_INVALID_ARG
    assert lib.fa_fwd_blocked(FA_F32, *args, 257, None) == FA_ERR_INVALID_ARG
    assert lib.fa_fwd_blocked(FA_BF16, *args, 4, None) == FA_ERR_UNSUPPORTED


def test_bwd_workspace_size(lib):
    # D and L*log2(e): 2*3*100 floats each -> 2400 B -> 2560 (256-aligned), twice
    assert lib.fa_bwd_workspace_size(FA_BF16, 2, 3, 100, 64) == 2 * 2560
    assert lib.fa_bwd_workspace_size(FA_BF16, 0, 3, 100, 64) == 0


def bwd(lib, **kw):
    need = lib.fa_bwd_workspace_size(FA_BF16, 1, 1, 8, 64)
    a = dict(dt=FA_BF16, ws=P, ws_bytes=need, d=64, Nq=8, scale=0.125, causal=1, dO=P)
    a.update(kw)
    return lib.fa_bwd(a["dt"], P, P, P, P, P, a["dO"], P, P, P, a["ws"], a["ws_bytes"], 1, 1,
                      a["Nq"], 8, a["d"], a["scale"], a["causal"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(ws=NULL), FA_ERR_INVALID_ARG),
    (dict(ws=P + 16), FA_ERR_INVALID_ARG),        # workspace must be 256-aligned
    (dict(ws_bytes=100), FA_ERR_INVALID_ARG),
    (dict(dO=NULL), FA_ERR_INVALID_ARG),
    (dict(scale=float("-inf")), FA_ERR_INVALID_ARG),
    (dict(d=32), FA_ERR_UNSUPPORTED),             # bf16 tiles exist for d = 64, 128
    (dict(dt=FA_F32, d=129), FA_ERR_UNSUPPORTED),  # fp32 path: d <= 128
])
def test_bwd_rejects(lib, kw, want):
    assert bwd(lib, **kw) == want


def bwd_noalloc(lib, **kw):
    a = dict(dt=FA_BF16, d=64, B=1, H=1, Nq=8, scale=0.125, causal=1, dO=P, dQ=P)
    a.update(kw)
    return lib.fa_bwd_noalloc(a["dt"], P, P, P, P, P, a["dO"], a["dQ"], P, P, a["B"], a["H"],
                              a["Nq"], 8, a["d"], a["scale"], a["causal"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(dO=NULL), FA_ERR_INVALID_ARG),
    (dict(dQ=P + 2), FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), FA_ERR_INVALID_ARG),
    (dict(causal=2), FA_ERR_INVALID_ARG),
    (dict(Nq=0), FA_ERR_INVALID_ARG),
    (dict(d=32), FA_ERR_UNSUPPORTED),
    # beyond the fixed array: 2^21 query rows fit, one more does not
    (dict(B=2, H=1 << 10, Nq=(1 << 10) + 1), FA_ERR_INVALID_ARG),
    (dict(B=1, H=1, Nq=(1 << 21) + 1), FA_ERR_INVALID_ARG),
])
def test_bwd_noalloc_rejects(lib, kw, want):
    """Rejected before any HIP call (there is no GPU here): bad arguments as
    for fa_bwd, and sizes whose workspace would not fit the fixed array."""
    assert bwd_noalloc(lib, **kw) == want


def test_bwd_noalloc_limit_matches_binding():
    import flashattention_online_softmax_fa_amd as fa
    text = open(HEADER).read()
    assert "#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)" in text
    assert fa.FA_NOALLOC_SCRATCH_BYTES == 16 << 20
    # 2^21 rows need exactly the whole array
    assert fa.fa_bwd_workspace_size(FA_BF16, 1, 1, 1 << 21, 64) == fa.FA_NOALLOC_SCRATCH_BYTES


def test_decode_rejects(lib):
    def call(n_split=4, d=128, dt=FA_BF16, Q=P, pm=P):
        return lib.fa_decode_split(dt, Q, P, P, pm, P, P, 1, 1, 1, 64, d, n_split, 0.1, None)
    assert call(n_split=0) == FA_ERR_INVALID_ARG     # at least one split
    assert call(n_split=-3) == FA_ERR_INVALID_ARG
    assert call(Q=NULL) == FA_ERR_INVALID_ARG
    assert call(pm=P + 1) == FA_ERR_INVALID_ARG
    assert call(d=80) == FA_ERR_UNSUPPORTED
    assert call(dt=FA_F32, d=200) == FA_ERR_UNSUPPORTED
    assert lib.fa_decode_split_offset(FA_BF16, P, P, P, P, P, P, 1, 1, 1, 64, 64, 4, 0.1, -1,
                                      None) == FA_ERR_INVALID_ARG
    assert lib.fa_decode_split_offset(FA_BF16, P, P, P, P, P, P, 1, 1, 1, 64, 96, 4, 0.1, 63,
                                      None) == FA_ERR_UNSUPPORTED


def test_merge_rejects(lib):
    def call(n_split=4, d=128, O=P):
        return lib.fa_merge_states(FA_BF16, P, P, P, O, P, 1, 1, 1, d, n_split, None)
    assert call(n_split=0) == FA_ERR_INVALID_ARG
    assert call(O=NULL) == FA_ERR_INVALID_ARG
    assert call(O=P + 1) == FA_ERR_INVALID_ARG
    assert call(d=513) == FA_ERR_UNSUPPORTED


STATS_SO = os.path.join(ROOT, "flashattention_online_softmax_fa_amd", "libfa_stats.so")
STATS_HEADER = os.path.join(ROOT, "include", "fa_stats.h")


def test_stats_build_exports():
    """The debug build exports the release calls plus include/fa_stats.h's;
    the release build exports none of the latter."""
    text = re.sub(r"/\*.*?\*/", "", open(STATS_HEADER).read(), flags=re.S)
    stats = sorted(set(re.findall(r"\b(fa_stats_[a-z_0-9]+)\s*\(", text)))
    assert stats == ["fa_stats_read", "fa_stats_reset", "fa_stats_tile"]
    dbg = ctypes.CDLL(STATS_SO)
    for name in _declared() + stats:
        assert hasattr(dbg, name), name
    rel = ctypes.CDLL(SO)
    for name in stats:
        assert not hasattr(rel, name), name


def test_stats_tile_shapes():
    """fa_stats_tile is host-only: block shapes of the counted kernels."""
    dbg = ctypes.CDLL(STATS_SO)
    i64p = ctypes.POINTER(ctypes.c_int64)
    dbg.fa_stats_tile.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int, i64p,
                                  i64p]
    r, c = ctypes.c_int64(), ctypes.c_int64()
    for kind in (0, 1, 2, 3):
        for d in (64, 128):
            for causal in (0, 1):
                assert dbg.fa_stats_tile(kind, FA_BF16, d, causal, ctypes.byref(r),
                                         ctypes.byref(c)) == FA_OK
                assert r.value >= 32 and r.value % 32 == 0 and c.value % 32 == 0
    # a forward workgroup holds whole wavefront blocks with the same key tile
    for d in (64, 128):
        wr, wc = ctypes.c_int64(), ctypes.c_int64()
        assert dbg.fa_stats_tile(0, FA_BF16, d, 0, ctypes.byref(r), ctypes.byref(c)) == FA_OK
        assert dbg.fa_stats_tile(3, FA_BF16, d, 0, ctypes.byref(wr), ctypes.byref(wc)) == FA_OK
        assert wr.value % r.value == 0 and wr.value >= 4 * r.value and wc.value == c.value
    assert dbg.fa_stats_tile(0, FA_F32, 64, 0, ctypes.byref(r), ctypes.byref(c)) == \
        FA_ERR_UNSUPPORTED
    assert dbg.fa_stats_tile(4, FA_BF16, 64, 0, ctypes.byref(r), ctypes.byref(c)) == \
        FA_ERR_INVALID_ARG
    assert dbg.fa_stats_tile(0, FA_BF16, 64, 0, None, ctypes.byref(c)) == FA_ERR_INVALID_ARG


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: any other --gpus exits with status 2 and a
    message, before touching the GPU."""
    import subprocess
    import sys as _sys
    r = subprocess.run([_sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr


def test_bench_reads_shader_clock(tmp_path):
    """The clock bench.py reports is the pp_dpm_sclk line the driver marks
    as current, both at a DPM level and in deep sleep; the matrix peak is
    scaled by it."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 2247Mhz *\n")
    assert bench.read_sclk(str(f)) == 2247.0
    f.write_text("S: 103Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    assert bench.read_sclk(str(f)) == 103.0
    f.write_text("0: 500Mhz\n1: 2400Mhz\n")
    assert bench.read_sclk(str(f)) is None
    assert bench.read_sclk(str(tmp_path / "missing")) is None
    run = {"work": 1e12, "unit": "TFLOP/s"}        # 1 TFLOP per step
    rf = {"bound": "mfma", "peak": 2500.0}
    bench.add_clock(rf, run, (2100.0, 1.0))       # 1 ms per step: 1000 TFLOP/s
    assert rf["peak_at_sclk"] == 2187.5 and rf["frac_at_sclk"] == round(1000 / 2187.5, 4)
    assert rf["sustained_ms"] == 1.0
    rf = {"bound": "hbm", "peak": 8000.0}
    bench.add_clock(rf, {"work": 7e9, "unit": "GB/s"}, (2100.0, 1.0))
    assert rf["sclk_mhz"] == 2100.0 and "frac_at_sclk" not in rf
    rf = {"bound": "mfma", "peak": 2500.0}
    bench.add_clock(rf, run, None)
    assert rf["sclk_mhz"] is None


def test_variant_build_rejects_bad_arguments():
    """build.py --variant takes a plain name and -DFA_... definitions only
    (checked before anything is compiled); FA_LIBRARY selects the library the
    package loads, and a missing one fails the import (no fallback)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "fa_build", os.path.join(ROOT, "flashattention_online_softmax_fa_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    with pytest.raises(ValueError):
        b.build_variant("../x", ["-DFA_FWD_WG64=4"])
    with pytest.raises(ValueError):
        b.build_variant("ok", ["-O0"])
    with pytest.raises(ValueError):
        b.build_variant("ok", ["-DNDEBUG"])
    import subprocess
    import sys as _sys
    env = dict(os.environ, FA_LIBRARY=os.path.join(ROOT, "no_such_libfa.so"))
    r = subprocess.run([_sys.executable, "-c", "import flashattention_online_softmax_fa_amd"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "no_such_libfa.so is not built" in r.stderr


def test_traffic_hash_ignores_comments_only(tmp_path):
    """The source hash that keeps measured HBM traffic valid is blind to
    comments and white space and changes with any change to the code,
    including the shared device headers."""
    import importlib.util
    import shutil
    spec = importlib.util.spec_from_file_location("bench_mod2", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    src = os.path.join(ROOT, "flashattention_online_softmax_fa_amd", "csrc")
    dst = tmp_path / "flashattention_online_softmax_fa_amd" / "csrc"
    dst.mkdir(parents=True)
    for f in ("bwd.hip", "fa_device.h", "fa_internal.h"):
        shutil.copy(os.path.join(src, f), dst / f)
    bench.ROOT = str(tmp_path)
    h0 = bench.source_hash("bwd.hip")
    p = dst / "bwd.hip"
    p.write_text(p.read_text() + "\n// a new comment\n/* and a block\n comment */\n\n")
    assert bench.source_hash("bwd.hip") == h0
    p.write_text(p.read_text().replace("constexpr int ST = T::ST;", "constexpr int ST = T::ST + 0;", 1))
    assert bench.source_hash("bwd.hip") != h0
    p.write_text(p.read_text().replace("constexpr int ST = T::ST + 0;", "constexpr int ST = T::ST;", 1))
    assert bench.source_hash("bwd.hip") == h0
    d = dst / "fa_device.h"
    d.write_text(d.read_text().replace("kLog2e = 1.4426950408889634f", "kLog2e = 1.4426950408889635f"))
    assert bench.source_hash("bwd.hip") != h0


def test_traffic_hash_covers_generated_step(tmp_path):
    """The forward's hash changes when the generated step it includes changes."""
    import importlib.util
    import shutil
    spec = importlib.util.spec_from_file_location("bench_mod3", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    src = os.path.join(ROOT, "flashattention_online_softmax_fa_amd", "csrc")
    dst = tmp_path / "flashattention_online_softmax_fa_amd" / "csrc"
    dst.mkdir(parents=True)
    for f in ("fwd_bf16.hip", "fa_device.h", "fa_internal.h", "fwd128_step.inc"):
        shutil.copy(os.path.join(src, f), dst / f)
    bench.ROOT = str(tmp_path)
    h0 = bench.source_hash("fwd_bf16.hip")
    p = dst / "fwd128_step.inc"
    p.write_text(p.read_text().replace("s_waitcnt lgkmcnt(0)", "s_waitcnt lgkmcnt(1)", 1))
    assert bench.source_hash("fwd_bf16.hip") != h0
