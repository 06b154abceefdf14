"""The C ABI without a GPU: libgemm.so loads, exports every function that
include/gemm.h declares, validates arguments before any HIP call, takes the
quick returns, and reports the chosen variant.  No test here launches work."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm.h")

FAKE = 0x10000        # a non-null, 64 KiB-aligned address; never dereferenced here


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("gemm_f32", "gemm_f16", "gemm_status_string", "gemm_describe", "gemm_set_load_mode",
              "gemm_set_tile_config"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import dense_gemm_fp32_amd as dg
    out = subprocess.run(["nm", "-D", "--defined-only", dg.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    for n in _declared():
        assert n in exported, n
        from dense_gemm_fp32_amd import binding
        assert hasattr(binding._lib, n)
    assert set(dg.EXPORTS) <= exported


def test_single_hip_runtime_loaded():
    import dense_gemm_fp32_amd as dg  # noqa: F401  (loads torch, then libgemm.so)
    dg.gemm_status_string(0)
    maps = open("/proc/self/maps").read()
    libs = set(re.findall(r"(\S*libamdhip64\S*)", maps))
    assert len(libs) == 1, libs


CASES = [
    # (expected, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
    (-1, -1, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4),
    (-2, 4, -1, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4),
    (-3, 4, 4, -1, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4),
    (-6, 4, 4, 8, 1.0, FAKE, 7, FAKE, 4, 0.0, FAKE, 4),
    (-6, 4, 4, 0, 1.0, FAKE, 0, FAKE, 4, 0.0, FAKE, 4),
    (-8, 4, 9, 4, 1.0, FAKE, 4, FAKE, 8, 0.0, FAKE, 9),
    (-11, 4, 9, 4, 1.0, FAKE, 4, FAKE, 9, 0.0, FAKE, 8),
    (-5, 4, 4, 4, 1.0, None, 4, FAKE, 4, 0.0, FAKE, 4),
    (-7, 4, 4, 4, 1.0, FAKE, 4, None, 4, 0.0, FAKE, 4),
    (-10, 4, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, None, 4),
    (-10, 4, 4, 4, 0.0, None, 4, None, 4, 0.5, None, 4),   # scale path needs C
    (-1, -1, -1, -1, 1.0, None, 0, None, 0, 0.0, None, 0),  # first failure wins
    (-6, 4, 4, 8, 1.0, None, 7, None, 3, 0.0, None, 3),
    # quick returns: nothing touched, no launch, null pointers allowed
    (0, 0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4),
    (0, 4, 0, 4, 1.0, None, 4, None, 1, 0.0, None, 1),
    (0, 4, 4, 4, 0.0, None, 4, None, 4, 1.0, None, 4),
    (0, 4, 4, 0, 1.0, None, 1, None, 4, 1.0, None, 4),
]


@pytest.mark.parametrize("fn", ["gemm_f32", "gemm_f16", "gemm_f16f32", "gemm_f32_valu",
                                "gemm_f32_noalloc"])
@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_argument_checks_and_quick_returns(fn, case):
    import dense_gemm_fp32_amd as dg
    expected, *args = case
    assert getattr(dg, fn)(*args, None) == expected
    # gemm_describe applies the same checks
    rc, text = dg.gemm_describe({"gemm_f32": "f32", "gemm_f16": "f16", "gemm_f16f32": "f16f32",
                                 "gemm_f32_valu": "f32", "gemm_f32_noalloc": "f32"}[fn], *args)
    assert rc == expected
    if expected < 0:
        assert text.startswith("invalid")


COLMAJOR_CASES = [
    # (expected, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc): lda >= M, ldb >= K, ldc >= M
    (-1, -1, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4),
    (-6, 5, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 5),
    (-8, 4, 4, 9, 1.0, FAKE, 4, FAKE, 8, 0.0, FAKE, 4),
    (-11, 9, 4, 4, 1.0, FAKE, 9, FAKE, 4, 0.0, FAKE, 8),
    (-5, 4, 4, 4, 1.0, None, 4, FAKE, 4, 0.0, FAKE, 4),
    (-7, 4, 4, 4, 1.0, FAKE, 4, None, 4, 0.0, FAKE, 4),
    (-10, 4, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, None, 4),
    # a row-major-valid call that is invalid column-major (lda = K < M)
    (-6, 8, 2, 3, 1.0, FAKE, 3, FAKE, 2, 0.0, FAKE, 8),
    (0, 0, 4, 4, 1.0, None, 1, None, 4, 0.0, None, 1),
    (0, 4, 4, 4, 0.0, None, 4, None, 4, 1.0, None, 4),
]


@pytest.mark.parametrize("fn", ["gemm_f32_colmajor", "gemm_f16_colmajor", "gemm_f16f32_colmajor"])
@pytest.mark.parametrize("case", COLMAJOR_CASES, ids=[str(i) for i in range(len(COLMAJOR_CASES))])
def test_colmajor_argument_checks(fn, case):
    import dense_gemm_fp32_amd as dg
    expected, *args = case
    assert getattr(dg, fn)(*args, None) == expected


def test_status_strings():
    import dense_gemm_fp32_amd as dg
    assert dg.gemm_status_string(0) == "success"
    for code in (-1, -2, -3, -5, -6, -7, -8, -10, -11):
        s = dg.gemm_status_string(code)
        assert s.startswith("invalid argument %d" % -code), s
    assert dg.gemm_status_string(-99) == "unknown status"
    assert len(dg.gemm_status_string(1)) > 0


def test_describe_picks_vector_or_scalar_loads():
    """Load widths per operand from its leading dimension and base (operand
    copies switched off: they would replace an unaligned fp32 operand by an
    aligned copy)."""
    import dense_gemm_fp32_amd as dg
    prev = dg.gemm_set_pack(1)
    try:
        _load_widths(dg)
    finally:
        dg.gemm_set_pack(prev)


def _load_widths(dg):
    rc, t = dg.gemm_describe("f32", 4096, 4096, 4096, 1.0, FAKE, 4096, FAKE, 4096, 0.0, FAKE, 4096)
    assert rc == 0 and "A:vec4" in t and "B:vec4" in t and "C:vec" in t and "beta0" in t
    # ragged, unaligned leading dimensions (K+13, N+5, N+3): lda = 530 is even,
    # so A takes element pairs (8 bytes of fp32, 4 of fp16; the SGEMM summary's
    # layout section: 64-bit accesses need an even leading dimension); the odd
    # ldb and ldc leave B and C element-wise
    rc, t = dg.gemm_describe("f32", 1000, 3000, 517, 1.5, FAKE, 530, FAKE, 3005, -0.75, FAKE, 3003)
    assert rc == 0 and "A:pair2" in t and "B:scalar1" in t and "C:scalar1" in t
    rc, t = dg.gemm_describe("f16", 1000, 3000, 517, 1.5, FAKE, 530, FAKE, 3005, -0.75, FAKE, 3003)
    assert rc == 0 and "A:pair2" in t and "B:scalar1" in t and "C:scalar1" in t
    # odd lda, even ldb: the other way round; a base aligned to one element only
    # keeps single elements even with an even leading dimension
    rc, t = dg.gemm_describe("f16", 1000, 3000, 517, 1.5, FAKE, 531, FAKE, 3006, -0.75, FAKE, 3003)
    assert "A:scalar1" in t and "B:pair2" in t
    rc, t = dg.gemm_describe("f32", 1000, 3000, 517, 1.5, FAKE + 4, 530, FAKE, 3005, -0.75, FAKE, 3003)
    assert "A:scalar1" in t
    rc, t = dg.gemm_describe("f16", 1000, 3000, 517, 1.5, FAKE + 2, 530, FAKE, 3005, -0.75, FAKE, 3003)
    assert "A:scalar1" in t
    rc, t = dg.gemm_describe("f16", 4096, 4096, 4096, 1.0, FAKE, 4096, FAKE, 4096, 0.5, FAKE, 4096)
    assert rc == 0 and "A:vec8" in t and "B:vec8" in t and "beta0" not in t
    # misaligned base pointer: scalar for that operand only
    rc, t = dg.gemm_describe("f32", 256, 256, 256, 1.0, FAKE + 4, 256, FAKE, 256, 0.0, FAKE, 256)
    assert "A:scalar1" in t and "B:vec4" in t
    # fp16 inputs with an fp32 C: 16-byte C accesses need a 16-byte aligned base
    rc, t = dg.gemm_describe("f16f32", 4096, 4096, 4096, 1.0, FAKE, 4096, FAKE, 4096, 0.5, FAKE, 4096)
    assert rc == 0 and "out f32" in t and "C:vec4" in t
    rc, t = dg.gemm_describe("f16f32", 4096, 4096, 4096, 1.0, FAKE, 4096, FAKE, 4096, 0.5, FAKE + 8, 4096)
    assert "C:scalar1" in t
    assert dg.gemm_describe(3, 8, 8, 8, 1.0, FAKE, 8, FAKE, 8, 0.0, FAKE, 8)[1].startswith("invalid")
    # degenerate routes
    assert "scale" in dg.gemm_describe("f32", 8, 8, 0, 1.0, None, 1, None, 8, 2.0, FAKE, 8)[1]
    assert "zero fill" in dg.gemm_describe("f32", 8, 8, 8, 0.0, None, 8, None, 8, 0.0, FAKE, 8)[1]
    assert "no-op" in dg.gemm_describe("f16", 8, 8, 8, 0.0, None, 8, None, 8, 1.0, None, 8)[1]


def test_force_scalar_mode_switch():
    import dense_gemm_fp32_amd as dg
    prev = dg.gemm_set_load_mode(1)
    try:
        rc, t = dg.gemm_describe("f32", 512, 512, 512, 1.0, FAKE, 512, FAKE, 512, 0.0, FAKE, 512)
        assert "A:scalar1" in t and "B:scalar1" in t and "C:scalar1" in t
    finally:
        assert dg.gemm_set_load_mode(prev) == 1
    assert dg.gemm_set_load_mode(7) == -1


def test_torch_wrapper_rejects_bad_layouts():
    import torch
    import dense_gemm_fp32_amd as dg
    A = torch.zeros(4, 6)
    with pytest.raises(ValueError):
        dg.gemm(A.t(), torch.zeros(4, 5), torch.zeros(6, 5))      # stride(1) != 1
    with pytest.raises(ValueError):
        dg.gemm(A, torch.zeros(5, 5), torch.zeros(4, 5))           # K mismatch
    with pytest.raises(ValueError):
        dg.gemm(A.double(), torch.zeros(6, 5).double(), torch.zeros(4, 5).double())


def test_missing_library_fails_loudly(tmp_path):
    """Without libgemm.so the binding raises instead of falling back."""
    import shutil
    import sys
    pkg = tmp_path / "dense_gemm_fp32_amd"
    shutil.copytree(os.path.join(ROOT, "dense_gemm_fp32_amd"), pkg,
                    ignore=shutil.ignore_patterns("*.so", "_build", "__pycache__"))
    code = ("import sys; sys.path.insert(0, %r); import dense_gemm_fp32_amd as d; d.gemm_f32" %
            str(tmp_path))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True)
    assert r.returncode != 0 and "not built" in r.stderr


def test_only_inline_asm_touches_m0():
    """The fp16 kernel sets m0 in inline assembly; no compiler-generated
    instruction of that translation unit may use m0 (checked on the gfx950
    assembly of the current source)."""
    import concurrent.futures
    from dense_gemm_fp32_amd import build as b
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(b.M0_ASM_SOURCES)) as ex:
        for f in [ex.submit(b.check_m0_only_in_asm, src) for src in b.M0_ASM_SOURCES]:
            f.result()


def test_library_override_loads_the_named_build(tmp_path):
    """DENSE_GEMM_FP32_AMD_LIB makes the binding load that file (the
    LDS-poison debug build runs the GPU suite this way) and only that file;
    a path that does not exist fails loudly."""
    import sys
    from dense_gemm_fp32_amd.build import LIB
    alt = tmp_path / "libgemm_copy.so"
    alt.write_bytes(open(LIB, "rb").read())
    code = ("import dense_gemm_fp32_amd as dg; dg.gemm_status_string(0); "
            "m = open('/proc/self/maps').read(); "
            "print(dg.LIB_PATH in m, %r in m)" % LIB)
    env = dict(os.environ, DENSE_GEMM_FP32_AMD_LIB=str(alt))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split() == ["True", "False"], r.stdout
    env["DENSE_GEMM_FP32_AMD_LIB"] = str(tmp_path / "missing.so")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0 and "ImportError" in r.stderr


def test_spill_check_reads_kernel_descriptors():
    """The build's spill check finds every kernel descriptor in gfx950
    assembly and refuses a GEMM kernel with a scratch segment (a synthetic
    descriptor as negative control; the real sources pass in
    test_only_inline_asm_touches_m0, which runs the same check)."""
    from dense_gemm_fp32_amd import build as b
    text = "\n".join([
        ".amdhsa_kernel _ZN5dgemm10hgemm_mfmaIXEEvNS_10GemmParamsE",
        "  .amdhsa_private_segment_fixed_size 0",
        ".end_amdhsa_kernel",
        ".amdhsa_kernel _ZN5dgemm10sgemm_mfmaIXEEvNS_10GemmParamsE",
        "  .amdhsa_private_segment_fixed_size 48",
        ".end_amdhsa_kernel",
        ".amdhsa_kernel _ZN5dgemm14scale_f32_kernelEv",
        "  .amdhsa_private_segment_fixed_size 16",
        ".end_amdhsa_kernel"])
    sizes = b.scratch_sizes(text)
    assert sizes == {"_ZN5dgemm10hgemm_mfmaIXEEvNS_10GemmParamsE": 0,
                     "_ZN5dgemm10sgemm_mfmaIXEEvNS_10GemmParamsE": 48,
                     "_ZN5dgemm14scale_f32_kernelEv": 16}
    with pytest.raises(RuntimeError, match="sgemm_mfma"):
        b.check_no_spills(text, "synthetic")
    b.check_no_spills(text.replace("fixed_size 48", "fixed_size 0"), "synthetic")
    with pytest.raises(RuntimeError, match="no kernel descriptors"):
        b.check_no_spills("", "empty")


def test_register_budget_check_reads_kernel_descriptors():
    """The build's register check compares each GEMM kernel's registers per
    lane with the budget of its tile's occupancy (512 registers per SIMD lane
    over the waves a SIMD is meant to hold) and refuses one over budget or
    with no occupancy entry (synthetic descriptors; the real sources pass in
    test_only_inline_asm_touches_m0, which runs the same check)."""
    from dense_gemm_fp32_amd import build as b
    assert b.register_budget(3, 4) == 168 and b.register_budget(1, 8) == 256
    assert b.register_budget(2, 4) == 256 and b.register_budget(1, 4) == 512
    mid = "_ZN5dgemm10sgemm_mfmaINS_7S32TileILi128ELi128ELi16ELi2ELi2ELi3ELi8ELb0EEELb0ELb0ELb1EEEvNS_10GemmParamsE"
    text = "\n".join([".amdhsa_kernel " + mid, "  .amdhsa_next_free_vgpr 168", ".end_amdhsa_kernel",
                      ".amdhsa_kernel _ZN5dgemm14scale_f32_kernelEv", "  .amdhsa_next_free_vgpr 400",
                      ".end_amdhsa_kernel"])
    assert b.register_counts(text) == {mid: 168, "_ZN5dgemm14scale_f32_kernelEv": 400}
    b.check_register_budget(text, "synthetic")          # at the budget; other kernels ignored
    with pytest.raises(RuntimeError, match="budget 168"):
        b.check_register_budget(text.replace("vgpr 168", "vgpr 176"), "synthetic")
    with pytest.raises(RuntimeError, match="no occupancy entry"):
        b.check_register_budget(text.replace("ILi128ELi128ELi16E", "ILi96ELi96ELi16E"), "synthetic")


def test_tile_table_choice_and_override():
    import dense_gemm_fp32_amd as dg
    def name(dt, n):
        return dg.gemm_describe(dt, n, n, n, 1.0, FAKE, n, FAKE, n, 0.0, FAKE, n)[1]
    assert "256x256x32" in name("f32", 4096) and "128x128x16" in name("f32", 3072)
    # past three and a third 64x64 tiles per CU, up to two 128x64 ones: the
    # four-wave 128x64 tile
    for n in (1888, 1920, 2048):
        assert "128x64x32 4 waves" in name("f32", n) and "split" not in name("f32", n), n
    # one to three 64x64 tiles per CU: that tile with four 32x32 waves,
    # unsplit; up to two per CU in 64-k steps through two slots
    for n in (1024, 1280):
        assert "64x64x64 4 waves 2 slots" in name("f32", n) and "split" not in name("f32", n), n
    for n in (1536, 1664, 1792):
        assert "64x64x32 4 waves 3 slots" in name("f32", n) and "split" not in name("f32", n), n
    for n in (1888, 768):
        assert "64x64x32 4 waves" not in name("f32", n) and "64x64x64" not in name("f32", n), n
    # the 32x32 tile, in 64-k steps up to 2.25 of them per CU
    assert "32x32x64 1 wave 2 slots" in name("f32", 256) and "32x32x64" in name("f32", 64)
    assert "32x32x32 1 wave 3 slots" in name("f32", 864)
    assert "split" not in name("f32", 256) and "split" not in name("f32", 768)
    # K split where the grid leaves CUs idle and K is long enough
    t = dg.gemm_describe("f32", 1024, 1024, 4096, 1.0, FAKE, 4096, FAKE, 1024, 0.0, FAKE, 1024)[1]
    assert "128x128x16" in t and "split-K 8" in t, t
    t = dg.gemm_describe("f32", 2304, 2304, 5000, 1.0, FAKE, 5000, FAKE, 2304, 0.0, FAKE, 2304)[1]
    assert "256x128x32" in t and "split-K 3" in t, t
    assert "split" not in name("f32", 4096) and "split" not in name("f16", 4096)
    assert "split" not in name("f16", 1536)
    assert "128x128x16" in name("f32", 3072) and "128x128x16" in name("f32", 4480)
    # the last round of 2944^3 (529 tiles: 2 rounds + 17) runs split; 5120^3
    # takes the 256x256 tile (400 tiles) with Stream-K after its first round
    # (test_stream_k_by_size_and_switches)
    assert "last round split-K 15" in name("f32", 2944) and "split" not in name("f32", 8192)
    assert "256x256x32" in name("f32", 5120) and "stream-K after 256 whole tiles" in name("f32", 5120)
    assert "256x256x32" in name("f32", 8192) and "256x128x32" in name("f32", 7808)
    assert "256x256x64" in name("f16", 4096) and "256x256x64" in name("f16", 3072)
    # the large fp16 tile: 16x16x32 blocks when its workgroups fill the CUs,
    # 32x32x16 blocks when part of the chip idles (the clock then stays high)
    assert "mfma16x16x32" in name("f16", 4096) and "mfma32x32x16" in name("f16", 3072)
    assert "mfma16x16x32" in name("f16", 8192) and "mfma16x16x32" in name("f16", 5120)
    assert "128x128x32" in name("f16", 2048) and "64x128x32" in name("f16", 512)
    prev = dg.gemm_set_tile_config(1)
    try:
        assert "256x128x32" in name("f32", 256) and "256x256x64" in name("f16", 256)
        dg.gemm_set_tile_config(3)
        assert "64x64x32" in name("f32", 4096)
        dg.gemm_set_tile_config(6)
        assert "256x256x32" in name("f32", 256) and "256x256x64" in name("f16", 256)
        dg.gemm_set_tile_config(4)
        assert "32x32x32" in name("f32", 4096) and "64x128x32" in name("f16", 4096)
        dg.gemm_set_tile_config(7)
        assert "64x64x32 4 waves" in name("f32", 4096) and "64x128x32" in name("f16", 4096)
        dg.gemm_set_tile_config(8)
        assert "128x64x32 4 waves" in name("f32", 4096) and "128x128x32" in name("f16", 4096)
        dg.gemm_set_tile_config(9)
        assert "64x64x64 4 waves 2 slots" in name("f32", 4096) and "64x128x32" in name("f16", 4096)
        dg.gemm_set_tile_config(10)
        assert "32x32x64 1 wave 2 slots" in name("f32", 4096) and "64x128x32" in name("f16", 4096)
    finally:
        dg.gemm_set_tile_config(prev)
    assert dg.gemm_set_tile_config(11) == -1 and dg.gemm_set_tile_config(-1) == -1


def test_staged_calls_split_the_medium_tile():
    """Unaligned operands (element-wise loads, operand copies switched off):
    fp32 grids under three 128x128 tiles per CU take that tile with the K
    split of least estimated time, fp16 grids under 1.5 take it with the
    smallest split reaching 1.5 workgroups per CU; larger grids keep the
    direct-path choice."""
    import dense_gemm_fp32_amd as dg
    prev_pack = dg.gemm_set_pack(1)
    try:
        _staged_choices(dg)
    finally:
        dg.gemm_set_pack(prev_pack)


def _staged_choices(dg):
    def d(M, N, K):
        return dg.gemm_describe("f32", M, N, K, 1.5, FAKE, K + 13, FAKE, N + 5, -0.75, FAKE, N + 3)[1]
    for (M, N, K), S in [((1000, 3000, 517), 4), ((2000, 2000, 1000), 3), ((3000, 3000, 3000), 4),
                         ((1000, 1000, 4000), 8), ((517, 3000, 1000), 4)]:
        t = d(M, N, K)
        assert "128x128x16" in t and ("split-K %d" % S) in t and "scalar1" in t, (M, N, K, t)
    assert "256x256x32" in d(4096, 4096, 4096) and "split" not in d(4096, 4096, 4096)
    assert "32x32x" in d(300, 300, 300)        # fewer 32x32 tiles than CUs: latency-bound
    # a misaligned base alone makes the call staged too
    t = dg.gemm_describe("f32", 1000, 3000, 512, 1.0, FAKE + 4, 512, FAKE, 3000, 0.0, FAKE, 3000)[1]
    assert "A:scalar1" in t and "split-K" in t
    # fp16: the 128x128 tile with the smallest split reaching 1.5 workgroups per CU
    def h(M, N, K):
        return dg.gemm_describe("f16", M, N, K, 1.5, FAKE, K + 13, FAKE, N + 5, -0.75, FAKE, N + 3)[1]
    for (M, N, K), S in [((1000, 3000, 517), 2), ((2000, 2000, 1000), 2), ((1500, 1500, 1500), 3),
                         ((517, 3000, 1000), 4), ((1000, 1000, 4000), 4)]:
        t = h(M, N, K)
        assert "128x128x32" in t and ("split-K %d" % S) in t and "scalar1" in t, (M, N, K, t)
    assert "256x256x64" in h(3000, 3000, 3000) and "split" not in h(3000, 3000, 3000)
    assert "64x128x32" in h(100, 100, 100)
    # forced tile or split settings still win
    prev = dg.gemm_set_split(1)
    try:
        assert "split" not in d(1000, 3000, 517) and "split" not in h(1000, 3000, 517)
    finally:
        dg.gemm_set_split(prev)


def test_wide_short_problems_take_the_four_wave_64x64_tile():
    """Aligned problems whose 64x64 tiles give every CU one to three of them
    (and whose K is not deeper than twice max(M, N)) take that tile with four
    32x32 waves, unsplit; beyond three per CU, or with fewer tiles than CUs,
    the other rules decide (wide, short problems whose 128x128 tiles leave CUs
    idle then split that tile in chunks of at least 512 k)."""
    import dense_gemm_fp32_amd as dg
    def d(M, N, K):
        return dg.gemm_describe("f32", M, N, K, 1.0, FAKE, K, FAKE, N, 0.0, FAKE, N)[1]
    for shape in [(517, 3000, 1000), (256, 8192, 1024), (128, 16384, 4096), (384, 3000, 600),
                  (256, 4096, 2048), (1000, 3000, 520), (1000, 1000, 1000)]:
        t = d(*shape)
        q = ((shape[0] + 63) // 64) * ((shape[1] + 63) // 64)
        # up to two tiles per CU in 64-k steps (two slots), else 32-k steps
        tile = "64x64x64 4 waves 2 slots" if q <= 512 else "64x64x32 4 waves 3 slots"
        assert tile in t and "split" not in t, (shape, t)
    assert "64x64x" not in d(1000, 8000, 700)              # 2000 tiles: over three per CU
    assert "64x64x" not in d(1024, 1024, 4096)             # deep K: the 128x128 tile in chunks
    t = d(2048, 384, 2048)                                 # 192 tiles, K 2048: the split stays
    assert "128x128x16" in t and "split-K" in t, t


def test_grids_under_one_round_take_the_four_wave_64x64_tile():
    """Grids of 170 to 255 64x64 tiles with K <= 1.5 max(M, N) take that tile
    with four 32x32 waves, unsplit, where the model would put a fourth 32x32
    workgroup on some CUs or split K at K <= 1536; grids under one round of
    them, with K <= max(M, N), take it in place of an unsplit larger tile
    that leaves over half the CUs idle; with at most three 32x32 tiles per
    CU or longer K the model's choice stands."""
    import dense_gemm_fp32_amd as dg
    def d(M, N, K):
        return dg.gemm_describe("f32", M, N, K, 1.0, FAKE, K, FAKE, N, 0.0, FAKE, N)[1]
    for shape in [(896, 896, 896), (928, 928, 928), (960, 960, 960), (600, 1600, 800),
                  (800, 1200, 1000), (1024, 768, 1024), (1000, 700, 1200), (960, 1024, 1400)]:
        t = d(*shape)
        assert "64x64x64 4 waves 2 slots" in t and "split" not in t, (shape, t)
    # 864^3: 729 32x32 tiles, at most three per CU; 832^3: 169 64x64 tiles;
    # 768^3: 576 32x32 tiles, which run in 64-k steps
    for n in (864, 832):
        assert "32x32x32 1 wave 3 slots" in d(n, n, n), n
    assert "32x32x64 1 wave 2 slots" in d(768, 768, 768)
    # longer K keeps the K split
    for shape in [(2048, 384, 2048), (768, 1024, 2048), (896, 896, 3000)]:
        t = d(*shape)
        assert "128x128x16" in t and "split-K" in t, (shape, t)
    # an unsplit larger tile that would leave over half the CUs idle, K <=
    # max(M, N): 512x1024x256 (32 128x128 tiles), 64x8192x512 (64 256x128
    # tiles), 128x8192x256, 2048x512x256, 200x3000x300
    for shape in [(512, 1024, 256), (64, 8192, 512), (128, 8192, 256), (2048, 512, 256),
                  (200, 3000, 300)]:
        t = d(*shape)
        assert "64x64x64 4 waves 2 slots" in t and "split" not in t, (shape, t)
    # small squares keep the 32x32 tile (in 64-k steps: at most 2.25 per CU)
    for n in (256, 512, 768):
        assert "32x32x64 1 wave 2 slots" in d(n, n, n), n
    # the switches that force a split or disable the last-round split leave
    # the model's choice
    prev = dg.gemm_set_tail_split(1)
    try:
        assert "32x32x32" in d(896, 896, 896)
        assert "128x128x16" in d(512, 1024, 256)
    finally:
        dg.gemm_set_tail_split(prev)


def test_split_choice_and_override():
    import dense_gemm_fp32_amd as dg
    def d(dt, M, N, K):
        return dg.gemm_describe(dt, M, N, K, 1.0, FAKE, K, FAKE, N, 0.0, FAKE, N)[1]
    assert "split-K 8" in d("f16", 1024, 1024, 8192) and "split-K 4" in d("f32", 512, 512, 8192)
    assert "split" not in d("f32", 1000, 3000, 512)
    prev = dg.gemm_set_split(1)
    try:
        assert "split" not in d("f16", 1024, 1024, 8192)
        dg.gemm_set_split(5)
        assert "split-K 5" in d("f32", 4096, 4096, 4096)
        assert "split-K 2" in d("f32", 64, 64, 40)       # only two 32-deep K steps
        assert "split" not in d("f32", 64, 64, 16)       # one K step: nothing to split
    finally:
        dg.gemm_set_split(prev)
    assert dg.gemm_set_split(65) == -1 and dg.gemm_set_split(-1) == -1


def test_probe_argument_checks():
    """gemm_probe_mfma validates its arguments in order before any HIP call."""
    import ctypes
    from dense_gemm_fp32_amd import binding
    lib = binding._lib
    fl = ctypes.c_double(-1.0)
    ok_ops, ok_out = 65536, 1 << 20
    cases = [
        (-101, (2, 1, FAKE, ok_ops, FAKE, ok_out, ctypes.byref(fl))),
        (-101, (-1, 1, FAKE, ok_ops, FAKE, ok_out, ctypes.byref(fl))),
        (-102, (1, 0, FAKE, ok_ops, FAKE, ok_out, ctypes.byref(fl))),
        (-103, (1, 1, None, ok_ops, FAKE, ok_out, ctypes.byref(fl))),
        (-104, (0, 1, FAKE, ok_ops - 1, FAKE, ok_out, ctypes.byref(fl))),
        (-105, (1, 1, FAKE, ok_ops, None, ok_out, ctypes.byref(fl))),
        (-106, (1, 1, FAKE, ok_ops, FAKE, ok_out - 4, ctypes.byref(fl))),
        (-107, (1, 1, FAKE, ok_ops, FAKE, ok_out, None)),
        (-101, (7, 0, None, 0, None, 0, None)),            # first failure wins
    ]
    for expected, args in cases:
        assert lib.gemm_probe_mfma(*args, None) == expected, (expected, args)
        assert "probe" in binding.gemm_status_string(expected)
    assert fl.value == -1.0        # no flop count written on a rejected call


LAYOUT_CASES = [
    # (layout, expected, M, N, K, lda, ldb, ldc): the stored row lengths
    # decide the leading-dimension checks
    ("nt", 0, 4, 9, 8, 8, 8, 9),        # A M x K (lda >= K), B N x K (ldb >= K)
    ("nt", -8, 4, 9, 8, 8, 7, 9),
    ("nt", -6, 4, 9, 8, 7, 8, 9),
    ("tn", 0, 6, 9, 8, 6, 9, 9),        # A K x M (lda >= M), B K x N (ldb >= N)
    ("tn", -6, 6, 9, 8, 5, 9, 9),
    ("tn", -8, 6, 9, 8, 6, 8, 9),
    ("tt", 0, 6, 9, 8, 6, 8, 9),        # both transposed
    ("tt", -6, 6, 9, 8, 5, 8, 9),
    ("tt", -8, 6, 9, 8, 6, 7, 9),
    ("tt", -11, 6, 9, 8, 6, 8, 8),
    ("tn", -1, -1, 9, 8, 6, 9, 9),
]


@pytest.mark.parametrize("dt", ["f32", "f16", "f16f32"])
@pytest.mark.parametrize("case", LAYOUT_CASES, ids=[str(i) for i in range(len(LAYOUT_CASES))])
def test_layout_argument_checks(dt, case):
    """The transposed-operand entry points check lda and ldb against the
    row lengths of A and B as stored, before any HIP call.  Successful cases
    use quick returns (alpha = 0, beta = 1) so nothing is launched."""
    import dense_gemm_fp32_amd as dg
    layout, expected, M, N, K, lda, ldb, ldc = case
    fn = getattr(dg, "gemm_%s_%s" % (dt, layout))
    assert fn(M, N, K, 0.0, FAKE, lda, FAKE, ldb, 1.0, FAKE, ldc, None) == expected
    if expected in (-6, -8):
        assert "stored transposed" in dg.gemm_status_string(expected)


def test_tail_split_in_descriptions():
    """The plan names the split of the last round when the model takes it,
    and the diagnostic switch turns it off or forces it."""
    import dense_gemm_fp32_amd as dg
    n = 5504
    args = (n, n, n, 1.0, FAKE, n, FAKE, n, 1.0, FAKE, n)
    rc, text = dg.gemm_describe("f32", *args)
    assert rc == 0 and "last round split-K" in text, text
    prev = dg.gemm_set_tail_split(1)
    try:
        rc, text = dg.gemm_describe("f32", *args)
        assert "last round" not in text, text
        dg.gemm_set_tail_split(3)
        rc, text = dg.gemm_describe("f32", 4096, 4096, 4096, 1.0, FAKE, 4096, FAKE, 4096, 0.0, FAKE,
                                    4096)
        assert "last round" not in text, text        # 512 tiles: whole rounds only
        rc, text = dg.gemm_describe("f32", 4200, 2000, 256, 1.0, FAKE, 256, FAKE, 2000, 0.0, FAKE,
                                    2000)
        assert "last round split-K 3" in text, text
    finally:
        dg.gemm_set_tail_split(prev)
    assert dg.gemm_set_tail_split(65) == -1 and dg.gemm_set_tail_split(-1) == -1
    # the square 4096 workload stays whole: 512 tiles fill two rounds
    rc, text = dg.gemm_describe("f32", 4096, 4096, 4096, 1.0, FAKE, 4096, FAKE, 4096, 0.0, FAKE, 4096)
    assert "split" not in text, text


def test_describe_reports_split_workspace():
    """The workspace a split call takes, worked out by hand: 2304 x 2304 x 5000
    splits the 256 x 128 tiles 3 ways into M x N fp32 slabs, 3 * 2304 * 2304 *
    4 bytes;
    2944^3 (23 x 23 = 529 tiles of 128 x 128, 2 whole rounds of 256 and 17
    left over) splits the 17 leftover tiles 15 ways into dense tile blocks,
    15 * 17 * 128 * 128 * 4 bytes.  An unsplit call takes none."""
    import dense_gemm_fp32_amd as dg
    cases = [((2304, 2304, 5000), "split-K 3", 63700992),
             ((2944, 2944, 2944), "last round split-K 15", 16711680)]
    for (m, n, k), split, nbytes in cases:
        rc, text = dg.gemm_describe("f32", m, n, k, 1.0, FAKE, k, FAKE, n, 1.0, FAKE, n)
        assert rc == 0 and split in text and ("workspace %d bytes" % nbytes) in text, text
    rc, text = dg.gemm_describe("f32", 4096, 4096, 4096, 1.0, FAKE, 4096, FAKE, 4096, 0.0, FAKE, 4096)
    assert rc == 0 and "workspace" not in text, text


def test_noalloc_refuses_workspace_beyond_the_scratch_region():
    """3000 x 3000 x 30000 splits K 8 ways into 288,000,000 bytes of slabs,
    more than the 64 MiB scratch region: gemm_f32_noalloc refuses before any
    HIP call (so this runs without a GPU; the pointers are never touched),
    while its argument checks come first."""
    import dense_gemm_fp32_amd as dg
    rc, text = dg.gemm_describe("f32", 3000, 3000, 30000, 1.0, FAKE, 30000, FAKE, 3000, 0.0, FAKE,
                                3000)
    assert "workspace 288000000 bytes" in text, text
    assert dg.gemm_f32_noalloc(3000, 3000, 30000, 1.0, FAKE, 30000, FAKE, 3000, 0.0, FAKE, 3000,
                               None) == dg.GEMM_ERR_SCRATCH_LIMIT
    assert dg.gemm_f32_noalloc(3000, 3000, 30000, 1.0, FAKE, 29999, FAKE, 3000, 0.0, FAKE, 3000,
                               None) == -6
    msg = dg.gemm_status_string(dg.GEMM_ERR_SCRATCH_LIMIT)
    assert "scratch" in msg and "nothing was enqueued" in msg


def test_workspace_limit_switch():
    import dense_gemm_fp32_amd as dg
    assert dg.gemm_set_workspace_limit(0) == -1
    assert dg.gemm_set_workspace_limit(1 << 20) == 0
    assert dg.gemm_set_workspace_limit(-5) == -2
    assert dg.gemm_set_workspace_limit(-1) == 1 << 20


def test_stream_k_by_size_and_switches():
    """Stream-K behind the whole rounds, with two fp32 tile blocks of
    workspace per Stream-K workgroup (one per CU): the four-wave 64x64 tile
    with two whole rounds and at most half a round more, or three and at
    most a third of a round more; the 128x64 tile with two to three and a
    half rounds (M, N, K >= 640); the 128x128 tile
    with two to seven rounds and a leftover of a quarter to seven eighths of
    a round, in place of any choice, and up to sixteen rounds in place of
    that tile; the 256x128 and 256x256 tiles with a round partly filled, in
    place of themselves.  Other sizes, deep K, and calls whose workspace
    cannot hold the blocks run without it.  The switch forces each
    decomposition, and refuses unknown modes."""
    import dense_gemm_fp32_amd as dg

    def d(M, N, K, lda=None, ldb=None, ldc=None):
        rc, t = dg.gemm_describe("f32", M, N, K, 1.0, FAKE, lda or K, FAKE, ldb or N, 0.5, FAKE,
                                 ldc or N)
        assert rc == 0
        return t

    def ws(t):
        return int(t.split("workspace ")[1].split()[0]) if "workspace" in t else 0

    block = 2 * 64 * 64 * 4
    # 1536^3: 576 tiles, 512 whole and 64 left over 256 workgroups
    t = d(1536, 1536, 1536)
    assert "64x64x32 4 waves" in t and "stream-K after 512 whole tiles" in t, t
    assert "blocks 768 " in t and ws(t) == 256 * block, t
    # 1472^3: 529 tiles, 17 left; their 46 K steps each, 782 in all, in runs
    # of 4 over 196 workgroups
    t = d(1472, 1472, 1472)
    assert "stream-K after 512 whole tiles" in t and "blocks 708 " in t and ws(t) == 196 * block, t
    assert "stream-K after 512 whole tiles" in d(1600, 1600, 1600)
    assert "stream-K after 512 whole tiles" in d(2048, 1152, 1024)
    # one round and a small leftover (1088^3, 1152^3), larger leftovers
    # (1664^3: 164 tiles), whole rounds (1024^3), other tiles: plain
    for n in (1024, 1088, 1152, 1216, 1280, 1408, 1664, 2048, 4096):
        assert "stream-K" not in d(n, n, n), n
    # past three whole rounds by at most a third of a round: 1792^3 (784
    # tiles), 1856^3 (841), 2048x1600x1800 (800); from 1888^3 (900) the
    # 128x64 tile, plain
    for s in ((1760, 1760, 1760), (1792, 1792, 1792), (1856, 1856, 1856), (2048, 1600, 1800)):
        t = d(*s)
        assert "64x64x32 4 waves" in t and "stream-K after 768 whole tiles" in t, (s, t)
    # 1792^3: 16 tiles left, their 56 K steps each in runs of 4 over 224
    # workgroups
    t = d(1792, 1792, 1792)
    assert "blocks 992 " in t and ws(t) == 224 * block, t
    for n in (1888, 1920, 1984):
        assert "128x64x32 4 waves" in d(n, n, n) and "stream-K" not in d(n, n, n), n
    # deep K (K > 2 max(M, N)) stays off it
    assert "stream-K" not in d(1792, 1792, 3600)
    # exactly 1536 64x64 tiles (six per CU), K >= 1024: that tile, plain
    for s in ((1536, 4096, 1536), (1024, 6144, 1024), (4096, 1536, 2048), (2048, 3072, 2048)):
        t = d(*s)
        assert "64x64x32 4 waves 3 slots" in t and "stream-K" not in t and "split" not in t, (s, t)
    assert "64x64x32" not in d(1536, 4096, 512) and "64x64x32" not in d(2048, 4096, 1024)
    assert "64x64x32" not in d(3072, 2048, 4000)
    # the 128x64 tile: two to three and a half rounds of its tiles, a round
    # partly filled, M, N and K at least 640.  2176^3: 578 tiles, 512 whole,
    # 66 left; their 68 K steps each, 4488 in all, in runs of 18 over 250
    # workgroups, two 128x64 blocks each
    t = d(2176, 2176, 2176)
    assert "128x64x32 4 waves" in t and "stream-K after 512 whole tiles" in t, t
    assert "blocks 762 " in t and ws(t) == 250 * 2 * 128 * 64 * 4, t
    for s in ((2304, 2304, 2304), (2432, 2432, 2432), (2048, 2304, 2048), (1536, 3072, 2048),
              (2176, 2176, 1536), (768, 6144, 2048), (6144, 768, 2048), (640, 8192, 1536),
              (2176, 2176, 768), (3072, 1536, 640)):
        assert "128x64x32 4 waves" in d(*s) and "stream-K after 512 whole tiles" in d(*s), s
    for n in (2560, 2688):
        assert "128x64x32 4 waves" in d(n, n, n) and "stream-K after 768 whole tiles" in d(n, n, n), n
    # not past three and a half rounds (2816^3: 968 tiles), at whole rounds
    # (2048 x 3072 x 2048: 768), with K or a side below 640, or deep K
    for s in ((2816, 2816, 2816), (2048, 3072, 2048), (2176, 2176, 512), (1000, 4000, 2000),
              (2304, 2304, 5000), (2560, 2560, 512), (600, 8192, 2048), (2176, 2176, 600)):
        assert not ("128x64x32" in d(*s) and "stream-K" in d(*s)), (s, d(*s))
    # copies and Stream-K share one workspace
    t = d(1536, 1536, 1536, 1537, 1537, 1537)
    assert "copies A B" in t and "stream-K after 512" in t and ws(t) == 2 * 1536 * 1536 * 4 + 256 * block, t
    # a workspace limit below the blocks drops Stream-K
    prev = dg.gemm_set_workspace_limit(256 * block - 1)
    try:
        assert "stream-K" not in d(1536, 1536, 1536)
        dg.gemm_set_workspace_limit(256 * block)
        assert "stream-K after 512" in d(1536, 1536, 1536)
    finally:
        dg.gemm_set_workspace_limit(prev)
    # the 128x128 tile: two to sixteen rounds of its tiles, a leftover of a
    # quarter to seven eighths of the CUs, K >= 1024.  3840^3: 900 tiles, 768
    # whole, 132 left, in runs of 124 of their 240 K steps over 256 workgroups
    t = d(3840, 3840, 3840)
    assert "128x128x16 4 waves 3 slots loads" in t and "stream-K after 768 whole tiles" in t, t
    assert "blocks 1024 " in t and ws(t) == 256 * 2 * 128 * 128 * 4, t
    # ... in place of a K split (3328^3, the 256x128 tile split 3) or the
    # larger tiles (3840^3) up to seven rounds of 128x128 tiles; from seven
    # to sixteen only in place of the 128x128 tile itself (6016^3)
    for n in (3072, 3328, 3840, 5248, 6016, 7040):
        assert "128x128x16" in d(n, n, n) and "stream-K after" in d(n, n, n), n
    # the 256x256 tile, wherever it has a round of tiles and at least 97% of
    # their area lies inside the matrix: 6400^3 (625 tiles, 512 whole),
    # 9344^3 (36.5 tiles a side: 97.3%), 4352^3; not at 7296^3 (28.5 a
    # side: 96.5%) nor under one round (3840^3: 225 tiles); plain with whole
    # rounds (8192^3, 12288^3)
    # (6400^3: the 113 leftover tiles' 200 K steps each, 22600 in all, in
    # runs of 89 over 254 workgroups)
    t = d(6400, 6400, 6400)
    assert "256x256x32" in t and "stream-K after 512 whole tiles" in t and "blocks 766 " in t, t
    assert ws(t) == 254 * 2 * 256 * 256 * 4, t
    for n in (4352, 9344, 10752, 12800):
        assert "256x256x32" in d(n, n, n) and "stream-K after" in d(n, n, n), n
    assert "256x256x32" not in d(7296, 7296, 7296) and "256x256x32" not in d(3840, 3840, 3840)
    for n in (8192, 12288):
        assert "256x256x32" in d(n, n, n) and "stream-K" not in d(n, n, n), n
    # the 256x128 tile, plain or with the last round split, takes Stream-K on
    # the same tile when a round is partly filled (7808^3: 30.5 256x256
    # tiles a side would be 96.7% inside)
    t = d(7808, 7808, 7808)
    assert "256x128x32" in t and "stream-K after 1792 whole tiles" in t, t
    assert ws(t) == 255 * 2 * 256 * 128 * 4, t
    # where the workspace cannot hold the partial blocks, the model's own
    # choice: 7808^3's last round split, 6400^3 whole on the 256x128 tile
    prev = dg.gemm_set_workspace_limit(60 << 20)
    try:
        t = d(7808, 7808, 7808)
        assert "256x128x32" in t and "last round split-K" in t and "stream-K" not in t, t
        t = d(6400, 6400, 6400)
        assert "256x128x32" in t and "split" not in t and "stream-K" not in t, t
    finally:
        dg.gemm_set_workspace_limit(prev)
    # 128x128 tiles with a leftover under a quarter (2944^3: 17 tiles) or
    # over seven eighths (4992^3: 241), whole rounds of 256x256 tiles
    # (4096^3), K under 1024, rows without 16-byte loads: no Stream-K
    for n in (2944, 4096, 4992):
        assert "stream-K" not in d(n, n, n), n
    assert "stream-K" not in d(3840, 3840, 1000)
    # deep K keeps the model's K split
    t = d(3000, 3000, 30000)
    assert "stream-K" not in t and "split-K" in t, t
    assert "stream-K after 512" in d(3000, 3000, 6000)
    # unaligned rows: copied (and then Stream-K on the copies), or, with
    # copies off, the register-staged path's own rule
    t = d(3840, 3840, 3840, 3841, 3841, 3840)
    assert "copies A B" in t and "stream-K after 768" in t, t
    pack = dg.gemm_set_pack(1)
    try:
        assert "stream-K" not in d(3840, 3840, 3840, 3841, 3841, 3840)
    finally:
        dg.gemm_set_pack(pack)
    # the switch
    prev = dg.gemm_set_stream_k(1)
    try:
        assert prev == 0
        assert "stream-K" not in d(1536, 1536, 1536)
        assert "stream-K" not in d(3840, 3840, 3840)
        # every tile's K steps: 400 tiles x 40 steps, in runs of 32 over 500
        # workgroups (two per CU asked for) ...
        assert dg.gemm_set_stream_k(3) == 1
        t = d(1280, 1280, 1280)
        assert "stream-K" in t and "whole tiles" not in t and "blocks 500 " in t, t
        # ... and with one per CU asked for, runs capped at one tile's steps
        dg.gemm_set_stream_k(2)
        assert "blocks 400 " in d(1280, 1280, 1280)
        # ... and with one round whole first (1024^3 has nothing left: plain)
        dg.gemm_set_stream_k(5)
        assert "stream-K after 256 whole tiles" in d(1280, 1280, 1280)
        assert "stream-K" not in d(1024, 1024, 1024)
        dg.gemm_set_stream_k(6)
        t = d(1280, 1280, 1280)
        assert "stream-K after 256 whole tiles" in t and ws(t) == (int(t.split("blocks ")[1].split()[0]) - 256) * block, t
        # only calls on the 64x64 tile
        assert "stream-K" not in d(4096, 4096, 4096)
    finally:
        dg.gemm_set_stream_k(prev)
    assert dg.gemm_set_stream_k(7) == -1 and dg.gemm_set_stream_k(-1) == -1


def test_operand_copies_by_size_and_switches():
    """Operands whose rows do not allow 16-byte loads are copied to 16-byte
    rows in fp32 calls above the size rule (5e9 flops, or 1.5e9 with N a
    multiple of 4), never in fp16 calls by size, never under gemm_set_pack(1)
    or the element-wise load switch, always under gemm_set_pack(2); the
    copies' bytes are part of the reported workspace and a workspace limit
    below them drops the copies."""
    import dense_gemm_fp32_amd as dg

    def d(dtype, M, N, K, lda, ldb, ldc, a=FAKE, b=FAKE):
        rc, t = dg.gemm_describe(dtype, M, N, K, 1.0, a, lda, b, ldb, 0.5, FAKE, ldc)
        assert rc == 0
        return t

    def ws(t):
        return int(t.split("workspace ")[1].split()[0]) if "workspace" in t else 0

    # fp32 2048^3, every ld 2049: two copies of 2048 x 2048 floats (rows of
    # 2048 already fill whole 16-byte chunks), and the GEMM on them is unsplit
    t = d("f32", 2048, 2048, 2048, 2049, 2049, 2049)
    assert "copies A B" in t and "A:vec4 B:vec4" in t and ws(t) == 2 * 2048 * 2048 * 4, t
    # one unaligned operand: only it is copied; 1001 columns pad to 1004
    t = d("f32", 2000, 2000, 1001, 1001, 2000, 2000)
    assert "copies A" in t and "copies A B" not in t and ws(t) >= 2000 * 1004 * 4, t
    t = d("f32", 2000, 2000, 1000, 1000, 2001, 2000)
    assert "copies B" in t, t
    # a base off a 16-byte boundary alone is enough
    assert "copies A" in d("f32", 2048, 2048, 2048, 2048, 2048, 2048, a=FAKE + 4)
    # the ragged workload (3.1e9 flops, N = 3000): copied, and the copies take
    # the four-wave 64x64 tile
    t = d("f32", 1000, 3000, 517, 530, 3005, 3003)
    assert "copies A B" in t and "64x64x32 4 waves" in t, t
    # the same size with a ragged N, and smaller calls: not copied
    assert "copies" not in d("f32", 3000, 517, 1000, 1001, 519, 519)
    assert "copies" not in d("f32", 768, 768, 768, 769, 769, 769)
    # fp16: not by size
    assert "copies" not in d("f16", 4096, 4096, 4096, 4097, 4097, 4097)
    assert "copies" not in d("f16", 1000, 3000, 517, 530, 3005, 3003)
    # aligned operands are never copied
    assert "copies" not in d("f32", 4096, 4096, 4096, 4096, 4096, 4097)
    # the switches
    prev = dg.gemm_set_pack(1)
    try:
        assert prev == 0
        assert "copies" not in d("f32", 2048, 2048, 2048, 2049, 2049, 2049)
        assert dg.gemm_set_pack(2) == 1
        t = d("f32", 300, 200, 100, 101, 201, 200)
        # A: 300 rows of K = 100 floats, B: 100 rows of N = 200 (both already
        # whole 16-byte chunks), each copy rounded up to 256 bytes
        assert "copies A B" in t and ws(t) == (300 * 100 * 4 + 255) // 256 * 256 + \
            (100 * 200 * 4 + 255) // 256 * 256, t
        t = d("f16", 300, 200, 100, 101, 201, 200)
        # fp16: 100 halves pad to 104, 200 to 200
        assert "copies A B" in t and ws(t) == (300 * 104 * 2 + 255) // 256 * 256 + \
            (100 * 200 * 2 + 255) // 256 * 256, t
        load = dg.gemm_set_load_mode(1)
        try:
            assert "copies" not in d("f32", 300, 200, 100, 101, 201, 200)
        finally:
            dg.gemm_set_load_mode(load)
    finally:
        dg.gemm_set_pack(prev)
    assert dg.gemm_set_pack(3) == -1 and dg.gemm_set_pack(-1) == -1
    # a workspace limit below the copies drops them (and the split, if any)
    need = ws(d("f32", 2048, 2048, 2048, 2049, 2049, 2049))
    prev = dg.gemm_set_workspace_limit(need - 1)
    try:
        assert "copies" not in d("f32", 2048, 2048, 2048, 2049, 2049, 2049)
        dg.gemm_set_workspace_limit(need)
        assert "copies A B" in d("f32", 2048, 2048, 2048, 2049, 2049, 2049)
    finally:
        dg.gemm_set_workspace_limit(prev)


def _profile_rows(name):
    """Data rows of the markdown table in profiles/<name> (lists of cells):
    the lines after the table's header and separator."""
    rows, seen_sep = [], False
    with open(os.path.join(ROOT, "profiles", name)) as f:
        for line in f:
            if not line.startswith("|"):
                continue
            if line.startswith("|---"):
                seen_sep = True
                continue
            if seen_sep:
                rows.append([c.strip() for c in line.strip().strip("|").split("|")])
    return rows


def _short_plan(plan, sweep):
    """The tile column the sweep and workload tables print for a plan."""
    body = plan.split(" tile ", 1)[1]
    if sweep:
        short = body.split(" loads A:")[0]
        if "stream-K" in plan:
            short += " stream-K" + plan.split("stream-K")[1].split(" workspace")[0]
        if "split-K" in plan:
            short += " " + ("last round " if "last round" in plan else "") + \
                "split-K " + plan.split("split-K ")[1].split()[0]
        return short
    short = body.split(" blocks ")[0]
    if "split-K" in plan:
        short += " split-K " + plan.split("split-K ")[1].split()[0]
    return short


def test_plans_match_the_committed_sweep_and_table():
    """Each size of the committed fp32 sweep and each workload of the
    committed table was measured with a plan (tile, loads, split) that the
    library still chooses for it: a change to the tile or split rules that
    moves any of them must come with new measurements."""
    import dense_gemm_fp32_amd as dg
    import workloads as wl
    sweep = _profile_rows("sweep_f32_1024_12800.md")
    assert len(sweep) == len(wl.sweep_sizes()), len(sweep)
    for cells in sweep:
        n = int(cells[0])
        rc, plan = dg.gemm_describe("f32", n, n, n, 1.0, FAKE, n, FAKE, n, 1.0, FAKE, n)
        assert rc == 0
        assert _short_plan(plan, True) == cells[-1], (n, plan, cells[-1])
    table = {c[0]: c for c in _profile_rows("workloads_table.md")}
    by_name = {w.name: w for w in wl.ALL}
    checked = 0
    for name, cells in table.items():
        w = by_name.get(name)
        if w is None:
            continue
        rc, plan = dg.gemm_describe(w.dtype, w.M, w.N, w.K, w.alpha, FAKE, w.lda, FAKE, w.ldb,
                                    w.beta, FAKE, w.ldc)
        assert rc == 0
        assert _short_plan(plan, False) == cells[-1], (name, plan, cells[-1])
        checked += 1
    assert checked >= 7, sorted(table)
