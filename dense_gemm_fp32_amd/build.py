"""Build libgemm.so (the gfx950 GEMM library) in-tree with hipcc.

    python -m dense_gemm_fp32_amd.build              # compile every source
    python -m dense_gemm_fp32_amd.build --lds-poison # debug build, see below

Every HIP source under csrc/ is compiled for gfx950 only, then linked into
dense_gemm_fp32_amd/libgemm.so next to this file.  The build also compiles the
kernel sources to gfx950 assembly and fails if compiler-generated code touches
m0 or if a GEMM kernel spills to scratch memory.

--lds-poison builds dense_gemm_fp32_amd/libgemm_lds_poison.so instead, in which
every kernel fills its shared memory with NaN before using it (DGEMM_LDS_POISON):
run the GPU tests against it with DENSE_GEMM_FP32_AMD_LIB pointing at that file.
"""
import concurrent.futures
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgemm.so")
BUILD_DIR = os.path.join(HERE, "_build")
POISON_LIB = os.path.join(HERE, "libgemm_lds_poison.so")
POISON_BUILD_DIR = os.path.join(HERE, "_build_lds_poison")
SOURCES = ["api.hip", "gemm_f32.hip", "gemm_f16.hip", "gemm_valu.hip", "scale.hip", "splitk.hip",
           "pack.hip", "probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# No packed-fp32 instructions: hipcc may otherwise fuse float pairs into
# v_pk_* forms.  (The host pass warns that it does not know the feature.)
HIP_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src, verbose=False, build_dir=BUILD_DIR, extra=()):
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *HIP_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, out))
    if verbose and out.strip():
        print(out)
    return obj


# Sources that set m0 in inline assembly (the kernels' direct
# global->LDS loads).  m0 is a register the compiler reserves for itself, so the
# build verifies that no compiler-generated instruction in these sources
# touches it: the asm's m0 writes then cannot disturb compiled code.  The
# same assembly is checked for spills (and that of gemm_valu.hip).
M0_ASM_SOURCES = ["gemm_f16.hip", "gemm_f32.hip"]
SPILL_ONLY_SOURCES = ["gemm_valu.hip"]


def check_spills_only(src):
    cmd = [HIPCC, *HIP_FLAGS, "--cuda-device-only", "-S", "-o", "-", os.path.join(CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc -S failed on %s:\n%s" % (src, r.stderr))
    check_no_spills(r.stdout, src)


# Kernels whose registers hold the accumulator tiles: a spill to scratch
# memory would put every MFMA's operands behind memory traffic, so the build
# refuses one.
NO_SPILL_KERNELS = ("hgemm_mfma", "sgemm_mfma", "sgemm_streamk", "sgemm_valu")


def scratch_sizes(asm_text):
    """{kernel symbol: scratch bytes per lane} from gfx950 assembly text."""
    sizes = {}
    current = None
    for line in asm_text.splitlines():
        t = line.strip()
        m = re.match(r"^\.amdhsa_kernel\s+(\S+)", t)
        if m:
            current = m.group(1)
            continue
        m = re.match(r"^\.amdhsa_private_segment_fixed_size\s+(\d+)", t)
        if m and current is not None:
            sizes[current] = int(m.group(1))
        if t.startswith(".end_amdhsa_kernel"):
            current = None
    return sizes


def check_no_spills(asm_text, src):
    """Raise RuntimeError if a GEMM kernel in `src`'s assembly uses scratch."""
    sizes = scratch_sizes(asm_text)
    if not sizes:
        raise RuntimeError("no kernel descriptors found in the assembly of %s" % src)
    bad = ["%s: %d bytes" % (k, v) for k, v in sizes.items()
           if v and any(n in k for n in NO_SPILL_KERNELS)]
    if bad:
        raise RuntimeError("GEMM kernels in %s spill to scratch memory:\n%s" % (src, "\n".join(bad)))


# Register budget per lane of each GEMM tile: a SIMD's 512 registers per lane
# (architected and accumulation) are shared by the waves it holds, so a tile
# meant to put W waves on each SIMD (its workgroups per CU, as its LDS allows,
# times its waves, over 4 SIMDs) may use at most 512 / W of them, in granules
# of 8.  One more register and fewer of its workgroups fit on a CU.
# (symbol fragment of the tile's template arguments, workgroups per CU, waves)
TILE_OCCUPANCY = (
    ("S32TileILi256ELi256ELi32E", 1, 8),
    ("S32TileILi256ELi128ELi32E", 1, 8),
    # the 128x128 tile with spread loads runs only on grids of at most one
    # workgroup per CU; with the loads issued together, three share a CU
    ("S32TileILi128ELi128ELi16ELi2ELi2ELi3ELi8ELb1E", 1, 4),
    ("S32TileILi128ELi128ELi16ELi2ELi2ELi3ELi8ELb0E", 3, 4),
    ("S32TileILi128ELi64ELi32E", 2, 4),
    ("S32TileILi64ELi64ELi64ELi2ELi2ELi2E", 2, 4),
    ("S32TileILi64ELi64ELi32ELi2ELi2E", 3, 4),
    ("S32TileILi64ELi64ELi32ELi1ELi1E", 3, 1),
    ("S32TileILi32ELi32ELi64E", 5, 1),
    ("S32TileILi32ELi32ELi32E", 6, 1),
    ("H16TileILi256ELi256ELi64E", 1, 8),
    ("H16TileILi128ELi128ELi32E", 2, 4),
    ("H16TileILi64ELi128ELi32E", 3, 2),
)


def register_budget(wgs_per_cu, waves):
    per_simd = max(1, -(-wgs_per_cu * waves // 4))
    return 512 // per_simd // 8 * 8


def register_counts(asm_text):
    """{kernel symbol: registers per lane (.amdhsa_next_free_vgpr)}."""
    counts = {}
    current = None
    for line in asm_text.splitlines():
        t = line.strip()
        m = re.match(r"^\.amdhsa_kernel\s+(\S+)", t)
        if m:
            current = m.group(1)
            continue
        m = re.match(r"^\.amdhsa_next_free_vgpr\s+(\d+)", t)
        if m and current is not None:
            counts[current] = int(m.group(1))
        if t.startswith(".end_amdhsa_kernel"):
            current = None
    return counts


def check_register_budget(asm_text, src):
    """Raise RuntimeError if a GEMM kernel in `src`'s assembly uses more
    registers than its tile's occupancy allows (TILE_OCCUPANCY), or if a GEMM
    kernel's tile has no entry there."""
    bad = []
    for kernel, regs in register_counts(asm_text).items():
        if not any(n in kernel for n in NO_SPILL_KERNELS) or "sgemm_valu" in kernel:
            continue
        entry = [e for e in TILE_OCCUPANCY if e[0] in kernel]
        if not entry:
            bad.append("%s: no occupancy entry for its tile" % kernel)
            continue
        budget = register_budget(entry[0][1], entry[0][2])
        if regs > budget:
            bad.append("%s: %d registers, budget %d (%d workgroups of %d waves per CU)"
                       % (kernel, regs, budget, entry[0][1], entry[0][2]))
    if bad:
        raise RuntimeError("GEMM kernels in %s exceed their register budget:\n%s"
                           % (src, "\n".join(bad)))


def check_m0_only_in_asm(src):
    """Compile `src` to gfx950 assembly and verify that every instruction
    mentioning m0 lies inside an inline-asm block, and that no GEMM kernel
    spills or exceeds its register budget.  Raises RuntimeError."""
    cmd = [HIPCC, *HIP_FLAGS, "--cuda-device-only", "-S", "-o", "-", os.path.join(CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc -S failed on %s:\n%s" % (src, r.stderr))
    check_no_spills(r.stdout, src)
    check_register_budget(r.stdout, src)
    inside = False
    bad = []
    for n, line in enumerate(r.stdout.splitlines(), 1):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            inside = True
            continue
        if t.startswith(";;#ASMEND"):
            inside = False
            continue
        if not t or t.startswith((";", ".")):
            continue
        code = t.split(";", 1)[0]
        if not inside and re.search(r"\bm0\b", code):
            bad.append("%d: %s" % (n, t))
    if bad:
        raise RuntimeError("compiler-generated code uses m0 in %s (inline asm clobbers it):\n%s"
                           % (src, "\n".join(bad[:20])))


def build(verbose=False, lds_poison=False):
    """Compile all sources and link libgemm.so (or, with lds_poison, the
    debug library libgemm_lds_poison.so); returns the library path."""
    build_dir = POISON_BUILD_DIR if lds_poison else BUILD_DIR
    lib = POISON_LIB if lds_poison else LIB
    extra = ("-DDGEMM_LDS_POISON",) if lds_poison else ()
    os.makedirs(build_dir, exist_ok=True)
    # The assembly checks and the object compiles are independent hipcc runs:
    # run them side by side (the two kernel sources dominate the build time).
    workers = min(os.cpu_count() or 4,
                  len(SOURCES) + len(M0_ASM_SOURCES) + len(SPILL_ONLY_SOURCES), 16)
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        checks = [] if lds_poison else (
            [ex.submit(check_m0_only_in_asm, src) for src in M0_ASM_SOURCES] +
            [ex.submit(check_spills_only, src) for src in SPILL_ONLY_SOURCES])
        compiles = [ex.submit(_compile, src, verbose, build_dir, extra) for src in SOURCES]
        for f in checks:
            f.result()
        objs = [f.result() for f in compiles]
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, lds_poison="--lds-poison" in sys.argv))
