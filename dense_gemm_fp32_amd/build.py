"""Build libgemm.so (the gfx950 GEMM library) in-tree with hipcc.

    python -m dense_gemm_fp32_amd.build          # compile every source

Every HIP source under csrc/ is compiled for gfx950 only, then linked into
dense_gemm_fp32_amd/libgemm.so next to this file.
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
SOURCES = ["api.hip", "gemm_f32.hip", "gemm_f16.hip", "gemm_valu.hip", "scale.hip", "splitk.hip",
           "probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# No packed-fp32 instructions: hipcc may otherwise fuse float pairs into
# v_pk_* forms.  (The host pass warns that it does not know the feature.)
HIP_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src, verbose=False):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
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
# touches it: the asm's m0 writes then cannot disturb compiled code.
M0_ASM_SOURCES = ["gemm_f16.hip", "gemm_f32.hip"]


def check_m0_only_in_asm(src):
    """Compile `src` to gfx950 assembly and verify that every instruction
    mentioning m0 lies inside an inline-asm block.  Raises RuntimeError."""
    cmd = [HIPCC, *HIP_FLAGS, "--cuda-device-only", "-S", "-o", "-", os.path.join(CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc -S failed on %s:\n%s" % (src, r.stderr))
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


def build(verbose=False):
    """Compile all sources and link libgemm.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    # The m0 checks and the object compiles are independent hipcc runs: run
    # them side by side (the two kernel sources dominate the build time).
    workers = min(os.cpu_count() or 4, len(SOURCES) + len(M0_ASM_SOURCES), 16)
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        checks = [ex.submit(check_m0_only_in_asm, src) for src in M0_ASM_SOURCES]
        compiles = [ex.submit(_compile, src, verbose) for src in SOURCES]
        for f in checks:
            f.result()
        objs = [f.result() for f in compiles]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
