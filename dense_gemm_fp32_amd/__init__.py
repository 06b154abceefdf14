"""MI355X (gfx950) GEMM library: row-major C := alpha*A*B + beta*C in fp32, in
fp16 with fp32 accumulation, and with fp16 inputs and an fp32 C; hand-written
HIP kernels behind a C ABI
(include/gemm.h, libgemm.so).

The binding is loaded on first use of one of its names, so that host-only
helpers of this package (the build script, the measurement model) import
without the library; using the GEMM entry points without a built library
raises ImportError.
"""
_LAYOUT_NAMES = tuple("gemm_%s_%s" % (t, l) for t in ("f32", "f16", "f16f32") for l in ("nt", "tn", "tt"))
_BINDING_NAMES = ("gemm_f32", "gemm_f16", "gemm_f16f32", "gemm_f32_valu", "gemm_f32_noalloc",
                  "gemm_f32_colmajor", "gemm_f16_colmajor", "gemm_f16f32_colmajor",
                  "gemm_status_string", "gemm_describe", "gemm_set_load_mode",
                  "gemm_set_tile_config", "gemm_set_split", "gemm_set_tail_split",
                  "gemm_set_pack", "gemm_set_stream_k", "gemm_set_workspace_limit", "gemm_probe_mfma", "gemm", "GemmError",
                  "GEMM_ERR_SCRATCH_LIMIT", "LIB_PATH", "EXPORTS", "LAYOUT_NAMES") + _LAYOUT_NAMES

__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
