"""gemm_f32_noalloc, the entry point for callers that cannot allocate, against
gemm_f32 on the same inputs: same plan, same kernels, so the results must be
the same bits, and both within the accuracy bound of the oracle.  The calls
come in a row on one device, so the library's fixed scratch region is reused
with the previous call's contents still in it; the second call is smaller
than the first."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gemm_harness import bits, check, check_sampled, note, run

pytestmark = pytest.mark.gpu


def _plan(w):
    import dense_gemm_fp32_amd as dg
    rc, text = dg.gemm_describe("f32", w.M, w.N, w.K, w.alpha, 4096, w.lda, 4096, w.ldb, w.beta,
                                4096, w.ldc)
    assert rc == 0
    return text


def _both(w):
    """Outputs of gemm_f32_noalloc and gemm_f32 on fresh copies of w's inputs."""
    A, B, C = wl.make(w)
    plan = _plan(w)
    rc, out_na = run("f32", w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc,
                     "%s noalloc (%s)" % (w.name, plan), entry="gemm_f32_noalloc")
    assert rc == 0
    rc, out_ref = run("f32", w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc,
                      "%s gemm_f32" % w.name)
    assert rc == 0
    return plan, (A, B, C), out_na, out_ref


def test_noalloc_matches_gemm_f32_on_calls_in_a_row():
    # 1) 2304 x 2304 x 5000, beta = 1: K split 3 ways into M x N slabs,
    #    63,700,992 bytes of the 64 MiB region.
    w1 = wl.Workload("noalloc_2304x2304x5000", "f32", 2304, 2304, 5000, 5000, 2304, 2304, 1.0, 1.0,
                     "uniform", "uniform", (5, 6, 7))
    plan, (A, B, C), out_na, out_ref = _both(w1)
    assert "split-K 3" in plan and "workspace 63700992 bytes" in plan, plan
    assert np.array_equal(bits(out_na, "f32"), bits(out_ref, "f32"))
    check_sampled("f32", w1, A, B, C, out_na, nrows=16, seed=3)

    # 2) smaller: the ragged 1000 x 3000 x 517 workload (unaligned lda and
    #    ldb, all three tails): A and B copied to 16-byte rows in the region
    #    (1000 x 520 and 517 x 3000 floats, 8,284,160 bytes), unsplit; the
    #    region still holds the first call's slabs beyond that.
    w2 = wl.RAGGED_F32
    plan, (A, B, C), out_na, out_ref = _both(w2)
    assert "copies A B" in plan and "workspace 8284160 bytes" in plan, plan
    assert np.array_equal(bits(out_na, "f32"), bits(out_ref, "f32"))
    check("f32", w2.M, w2.N, w2.K, w2.alpha, A, w2.lda, B, w2.ldb, w2.beta, C, w2.ldc, out_na,
          "ragged noalloc")

    # 3) the last-round split: 2944^3, 17 leftover tiles in 15 K chunks,
    #    16,711,680 bytes of dense tile blocks.
    w3 = wl.sweep(2944)
    plan, (A, B, C), out_na, out_ref = _both(w3)
    assert "last round split-K 15" in plan, plan
    assert np.array_equal(bits(out_na, "f32"), bits(out_ref, "f32"))
    check_sampled("f32", w3, A, B, C, out_na, nrows=16, seed=5,
                  extra_rows=[2944 - 1 - 128 * i - 37 for i in range(8)])

    # 4) unaligned leading dimensions above the size rule for operand copies:
    #    2048^3 with every ld = 2049.  A and B are copied into the region (two
    #    2048 x 2048 fp32 copies, 33,554,432 bytes) and the GEMM runs on the
    #    copies, unsplit.
    w4 = wl.Workload("noalloc_copies_2048", "f32", 2048, 2048, 2048, 2049, 2049, 2049, 1.0, 0.5,
                     "uniform", "uniform", (12, 13, 14))
    plan, (A, B, C), out_na, out_ref = _both(w4)
    assert "copies A B" in plan and "workspace 33554432 bytes" in plan, plan
    assert np.array_equal(bits(out_na, "f32"), bits(out_ref, "f32"))
    check_sampled("f32", w4, A, B, C, out_na, nrows=12, seed=6, extra_rows=[2047])

    # 5) a call that does not split uses no workspace at all.
    w5 = wl.square(384, seeds=(8, 9, 10))
    plan, (A, B, C), out_na, out_ref = _both(w5)
    assert "workspace" not in plan, plan
    assert np.array_equal(bits(out_na, "f32"), bits(out_ref, "f32"))
    check("f32", w5.M, w5.N, w5.K, w5.alpha, A, w5.lda, B, w5.ldb, w5.beta, C, w5.ldc, out_na,
          "384 noalloc")


def test_noalloc_refuses_a_call_beyond_the_region_and_touches_nothing():
    """3000 x 3000 x 30000 would split into 288,000,000 bytes of slabs: refused
    with GEMM_ERR_SCRATCH_LIMIT before anything is enqueued, C unchanged."""
    import torch
    import dense_gemm_fp32_amd as dg
    note("noalloc refusal 3000x3000x30000")
    dev = torch.device("cuda:0")
    # full-size buffers, so that even a launch could not reach past them
    A = torch.zeros(3000 * 30000, device=dev)
    B = torch.zeros(30000 * 3000, device=dev)
    C = torch.full((3000 * 3000,), 7.0, device=dev)
    rc = dg.gemm_f32_noalloc(3000, 3000, 30000, 1.0, A, 30000, B, 3000, 0.0, C, 3000,
                             torch.cuda.current_stream(dev))
    torch.cuda.synchronize(dev)
    assert rc == dg.GEMM_ERR_SCRATCH_LIMIT
    assert bool((C == 7.0).all())
