"""Host-side model and benchmark schedule, pinned to the worked numbers the
pages print (fixtures under tests/golden/, each citing its page)."""
import os

import pytest

from dense_gemm_fp32_amd import model

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [list(map(int, l.split())) for l in f if l.strip() and not l.startswith("#")]


def test_replay_schedule_matches_page_example():
    for n, replays, averaged in _rows("replay_schedule.txt"):
        assert model.replay_count(n) == replays
        assert model.replays_averaged(n) == averaged


def test_replay_schedule_shape():
    assert model.replay_count(1024) == 1000
    sizes = list(range(1024, 12801, 128))
    counts = [model.replay_count(n) for n in sizes]
    assert all(a >= b for a, b in zip(counts, counts[1:]))
    assert counts[-1] >= 2


def test_reads_per_output_matches_page():
    for K, tm, tn, reads in _rows("global_reads_per_output.txt"):
        assert model.global_reads_per_output(K, tm, tn) == reads


def test_lds_budget_matches_page():
    for tm, tn, tk, eb, st, nbytes in _rows("lds_budget.txt"):
        assert model.lds_tile_bytes(tm, tn, tk, eb, st) == nbytes


def test_algorithmic_work():
    assert model.flops(4096, 4096, 4096) == 2 * 4096 ** 3
    assert model.algorithmic_bytes(4096, 4096, 4096, 4, False) == 3 * 4 * 4096 ** 2
    assert model.algorithmic_bytes(4096, 4096, 4096, 2, True) == 4 * 2 * 4096 ** 2


def test_bench_uses_model_schedule():
    import bench
    for n in (1024, 4096, 12800):
        assert bench.replay_count(n) == model.replay_count(n)
