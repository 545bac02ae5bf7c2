"""Host logic of the benchmark (no GPU): the counter-summary guard and the
block-aligned pieces of the CPU baseline."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_source_digest_ignores_comments_and_whitespace(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one\n}\n/* block */\n")
    b.write_text("int f(int x) { return x + 1; }\n// a different comment\n")
    assert bench.source_digest([str(a)]) == bench.source_digest([str(b)])
    b.write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_digest([str(a)]) != bench.source_digest([str(b)])


def test_read_traffic_refuses_a_changed_kernel(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k() {}\n")
    assert bench.read_traffic([str(src)]) is None


@pytest.mark.parametrize("total,parts,multiple", [(1, 1, 128), (127, 4, 128), (437_499_904, 64, 128),
                                                  (5_000, 64, 1), (128 * 1000 + 77, 7, 128)])
def test_cpu_pieces_tile_the_range(total, parts, multiple):
    step = bench._piece(total, parts, multiple)
    assert step % multiple == 0 and step >= multiple
    starts = list(range(0, total, step))
    assert len(starts) <= max(parts, 1) + 1
    assert all(s % multiple == 0 for s in starts)
    assert min(total, starts[-1] + step) == total
