"""Host-side checks of the benchmark's contract (no GPU): it refuses more than one GPU
with a message, counts flop per visited block at the block size, and keys the stored
counter summaries by the kernel code (comments and spacing aside)."""
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_flop_per_block():
    assert bench.block_flop(64) == 2 * 64 * 64 * 128
    assert bench.block_flop(128) == 2 * 128 * 128 * 128


def test_kernel_hash_ignores_comments_but_not_code(tmp_path):
    for p in bench.KERNEL_SOURCES:
        dst = tmp_path / p
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, p), dst)
    old_root = bench.ROOT
    try:
        bench.ROOT = str(tmp_path)
        base = bench.kernel_source_hash()
        src = tmp_path / bench.KERNEL_SOURCES[0]
        text = src.read_text()
        src.write_text("// a note\n/* another\n note */\n" + text.replace("\n", "\n\n", 3))
        assert bench.kernel_source_hash() == base
        src.write_text(text.replace("constexpr int kRing = 4;", "constexpr int kRing = 3;"))
        assert bench.kernel_source_hash() != base
    finally:
        bench.ROOT = old_root
