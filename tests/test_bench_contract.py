"""bench.py's host-side contract, on the CPU: the one-GPU refusal and the
algorithmic byte counts its roofline entries divide by."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=60)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_pool_bytes_of_the_configured_workloads():
    # 65536 tokens, ratio 4, 512 wide, fp4 out: every value of both 2 x 512
    # planes read once, 256 code bytes + 32 scale bytes per entry written
    assert bench.pool_bytes(1, 65536, 4, 512, True, False) == 2 * 65536 * 1024 * 4 + 16384 * (256 + 32)
    # the 128-wide indexer compressor, bf16 latent out
    assert bench.pool_bytes(1, 65536, 4, 128, False, True) == 2 * 65536 * 256 * 4 + 16384 * 128 * 2
    # ratio 128, 2 x 16384 tokens, 512 wide, bf16 latent out
    assert bench.pool_bytes(2, 16384, 128, 512, False, True) == 2 * 2 * 16384 * 512 * 4 + 2 * 128 * 512 * 2
    # e8m0 keys: blocks of 32
    assert bench.pool_bytes(1, 65536, 4, 128, True, False, block=32) == 2 * 65536 * 256 * 4 + 16384 * (64 + 4)


def test_post_projection_bytes_of_the_long_workload():
    tiles = 65536 // 256
    boundary = (tiles - 1) * (8 * 512 * 2 * 4 + 512 * 4)
    finish = 16384 * 512 * 4 + 16384 * (256 + 32)
    state = 4 * 1024 * 2 * 4 * 2
    assert bench.post_projection_bytes(1, 65536, 512, True) == boundary + finish + state


def test_kernel_source_hashes_cover_existing_files():
    for name in bench.KERNEL_SOURCES:
        assert len(bench.source_sha(name)) == 16
