"""Host-side checks of bench.py's accounting (no GPU needed)."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_flops_per_token_head_match_the_chunk_table():
    # (C+1)(dk+dv) intra-chunk causal half + 2*dk*dv read-out + 2*dk*dv update, per token-head.
    for c, per in bench.FLOP_PER_TOKEN_HEAD.items():
        assert bench.algorithmic_flops(1, 1, 1, c) == per
    assert bench.algorithmic_flops(8, 16, 8192, 512) == 918_272 * 8 * 16 * 8192


def test_output_and_walk_shares_add_up():
    total = bench.algorithmic_flops(8, 16, 8192, 512)
    out = bench.output_flops(8, 16, 8192, 512)
    assert total - out == 2 * 256 * 512 * 8 * 16 * 8192


def test_decode_bytes():
    assert bench.decode_bytes(8, 16) == 134_610_944


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_measured_traffic_is_keyed_by_kernel_source():
    t = bench.measured_traffic()
    assert set(t) == {"chunk_out", "state_walk", "decode_step"}
    for v in t.values():
        assert v is None or v > 0
