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
    assert set(t) == {"chunk_out", "chunk_out_gated", "state_walk", "decode_step"}
    for v in t.values():
        assert v is None or v > 0


def test_output_and_walk_bytes():
    # Output stage: bf16 Q, K (dk) and V, O (dv) per token-head, plus the bf16
    # dk x dv state of every chunk but the first (no state_in).
    per_tok = (2 * 256 + 2 * 512) * 2
    states = 8 * 16 * 15 * 256 * 512 * 2
    assert bench.output_bytes(8, 16, 8192, 512) == 8 * 16 * 8192 * per_tok + states
    assert bench.output_bytes(8, 16, 8192, 512, state_in=True) == 8 * 16 * 8192 * per_tok + states * 16 // 15
    # State stage: K, V read; the bf16 state of all 16 chunks and the fp32 final state written.
    assert bench.walk_bytes(8, 16, 8192, 512) == 8 * 16 * 8192 * 768 * 2 + 8 * 16 * 16 * 256 * 512 * 2 + 8 * 16 * 256 * 512 * 4
    # Both stages sit below the ridge point of 2.5 PFLOP/s over 8 TB/s.
    assert bench.output_flops(8, 16, 8192, 512) / bench.output_bytes(8, 16, 8192, 512) < bench.PEAK_BF16 / bench.PEAK_HBM
