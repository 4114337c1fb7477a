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
    assert set(t) == {"fused", "xpos", "chunk_out", "chunk_out_gated", "state_walk", "decode_step"}
    for v in t.values():
        assert v is None or v > 0


def test_method_bytes_flops_and_intensity_at_the_prefill():
    # Q, K, V read once and O written once: (2*256 + 2*512) * 2 = 3,072 bytes per token-head.
    assert bench.method_bytes(1, 1, 1) == 3072
    assert bench.method_bytes(8, 16, 8192) == 3072 * 8 * 16 * 8192 == 3_221_225_472
    flop = bench.algorithmic_flops(8, 16, 8192, 512)
    assert round(flop / 1e9, 1) == 962.9  # 9.629e11 flop per forward
    assert round(flop / bench.method_bytes(8, 16, 8192)) == 299  # flop/B, below the 312.5 ridge
    assert flop / bench.method_bytes(8, 16, 8192) < bench.PEAK_BF16 / bench.PEAK_HBM
    # The output stage's share: 656,128 flop per token-head at chunk 512.
    assert bench.output_flops(1, 1, 1, 512) == 656_128


def test_roofline_fractions_use_the_binding_roof():
    # At chunk 512 the forward is HBM-bound (AI 299): the binding-roof fraction equals the HBM fraction.
    flop, nbytes = bench.algorithmic_flops(8, 16, 8192, 512), bench.method_bytes(8, 16, 8192)
    f = bench.roofline_fracs(flop, nbytes, 1e-3)
    assert f["binding_roof"] == "hbm"
    assert abs(f["binding_roof_frac"] - f["hbm_frac"]) < 1e-12
    assert abs(f["hbm_frac"] - nbytes / 1e-3 / 8e12) < 1e-12
    assert abs(f["mfma_frac"] - flop / 1e-3 / 2.5e15) < 1e-12
    # One row of 16 heads, 65,536 tokens at chunk 64: AI 187 flop/B; 20.4 M tokens/s reads about 0.13.
    flop64, bytes64 = bench.algorithmic_flops(1, 16, 65536, 64), bench.method_bytes(1, 16, 65536)
    assert round(flop64 / bytes64) == 187
    t = 65536 / 20.4e6
    assert abs(bench.roofline_fracs(flop64, bytes64, t)["binding_roof_frac"] - 0.128) < 0.005


def test_two_stage_design_bytes():
    # Method bytes, K and V again, the bf16 state of all 16 chunks written and
    # of 15 read back, and the fp32 final state.
    B, H, N = 8, 16, 8192
    st = 256 * 512 * 2
    expect = 3072 * B * H * N + 768 * 2 * B * H * N + B * H * (16 + 15) * st + B * H * 256 * 512 * 4
    assert bench.two_stage_design_bytes(B, H, N, 512) == expect
    assert bench.chunk_state_bytes(B, H, N, 512) == B * H * 15 * st
    assert bench.chunk_state_bytes(B, H, N, 512, state_in=True) == B * H * 16 * st


def test_single_pass_design_bytes_and_executed_flops():
    B, H, N = 8, 16, 8192
    # Each of the two 256-column v tiles of a head reads Q and K whole: (2*2*256 + 2*512) * 2 B per token-head,
    # plus the fp32 final state.
    assert bench.single_pass_design_bytes(B, H, N) == 4096 * B * H * N + B * H * 256 * 512 * 4
    # Scores and values over whole 32-key blocks up to each 64-row block's end: 64 keys per query at chunk 64
    # (against 32.5 for the causal half), 96 at chunk 128, 288 at chunk 512; scores once per v tile.
    for C, keys in ((64, 64), (128, 96), (512, 288)):
        per = keys * (2 * 256 * 2 + 2 * 512) + 4 * 256 * 512
        assert bench.single_pass_executed_flops(B, H, N, C) == per * B * H * N
        assert bench.single_pass_executed_flops(B, H, N, C) > bench.algorithmic_flops(B, H, N, C)


def test_backward_method_and_executed_flops():
    # Three retentions of the forward's kind (the count is symmetric in the
    # two widths): 3 * 918,272 flop per token-head at chunk 512.
    tok = 8 * 16 * 8192
    assert bench.backward_method_flops(8, 16, 8192, 512) == 3 * 918_272 * tok
    # Executed: dQ and dK each as two 256-wide parts, whose value products
    # (width dk) are formed once per part.
    per_part = 513 * (256 + 256) + 4 * 256 * 256
    assert bench.backward_flops(8, 16, 8192, 512) == (918_272 + 4 * per_part) * tok
    assert bench.backward_flops(8, 16, 8192, 64) > bench.backward_method_flops(8, 16, 8192, 64)
