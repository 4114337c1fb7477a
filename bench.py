#!/usr/bin/env python3
"""Benchmark of Multi-Scale Retention on one MI355X.

Step = one chunkwise MSR forward of a 6.7B-shaped prefill: B=8, H=16, N=8192,
dk=256, dv=512, chunk 512, bf16 in / fp32 accumulate, per-head GroupNorm
epilogue, fp32 state out (decay constants, intra-chunk products, cross-chunk
read-out, state carry, GroupNorm and state output all run inside the timed
call). Inputs are synthetic (seeded Gaussians, already resident in HBM).

Also timed: the recurrent decode step from the prefill's final state
(fp32 [8,16,256,512]), 1024 single-token steps back to back.

Prints ONE JSON line. `value` is prefill tokens/s (B*N tokens per step).
`roofline` is that of the dominant kernel, the output stage: its arithmetic
intensity (algorithmic flops over algorithmic HBM bytes, about 185 flop/B) is
below MI355X's ridge point (2.5 PFLOP/s / 8 TB/s = 312.5 flop/B), so its
binding roof is HBM: achieved = algorithmic bytes per launch (Q, K, V, the
bf16 chunk states it reads, O) over the launch time measured with HIP events,
against 8 TB/s. The same object also gives the matrix-core view (algorithmic
flops over time against the 2.5 PFLOP/s dense bf16 peak). `step_roofline`
does the same for the whole step (both stages), `state_walk` for the first
stage. `gated` times the same prefill with the gated epilogue
swish(gate) * GroupNorm(O) (the output kernel then also reads the bf16 gate).
`backward` times the backward pass (dQ, dK, dV) of the same prefill, with
the flops its decomposition executes against the bf16 MFMA peak and its
irreducible bytes against HBM.
`decode` carries the decode step's latency and its HBM roofline
(134,610,944 algorithmic bytes per step against 8 TB/s);
`decode_cache_defeating` repeats it at B=32, whose 256 MiB state does not fit
the Infinity Cache. `small_config` times the parallel and chunkwise forms at
B=2 H=8 N=2048, `long_sequence` the chunkwise form at B=1 H=16 from 8k to 64k
tokens and chunk 64..512, each with its binding-roofline fraction.
`cpu_baseline` is the fp64 CPU oracle on a bounded sample of the prefill
(plus, under `other_cases`, the decode step, the B=2 chunkwise case and the
65,536-token B=1 chunkwise case). `device` records the GPU, the HIP and torch
versions and the clocks rocm-smi reports after the timed work.

The default 30 untimed warm-up steps (about 60 ms of load) let the GPU reach
its sustained clocks first: from idle, the first 40 ms or so of this workload
run up to 20% slower.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

B, H, N, DK, DV, CHUNK = 8, 16, 8192, 256, 512, 512
SEED = 1003
DECODE_SEED = 1004
GATE_SEED = 1006
BACKWARD_SEED = 1007
PEAK_BF16 = 2.5e15
PEAK_HBM = 8.0e12
FLOP_PER_TOKEN_HEAD = {64: 574_208, 128: 623_360, 256: 721_664, 512: 918_272}


def algorithmic_flops(B, H, N, chunk, dk=DK, dv=DV):
    """Intra-chunk causal half (C+1)/2 * 2 * (dk+dv), read-out 2*dk*dv, update 2*dk*dv, per token-head.

    Exact for N a multiple of the chunk: the causal half of a chunk of length C
    has C(C+1)/2 score entries, each costing 2*dk (scores) + 2*dv (values).
    """
    per = (chunk + 1) * (dk + dv) + 4 * dk * dv
    return float(per) * B * H * N


def output_flops(B, H, N, chunk, dk=DK, dv=DV):
    """The output stage's share: intra-chunk causal half plus the cross-chunk read-out."""
    return float((chunk + 1) * (dk + dv) + 2 * dk * dv) * B * H * N


def method_bytes(B, H, N, dk=DK, dv=DV):
    """HBM bytes the method itself must move: bf16 Q, K, V read once and O
    written once, (2*dk + 2*dv) * 2 bytes per token-head (3,072 at dk 256,
    dv 512; 3.221e9 B for B8 H16 N8192). Whatever a design moves beyond this
    (states written and read back, operands read twice) is reported apart, as
    design bytes."""
    return float(B * H * N * (2 * dk + 2 * dv) * 2)


def chunk_state_bytes(B, H, N, chunk, dk=DK, dv=DV, state_in=False):
    """The bf16 state carried into every chunk that has one, as the two-stage
    design writes it once (state stage) and reads it once (output stage)."""
    nchunks = -(-N // chunk)
    states = nchunks if state_in else nchunks - 1
    return float(B * H * states * dk * dv * 2)


def two_stage_design_bytes(B, H, N, chunk, dk=DK, dv=DV):
    """Bytes the two-stage design moves per forward: method bytes, plus K and V
    read a second time by the state stage, plus the bf16 chunk states written
    by the state stage (every chunk) and read by the output stage (all but the
    first), plus the fp32 final state."""
    nchunks = -(-N // chunk)
    return (method_bytes(B, H, N, dk, dv) + float(B * H * N * (dk + dv) * 2)
            + float(B * H * nchunks * dk * dv * 2) + chunk_state_bytes(B, H, N, chunk, dk, dv)
            + float(B * H * dk * dv * 4))


def single_pass_design_bytes(B, H, N, dk=DK, dv=DV):
    """Bytes the single-pass kernel's workgroups request: each (head, 256-column
    v tile) reads Q and K whole and its V columns, and writes its O columns and
    its columns of the final fp32 state. Q and K are requested once per v tile
    (the v tiles of a head share an XCD, so the repeat is meant to hit L2)."""
    nvt = dv // 256
    return float(B * H * N * (nvt * 2 * dk + 2 * dv) * 2 + B * H * dk * dv * 4)


def single_pass_executed_flops(B, H, N, chunk, dk=DK, dv=DV):
    """Flops the single-pass kernel executes: the method's, with the scores of
    every 64-row query block against whole 32-key blocks up to its end
    (computed by each of the dv/256 v tiles) and the products with V over whole
    blocks, for N a multiple of the chunk and the chunk a multiple of 64."""
    nvt = dv // 256
    per_chunk_keys = sum(64 * (qb * 64 + 64) for qb in range(chunk // 64))
    per_token = per_chunk_keys / chunk
    return float(B * H * N * (per_token * 2 * dk * nvt + per_token * 2 * dv + 4 * dk * dv))


def roofline_fracs(flop, nbytes, seconds):
    """Fractions of the binding roof min(MFMA peak, AI * HBM peak), of HBM
    bandwidth and of the MFMA peak, for method flops and bytes over a time."""
    roof = min(PEAK_BF16, flop / nbytes * PEAK_HBM)
    return {"binding_roof": "mfma" if roof == PEAK_BF16 else "hbm",
            "binding_roof_frac": flop / seconds / roof,
            "hbm_frac": nbytes / seconds / PEAK_HBM,
            "mfma_frac": flop / seconds / PEAK_BF16}


def decode_bytes(B, H, dk=DK, dv=DV):
    """fp32 state read + written, bf16 q, k, v in and o out."""
    return 2 * B * H * dk * dv * 4 + B * H * (2 * dk + 2 * dv) * 2


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_6p7b_prefill_and_decode.md")
CSRC = os.path.join(ROOT, "retnet_retention_msr_amd", "csrc")


def _source_hash(names):
    import hashlib

    m = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            m.update(f.read())
    return m.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary.

    A figure is used only while the kernel source it was measured on is
    unchanged (hash of the kernel file, the headers it includes and, for the
    MFMA kernels, the build script that sets their flags); otherwise it is
    None.
    """
    current = {
        "fused": _source_hash(["fused.hip", "mfma_tiles.h", "common.h", "../build.py"]),
        "xpos": _source_hash(["xpos.hip", "common.h", "../build.py"]),
        "chunk_out": _source_hash(["mfma_out.hip", "mfma_tiles.h", "common.h", "../build.py"]),
        "chunk_out_gated": _source_hash(["mfma_out.hip", "mfma_tiles.h", "common.h", "../build.py"]),
        "state_walk": _source_hash(["mfma.hip", "mfma_tiles.h", "common.h", "../build.py"]),
        "decode_step": _source_hash(["decode.hip", "common.h"]),
    }
    out = {k: None for k in current}
    try:
        with open(TRAFFIC_FILE) as f:
            for line in f:
                parts = line.split()
                if len(parts) == 4 and parts[0] == "traffic" and parts[1] in current and parts[2] == current[parts[1]]:
                    out[parts[1]] = float(parts[3])
    except OSError:
        pass
    return out


def _cpu_threads():
    try:
        import threadpoolctl

        info = threadpoolctl.threadpool_info()
        blas = [i for i in info if i.get("user_api") == "blas"]
        if blas:
            return int(max(i["num_threads"] for i in blas)), blas[0].get("internal_api", "?")
    except Exception:
        pass
    return len(os.sched_getaffinity(0)), "unknown"


LONG_LENGTHS = (8192, 16384, 32768, 65536)
LONG_CHUNKS = (64, 128, 256, 512)


def long_sequence_sweep(ret, synthetic, dev, min_reps=5, warm_s=0.05, timed_s=0.02):
    """Tokens/s of the chunkwise forward (GroupNorm, fp32 state out) for one
    batch row of 16 heads as the sequence grows (chunk 512), and across chunk
    sizes at 65,536 tokens. Each point: calls back to back for `warm_s`
    seconds first (the clocks drop while the GPU idles, e.g. during the CPU
    baseline, and the shortest points last well under a millisecond), then
    HIP events around at least `min_reps` calls and at least `timed_s`
    seconds of them."""
    import torch

    H_ = 16
    gamma = synthetic.head_gammas(H_)
    gn = ret.GroupNorm(1e-5)
    q, k, v = synthetic.make_qkv(1, H_, max(LONG_LENGTHS), DK, DV, dtype=torch.bfloat16, seed=SEED + 7)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    del q, k, v

    def run(n, chunk):
        qs, ks, vs = qd[:, :, :n].contiguous(), kd[:, :, :n].contiguous(), vd[:, :, :n].contiguous()
        out = torch.empty(1, H_, n, DV, dtype=torch.bfloat16, device=dev)
        st = torch.empty(1, H_, DK, DV, dtype=torch.float32, device=dev)
        ws = torch.empty(ret.chunkwise_workspace_bytes(1, H_, n, DK, DV, chunk), dtype=torch.uint8, device=dev)
        f = lambda: ret.chunkwise(qs, ks, vs, gamma, chunk, state_out=st, gn=gn, out=out, workspace=ws)
        t0, calls = time.perf_counter(), 0
        while True:
            f()
            calls += 1
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= warm_s:
                break
        per_call = (time.perf_counter() - t0) / calls
        reps = max(min_reps, int(timed_s / per_call) + 1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        flop = algorithmic_flops(1, H_, n, chunk)
        byts = method_bytes(1, H_, n)
        return {"N": n, "chunk": chunk, "ms": ms, "reps": reps, "tokens_per_s": n / (ms * 1e-3),
                "algorithmic_flop": flop, "method_bytes": byts,
                **roofline_fracs(flop, byts, ms * 1e-3)}

    by_length = [run(n, 512) for n in LONG_LENGTHS]
    by_chunk = [run(max(LONG_LENGTHS), c) for c in LONG_CHUNKS]
    by_chunk_short = [run(min(LONG_LENGTHS), c) for c in LONG_CHUNKS]
    tps = [r["tokens_per_s"] for r in by_length]
    return {
        "workload": "B=1 H=16 dk=256 dv=512 bf16, GroupNorm, fp32 state out",
        "by_length_chunk512": by_length,
        "by_chunk_N65536": by_chunk,
        "by_chunk_N8192": by_chunk_short,
        "flatness_min_over_max": min(tps) / max(tps),
        # tokens/s at the longest length over tokens/s at the shortest, per chunk size
        "flatness_by_chunk": {str(c): hi["tokens_per_s"] / lo["tokens_per_s"]
                              for c, lo, hi in zip(LONG_CHUNKS, by_chunk_short, by_chunk)},
    }


def small_config(ret, synthetic, dev, reps=200, warm_s=0.05):
    """The 1.3B-shaped case (B=2, H=8, N=2048, dk=256, dv=512, chunk 256,
    bf16, seed 1002): parallel and chunkwise forward, µs per call from HIP
    events around `reps` calls after `warm_s` seconds of calls back to back
    (clocks settle), with tokens/s and the binding-roofline fraction
    (algorithmic flop and bytes as for the prefill)."""
    import torch

    b, h, n, c = 2, 8, 2048, 256
    gamma = synthetic.head_gammas(h)
    q, k, v = synthetic.make_qkv(b, h, n, DK, DV, dtype=torch.bfloat16, seed=1002)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty(b, h, n, DV, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(ret.chunkwise_workspace_bytes(b, h, n, DK, DV, c), dtype=torch.uint8, device=dev)

    def timed(f):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < warm_s:
            f()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    res = {"workload": "B=2 H=8 N=2048 dk=256 dv=512 bf16, no GroupNorm", "reps": reps}
    # parallel: N(N+1)/2 score entries per head, each 2*dk + 2*dv flop; bytes Q, K, V, O.
    par_flop = float(b * h * n * (n + 1) * (DK + DV))
    par_bytes = method_bytes(b, h, n)
    us = timed(lambda: ret.parallel(qd, kd, vd, gamma, out=out))
    res["parallel"] = {"us": us, "tokens_per_s": b * n / (us * 1e-6), "algorithmic_flop": par_flop,
                       "method_bytes": par_bytes, **roofline_fracs(par_flop, par_bytes, us * 1e-6)}
    ch_flop = algorithmic_flops(b, h, n, c)
    ch_bytes = method_bytes(b, h, n)
    us = timed(lambda: ret.chunkwise(qd, kd, vd, gamma, c, out=out, workspace=ws))
    res["chunkwise"] = {"us": us, "chunk": c, "tokens_per_s": b * n / (us * 1e-6), "algorithmic_flop": ch_flop,
                        "method_bytes": ch_bytes, **roofline_fracs(ch_flop, ch_bytes, us * 1e-6)}
    return res


def decode_cache_defeating(ret, synthetic, dev, steps=64):
    """Secondary decode measurement at B=32, H=16 (the fp32 state, 256 MiB,
    exceeds the 256 MB Infinity Cache, so each step's state read and write
    reach HBM): µs per step and algorithmic GB/s."""
    import torch

    b = 32
    gamma = synthetic.head_gammas(H)
    gen = torch.Generator().manual_seed(DECODE_SEED + 1)
    st = torch.randn(b, H, DK, DV, generator=gen).to(dev)
    qs = torch.randn(steps, b, H, DK, generator=gen).to(torch.bfloat16).to(dev)
    ks = torch.randn(steps, b, H, DK, generator=gen).to(torch.bfloat16).to(dev)
    vs = torch.randn(steps, b, H, DV, generator=gen).to(torch.bfloat16).to(dev)
    o = torch.empty(b, H, DV, dtype=torch.bfloat16, device=dev)
    for i in range(4):
        ret.recurrent_step(qs[i], ks[i], vs[i], gamma, st, out=o)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        ret.recurrent_step(qs[i], ks[i], vs[i], gamma, st, out=o)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    byts = decode_bytes(b, H)
    return {"B": b, "H": H, "steps": steps, "us_per_step": us, "algorithmic_bytes_per_step": byts,
            "achieved_gbps": byts / (us * 1e-6) / 1e9, "frac": byts / (us * 1e-6) / PEAK_HBM}


def cpu_extra(synthetic, gamma):
    """The fp64 oracle on the other measured cases: the decode step over all
    B*H heads (16 steps from a random state), the 1.3B-shaped chunkwise
    forward in full and the 65,536-token B=1 chunkwise forward (chunk 512,
    GroupNorm) in full."""
    import torch

    from oracle import retention_oracle as orc

    gen = torch.Generator().manual_seed(DECODE_SEED)
    st = torch.randn(B, H, DK, DV, generator=gen)
    qs = torch.randn(16, B, H, DK, generator=gen).to(torch.bfloat16)
    ks = torch.randn(16, B, H, DK, generator=gen).to(torch.bfloat16)
    vs = torch.randn(16, B, H, DV, generator=gen).to(torch.bfloat16)
    t0 = time.perf_counter()
    S = st
    for i in range(16):
        _, S = orc.recurrent_step(qs[i], ks[i], vs[i], gamma, S)
    dec_us = (time.perf_counter() - t0) / 16 * 1e6
    q2, k2, v2 = synthetic.make_qkv(2, 8, 2048, DK, DV, dtype=torch.bfloat16, seed=1002)
    t0 = time.perf_counter()
    orc.chunkwise(q2, k2, v2, synthetic.head_gammas(8), 256)
    small_s = time.perf_counter() - t0
    n_long = max(LONG_LENGTHS)
    q3, k3, v3 = synthetic.make_qkv(1, H, n_long, DK, DV, dtype=torch.bfloat16, seed=SEED + 7)
    t0 = time.perf_counter()
    o3, _ = orc.chunkwise(q3, k3, v3, synthetic.head_gammas(H), CHUNK)
    orc.group_norm(o3, eps=1e-5)
    long_s = time.perf_counter() - t0
    return {"decode_us_per_step": dec_us, "decode_workload": f"B={B} H={H} dk={DK} dv={DV}, 16 steps",
            "small_chunkwise_s": small_s, "small_tokens_per_s": 2 * 2048 / small_s,
            "small_workload": "B=2 H=8 N=2048 dk=256 dv=512 chunk 256",
            "long_chunkwise_s": long_s, "long_tokens_per_s": n_long / long_s,
            "long_workload": f"B=1 H={H} N={n_long} dk={DK} dv={DV} chunk {CHUNK}, GroupNorm"}


def device_info():
    """GPU name and architecture, HIP and torch versions, and the clocks rocm-smi
    reports right after the timed work (None where unavailable)."""
    import subprocess

    import torch

    props = torch.cuda.get_device_properties(0)
    info = {"name": props.name, "arch": getattr(props, "gcnArchName", None), "hip": torch.version.hip,
            "torch": torch.__version__, "rocm_smi_clocks": None}
    # Under a profiler (rocprofv3 preloads its tool library into every child,
    # which then holds the GPU before rocm-smi's interpreter starts) the
    # clocks are not read.
    if any(k.startswith(("ROCPROF_", "ROCPROFILER_")) for k in os.environ):
        return info
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        if r.returncode == 0:
            data = json.loads(r.stdout)
            card = next(iter(data.values())) if data else {}
            info["rocm_smi_clocks"] = {k: v for k, v in card.items() if "clock" in k.lower()}
    except (OSError, ValueError, subprocess.SubprocessError, StopIteration):
        pass
    return info


def cpu_baseline(q, k, v, gamma, n_batch_rows=2):
    """The fp64 oracle (as written, untuned) on batch rows 0..n_batch_rows-1 of the prefill."""
    import numpy as np

    from oracle import retention_oracle as orc

    qs, ks, vs = q[:n_batch_rows], k[:n_batch_rows], v[:n_batch_rows]
    t0 = time.perf_counter()
    o, _ = orc.chunkwise(qs, ks, vs, gamma, CHUNK)
    orc.group_norm(o, eps=1e-5)
    dt = time.perf_counter() - t0
    head_seqs = n_batch_rows * H
    # Equivalent full-workload tokens/s: every token spans H heads.
    tokens_per_s = head_seqs * N / H / dt
    threads, blas = _cpu_threads()
    del np
    return {
        "value": tokens_per_s,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"chunkwise+GroupNorm oracle (fp64, {blas} BLAS) on batch rows 0..{n_batch_rows - 1} "
                  f"({head_seqs} of {B * H} head-sequences, N={N}, chunk {CHUNK}), {dt:.1f} s, "
                  "scaled to full-workload tokens/s",
        "seconds": dt,
    }


def backward_flops(B, H, N, chunk, dk=DK, dv=DV, part=256):
    """Flops the backward executes: one retention of the forward's size for dV,
    and for dQ and dK one retention per part of the dv-wide query/key width
    (parts of at most 256, value width dk), each counted like the forward."""
    total = algorithmic_flops(B, H, N, chunk, dk, dv)
    for c in range(0, dv, part if dv > part else dv):
        w = min(part if dv > part else dv, dv - c)
        total += 2 * algorithmic_flops(B, H, N, chunk, w, dk)
    return total


def backward_method_flops(B, H, N, chunk, dk=DK, dv=DV):
    """The backward's own flops: three retentions of the forward's kind, dV
    with query/key width dk and value width dv, dQ and dK with query/key
    width dv and value width dk, each counted like the forward (what splitting
    the dv-wide query/key width into parts redoes is not counted)."""
    return algorithmic_flops(B, H, N, chunk, dk, dv) + 2 * algorithmic_flops(B, H, N, chunk, dv, dk)


def backward_min_bytes(B, H, N, dk=DK, dv=DV):
    """The backward's irreducible HBM traffic: bf16 Q, K, V and dO read, dQ, dK, dV written."""
    return float(B * H * N * ((2 * dk + 2 * dv) + (2 * dk + dv)) * 2)


def backward_pass(ret, torch, dev, stream, qd, kd, vd, gamma, steps, warmup=3, chunks=(CHUNK, 64)):
    """The backward pass of the same prefill (no states): dQ, dK, dV for a
    seeded dO, at the forward's chunk and at chunk 64, where its retentions
    plan the single-pass kernel (the gradients do not depend on the chunk)."""
    gen = torch.Generator(device=dev).manual_seed(BACKWARD_SEED)
    dO = torch.randn(B, H, N, DV, generator=gen, device=dev).to(torch.bfloat16)
    grads = (torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd))
    out = {}
    for C in chunks:
        ws = torch.empty(ret.chunkwise_backward_workspace_bytes(B, H, N, DK, DV, C), dtype=torch.uint8, device=dev)
        for _ in range(warmup):
            ret.chunkwise_backward(qd, kd, vd, dO, gamma, C, workspace=ws, grads=grads)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            ret.chunkwise_backward(qd, kd, vd, dO, gamma, C, workspace=ws, grads=grads)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        flop = backward_flops(B, H, N, C)
        mflop = backward_method_flops(B, H, N, C)
        nbytes = backward_min_bytes(B, H, N)
        del ws
        out[C] = {
            "workload": f"backward of the prefill above without GroupNorm or states at chunk {C}: dQ, dK, dV "
                        "for bf16 dO ~ N(0,1)",
            "chunk": C,
            "steps": steps,
            "ms": ms,
            "tokens_per_s": B * N / (ms * 1e-3),
            "method_flop": mflop,
            "mfma_frac": mflop / (ms * 1e-3) / PEAK_BF16,
            "executed_flop": flop,
            "mfma_tflops_executed": flop / (ms * 1e-3) / 1e12,
            "min_bytes": nbytes,
            "hbm_frac_of_min_bytes": nbytes / (ms * 1e-3) / PEAK_HBM,
        }
    del dO, grads
    res = dict(out[chunks[0]])
    for C in chunks[1:]:
        res[f"chunk_{C}"] = out[C]
    return res


def xpos_prologue(ret, torch, dev, stream, qd, kd, steps, warmup=5):
    """The xPos rotation of Q and K (retention_xpos_rotate, one launch over
    both) at the headline shape, out of place: Q and K read and written once,
    4 * B * H * N * dk * 2 bytes per call, bound by HBM."""
    B, H, N, d = qd.shape
    theta = ret.xpos_theta(d)
    oq, ok = torch.empty_like(qd), torch.empty_like(kd)
    for _ in range(warmup):
        ret.xpos_rotate(qd, kd, theta, pos0=0, out_q=oq, out_k=ok)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        ret.xpos_rotate(qd, kd, theta, pos0=0, out_q=oq, out_k=ok)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = 4.0 * B * H * N * d * 2
    del oq, ok
    return {
        "kernel": "xpos_kernel (retention_xpos_rotate on Q and K of B8 H16 N8192 dk256, bf16)",
        "launch_ms": ms,
        "roofline": {
            "bound": "hbm",
            "achieved": nbytes / (ms * 1e-3) / 1e9,
            "peak": PEAK_HBM / 1e9,
            "unit": "GB/s",
            "frac": nbytes / (ms * 1e-3) / PEAK_HBM,
            "algorithmic_bytes_per_launch": nbytes,
            "traffic": measured_traffic()["xpos"],
        },
    }


SINGLE_PASS_CHUNKS = (64, 128)


def single_pass_prefill(ret, torch, dev, stream, qd, kd, vd, gamma, state, out, gn, steps, warmup=10,
                        chunks=SINGLE_PASS_CHUNKS):
    """The headline shape at the chunk lengths that plan the single-pass
    kernel (retention_chunkwise, one launch after a small zeroing kernel).
    The chunk length changes only the blocking of the same retention (every
    chunk length gives the same outputs up to rounding) and the method's flop
    count; these are not the headline configuration, whose chunk is 512."""
    B, H, N = qd.shape[0], qd.shape[1], qd.shape[2]
    res = {}
    for C in chunks:
        ws = torch.empty(max(ret.chunkwise_workspace_bytes(B, H, N, DK, DV, C), 1), dtype=torch.uint8, device=dev)
        assert ret.chunkwise_workspace_bytes(B, H, N, DK, DV, C) == B * H * (DV // 256) * 2048, "not the single pass"

        def step():
            ret.chunkwise(qd, kd, vd, gamma, C, state_out=state, gn=gn, out=out, workspace=ws)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        flop = algorithmic_flops(B, H, N, C)
        mbytes = method_bytes(B, H, N)
        res[f"chunk_{C}"] = {
            "ms_per_step": ms,
            "tokens_per_s": B * N / (ms * 1e-3),
            "hbm_frac_of_method_bytes": mbytes / (ms * 1e-3) / PEAK_HBM,
            "method_flop": flop,
            "mfma_frac_of_method_flop": flop / (ms * 1e-3) / PEAK_BF16,
            "executed_flop": single_pass_executed_flops(B, H, N, C),
            "design_bytes": single_pass_design_bytes(B, H, N),
        }
        del ws
    res["kernel"] = "fused_chunk_kernel (retention_chunkwise at chunk 64 and 128: read-out, intra-chunk products, " \
                    "state update, GroupNorm and state out in one launch)"
    res["traffic_chunk_64"] = measured_traffic()["fused"]
    return res


def gated_prefill(ret, torch, dev, stream, qd, kd, vd, gamma, ws, state, out, gn, steps, warmup=5):
    """The same prefill with the gated epilogue, swish(gate) * GroupNorm(O).

    The gate ([B,H,N,dv] bf16, N(0, 4)) is drawn on the device from a seeded
    generator. The output kernel then also reads the gate: 2 bytes per output
    element more than the plain GroupNorm epilogue.
    """
    gen = torch.Generator(device=dev).manual_seed(GATE_SEED)
    gate = (torch.randn(B, H, N, DV, generator=gen, device=dev) * 2.0).to(torch.bfloat16)

    def step(events=None):
        if events is not None:
            events[0].record(stream)
        ret.chunk_states(kd, vd, gamma, CHUNK, ws, state_out=state)
        if events is not None:
            events[1].record(stream)
        ret.chunk_output(qd, kd, vd, gamma, CHUNK, ws, gn=gn, out=out, gate=gate)
        if events is not None:
            events[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(ev[i])
    torch.cuda.synchronize()
    ms = ev[0][0].elapsed_time(ev[-1][2]) / steps
    out_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    # Method bytes of the gated output: Q, K, V, O plus the gate read once.
    bytes_out = method_bytes(B, H, N) + B * H * N * DV * 2
    # The same gated prefill at chunk 64, where retention_chunkwise plans the
    # single pass (gate applied in its epilogue); one call per step.
    c64 = 64
    ws64 = torch.empty(max(ret.chunkwise_workspace_bytes(B, H, N, DK, DV, c64), 1), dtype=torch.uint8, device=dev)
    for _ in range(warmup):
        ret.chunkwise(qd, kd, vd, gamma, c64, state_out=state, gn=gn, out=out, workspace=ws64, gate=gate)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        ret.chunkwise(qd, kd, vd, gamma, c64, state_out=state, gn=gn, out=out, workspace=ws64, gate=gate)
    e1.record(stream)
    torch.cuda.synchronize()
    ms64 = e0.elapsed_time(e1) / steps
    del gate, ws64
    return {
        "workload": "the prefill above with the gated epilogue swish(gate) * GroupNorm(O), gate bf16 [B,H,N,dv]",
        "steps": steps,
        "ms_per_step": ms,
        "tokens_per_s": B * N / (ms * 1e-3),
        "output_launch_ms": out_ms,
        "output_roofline": {
            "bound": "hbm",
            "method_bytes_per_launch": bytes_out,
            "achieved": bytes_out / (out_ms * 1e-3) / 1e9,
            "peak": PEAK_HBM / 1e9,
            "unit": "GB/s",
            "frac": bytes_out / (out_ms * 1e-3) / PEAK_HBM,
            "traffic": measured_traffic()["chunk_out_gated"],
        },
        "single_pass_chunk_64": {
            "ms_per_step": ms64,
            "tokens_per_s": B * N / (ms64 * 1e-3),
            "hbm_frac_of_method_bytes": bytes_out / (ms64 * 1e-3) / PEAK_HBM,
        },
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-batch-rows", type=int, default=8)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (reference for HBM byte counters)")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-long", action="store_true", help="skip the long-sequence flatness sweep")
    ap.add_argument("--skip-small", action="store_true", help="skip the B=2 H=8 N=2048 timings")
    ap.add_argument("--skip-decode-b32", action="store_true", help="skip the cache-defeating B=32 decode timing")
    ap.add_argument("--skip-gated", action="store_true", help="skip the swish-gated prefill timing")
    ap.add_argument("--skip-backward", action="store_true", help="skip the backward-pass timing")
    ap.add_argument("--skip-xpos", action="store_true", help="skip the xPos rotation timing")
    ap.add_argument("--single-pass-chunks", default="64,128",
                    help="chunk lengths of the single-pass timings (each must plan the single pass)")
    ap.add_argument("--skip-single-pass", action="store_true",
                    help="skip the single-pass kernel timings at chunks 64 and 128")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the retention path here is a single-GPU build: a multi-GPU run would shard heads with "
              "no communication, which this bench does not launch.", file=sys.stderr)
        sys.exit(2)

    import torch

    import retnet_retention_msr_amd as ret
    from retnet_retention_msr_amd import synthetic

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(f"[bench] generating inputs B={B} H={H} N={N} dk={DK} dv={DV}", file=sys.stderr, flush=True)
    q, k, v = synthetic.make_qkv(B, H, N, DK, DV, dtype=torch.bfloat16, seed=SEED)
    gamma = synthetic.head_gammas(H)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty(B, H, N, DV, dtype=torch.bfloat16, device=dev)
    state = torch.empty(B, H, DK, DV, dtype=torch.float32, device=dev)
    ws = torch.empty(ret.chunkwise_workspace_bytes(B, H, N, DK, DV, CHUNK), dtype=torch.uint8, device=dev)
    gn = ret.GroupNorm(1e-5)

    def step(events=None):
        # One chunkwise forward as its two stages (the same work retention_chunkwise
        # launches); optional events bracket each stage on the current stream.
        if events is not None:
            events[0].record(stream)
        ret.chunk_states(kd, vd, gamma, CHUNK, ws, state_out=state)
        if events is not None:
            events[1].record(stream)
        ret.chunk_output(qd, kd, vd, gamma, CHUNK, ws, gn=gn, out=out)
        if events is not None:
            events[2].record(stream)

    stream = torch.cuda.current_stream()

    # The CPU oracle first, while the GPU has nothing to do; then the other
    # GPU measurements; the headline prefill last, so that its warm-up and
    # timed steps run at the clocks the GPU holds under sustained load (from
    # idle, the first tens of milliseconds of this load run slower).
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(q, k, v, gamma, args.cpu_batch_rows)
        cpu["other_cases"] = cpu_extra(synthetic, gamma)

    gated = None
    if not args.skip_gated:
        print(f"[bench] timing {args.steps} swish-gated prefill steps", file=sys.stderr, flush=True)
        gated = gated_prefill(ret, torch, dev, stream, qd, kd, vd, gamma, ws, state, out, gn, args.steps)

    xpos = None
    if not args.skip_xpos:
        print(f"[bench] timing {args.steps} xPos rotations of Q and K", file=sys.stderr, flush=True)
        xpos = xpos_prologue(ret, torch, dev, stream, qd, kd, args.steps)

    single_pass = None
    if not args.skip_single_pass:
        print(f"[bench] timing the single-pass kernel at chunks {args.single_pass_chunks}", file=sys.stderr,
              flush=True)
        chunks = tuple(int(c) for c in args.single_pass_chunks.split(","))
        single_pass = single_pass_prefill(ret, torch, dev, stream, qd, kd, vd, gamma, state, out, gn, args.steps,
                                          chunks=chunks)

    backward = None
    if not args.skip_backward:
        print(f"[bench] timing {args.steps} backward passes", file=sys.stderr, flush=True)
        backward = backward_pass(ret, torch, dev, stream, qd, kd, vd, gamma, args.steps)

    # Decode: single-token steps from the prefill's state.
    step()
    torch.cuda.synchronize()
    if args.skip_decode:
        args.decode_steps = 0
    print(f"[bench] timing {args.decode_steps} decode steps", file=sys.stderr, flush=True)
    gen = torch.Generator().manual_seed(DECODE_SEED)
    T = args.decode_steps
    dq = torch.randn(T, B, H, DK, generator=gen).to(torch.bfloat16).to(dev)
    dk_ = torch.randn(T, B, H, DK, generator=gen).to(torch.bfloat16).to(dev)
    dvv = torch.randn(T, B, H, DV, generator=gen).to(torch.bfloat16).to(dev)
    dstate = state.clone()
    dout = torch.empty(B, H, DV, dtype=torch.bfloat16, device=dev)
    for i in range(min(8, T)):
        ret.recurrent_step(dq[i], dk_[i], dvv[i], gamma, dstate, out=dout)
    torch.cuda.synchronize()
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    for i in range(T):
        ret.recurrent_step(dq[i], dk_[i], dvv[i], gamma, dstate, out=dout)
    d1.record(stream)
    torch.cuda.synchronize()
    us_step = d0.elapsed_time(d1) * 1e3 / T if T else float("nan")
    dbytes = decode_bytes(B, H)
    dgbps = dbytes / (us_step * 1e-6) / 1e9
    del dq, dk_, dvv, dstate

    decode_b32 = None
    if not args.skip_decode and not args.skip_decode_b32:
        print("[bench] cache-defeating decode (B=32)", file=sys.stderr, flush=True)
        decode_b32 = decode_cache_defeating(ret, synthetic, dev)

    small = None
    if not args.skip_small:
        print("[bench] B=2 H=8 N=2048 parallel and chunkwise", file=sys.stderr, flush=True)
        small = small_config(ret, synthetic, dev)

    long_seq = None
    if not args.skip_long:
        print("[bench] long-sequence sweep", file=sys.stderr, flush=True)
        long_seq = long_sequence_sweep(ret, synthetic, dev)

    # The headline: W untimed steps, then exactly K timed steps between two
    # synchronisations, HIP events on the launch stream around every stage.
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} prefill steps", file=sys.stderr, flush=True)
    t_wall = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = ev[0][0].elapsed_time(ev[-1][2]) / args.steps
    per_step = sorted(e[0].elapsed_time(e[2]) for e in ev)
    ms_median, ms_min = per_step[len(per_step) // 2], per_step[0]
    walk_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    out_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    tokens_per_s = B * N / (ms * 1e-3)
    flops = algorithmic_flops(B, H, N, CHUNK)
    achieved = flops / (ms * 1e-3)
    flops_out = output_flops(B, H, N, CHUNK)
    flops_walk = flops - flops_out
    mbytes = method_bytes(B, H, N)
    # What the two stages move by design: the output stage reads Q, K, V and
    # the bf16 chunk states and writes O; the state stage reads K and V again
    # and writes the chunk states and the final state.
    design_out = mbytes + chunk_state_bytes(B, H, N, CHUNK)
    design_step = two_stage_design_bytes(B, H, N, CHUNK)
    design_walk = design_step - design_out

    traffic = measured_traffic()
    line = {
        "metric": "chunkwise MSR tokens/s @B8 H16 N8k; decode-step µs; % of MFMA/HBM roofline",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": ms_median,
        "ms_per_step_min": ms_min,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "chunkwise MSR forward + per-head GroupNorm + fp32 state out, 6.7B-shaped prefill",
            "B": B, "H": H, "N": N, "dk": DK, "dv": DV, "chunk": CHUNK,
            "gamma": "1 - 2^(-5-h)", "parallelism": "single GPU",
        },
        # The dominant kernel is the output stage. Its fractions count the
        # method's bytes (Q, K, V read, O written) and the output stage's share
        # of the method's flops; the arithmetic intensity of the whole forward
        # (299 flop/B) and of this stage (214 flop/B) are both below the ridge
        # (312.5 flop/B), so the binding roof is HBM.
        "roofline": {
            "bound": "hbm",
            "achieved": mbytes / (out_ms * 1e-3) / 1e9,
            "peak": PEAK_HBM / 1e9,
            "unit": "GB/s",
            "frac": mbytes / (out_ms * 1e-3) / PEAK_HBM,
            "traffic": traffic["chunk_out"],
            "kernel": "mfma_chunk_out_kernel (retention_chunk_output: intra-chunk products, read-out, GroupNorm)",
            "method_bytes_per_launch": mbytes,
            "method_flop_per_launch": flops_out,
            "arithmetic_intensity_flop_per_byte": flops_out / mbytes,
            "ridge_flop_per_byte": PEAK_BF16 / PEAK_HBM,
            "design_bytes_per_launch": design_out,
            "design_over_method": design_out / mbytes,
            "traffic_over_method": traffic["chunk_out"] / mbytes if traffic["chunk_out"] else None,
            "mfma_tflops": flops_out / (out_ms * 1e-3) / 1e12,
            "mfma_frac": flops_out / (out_ms * 1e-3) / PEAK_BF16,
            "launch_ms": out_ms,
        },
        "step_roofline": {
            "bound": "hbm",
            "achieved": mbytes / (ms * 1e-3) / 1e9,
            "peak": PEAK_HBM / 1e9,
            "unit": "GB/s",
            "frac": mbytes / (ms * 1e-3) / PEAK_HBM,
            "method_bytes_per_step": mbytes,
            "method_flop_per_step": flops,
            "arithmetic_intensity_flop_per_byte": flops / mbytes,
            "design_bytes_per_step": design_step,
            "design_over_method": design_step / mbytes,
            "mfma_tflops": achieved / 1e12,
            "mfma_frac": achieved / PEAK_BF16,
        },
        "state_walk": {
            "kernel": "mfma_state_walk2_kernel (retention_chunk_states: chunk-state carry)",
            "launch_ms": walk_ms,
            "design_bytes_per_launch": design_walk,
            "design_gbps": design_walk / (walk_ms * 1e-3) / 1e9,
            "method_flop_per_launch": flops_walk,
            "mfma_tflops": flops_walk / (walk_ms * 1e-3) / 1e12,
            "traffic": traffic["state_walk"],
        },
        "gated": gated,
        "single_pass": single_pass,
        "xpos": xpos,
        "backward": backward,
        "decode": {
            "steps": T,
            "us_per_step": us_step,
            "roofline": {
                "bound": "hbm",
                "achieved": dgbps,
                "peak": PEAK_HBM / 1e9,
                "unit": "GB/s",
                "frac": dgbps * 1e9 / PEAK_HBM,
                "traffic": traffic["decode_step"],
                "algorithmic_bytes_per_step": dbytes,
            },
        },
        "decode_cache_defeating": decode_b32,
        "small_config": small,
        "long_sequence": long_seq,
        "cpu_baseline": cpu,
        "device": device_info(),
        "wall_s_timed": wall,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
