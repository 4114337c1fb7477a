"""GPU parity of the single-pass chunkwise kernel against the fp64 oracle.

retention_chunkwise takes the single-pass kernel (one workgroup per head and
256-column v tile walking the chunks with its state in registers, GroupNorm
statistics exchanged between the v tiles of a head) for bf16, dk 128 or 256,
dv a multiple of 256, chunk 64 or 128 (after clamping to the sequence), once
heads times v tiles reach 192. Every case here has that many, so every
chunkwise call below runs it (the workspace size, checked first, says which
path was planned); longer chunks plan the two stages. Outputs and
states are compared element by element with the oracle, per (b, h) slice at
2e-2 * max|o|. Cases: ragged tails and several chunk lengths, state in and
out (aliased too), GroupNorm with and without affine, the swish gate, dk 128
with one v tile, dv 1024 with four, sequences shorter than a block, extreme
decays, agreement with the two-stage entry points, and backward passes whose
retentions all take this kernel with the inputs read in place (reverse order,
row pitch, two retentions in one launch, later parts accumulating).
"""

import numpy as np
import pytest
import torch

import retnet_retention_msr_amd as ret
from oracle import retention_oracle as orc
from retnet_retention_msr_amd import synthetic

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-2


def _np(t):
    return t.detach().to("cpu").double().numpy()


def _check(got, ref, what=""):
    got = _np(got) if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what
    for b in range(ref.shape[0]):
        for h in range(ref.shape[1]):
            scale = float(np.max(np.abs(ref[b, h])))
            err = float(np.max(np.abs(got[b, h] - ref[b, h])))
            assert err <= TOL * max(scale, 1e-30), f"{what} b={b} h={h}: err {err:.3e} > {TOL} * {scale:.3e}"


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _is_single_pass(B, H, N, dk, dv, C):
    """The plan: the single-pass kernel's workspace is the GroupNorm exchange only."""
    units = B * H * (dv // 256)
    return ret.chunkwise_workspace_bytes(B, H, N, dk, dv, C) == units * 2048


def _align(x):
    return (x + 255) // 256 * 256


def _segments(B, H, N, dk, dv, C):
    """Segments the planner cuts each sequence into for the single pass (the
    rule the header states): enough for about 256 (head, segment, v tile)
    units, at least 4 chunks each, at least 192 units in all."""
    base = B * H * (dv // 256)
    nchunks = -(-N // C)
    nseg = min(-(-256 // base), nchunks // 4)
    assert nseg >= 2 and base * nseg >= 192, "not a segmented plan"
    cps = -(-nchunks // nseg)
    return -(-nchunks // cps)


def _is_segmented_single_pass(B, H, N, dk, dv, C):
    """Workspace of the segmented single pass: the exchange mailbox of every
    (head, segment, v tile), the segments' fp32 end states, and room for a copy
    of state_in."""
    nseg = _segments(B, H, N, dk, dv, C)
    want = (_align(B * H * nseg * (dv // 256) * 2048) + _align(B * H * nseg * dk * dv * 4)
            + _align(B * H * dk * dv * 4))
    return ret.chunkwise_workspace_bytes(B, H, N, dk, dv, C) == want


CASES = [
    # B, H, N, dk, dv, chunk, gn, affine, state
    (6, 16, 600, 256, 512, 128, True, True, True),     # ragged last chunk (64 + 24 rows), state in/out
    (6, 16, 200, 256, 512, 128, True, False, False),   # one full chunk and a 72-row tail
    (6, 16, 1000, 256, 512, 128, False, False, True),  # many chunks, ragged last chunk, no GroupNorm
    (12, 16, 384, 128, 256, 64, True, True, True),     # dk 128, one v tile (no exchange), chunk 64
    (3, 16, 512, 256, 1024, 128, True, True, False),   # four v tiles
    (4, 16, 300, 256, 768, 64, True, True, True),      # three v tiles (exchange among three), ragged
    (6, 16, 200, 256, 512, 64, True, False, True),     # chunk 64, N not a multiple of 32
]


@pytest.mark.parametrize("B, H, N, dk, dv, C, gn_on, affine, with_state", CASES)
def test_single_pass_matches_oracle(B, H, N, dk, dv, C, gn_on, affine, with_state):
    _announce(f"single pass B={B} H={H} N={N} dk={dk} dv={dv} chunk={C} gn={gn_on} affine={affine} "
              f"state={with_state}")
    assert _is_single_pass(B, H, N, dk, dv, C)
    q, k, v = synthetic.make_qkv(B, H, N, dk, dv, dtype=torch.bfloat16, seed=3000 + N + C)
    g = synthetic.head_gammas(H)
    S0 = synthetic.make_state(B, H, dk, dv, seed=3001 + N, std=0.5) if with_state else None
    w = b = None
    if affine:
        w, b = synthetic.make_gn_affine(H, dv, seed=3002)
    gn = ret.GroupNorm(1e-5, w.to(DEV) if w is not None else None, b.to(DEV) if b is not None else None) \
        if gn_on else None
    raw, S_ref = orc.chunkwise(q, k, v, g, C, state_in=S0)
    ref = orc.group_norm(raw, eps=1e-5, weight=w, bias=b) if gn_on else raw
    o, S = ret.chunkwise(q.to(DEV), k.to(DEV), v.to(DEV), g, C, state_in=None if S0 is None else S0.to(DEV),
                         state_out=True, gn=gn)
    torch.cuda.synchronize()
    _check(o, ref, "o")
    _check(S, S_ref, "state")


def test_single_pass_gated():
    B, H, N, dk, dv, C = 6, 16, 640, 256, 512, 128
    _announce(f"single pass gated B={B} H={H} N={N} chunk={C}")
    assert _is_single_pass(B, H, N, dk, dv, C)
    q, k, v = synthetic.make_qkv(B, H, N, dk, dv, dtype=torch.bfloat16, seed=3100)
    g = synthetic.head_gammas(H)
    gate = synthetic.make_gate((B, H, N, dv), dtype=torch.bfloat16, seed=3101)
    w, b = synthetic.make_gn_affine(H, dv, seed=3102)
    raw, _ = orc.chunkwise(q, k, v, g, C)
    ref = orc.gated_group_norm(raw, _np(gate), eps=1e-5, weight=w, bias=b)
    o, _ = ret.chunkwise(q.to(DEV), k.to(DEV), v.to(DEV), g, C, gn=ret.GroupNorm(1e-5, w.to(DEV), b.to(DEV)),
                         gate=gate.to(DEV))
    torch.cuda.synchronize()
    _check(o, ref, "gated o")


@pytest.mark.parametrize("N", [1, 31, 64, 65])
def test_single_pass_short_sequences_with_state(N):
    """A chunk of 512 is clamped to the sequence (at most 128 rows here), so
    these take the single pass."""
    B, H, dk, dv, C = 6, 16, 256, 512, 512
    _announce(f"single pass short N={N}")
    assert _is_single_pass(B, H, N, dk, dv, C)
    q, k, v = synthetic.make_qkv(B, H, N, dk, dv, dtype=torch.bfloat16, seed=3200 + N)
    g = synthetic.head_gammas(H)
    S0 = synthetic.make_state(B, H, dk, dv, seed=3201, std=0.5)
    raw, S_ref = orc.chunkwise(q, k, v, g, C, state_in=S0)
    Sd = S0.to(DEV)
    # state_out aliases state_in.
    o, S = ret.chunkwise(q.to(DEV), k.to(DEV), v.to(DEV), g, C, state_in=Sd, state_out=Sd, gn=ret.GroupNorm(1e-5))
    torch.cuda.synchronize()
    _check(o, orc.group_norm(raw, eps=1e-5), "o")
    _check(S, S_ref, "state")


def test_single_pass_extreme_decays():
    B, H, N, dk, dv, C = 6, 16, 384, 256, 512, 128
    _announce("single pass extreme decays")
    assert _is_single_pass(B, H, N, dk, dv, C)
    q, k, v = synthetic.make_qkv(B, H, N, dk, dv, dtype=torch.bfloat16, seed=3300)
    g = torch.tensor([1e-6, 1 - 2.0 ** -20, 0.05, 0.5, 0.3, 0.999] + [0.9] * 10, dtype=torch.float32)
    S0 = synthetic.make_state(B, H, dk, dv, seed=3301, std=0.5)
    raw, S_ref = orc.chunkwise(q, k, v, g, C, state_in=S0)
    o, S = ret.chunkwise(q.to(DEV), k.to(DEV), v.to(DEV), g, C, state_in=S0.to(DEV), state_out=True,
                         gn=ret.GroupNorm(1e-5))
    torch.cuda.synchronize()
    _check(o, orc.group_norm(raw, eps=1e-5), "o")
    _check(S, S_ref, "state")


def test_single_pass_agrees_with_the_two_stage_path():
    B, H, N, dk, dv, C = 6, 16, 1024, 256, 512, 128
    _announce("single pass vs two stages")
    assert _is_single_pass(B, H, N, dk, dv, C)
    q, k, v = (t.to(DEV) for t in synthetic.make_qkv(B, H, N, dk, dv, dtype=torch.bfloat16, seed=3400))
    g = synthetic.head_gammas(H)
    gn = ret.GroupNorm(1e-5)
    o1, S1 = ret.chunkwise(q, k, v, g, C, state_out=True, gn=gn)
    ws = torch.empty(ret.chunk_stages_workspace_bytes(B, H, N, dk, dv, C), dtype=torch.uint8, device=DEV)
    S2 = torch.empty_like(S1)
    ret.chunk_states(k, v, g, C, ws, state_out=S2)
    o2 = ret.chunk_output(q, k, v, g, C, ws, gn=gn)
    torch.cuda.synchronize()
    _check(o1, _np(o2), "o vs two stages")
    _check(S1, _np(S2), "state vs two stages")


def test_single_pass_repeatable():
    """No atomics on the output path: repeated calls give identical bits."""
    B, H, N, dk, dv, C = 6, 16, 512, 256, 512, 64
    _announce("single pass repeatable")
    q, k, v = (t.to(DEV) for t in synthetic.make_qkv(B, H, N, dk, dv, dtype=torch.bfloat16, seed=3500))
    g = synthetic.head_gammas(H)
    outs = [ret.chunkwise(q, k, v, g, C, state_out=True, gn=ret.GroupNorm(1e-5)) for _ in range(3)]
    torch.cuda.synchronize()
    for o, S in outs[1:]:
        assert torch.equal(o, outs[0][0])
        assert torch.equal(S, outs[0][1])


def _is_direct_backward(B, H, N, dk, dv, C):
    """Workspace of the backward on the single pass with in-place operands:
    four fp32 state buffers and the exchange words of the wider of its
    launches (dV: (head, v tile) units; a part of dQ and dK: two retentions)."""
    st = B * H * dk * dv * 4
    want = 4 * _align(st) + _align(max(B * H * (dv // 256), 2 * B * H * (dk // 256)) * 2048)
    return ret.chunkwise_backward_workspace_bytes(B, H, N, dk, dv, C) == want


BACKWARD_CASES = [
    # B, H, N, dv, chunk, state in / final-state gradient, decays
    (12, 16, 320, 512, 128, True, "schedule"),   # 192 units per retention, state in and out
    (12, 16, 200, 512, 64, False, "schedule"),   # ragged last chunk (8 rows), no states
    (6, 16, 150, 768, 64, True, "schedule"),     # three parts of dO / V (two adding), three v tiles of dV
    (12, 16, 130, 512, 64, True, "extreme"),     # gamma 1e-6 and 1 - 2^-20 with dS_N (divided by gamma)
    (12, 16, 600, 512, 256, True, "schedule"),   # chunk 256: four query blocks a chunk, ragged last chunk
    (12, 16, 1100, 512, 512, False, "schedule"), # chunk 512: eight query blocks, 76-row last chunk
    (12, 16, 200, 256, 64, True, "schedule"),    # dv 256: one part, dQ and dK in a single launch
    (6, 16, 140, 1024, 64, True, "schedule"),    # dv 1024: four parts (three adding), four v tiles of dV
    (12, 16, 40, 512, 512, True, "schedule"),    # one chunk shorter than a query block (40 rows)
]


@pytest.mark.parametrize("B, H, N, dv, C, with_state, decays", BACKWARD_CASES)
def test_backward_through_the_single_pass_kernel(B, H, N, dv, C, with_state, decays):
    """Every retention of the backward takes the single-pass kernel with the
    inputs where they are: dV over the v tiles of dO (reversed), then one
    launch per 256-wide part of V and dO holding both the dQ and the
    (reversed) dK retention, later parts adding to the first; all four
    gradients against the oracle."""
    dk = 256
    _announce(f"backward B={B} H={H} N={N} dv={dv} chunk={C} state={with_state} {decays} via the single pass")
    assert _is_direct_backward(B, H, N, dk, dv, C)
    q, k, v = synthetic.make_qkv(B, H, N, dk, dv, dtype=torch.bfloat16, seed=3600 + N)
    g = synthetic.head_gammas(H)
    if decays == "extreme":
        g = g.clone()
        g[0], g[H - 1] = 1e-6, 1.0 - 2.0 ** -20
    dO = synthetic.make_qkv(B, H, N, dk, dv, dtype=torch.bfloat16, seed=3601 + N)[2]
    S0 = synthetic.make_state(B, H, dk, dv, seed=3602, std=0.5) if with_state else None
    dSN = synthetic.make_state(B, H, dk, dv, seed=3603, std=0.05) if with_state else None
    dev = lambda t: None if t is None else t.to(DEV)
    gq, gk, gv, gs = ret.chunkwise_backward(dev(q), dev(k), dev(v), dev(dO), g, C, state_in=dev(S0),
                                            grad_state_out=dev(dSN), grad_state_in=True)
    torch.cuda.synchronize()
    S0_ref = S0 if S0 is not None else torch.zeros(B, H, dk, dv)
    refs = orc.backward(q, k, v, g, dO, state_in=S0_ref, d_state_out=dSN)
    for name, got, r in zip(("dq", "dk", "dv", "dS0"), (gq, gk, gv, gs), refs):
        _check(got, r, name)


@pytest.mark.parametrize("C", [256, 512])
def test_long_chunks_plan_the_two_stages(C):
    """Chunks above 128 plan the two stages: the workspace holds the chunk states."""
    B, H, N, dk, dv = 6, 16, 1024, 256, 512
    assert not _is_single_pass(B, H, N, dk, dv, C)
    assert ret.chunkwise_workspace_bytes(B, H, N, dk, dv, C) == ret.chunk_stages_workspace_bytes(B, H, N, dk, dv, C)


SEG_CASES = [
    # B, H, N, dk, dv, chunk, gn, affine, state: few heads, the sequence cut into segments
    (1, 16, 4096, 256, 512, 64, True, True, True),     # 8 segments of 8 chunks, state in and out
    (1, 8, 4100, 256, 512, 64, True, False, True),     # 13 segments, ragged last chunk (4 rows)
    (1, 16, 4096, 256, 512, 128, False, False, False), # chunk 128, no GroupNorm
    (2, 16, 2048, 128, 256, 64, True, True, True),     # dk 128, one v tile
]


@pytest.mark.parametrize("B, H, N, dk, dv, C, gn_on, affine, with_state", SEG_CASES)
def test_segmented_single_pass_matches_oracle(B, H, N, dk, dv, C, gn_on, affine, with_state):
    _announce(f"segmented single pass B={B} H={H} N={N} dk={dk} dv={dv} chunk={C} gn={gn_on} state={with_state}")
    assert _is_segmented_single_pass(B, H, N, dk, dv, C)
    q, k, v = synthetic.make_qkv(B, H, N, dk, dv, dtype=torch.bfloat16, seed=3700 + N + C)
    g = synthetic.head_gammas(H)
    S0 = synthetic.make_state(B, H, dk, dv, seed=3701 + N, std=0.5) if with_state else None
    w = b = None
    if affine:
        w, b = synthetic.make_gn_affine(H, dv, seed=3702)
    gn = ret.GroupNorm(1e-5, w.to(DEV) if w is not None else None, b.to(DEV) if b is not None else None) \
        if gn_on else None
    raw, S_ref = orc.chunkwise(q, k, v, g, C, state_in=S0)
    ref = orc.group_norm(raw, eps=1e-5, weight=w, bias=b) if gn_on else raw
    o, S = ret.chunkwise(q.to(DEV), k.to(DEV), v.to(DEV), g, C, state_in=None if S0 is None else S0.to(DEV),
                         state_out=True, gn=gn)
    torch.cuda.synchronize()
    _check(o, ref, "o")
    _check(S, S_ref, "state")


def test_segmented_single_pass_aliased_state_and_gate():
    """state_out aliasing state_in (read from a copy, since the first segment's
    workgroups may still read it while the last one's write), with the gate."""
    B, H, N, dk, dv, C = 1, 16, 2048, 256, 512, 64
    _announce("segmented single pass, aliased state, gated")
    assert _is_segmented_single_pass(B, H, N, dk, dv, C)
    q, k, v = synthetic.make_qkv(B, H, N, dk, dv, dtype=torch.bfloat16, seed=3800)
    g = synthetic.head_gammas(H)
    S0 = synthetic.make_state(B, H, dk, dv, seed=3801, std=0.5)
    gate = synthetic.make_gate((B, H, N, dv), dtype=torch.bfloat16, seed=3802)
    raw, S_ref = orc.chunkwise(q, k, v, g, C, state_in=S0)
    Sd = S0.to(DEV)
    o, S = ret.chunkwise(q.to(DEV), k.to(DEV), v.to(DEV), g, C, state_in=Sd, state_out=Sd, gn=ret.GroupNorm(1e-5),
                         gate=gate.to(DEV))
    torch.cuda.synchronize()
    assert S.data_ptr() == Sd.data_ptr()
    _check(o, orc.gated_group_norm(raw, _np(gate), eps=1e-5), "gated o")
    _check(S, S_ref, "state")


@pytest.mark.parametrize("with_state", [False, True])
def test_backward_single_token_within_the_part_rounding(with_state):
    """One token (every other row of each tile lies outside the sequence).
    dQ and dK are summed over the two 256-wide parts of dO and V, each part
    rounded to bf16 before the next adds to it; with one key the parts of an
    element can cancel (the score over 512 columns, |s| ~ 20, against a sum
    near zero), so their bound is the usual one plus the parts' own rounding,
    2^-8 * (|part 0| + |part 1|), with each part the oracle's gradient of the
    retention on that part's columns (the gradients are linear in that
    split). dV and the state gradient take no parts: the usual bound."""
    B, H, N, dk, dv, C = 12, 16, 1, 256, 512, 64
    _announce(f"backward B={B} H={H} N=1 state={with_state} within the part rounding")
    assert _is_direct_backward(B, H, N, dk, dv, C)
    q, k, v = synthetic.make_qkv(B, H, N, dk, dv, dtype=torch.bfloat16, seed=3950)
    g = synthetic.head_gammas(H)
    dO = synthetic.make_qkv(B, H, N, dk, dv, dtype=torch.bfloat16, seed=3951)[2]
    S0 = synthetic.make_state(B, H, dk, dv, seed=3952, std=0.5) if with_state else None
    dSN = synthetic.make_state(B, H, dk, dv, seed=3953, std=0.05) if with_state else None
    dev = lambda t: None if t is None else t.to(DEV)
    gq, gk, gv, gs = ret.chunkwise_backward(dev(q), dev(k), dev(v), dev(dO), g, C, state_in=dev(S0),
                                            grad_state_out=dev(dSN), grad_state_in=True)
    torch.cuda.synchronize()
    S0_ref = S0 if S0 is not None else torch.zeros(B, H, dk, dv)
    refs = orc.backward(q, k, v, g, dO, state_in=S0_ref, d_state_out=dSN)
    _check(gv, refs[2], "dv")
    _check(gs, refs[3], "dS0")
    parts = []
    for p in range(2):
        cols = slice(256 * p, 256 * (p + 1))
        parts.append(orc.backward(q, k, v[..., cols], g, dO[..., cols],
                                  state_in=S0_ref[..., cols],
                                  d_state_out=None if dSN is None else dSN[..., cols]))
    for name, got, r, idx in (("dq", gq, refs[0], 0), ("dk", gk, refs[1], 1)):
        got = _np(got)
        mag = np.abs(parts[0][idx]) + np.abs(parts[1][idx])
        for b in range(B):
            for h in range(H):
                err = float(np.max(np.abs(got[b, h] - r[b, h])))
                bound = TOL * float(np.max(np.abs(r[b, h]))) + 2.0 ** -8 * float(np.max(mag[b, h]))
                assert err <= bound, f"{name} b={b} h={h}: err {err:.3e} > {bound:.3e}"


def test_repeated_calls_are_bit_identical():
    """The single pass has no atomics in its arithmetic: repeated calls give
    the same bits. A read of LDS tiles before every wave's copies have landed
    (the first key block of each query block, before its wait was added)
    showed here as outputs that changed from call to call."""
    B, H, N, dk, dv = 12, 16, 1024, 256, 512
    _announce(f"repeat B={B} H={H} N={N}: forward chunk 64, backward chunks 64 and 256")
    q, k, v = (t.to(DEV) for t in synthetic.make_qkv(B, H, N, dk, dv, dtype=torch.bfloat16, seed=3900))
    dO = synthetic.make_qkv(B, H, N, dk, dv, dtype=torch.bfloat16, seed=3901)[2].to(DEV)
    g = synthetic.head_gammas(H)
    ref = None
    for _ in range(8):
        o, S = ret.chunkwise(q, k, v, g, 64, state_out=True, gn=ret.GroupNorm(1e-5))
        if ref is None:
            ref = (o.clone(), S.clone())
        assert torch.equal(o, ref[0]) and torch.equal(S, ref[1])
    for C in (64, 256):
        ref = None
        for _ in range(8):
            grads = ret.chunkwise_backward(q, k, v, dO, g, C)[:3]
            if ref is None:
                ref = tuple(x.clone() for x in grads)
            assert all(torch.equal(a, b) for a, b in zip(grads, ref)), C

