"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Tolerances are those fixed for the operator: max|err| <= 1e-4 * max|o| for
fp32 inputs and <= 2e-2 * max|o| for bf16 inputs, checked per (b, h) head
slice against that slice's own max|o_ref| (stricter than one global max,
because short-memory heads have much smaller outputs than long-memory ones).
Both sides see identical inputs: bf16 tensors are widened exactly for the
oracle. Inputs come from the seeded generators in
retnet_retention_msr_amd.synthetic.
"""

import numpy as np
import pytest
import torch

import retnet_retention_msr_amd as ret
from oracle import retention_oracle as orc
from retnet_retention_msr_amd import synthetic

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
DEV = "cuda:0"


def _np(t):
    return t.detach().to("cpu").double().numpy()


def _check(got, ref, tol, what=""):
    """Per-head check: max |got - ref| <= tol * max|ref| over each [b, h] slice."""
    got = _np(got) if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what
    B, H = ref.shape[:2]
    for b in range(B):
        for h in range(H):
            scale = float(np.max(np.abs(ref[b, h])))
            err = float(np.max(np.abs(got[b, h] - ref[b, h])))
            assert err <= tol * max(scale, 1e-30), f"{what} b={b} h={h}: err {err:.3e} > {tol} * {scale:.3e}"


def _inputs(B, H, N, dk, dv, dtype, seed, with_state=False):
    q, k, v = synthetic.make_qkv(B, H, N, dk, dv, dtype=dtype, seed=seed)
    g = synthetic.head_gammas(H)
    S0 = synthetic.make_state(B, H, dk, dv, seed=seed + 1, std=0.5) if with_state else None
    return q, k, v, g, S0


def _dev(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


def _announce(msg):
    print(f"[case] {msg}", flush=True)


# ---------------------------------------------------------------------------
# Single-head fp32 case: B=1, H=1, N=64, d=16, gamma = 1 - 2^-5, chunk 16
# ---------------------------------------------------------------------------


def test_fp32_single_head_three_forms():
    _announce("fp32 single head: parallel, chunkwise, recurrent steps")
    q, k, v = synthetic.make_qkv(1, 1, 64, 16, 16, dtype=torch.float32, seed=1001, qk_var=1.0)
    g = torch.tensor([1 - 2.0 ** -5], dtype=torch.float32)
    ref, Sref = orc.recurrent(q, k, v, g)
    qd, kd, vd = _dev(q, k, v)
    _check(ret.parallel(qd, kd, vd, g), ref, 1e-4, "parallel")
    o, S = ret.chunkwise(qd, kd, vd, g, 16, state_out=True)
    _check(o, ref, 1e-4, "chunkwise")
    _check(S, Sref, 1e-4, "chunkwise state")
    state = torch.zeros(1, 1, 16, 16, device=DEV)
    outs = [ret.recurrent_step(qd[:, :, n].contiguous(), kd[:, :, n].contiguous(), vd[:, :, n].contiguous(), g, state)
            for n in range(64)]
    _check(torch.stack(outs, dim=2), ref, 1e-4, "recurrent steps")
    _check(state, Sref, 1e-4, "recurrent state")


def test_fp32_closed_form_all_ones():
    _announce("fp32 d=1 all-ones closed form")
    N = 64
    gamma = 1 - 2.0 ** -5
    ones = torch.ones(1, 1, N, 1, device=DEV)
    g = torch.tensor([gamma])
    n = np.arange(N)
    expect = ((1 - gamma ** (n + 1)) / (1 - gamma))[None, None, :, None]
    _check(ret.parallel(ones, ones, ones, g), expect, 1e-4, "parallel")
    _check(ret.chunkwise(ones, ones, ones, g, 16)[0], expect, 1e-4, "chunkwise")
    state = torch.zeros(1, 1, 1, 1, device=DEV)
    o = [ret.recurrent_step(ones[:, :, i].contiguous(), ones[:, :, i].contiguous(), ones[:, :, i].contiguous(), g,
                            state) for i in range(N)]
    _check(torch.stack(o, dim=2), expect, 1e-4, "recurrent")


@pytest.mark.parametrize("N,C", [(61, 16), (100, 7), (33, 64)])
def test_fp32_chunkwise_with_state_ragged(N, C):
    _announce(f"fp32 chunkwise with state N={N} C={C}")
    q, k, v, g, S0 = _inputs(2, 4, N, 24, 40, torch.float32, seed=N + C, with_state=True)
    ref, Sref = orc.chunkwise(q, k, v, g, C, state_in=S0)
    qd, kd, vd, S0d = _dev(q, k, v, S0)
    o, S = ret.chunkwise(qd, kd, vd, g, C, state_in=S0d, state_out=True)
    _check(o, ref, 1e-4, "o")
    _check(S, Sref, 1e-4, "state")


# ---------------------------------------------------------------------------
# bf16 on the MFMA kernels: small sizes spanning several tiles and a ragged tail
# ---------------------------------------------------------------------------

BF16_SHAPES = [
    # B, H, N, dk, dv, chunk
    (2, 3, 200, 64, 128, 64),
    (1, 2, 200, 64, 128, 128),
    (1, 2, 130, 256, 512, 64),
    (2, 2, 190, 96, 256, 128),
    (1, 3, 300, 32, 128, 192),
]


@pytest.mark.parametrize("B,H,N,dk,dv,C", BF16_SHAPES)
@pytest.mark.parametrize("with_state", [False, True])
def test_bf16_chunkwise_matches_oracle(B, H, N, dk, dv, C, with_state):
    _announce(f"bf16 chunkwise {B}x{H}x{N} dk={dk} dv={dv} C={C} state={with_state}")
    q, k, v, g, S0 = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=N * 7 + dk + C, with_state=with_state)
    ref, Sref = orc.chunkwise(q, k, v, g, C, state_in=S0)
    qd, kd, vd, S0d = _dev(q, k, v, S0)
    o, S = ret.chunkwise(qd, kd, vd, g, C, state_in=S0d, state_out=True)
    _check(o, ref, 2e-2, "o")
    _check(S, Sref, 2e-2, "state")


@pytest.mark.parametrize("B,H,N,dk,dv,C", BF16_SHAPES[:4])
def test_bf16_parallel_matches_oracle(B, H, N, dk, dv, C):
    _announce(f"bf16 parallel {B}x{H}x{N} dk={dk} dv={dv}")
    q, k, v, g, _ = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=N * 3 + dk)
    ref = orc.parallel(q, k, v, g)
    qd, kd, vd = _dev(q, k, v)
    _check(ret.parallel(qd, kd, vd, g), ref, 2e-2, "parallel")


@pytest.mark.parametrize("affine", [False, True])
@pytest.mark.parametrize("form", ["parallel", "chunkwise"])
def test_bf16_groupnorm_epilogue(affine, form):
    _announce(f"bf16 GroupNorm {form} affine={affine}")
    B, H, N, dk, dv, C = 2, 3, 200, 64, 256, 64
    q, k, v, g, S0 = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=77, with_state=(form == "chunkwise"))
    w, bvec = synthetic.make_gn_affine(H, dv, seed=78) if affine else (None, None)
    if form == "parallel":
        raw = orc.parallel(q, k, v, g)
    else:
        raw = orc.chunkwise(q, k, v, g, C, state_in=S0)[0]
    ref = orc.group_norm(raw, eps=1e-5, weight=w, bias=bvec)
    qd, kd, vd, S0d, wd, bd = _dev(q, k, v, S0, w, bvec)
    gn = ret.GroupNorm(1e-5, wd, bd)
    if form == "parallel":
        o = ret.parallel(qd, kd, vd, g, gn=gn)
    else:
        o = ret.chunkwise(qd, kd, vd, g, C, state_in=S0d, gn=gn)[0]
    _check(o, ref, 2e-2, "gn")


# Gated epilogue, swish(gate) * GroupNorm(O): every MFMA output-kernel
# instance (dv 128, 256, 512), a ragged last query block, state read-out and
# affine GroupNorm; and the fp32 generic kernel.
GATED_SHAPES = [
    # B, H, N, dk, dv, chunk, dtype
    (2, 3, 200, 64, 128, 64, torch.bfloat16),
    (1, 4, 333, 128, 256, 128, torch.bfloat16),
    (2, 2, 301, 256, 512, 256, torch.bfloat16),
    (1, 2, 45, 24, 40, 16, torch.float32),
]


@pytest.mark.parametrize("B,H,N,dk,dv,C,dtype", GATED_SHAPES)
@pytest.mark.parametrize("form", ["parallel", "chunkwise"])
def test_gated_groupnorm_epilogue(B, H, N, dk, dv, C, dtype, form):
    _announce(f"gated GroupNorm {form} {B}x{H}x{N} dk={dk} dv={dv} C={C} {dtype}")
    q, k, v, g, S0 = _inputs(B, H, N, dk, dv, dtype, seed=N + dv, with_state=(form == "chunkwise"))
    w, bvec = synthetic.make_gn_affine(H, dv, seed=N + 9)
    gate = synthetic.make_gate((B, H, N, dv), dtype=dtype, seed=N + 11)
    if form == "parallel":
        raw = orc.parallel(q, k, v, g)
    else:
        raw = orc.chunkwise(q, k, v, g, C, state_in=S0)[0]
    ref = orc.gated_group_norm(raw, gate, eps=1e-5, weight=w, bias=bvec)
    qd, kd, vd, S0d, wd, bd, gd = _dev(q, k, v, S0, w, bvec, gate)
    gn = ret.GroupNorm(1e-5, wd, bd)
    if form == "parallel":
        o = ret.parallel(qd, kd, vd, g, gn=gn, gate=gd)
    else:
        o = ret.chunkwise(qd, kd, vd, g, C, state_in=S0d, gn=gn, gate=gd)[0]
    _check(o, ref, TOL[dtype], "gated")
    # the ungated call on the same inputs still gives the plain GroupNorm
    if form == "chunkwise":
        o2 = ret.chunkwise(qd, kd, vd, g, C, state_in=S0d, gn=gn)[0]
        _check(o2, orc.group_norm(raw, eps=1e-5, weight=w, bias=bvec), TOL[dtype], "ungated")


def test_gated_large_gates_saturate():
    """Gates far out on both sides: swish(g) = g for g >> 0 and 0 for g << 0."""
    _announce("gated GroupNorm, saturating gates")
    B, H, N, dk, dv, C = 1, 2, 130, 64, 128, 64
    q, k, v, g, _ = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=5)
    gate = synthetic.make_gate((B, H, N, dv), dtype=torch.float32, seed=6)
    gate = (torch.sign(gate) * 100.0).to(torch.bfloat16)
    ref = orc.gated_group_norm(orc.chunkwise(q, k, v, g, C)[0], gate, eps=1e-5)
    qd, kd, vd, gd = _dev(q, k, v, gate)
    o = ret.chunkwise(qd, kd, vd, g, C, gn=ret.GroupNorm(1e-5), gate=gd)[0]
    _check(o, ref, 2e-2, "saturated")
    assert torch.all(o[(gd < 0)] == 0)


# Shapes with more 64-row query blocks than the output kernel runs workgroups
# (one per CU), so each workgroup takes several blocks, from different heads,
# chunk positions and a ragged tail, with state read-out and affine GroupNorm.
MANY_BLOCK_SHAPES = [
    # B, H, N, dk, dv, chunk
    (4, 16, 1000, 32, 128, 128),
    (4, 8, 700, 128, 256, 64),
    (2, 8, 1100, 256, 512, 256),
]


@pytest.mark.parametrize("B,H,N,dk,dv,C", MANY_BLOCK_SHAPES)
def test_bf16_chunkwise_many_blocks_per_workgroup(B, H, N, dk, dv, C):
    _announce(f"bf16 chunkwise many blocks {B}x{H}x{N} dk={dk} dv={dv} C={C}")
    q, k, v, g, S0 = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=N + dk + dv, with_state=True)
    w, bvec = synthetic.make_gn_affine(H, dv, seed=N + 5)
    raw, Sref = orc.chunkwise(q, k, v, g, C, state_in=S0)
    ref = orc.group_norm(raw, eps=1e-5, weight=w, bias=bvec)
    qd, kd, vd, S0d, wd, bd = _dev(q, k, v, S0, w, bvec)
    o, S = ret.chunkwise(qd, kd, vd, g, C, state_in=S0d, state_out=True, gn=ret.GroupNorm(1e-5, wd, bd))
    _check(o, ref, 2e-2, "o")
    _check(S, Sref, 2e-2, "state")


def test_bf16_generic_fallback_shapes():
    """bf16 sizes outside the MFMA kernels (dv=64, chunk not a multiple of 64) use the generic kernels."""
    _announce("bf16 generic fallback")
    q, k, v, g, S0 = _inputs(1, 2, 150, 48, 64, torch.bfloat16, seed=5, with_state=True)
    ref, Sref = orc.chunkwise(q, k, v, g, 50, state_in=S0)
    qd, kd, vd, S0d = _dev(q, k, v, S0)
    o, S = ret.chunkwise(qd, kd, vd, g, 50, state_in=S0d, state_out=True)
    _check(o, ref, 2e-2, "o")
    _check(S, Sref, 2e-2, "state")
    q, k, v, g, _ = _inputs(1, 2, 150, 64, 128, torch.bfloat16, seed=6)
    ref, _ = orc.chunkwise(q, k, v, g, 40)
    qd, kd, vd = _dev(q, k, v)
    _check(ret.chunkwise(qd, kd, vd, g, 40)[0], ref, 2e-2, "o chunk 40")


@pytest.mark.parametrize(
    "B,H,N,dk,dv,C",
    [
        # two walks (segment end states, then every segment from its true start):
        (1, 2, 1024 + 40, 96, 512, 64),  # 32-row k tiles
        (1, 2, 1024 + 40, 128, 256, 64),  # full-dk walk
        # one walk from zero per segment, then the fix-up pass:
        (1, 2, 1024 + 40, 64, 128, 192),  # 64-row k tiles
        (1, 3, 1000, 128, 256, 256),  # full-dk walk (dk 128)
        (1, 2, 1600, 256, 512, 512),  # full-dk walk (dk 256), ragged last chunk
    ],
)
def test_bf16_segmented_walk_and_aliased_state(B, H, N, dk, dv, C):
    """Few heads, many chunks: the state walk is cut into segments; state_out aliases state_in."""
    _announce(f"bf16 segmented walk {B}x{H}x{N} dk={dk} dv={dv} C={C}")
    q, k, v, g, S0 = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=11 + N + C, with_state=True)
    ref, Sref = orc.chunkwise(q, k, v, g, C, state_in=S0)
    qd, kd, vd, Sd = _dev(q, k, v, S0)
    o, S = ret.chunkwise(qd, kd, vd, g, C, state_in=Sd, state_out=Sd)
    assert S is Sd
    _check(o, ref, 2e-2, "o")
    _check(Sd, Sref, 2e-2, "state")


@pytest.mark.parametrize(
    "B,H,N,dk,dv,C",
    [
        (16, 16, 200, 256, 512, 64),  # 256 heads x 2 wide tiles: 256-column walk, dk 256
        (16, 16, 150, 128, 256, 64),  # 256 heads x 1 wide tile: 256-column walk, dk 128
    ],
)
def test_bf16_wide_walk_many_heads(B, H, N, dk, dv, C):
    """Enough heads for 256-column walk workgroups (no segmentation); ragged last chunk and a state in."""
    _announce(f"bf16 wide walk {B}x{H}x{N} dk={dk} dv={dv} C={C}")
    q, k, v, g, S0 = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=21 + N + dk, with_state=True)
    ref, Sref = orc.chunkwise(q, k, v, g, C, state_in=S0)
    qd, kd, vd, S0d = _dev(q, k, v, S0)
    o, S = ret.chunkwise(qd, kd, vd, g, C, state_in=S0d, state_out=True)
    _check(o, ref, 2e-2, "o")
    _check(S, Sref, 2e-2, "state")


# ---------------------------------------------------------------------------
# Decode step
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("gn_on", [False, True])
@pytest.mark.parametrize("dv", [128, 100])
def test_decode_steps_match_oracle(dtype, gn_on, dv):
    _announce(f"decode dtype={dtype} gn={gn_on} dv={dv}")
    B, H, dk, steps = 2, 3, 64, 5
    q, k, v = synthetic.make_qkv(B, H, steps, dk, dv, dtype=dtype, seed=21, qk_var=1.0)
    g = synthetic.head_gammas(H)
    S = synthetic.make_state(B, H, dk, dv, seed=22)
    w, bvec = synthetic.make_gn_affine(H, dv, seed=23)
    Sd = S.to(DEV)
    qd, kd, vd, wd, bd = _dev(q, k, v, w, bvec)
    Sref = S.double().numpy()
    tol = TOL[dtype]
    for n in range(steps):
        o_ref, Sref = orc.recurrent_step(q[:, :, n], k[:, :, n], v[:, :, n], g, Sref)
        if gn_on:
            o_ref = orc.group_norm(o_ref[:, :, None, :], 1e-5, w, bvec)[:, :, 0]
        gn = ret.GroupNorm(1e-5, wd, bd) if gn_on else None
        o = ret.recurrent_step(qd[:, :, n].contiguous(), kd[:, :, n].contiguous(), vd[:, :, n].contiguous(), g, Sd,
                               gn=gn)
        _check(o, o_ref, tol, f"o step {n}")
    _check(Sd, Sref, 1e-5, "state")


@pytest.mark.parametrize("dk", [128, 256])
@pytest.mark.parametrize("gn_on", [False, True])
def test_decode_batched_rows(dk, gn_on):
    """dk = 128 and 256 take the path that loads all of a thread's state rows first."""
    _announce(f"decode dk={dk} gn={gn_on}")
    B, H, dv, steps = 2, 3, 192, 3
    q, k, v = synthetic.make_qkv(B, H, steps, dk, dv, dtype=torch.bfloat16, seed=41, qk_var=1.0)
    g = synthetic.head_gammas(H)
    S = synthetic.make_state(B, H, dk, dv, seed=42)
    Sd = S.to(DEV)
    qd, kd, vd = _dev(q, k, v)
    Sref = S.double().numpy()
    for n in range(steps):
        o_ref, Sref = orc.recurrent_step(q[:, :, n], k[:, :, n], v[:, :, n], g, Sref)
        if gn_on:
            o_ref = orc.group_norm(o_ref[:, :, None, :], 1e-5)[:, :, 0]
        o = ret.recurrent_step(qd[:, :, n].contiguous(), kd[:, :, n].contiguous(), vd[:, :, n].contiguous(), g, Sd,
                               gn=ret.GroupNorm(1e-5) if gn_on else None)
        _check(o, o_ref, 2e-2, f"o step {n}")
    _check(Sd, Sref, 1e-5, "state")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dv", [128, 100])
def test_decode_gated_groupnorm(dtype, dv):
    _announce(f"decode gated dtype={dtype} dv={dv}")
    B, H, dk, steps = 2, 3, 64, 3
    q, k, v = synthetic.make_qkv(B, H, steps, dk, dv, dtype=dtype, seed=31, qk_var=1.0)
    g = synthetic.head_gammas(H)
    S = synthetic.make_state(B, H, dk, dv, seed=32)
    w, bvec = synthetic.make_gn_affine(H, dv, seed=33)
    gate = synthetic.make_gate((B, H, steps, dv), dtype=dtype, seed=34)
    Sd = S.to(DEV)
    qd, kd, vd, wd, bd, gd = _dev(q, k, v, w, bvec, gate)
    Sref = S.double().numpy()
    for n in range(steps):
        o_ref, Sref = orc.recurrent_step(q[:, :, n], k[:, :, n], v[:, :, n], g, Sref)
        o_ref = orc.gated_group_norm(o_ref[:, :, None, :], gate[:, :, n : n + 1], 1e-5, w, bvec)[:, :, 0]
        o = ret.recurrent_step(qd[:, :, n].contiguous(), kd[:, :, n].contiguous(), vd[:, :, n].contiguous(), g, Sd,
                               gn=ret.GroupNorm(1e-5, wd, bd), gate=gd[:, :, n].contiguous())
        _check(o, o_ref, TOL[dtype], f"o step {n}")
    _check(Sd, Sref, 1e-5, "state")


# ---------------------------------------------------------------------------
# Agreement between the GPU forms, the prefill seam, determinism
# ---------------------------------------------------------------------------


def test_gpu_forms_agree_bf16():
    _announce("bf16 GPU forms agree")
    B, H, N, dk, dv = 1, 4, 192, 64, 128
    q, k, v, g, _ = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=31)
    qd, kd, vd = _dev(q, k, v)
    o_par = ret.parallel(qd, kd, vd, g)
    o_chk, _ = ret.chunkwise(qd, kd, vd, g, 64)
    state = torch.zeros(B, H, dk, dv, device=DEV)
    o_rec = torch.stack([ret.recurrent_step(qd[:, :, n].contiguous(), kd[:, :, n].contiguous(),
                                            vd[:, :, n].contiguous(), g, state) for n in range(N)], dim=2)
    ref = _np(o_rec)
    _check(o_par, ref, 2e-2, "parallel vs recurrent")
    _check(o_chk, ref, 2e-2, "chunkwise vs recurrent")
    _check(o_chk, _np(o_par), 2e-2, "chunkwise vs parallel")


def test_prefill_seam_bf16():
    _announce("bf16 prefill seam")
    B, H, N, dk, dv, C, N1 = 1, 3, 320, 64, 128, 64, 128
    q, k, v, g, _ = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=41)
    qd, kd, vd = _dev(q, k, v)
    o_all, S_all = ret.chunkwise(qd, kd, vd, g, C, state_out=True)
    o1, S1 = ret.chunkwise(qd[:, :, :N1].contiguous(), kd[:, :, :N1].contiguous(), vd[:, :, :N1].contiguous(), g, C,
                           state_out=True)
    o2, S2 = ret.chunkwise(qd[:, :, N1:].contiguous(), kd[:, :, N1:].contiguous(), vd[:, :, N1:].contiguous(), g, C,
                           state_in=S1, state_out=True)
    _check(torch.cat([o1, o2], dim=2), _np(o_all), 2e-2, "seam o")
    _check(S2, _np(S_all), 2e-2, "seam state")


def test_bitwise_reproducible():
    _announce("bitwise reproducibility")
    q, k, v, g, S0 = _inputs(2, 4, 256, 128, 256, torch.bfloat16, seed=51, with_state=True)
    qd, kd, vd, S0d = _dev(q, k, v, S0)
    gn = ret.GroupNorm(1e-5)
    a, Sa = ret.chunkwise(qd, kd, vd, g, 64, state_in=S0d, state_out=True, gn=gn)
    b, Sb = ret.chunkwise(qd, kd, vd, g, 64, state_in=S0d, state_out=True, gn=gn)
    assert torch.equal(a, b) and torch.equal(Sa, Sb)


def test_invalid_gamma_raises():
    q, k, v, g, _ = _inputs(1, 2, 64, 32, 128, torch.bfloat16, seed=61)
    qd, kd, vd = _dev(q, k, v)
    with pytest.raises(ret.RetentionError):
        ret.parallel(qd, kd, vd, [0.5, 1.0])


@pytest.mark.parametrize("dtype,dk,dv,C", [(torch.bfloat16, 64, 128, 64), (torch.float32, 24, 40, 16)])
def test_stage_entry_points_equal_chunkwise(dtype, dk, dv, C):
    """retention_chunk_states + retention_chunk_output reproduce retention_chunkwise bit for bit."""
    _announce(f"stage entry points {dtype} dk={dk} dv={dv} C={C}")
    B, H, N = 2, 3, 200
    q, k, v, g, S0 = _inputs(B, H, N, dk, dv, dtype, seed=71, with_state=True)
    qd, kd, vd, S0d = _dev(q, k, v, S0)
    gn = ret.GroupNorm(1e-5)
    o_ref, S_ref = ret.chunkwise(qd, kd, vd, g, C, state_in=S0d, state_out=True, gn=gn)
    ws = torch.empty(ret.chunkwise_workspace_bytes(B, H, N, dk, dv, C, dtype), dtype=torch.uint8, device=DEV)
    S = torch.empty_like(S_ref)
    ret.chunk_states(kd, vd, g, C, ws, state_in=S0d, state_out=S)
    o = ret.chunk_output(qd, kd, vd, g, C, ws, has_state_in=True, gn=gn)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


# ---------------------------------------------------------------------------
# Backward pass: gradients against the oracle's (pinned) backward
# ---------------------------------------------------------------------------
BACKWARD_SHAPES = [
    # B, H, N, dk, dv, chunk, dtype
    (2, 2, 300, 64, 128, 64, torch.bfloat16),   # gradient retentions on MFMA (dV) and generic (dQ, dK)
    (1, 2, 257, 128, 256, 128, torch.bfloat16),  # all on MFMA, one part
    (1, 2, 200, 256, 512, 64, torch.bfloat16),   # all on MFMA, dv split into two 256-wide parts
    (1, 2, 45, 24, 300, 16, torch.float32),      # generic, dv split 256 + 44
]


@pytest.mark.parametrize("B,H,N,dk,dv,C,dtype", BACKWARD_SHAPES)
@pytest.mark.parametrize("with_state", [False, True])
def test_chunkwise_backward_matches_oracle(B, H, N, dk, dv, C, dtype, with_state):
    _announce(f"backward {B}x{H}x{N} dk={dk} dv={dv} C={C} {dtype} state={with_state}")
    q, k, v, g, S0 = _inputs(B, H, N, dk, dv, dtype, seed=N + dk, with_state=with_state)
    dO = synthetic.make_qkv(B, H, N, dk, dv, dtype=dtype, seed=N + 77)[2]
    dSN = synthetic.make_state(B, H, dk, dv, seed=N + 78, std=0.5) if with_state else None
    # (a zero starting state for the oracle when there is none, so that it also
    # returns the state gradient, which the GPU computes regardless)
    S0_ref = S0 if S0 is not None else torch.zeros(B, H, dk, dv)
    ref = orc.backward(q, k, v, g, dO, state_in=S0_ref, d_state_out=dSN)
    qd, kd, vd, dOd, S0d, dSNd = _dev(q, k, v, dO, S0, dSN)
    gq, gk, gv, gs = ret.chunkwise_backward(qd, kd, vd, dOd, g, C, state_in=S0d, grad_state_out=dSNd,
                                            grad_state_in=True)
    tol = TOL[dtype]
    _check(gq, ref[0], tol, "grad_q")
    _check(gk, ref[1], tol, "grad_k")
    _check(gv, ref[2], tol, "grad_v")
    _check(gs, ref[3], tol, "grad_state_in")


# ---------------------------------------------------------------------------
# Edge cases: a single token, a chunk longer than the sequence, the largest
# head count and value width the ABI takes, decays near 0 and near 1
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("N,C", [(1, 64), (5, 64), (63, 512)])
def test_short_sequences(dtype, N, C):
    _announce(f"short sequence N={N} C={C} {dtype}")
    B, H, dk, dv = 2, 2, 64, 128
    q, k, v, g, S0 = _inputs(B, H, N, dk, dv, dtype, seed=300 + N, with_state=True)
    ref, Sref = orc.chunkwise(q, k, v, g, C, state_in=S0)
    qd, kd, vd, S0d = _dev(q, k, v, S0)
    o, S = ret.chunkwise(qd, kd, vd, g, C, state_in=S0d, state_out=True)
    _check(o, ref, TOL[dtype], "o")
    _check(S, Sref, TOL[dtype], "state")
    _check(ret.parallel(qd, kd, vd, g), orc.parallel(q, k, v, g), TOL[dtype], "parallel")
    gq, gk, gv, gs = ret.chunkwise_backward(qd, kd, vd, vd, g, C, state_in=S0d, grad_state_in=True)
    bref = orc.backward(q, k, v, g, v, state_in=S0)
    for name, got, r in zip(("dq", "dk", "dv", "ds0"), (gq, gk, gv, gs), bref):
        _check(got, r, TOL[dtype], name)


def test_max_heads_and_wide_values():
    """256 heads (the ABI maximum; the decays are spread over [0.05, 0.999],
    since the 1 - 2^(-5-h) schedule rounds to 1 in fp32 from h = 19 on) and
    dv = 1024 (the widest value row, on the generic path)."""
    _announce("H=256 and dv=1024")
    B, H, N, dk, dv, C = 1, 256, 70, 32, 128, 64
    q, k, v, _, S0 = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=400, with_state=True)
    g = torch.linspace(0.05, 0.999, H)
    ref = orc.chunkwise(q, k, v, g, C, state_in=S0)[0]
    qd, kd, vd, S0d = _dev(q, k, v, S0)
    _check(ret.chunkwise(qd, kd, vd, g, C, state_in=S0d)[0], ref, 2e-2, "H=256")
    B, H, N, dk, dv = 1, 2, 90, 64, 1024
    q, k, v, g, _ = _inputs(B, H, N, dk, dv, torch.bfloat16, seed=401)
    qd, kd, vd = _dev(q, k, v)
    gn = ret.GroupNorm(1e-5)
    _check(ret.chunkwise(qd, kd, vd, g, 32, gn=gn)[0], orc.group_norm(orc.chunkwise(q, k, v, g, 32)[0]), 2e-2,
           "dv=1024")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_extreme_decays(dtype):
    """gamma near 0 (each token sees almost only itself) and near 1 (almost no decay)."""
    _announce(f"extreme decays {dtype}")
    B, H, N, dk, dv, C = 1, 2, 300, 64, 128, 64
    q, k, v, _, S0 = _inputs(B, H, N, dk, dv, dtype, seed=500, with_state=True)
    g = torch.tensor([1e-6, 1.0 - 2.0 ** -20])
    ref, Sref = orc.chunkwise(q, k, v, g, C, state_in=S0)
    qd, kd, vd, S0d = _dev(q, k, v, S0)
    o, S = ret.chunkwise(qd, kd, vd, g, C, state_in=S0d, state_out=True)
    _check(o, ref, TOL[dtype], "o")
    _check(S, Sref, TOL[dtype], "state")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_backward_extreme_decays_with_final_state_gradient(dtype):
    """gamma = 1e-6 and 1 - 2^-20 with a starting state and a final-state
    gradient (which enters the reverse-time retentions divided by gamma: 1e6
    for the first head), all four gradients against the oracle."""
    _announce(f"backward extreme decays with dS_N {dtype}")
    B, H, N, dk, dv, C = 1, 2, 300, 64, 128, 64
    q, k, v, _, S0 = _inputs(B, H, N, dk, dv, dtype, seed=510, with_state=True)
    g = torch.tensor([1e-6, 1.0 - 2.0 ** -20])
    dO = synthetic.make_qkv(B, H, N, dk, dv, dtype=dtype, seed=511)[2]
    dSN = synthetic.make_state(B, H, dk, dv, seed=512, std=0.1)
    qd, kd, vd, dOd, S0d, dSNd = _dev(q, k, v, dO, S0, dSN)
    gq, gk, gv, gs = ret.chunkwise_backward(qd, kd, vd, dOd, g, C, state_in=S0d, grad_state_out=dSNd,
                                            grad_state_in=True)
    torch.cuda.synchronize()
    refs = orc.backward(q, k, v, g, dO, state_in=S0, d_state_out=dSN)
    for name, got, r in zip(("dq", "dk", "dv", "dS0"), (gq, gk, gv, gs), refs):
        _check(got, r, TOL[dtype], name)
