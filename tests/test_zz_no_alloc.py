"""The allocation-free chunkwise entry point against retention_chunkwise (GPU).

retention_chunkwise_noalloc runs the same kernels as retention_chunkwise with
the library's own device scratch as workspace. Called through the C ABI, its
outputs and final states must equal those of retention_chunkwise with a
caller workspace (same kernels, same inputs: bit for bit, which implies the
2e-2 * max|o| bar), on two calls in a row, the second with a smaller input,
so the second runs over what the first left in the scratch. Sizes whose
workspace exceeds the scratch are refused with RET_ERR_UNSUPPORTED.
"""

import ctypes

import pytest
import torch

import retnet_retention_msr_amd as ret
from retnet_retention_msr_amd import _lib, synthetic

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _both(B, H, N, dk, dv, C, seed, gn=None, with_state=True):
    q, k, v = (t.to(DEV) for t in synthetic.make_qkv(B, H, N, dk, dv, dtype=torch.bfloat16, seed=seed))
    g = synthetic.head_gammas(H)
    s0 = synthetic.make_state(B, H, dk, dv, seed=seed + 1).to(DEV) if with_state else None
    ref, s_ref = ret.chunkwise(q, k, v, g, C, state_in=s0, state_out=True, gn=gn)
    out = torch.full((B, H, N, dv), float("nan"), dtype=torch.bfloat16, device=DEV)
    s_out = torch.full((B, H, dk, dv), float("nan"), dtype=torch.float32, device=DEV)
    ret.chunkwise_noalloc(q, k, v, g, C, out, state_in=s0, state_out=s_out, gn=gn)
    torch.cuda.synchronize()
    return ref, s_ref, out, s_out


@pytest.mark.parametrize("first, second", [
    ((1, 8, 2048, 256, 512, 256), (1, 4, 640, 256, 512, 128)),   # MFMA path (48 MiB), smaller second call
    ((1, 16, 2048, 256, 512, 512), (1, 2, 300, 128, 256, 64)),   # segmented walk (48 MiB), then a ragged tail
    ((1, 4, 200, 64, 96, 64), (1, 2, 77, 64, 96, 32)),            # generic kernels (dv 96)
])
def test_noalloc_equals_chunkwise_on_two_calls(first, second):
    print(f"[case] noalloc vs chunkwise: {first} then {second}", flush=True)
    for i, (shape, gn) in enumerate(((first, ret.GroupNorm(1e-5)), (second, None))):
        assert ret.chunkwise_workspace_bytes(*shape) <= _lib.NOALLOC_MAX_WORKSPACE_BYTES
        ref, s_ref, out, s_out = _both(*shape, seed=2000 + i, gn=gn)
        assert torch.equal(out, ref), (shape, (out.float() - ref.float()).abs().max().item())
        assert torch.equal(s_out, s_ref), (shape, (s_out - s_ref).abs().max().item())


def test_noalloc_refuses_sizes_beyond_its_scratch():
    lib = _lib.load()
    B, H, N, dk, dv, C = 8, 16, 8192, 256, 512, 512
    need = ret.chunkwise_workspace_bytes(B, H, N, dk, dv, C)
    if need <= _lib.NOALLOC_MAX_WORKSPACE_BYTES:
        pytest.skip("the 6.7B-shaped prefill fits the scratch")
    q = torch.empty(1, dtype=torch.bfloat16, device=DEV)
    g = (ctypes.c_float * H)(*synthetic.head_gammas(H).tolist())
    p = q.data_ptr()
    rc = lib.retention_chunkwise_noalloc(p, p, p, g, p, B, H, N, dk, dv, C, 1, None, None, None, None)
    assert rc == _lib.RET_ERR_UNSUPPORTED
