"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/retention.h declares,
and reject invalid or unsupported arguments before making any HIP call. Only
argument combinations that fail validation are passed to the real library;
the fake device pointers below are never dereferenced.

With RETENTION_ABI_TEST_LIB naming the host-only build of the validation and
planning code (tests/host_shim: the launchers replaced by stubs that record
the call and touch nothing; test_abi_sanitized.py builds it with the address
and undefined-behaviour sanitizers and runs this file against it), the same
checks run there, plus valid-argument calls that go through planning to the
stub launchers.
"""

import ctypes
import os
import re
import subprocess

import pytest

from retnet_retention_msr_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "retention.h")

FAKE = 0x10000  # never dereferenced: every call below fails validation first (or reaches a stub launcher)

SHIM = os.environ.get("RETENTION_ABI_TEST_LIB")
shim_only = pytest.mark.skipif(not SHIM, reason="valid-argument calls only run against the host shim")


@pytest.fixture(scope="module")
def lib():
    if SHIM:
        lib = _lib.open_library(SHIM)
        lib.retention_shim_launches.restype = ctypes.c_int
        return lib
    return _lib.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(retention_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert _declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.retention_abi_version() == _lib.ABI_VERSION == 4
    assert _lib.status_string(0) == "ok"
    assert _lib.status_string(-1) == "invalid argument"
    assert _lib.status_string(-2) == "unsupported arguments"
    assert _lib.status_string(-3) == "HIP runtime error"
    assert _lib.status_string(7) == "unknown status"


def _gamma(vals):
    return (ctypes.c_float * len(vals))(*vals)


def _parallel(lib, B=1, H=2, N=8, dk=32, dv=128, dtype=1, gamma=None, q=FAKE, o=FAKE, gn=None):
    g = _gamma(gamma if gamma is not None else [0.9] * H)
    return lib.retention_parallel(q, FAKE, FAKE, g, o, B, H, N, dk, dv, dtype, gn, None)


@pytest.mark.parametrize(
    "kw",
    [
        dict(q=None),
        dict(o=None),
        dict(B=0),
        dict(H=-1),
        dict(N=0),
        dict(dk=0),
        dict(dv=-5),
        dict(dtype=2),
        dict(dtype=-1),
        dict(gamma=[0.9, 1.0]),
        dict(gamma=[0.0, 0.5]),
        dict(gamma=[0.5, 1.5]),
        dict(gamma=[float("nan"), 0.5]),
        dict(gamma=[float("inf"), 0.5]),
        dict(gamma=[-0.5, 0.5]),
    ],
)
def test_parallel_rejects_invalid_arguments(lib, kw):
    assert _parallel(lib, **kw) == _lib.RET_ERR_INVALID_ARG


def test_parallel_rejects_null_gamma(lib):
    assert lib.retention_parallel(FAKE, FAKE, FAKE, None, FAKE, 1, 1, 8, 32, 128, 1, None, None) == -1


def test_groupnorm_eps_is_validated(lib):
    for eps in (-1e-5, float("nan"), float("inf")):
        gn = _lib.GnStruct(eps, None, None, None)
        assert _parallel(lib, gn=ctypes.byref(gn)) == _lib.RET_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(H=257), dict(dk=257), dict(dv=1025)])
def test_parallel_reports_unsupported_sizes(lib, kw):
    assert _parallel(lib, **kw) == _lib.RET_ERR_UNSUPPORTED


def _chunkwise(lib, chunk=64, ws=FAKE, ws_bytes=1 << 40, q=FAKE, B=1, H=2, N=256, dk=64, dv=128, dtype=1):
    g = _gamma([0.9] * H)
    return lib.retention_chunkwise(q, FAKE, FAKE, g, FAKE, B, H, N, dk, dv, chunk, dtype, None, None, None, ws,
                                   ws_bytes, None)


def test_chunkwise_rejects_invalid_arguments(lib):
    assert _chunkwise(lib, chunk=0) == -1
    assert _chunkwise(lib, chunk=-64) == -1
    assert _chunkwise(lib, q=None) == -1
    assert _chunkwise(lib, ws=None) == -1
    need = lib.retention_chunkwise_workspace_bytes(1, 2, 256, 64, 128, 64, 1)
    assert need > 0
    assert _chunkwise(lib, ws_bytes=need - 1) == -1


def test_recurrent_step_rejects_invalid_arguments(lib):
    g = _gamma([0.9])
    assert lib.retention_recurrent_step(FAKE, FAKE, FAKE, g, None, FAKE, 1, 1, 32, 32, 1, None, None) == -1
    assert lib.retention_recurrent_step(FAKE, FAKE, FAKE, g, FAKE, FAKE, 1, 1, 0, 32, 1, None, None) == -1
    assert lib.retention_recurrent_step(FAKE, FAKE, FAKE, _gamma([1.0]), FAKE, FAKE, 1, 1, 32, 32, 1, None,
                                        None) == -1
    assert lib.retention_recurrent_step(FAKE, FAKE, FAKE, g, FAKE, FAKE, 1, 1, 512, 32, 1, None, None) == -2


def test_workspace_bytes(lib):
    ws = lib.retention_chunkwise_workspace_bytes
    st = lib.retention_chunk_stages_workspace_bytes
    # The 6.7B-shaped prefill at chunks of 64 or 128 runs the single-pass
    # kernel: its workspace is only the GroupNorm exchange, two slots per
    # (head, 256-column v tile) of 64 rows of two tagged 64-bit words (mean,
    # sum of squared deviations): 2 KiB.
    units = 8 * 16 * 2
    assert ws(8, 16, 8192, 256, 512, 128, 1) == units * 2048
    # It does not grow with the sequence or with the chunk length.
    assert ws(8, 16, 65536, 256, 512, 64, 1) == ws(8, 16, 8192, 256, 512, 128, 1)
    # dk 128, dv 1024 (four v tiles).
    assert ws(4, 16, 4096, 128, 1024, 64, 1) == 256 * 2048
    # A chunk past 128 is clamped to the sequence first: N = 100 takes chunk 128.
    assert ws(8, 16, 100, 256, 512, 512, 1) == units * 2048
    # Longer chunks plan the two stages, whose entry points keep one bf16 state
    # per chunk and head (no segments here).
    assert st(8, 16, 8192, 256, 512, 512, 1) == 8 * 16 * 16 * 256 * 512 * 2
    assert ws(8, 16, 8192, 256, 512, 512, 1) == st(8, 16, 8192, 256, 512, 512, 1)
    # Few heads at chunk 64: the single pass over segments of the sequence (32
    # (head, v tile) pairs, so 8 segments of 128 chunks): the mailbox of 256
    # units, the segments' fp32 end states and room for a copy of state_in,
    # 72.5 MiB instead of the 4 GiB of bf16 chunk states the two stages need.
    seg = 16 * 8 * 2 * 2048 + 16 * 8 * 256 * 512 * 4 + 16 * 256 * 512 * 4
    assert ws(1, 16, 65536, 256, 512, 64, 1) == seg
    assert st(1, 16, 65536, 256, 512, 64, 1) > 4 * 2**30
    assert ws(8, 16, 8192, 256, 512, 256, 1) == st(8, 16, 8192, 256, 512, 256, 1)
    # Few heads (the single-pass kernel would leave most of the GPU idle): the
    # two-stage path and its chunk states, cut into segments whose fp32 end
    # states follow the chunk states.
    n = ws(1, 16, 65536, 256, 512, 512, 1)
    chunk_states = 16 * 128 * 256 * 512 * 2
    assert n == st(1, 16, 65536, 256, 512, 512, 1)
    assert n > chunk_states and (n - chunk_states) % (16 * 256 * 512 * 4) == 0
    # fp32 path: one fp32 state per chunk and head.
    assert ws(1, 1, 64, 16, 16, 16, 0) == 4 * 16 * 16 * 4
    # Invalid sizes give 0.
    assert ws(0, 16, 8192, 256, 512, 512, 1) == 0
    assert ws(1, 16, 8192, 256, 512, 0, 1) == 0
    assert st(0, 16, 8192, 256, 512, 512, 1) == 0


def test_chunk_stage_entry_points_validate(lib):
    g = _gamma([0.9, 0.8])
    need = lib.retention_chunk_stages_workspace_bytes(1, 2, 256, 64, 128, 64, 1)
    # states: null k, bad chunk, short workspace, bad gamma
    assert lib.retention_chunk_states(None, FAKE, g, 1, 2, 256, 64, 128, 64, 1, None, None, FAKE, need, None) == -1
    assert lib.retention_chunk_states(FAKE, FAKE, g, 1, 2, 256, 64, 128, 0, 1, None, None, FAKE, need, None) == -1
    assert lib.retention_chunk_states(FAKE, FAKE, g, 1, 2, 256, 64, 128, 64, 1, None, None, FAKE, need - 1,
                                      None) == -1
    assert lib.retention_chunk_states(FAKE, FAKE, _gamma([0.9, 1.0]), 1, 2, 256, 64, 128, 64, 1, None, None, FAKE,
                                      need, None) == -1
    # output: null o, unknown dtype, missing workspace
    assert lib.retention_chunk_output(FAKE, FAKE, FAKE, g, None, 1, 2, 256, 64, 128, 64, 1, 0, None, FAKE, need,
                                      None) == -1
    assert lib.retention_chunk_output(FAKE, FAKE, FAKE, g, FAKE, 1, 2, 256, 64, 128, 64, 3, 0, None, FAKE, need,
                                      None) == -1
    assert lib.retention_chunk_output(FAKE, FAKE, FAKE, g, FAKE, 1, 2, 256, 64, 128, 64, 1, 0, None, None, 0,
                                      None) == -1


def test_gn_struct_layout_matches_the_header(tmp_path):
    """ctypes' retention_gn_t has the C compiler's size and field offsets."""
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "retention.h"\n'
        "int main(void) { printf(\"%zu %zu %zu %zu %zu\\n\", sizeof(retention_gn_t),"
        " offsetof(retention_gn_t, eps), offsetof(retention_gn_t, weight),"
        " offsetof(retention_gn_t, bias), offsetof(retention_gn_t, gate)); return 0; }\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    S = _lib.GnStruct
    assert got == [ctypes.sizeof(S), S.eps.offset, S.weight.offset, S.bias.offset, S.gate.offset]


def test_gate_needs_groupnorm():
    import retnet_retention_msr_amd as ret

    with pytest.raises(ValueError, match="needs the GroupNorm"):
        ret._gn_struct(None, 2, 128, None, gate=object())


# Distinct fake addresses (1 TiB apart, never dereferenced) for the backward's
# q, k, v, dO and its three gradients, which may not share bytes.
BW = [FAKE + (i << 40) for i in range(7)]


def _backward(lib, gq=BW[4], ws=FAKE, ws_bytes=1 << 40, chunk=64, gamma=None, B=1, H=2, N=256, dk=64, dv=128,
              dtype=1, ptrs=None):
    g = _gamma(gamma or [0.9] * H)
    q, k, v, do, _, gk, gv = ptrs or BW
    return lib.retention_chunkwise_backward(q, k, v, do, g, gq, gk, gv, B, H, N, dk, dv, chunk, dtype,
                                            None, None, None, ws, ws_bytes, None)


def test_backward_rejects_invalid_arguments(lib):
    need = lib.retention_chunkwise_backward_workspace_bytes(1, 2, 256, 64, 128, 64, 1)
    assert need > 0
    assert _backward(lib, gq=None) == -1
    assert _backward(lib, ws=None) == -1
    assert _backward(lib, ws_bytes=need - 1) == -1
    assert _backward(lib, chunk=0) == -1
    assert _backward(lib, gamma=[0.9, 1.0]) == -1
    assert _backward(lib, N=0) == -1
    assert _backward(lib, dtype=2) == -1
    assert _backward(lib, H=257, gamma=[0.9] * 257) == -2


def test_outputs_that_share_bytes_with_inputs_are_refused(lib):
    """O is written while other workgroups still read Q, K and V (and the
    gate where they store): an O sharing bytes with any of them, or a gate
    sharing bytes with O, is refused before anything is launched; so is a
    decode state sharing bytes with the token's vectors."""
    B, H, N, dk, dv = 1, 2, 256, 64, 128
    nk, nv = B * H * N * dk * 2, B * H * N * dv * 2
    q, k, v, o = BW[:4]
    g = _gamma([0.9] * H)
    need = lib.retention_chunkwise_workspace_bytes(B, H, N, dk, dv, 64, 1)
    for oo in (q + nk - 2, k - nv + 2, v + 64):
        assert lib.retention_parallel(q, k, v, g, oo, B, H, N, dk, dv, 1, None, None) == -1
        assert lib.retention_chunkwise(q, k, v, g, oo, B, H, N, dk, dv, 64, 1, None, None, None, FAKE, need,
                                       None) == -1
    gate = _lib.GnStruct(1e-5, None, None, o + nv // 2)
    assert lib.retention_chunkwise(q, k, v, g, o, B, H, N, dk, dv, 64, 1, None, None, ctypes.byref(gate), FAKE,
                                   need, None) == -1
    snb = B * H * dk * dv * 4
    assert lib.retention_recurrent_step(q, k, v, g, q - snb + 4, o, B, H, dk, dv, 1, None, None) == -1
    assert lib.retention_recurrent_step(q, k, v, g, BW[4], q, B, H, dk, dv, 1, None, None) == -1


def test_backward_rejects_gradients_that_share_bytes(lib):
    """The gradients are written while the inputs are still being read: a
    gradient sharing bytes with an input or with another gradient is refused
    (before anything is launched)."""
    nk = 1 * 2 * 256 * 64 * 2  # bytes of q, k, grad_q, grad_k at the helper's shape (bf16)
    q, k, v, do, gq, gk, gv = BW
    assert _backward(lib, gq=q + nk - 2) == -1                                     # grad_q's first element in q
    assert _backward(lib, ptrs=[q, k, v, do, None, q - 2, gv]) == -1               # grad_k's last element in q
    assert _backward(lib, ptrs=[q, k, v, do, None, gk, do + 64]) == -1             # grad_v inside dO
    assert _backward(lib, gq=gk + nk // 2) == -1                                   # grad_q inside grad_k
    assert _backward(lib, ptrs=[q, k, v, do, None, gk, gq + 2], gq=gq) == -1       # grad_v inside grad_q


def _align(x):
    return (x + 255) // 256 * 256


def test_backward_workspace_bytes(lib):
    ws = lib.retention_chunkwise_backward_workspace_bytes
    B, H, N, dk, dv = 8, 16, 8192, 256, 512
    tok = B * H * N
    st = B * H * dk * dv * 4
    # bf16 on the single pass (any chunk that is a multiple of 64): four fp32
    # state buffers and the exchange words of 256 units.
    direct = 4 * _align(st) + _align(256 * 2048)
    for C in (64, 128, 256, 512):
        assert ws(B, H, N, dk, dv, C, 1) == direct, C
    # fp32 (two stages): at least the reversed Q, K, dO and V copies and the
    # forward-size chunk workspace.
    assert ws(B, H, N, dk, dv, 512, 0) >= (2 * tok * dk + 2 * tok * dv) * 4 + \
        lib.retention_chunkwise_workspace_bytes(B, H, N, dk, dv, 512, 0)
    # Too few heads for the single pass (16 (head, v tile) units): copies again.
    assert ws(1, 8, N, dk, dv, 512, 1) >= (2 * N * 8 * dk + 2 * N * 8 * dv) * 2
    # dk 128 (the dQ and dK retentions would have 128-wide values) and a chunk
    # that is no multiple of 64: copies.
    assert ws(B, H, N, 128, dv, 64, 1) >= (2 * tok * 128 + 2 * tok * dv) * 2
    assert ws(B, H, N, dk, dv, 96, 1) >= (2 * tok * dk + 2 * tok * dv) * 2
    # Reverse-order offsets must stay below 2^30 bytes: (N-1) * 512 * 2 + 1024
    # reaches it at N = 2^20, so that sequence takes the copies.
    big = 1 << 20
    st192 = 192 * dk * dv * 4
    assert ws(1, 192, big - 1, dk, dv, 64, 1) == 4 * _align(st192) + _align(2 * 192 * 2048)
    assert ws(1, 192, big, dk, dv, 64, 1) > 4 * _align(st192) + _align(2 * 192 * 2048)
    assert ws(0, H, N, dk, dv, 512, 1) == 0
    assert ws(B, H, N, dk, dv, 0, 1) == 0


def test_backward_rejects_subnormal_gamma_with_a_final_state_gradient(lib):
    """dL/dS_N enters divided by gamma: a subnormal gamma would overflow that quotient."""
    need = lib.retention_chunkwise_backward_workspace_bytes(1, 2, 256, 64, 128, 64, 1)
    g = _gamma([1e-39, 0.9])
    assert lib.retention_chunkwise_backward(*BW[:4], g, *BW[4:], 1, 2, 256, 64, 128, 64, 1,
                                            None, FAKE, None, FAKE, need, None) == _lib.RET_ERR_UNSUPPORTED


def test_huge_chunk_plans_like_one_chunk(lib):
    """A chunk at or above N is one chunk: the workspace equals that of the smallest such chunk."""
    ws = lib.retention_chunkwise_workspace_bytes
    one = ws(1, 2, 1000, 64, 128, 1024, 1)
    assert one > 0
    assert ws(1, 2, 1000, 64, 128, 2**31 - 1, 1) == one
    assert ws(1, 2, 1000, 64, 128, 2**31 - 64, 1) == one
    assert lib.retention_chunkwise_backward_workspace_bytes(1, 2, 1000, 64, 128, 2**31 - 1, 1) == \
        lib.retention_chunkwise_backward_workspace_bytes(1, 2, 1000, 64, 128, 1024, 1)


def _launches(lib):
    return lib.retention_shim_launches()


@shim_only
@pytest.mark.parametrize("shape", [
    (8, 16, 8192, 256, 512, 512, 1),   # the 6.7B-shaped prefill
    (1, 16, 65536, 256, 512, 64, 1),   # one long sequence, small chunks (segmented single pass)
    (1, 16, 65536, 256, 128, 64, 1),   # one long sequence, dv 128: segmented walk (two passes)
    (1, 16, 65536, 256, 512, 512, 1),  # segmented walk with the fix-up pass
    (2, 8, 2048, 256, 512, 256, 1),
    (1, 1, 64, 16, 16, 16, 0),         # fp32 generic path
    (1, 3, 77, 48, 96, 2**31 - 1, 1),  # generic bf16 shape, chunk near INT_MAX
    (2, 4, 1000, 128, 256, 2**31 - 64, 1),
])
def test_valid_chunkwise_calls_reach_the_launchers(lib, shape):
    B, H, N, dk, dv, chunk, dtype = shape
    need = lib.retention_chunkwise_workspace_bytes(B, H, N, dk, dv, chunk, dtype)
    g = _gamma([1 - 2.0 ** (-5 - h) for h in range(H)])
    before = _launches(lib)
    q, k, v, o = BW[:4]
    assert lib.retention_chunkwise(q, k, v, g, o, B, H, N, dk, dv, chunk, dtype, None, FAKE, None,
                                   FAKE if need else None, need, None) == 0
    gn = _lib.GnStruct(1e-5, None, None, None)
    assert lib.retention_chunkwise(q, k, v, g, o, B, H, N, dk, dv, chunk, dtype, FAKE, FAKE,
                                   ctypes.byref(gn), FAKE if need else None, need, None) == 0
    assert lib.retention_parallel(q, k, v, g, o, B, H, N, dk, dv, dtype, ctypes.byref(gn), None) == 0
    assert _launches(lib) > before


@shim_only
@pytest.mark.parametrize("shape", [
    (8, 16, 8192, 256, 512, 512, 1),
    (1, 2, 300, 64, 320, 64, 1),   # dv above the 256-column part width: two parts
    (1, 1, 64, 16, 16, 16, 0),
])
def test_valid_backward_and_decode_calls_reach_the_launchers(lib, shape):
    B, H, N, dk, dv, chunk, dtype = shape
    need = lib.retention_chunkwise_backward_workspace_bytes(B, H, N, dk, dv, chunk, dtype)
    g = _gamma([1 - 2.0 ** (-5 - h) for h in range(H)])
    before = _launches(lib)
    assert lib.retention_chunkwise_backward(*BW[:4], g, *BW[4:], B, H, N, dk, dv, chunk,
                                            dtype, FAKE, FAKE, FAKE, FAKE, need, None) == 0
    assert lib.retention_recurrent_step(*BW[:3], g, BW[4], BW[5], B, H, dk, dv, dtype, None, None) == 0
    assert _launches(lib) > before


def _theta(n, value=0.5):
    return (ctypes.c_float * n)(*([value] * n))


def test_xpos_rotate_rejects_invalid_arguments(lib):
    th = _theta(128)
    A, B_ = 0x100000, 0x900000  # two fake buffers far apart (the 2x2x8x256 bf16 tensors span 16 KiB)
    call = lambda q=A, k=B_, qo=A, ko=B_, th=th, B=2, H=2, N=8, d=256, pos0=0, dtype=1: \
        lib.retention_xpos_rotate(q, k, qo, ko, th, B, H, N, d, pos0, dtype, None)
    assert call(q=None) == -1
    assert call(qo=None) == -1
    assert call(th=None) == -1
    assert call(k=None) == -1                      # k_out without k
    assert call(ko=None) == -1                     # k without k_out
    assert call(d=255) == -1                       # odd width
    assert call(d=0) == -1 and call(N=0) == -1 and call(B=0) == -1
    assert call(dtype=2) == -1
    assert call(d=258, th=_theta(129)) == -2       # wider than RETENTION_MAX_DK
    assert call(pos0=-1) == -1
    assert call(pos0=2**53 - 7) == -1              # pos0 + N past 2^53
    assert call(q=A + 2, qo=A + 2) == -1           # bf16 pairs need 4-byte alignment
    assert call(q=A + 4, qo=A + 4, dtype=0) == -1  # fp32 pairs need 8
    bad = _theta(128)
    bad[7] = float("nan")
    assert call(th=bad) == -1
    bad[7] = float("inf")
    assert call(th=bad) == -1
    # Overlaps: an output inside another buffer, the outputs on each other, or
    # in place with q and k overlapping.
    assert call(qo=A + 64) == -1                   # q_out partly over q
    assert call(qo=B_ + 64, ko=0x2000000) == -1    # q_out over k
    assert call(qo=0x2000000, ko=0x2000000 + 64) == -1
    assert call(k=A + 1024, ko=0x3000000) == -1    # in-place q with k overlapping q


@shim_only
def test_valid_xpos_calls_reach_the_launcher(lib):
    th = _theta(128)
    before = _launches(lib)
    A, B_ = 0x100000, 0x900000
    # In place, out of place, q alone, the largest position, a narrow odd-pair width.
    assert lib.retention_xpos_rotate(A, B_, A, B_, th, 2, 2, 8, 256, 0, 1, None) == 0
    assert lib.retention_xpos_rotate(A, B_, 0x2000000, 0x3000000, th, 2, 2, 8, 256, 0, 0, None) == 0
    assert lib.retention_xpos_rotate(A, None, A, None, th, 8, 16, 8192, 256, 123456789, 1, None) == 0
    assert lib.retention_xpos_rotate(A, None, A, None, th, 1, 1, 1, 256, 2**53 - 1, 1, None) == 0
    assert lib.retention_xpos_rotate(A, B_, A, B_, _theta(3), 1, 3, 5, 6, 7, 1, None) == 0
    assert _launches(lib) == before + 5
