"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/retention.h declares,
and reject invalid or unsupported arguments before making any HIP call. Only
argument combinations that fail validation are passed here; the fake device
pointers below are never dereferenced.
"""

import ctypes
import os
import re
import subprocess

import pytest

from retnet_retention_msr_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "retention.h")

FAKE = 0x10000  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
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
    assert lib.retention_abi_version() == _lib.ABI_VERSION == 2
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
    # bf16 MFMA path, 6.7B-shaped prefill: one bf16 [dv][dk] state per chunk and head, no segments.
    assert ws(8, 16, 8192, 256, 512, 512, 1) == 8 * 16 * 16 * 256 * 512 * 2
    # fp32 path: one fp32 state per chunk and head.
    assert ws(1, 1, 64, 16, 16, 16, 0) == 4 * 16 * 16 * 4
    # Long sequence with 16 heads: the walk is cut into segments whose fp32 end states follow the chunk states.
    n = ws(1, 16, 65536, 256, 512, 512, 1)
    chunk_states = 16 * 128 * 256 * 512 * 2
    assert n > chunk_states and (n - chunk_states) % (16 * 256 * 512 * 4) == 0
    # Invalid sizes give 0.
    assert ws(0, 16, 8192, 256, 512, 512, 1) == 0
    assert ws(1, 16, 8192, 256, 512, 0, 1) == 0


def test_chunk_stage_entry_points_validate(lib):
    g = _gamma([0.9, 0.8])
    need = lib.retention_chunkwise_workspace_bytes(1, 2, 256, 64, 128, 64, 1)
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


def _backward(lib, gq=FAKE, ws=FAKE, ws_bytes=1 << 40, chunk=64, gamma=None, B=1, H=2, N=256, dk=64, dv=128,
              dtype=1):
    g = _gamma(gamma or [0.9] * H)
    return lib.retention_chunkwise_backward(FAKE, FAKE, FAKE, FAKE, g, gq, FAKE, FAKE, B, H, N, dk, dv, chunk, dtype,
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


def test_backward_workspace_bytes(lib):
    ws = lib.retention_chunkwise_backward_workspace_bytes
    # It holds at least the reversed Q, K, dO and V copies and the forward-size chunk workspace.
    B, H, N, dk, dv = 8, 16, 8192, 256, 512
    tok = B * H * N
    assert ws(B, H, N, dk, dv, 512, 1) >= (2 * tok * dk + 2 * tok * dv) * 2 + \
        lib.retention_chunkwise_workspace_bytes(B, H, N, dk, dv, 512, 1)
    assert ws(0, H, N, dk, dv, 512, 1) == 0
    assert ws(B, H, N, dk, dv, 0, 1) == 0
