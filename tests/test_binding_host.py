"""Argument checks of the torch binding (no GPU needed).

Every tensor the binding hands to the C ABI becomes a raw pointer, so a host
tensor, a wrong shape or dtype, a short workspace or an output overlapping an
input must be refused in Python, before the library is loaded or called.
These tests make the library unloadable and check that each bad argument
raises ValueError (or TypeError for an unsupported dtype) first.
"""

import pytest
import torch

import retnet_retention_msr_amd as ret
from retnet_retention_msr_amd import _lib


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def refuse():
        raise AssertionError("the C library was reached before the arguments were checked")

    monkeypatch.setattr(_lib, "load", refuse)


CPU = torch.device("cpu")
META = torch.device("meta")


def _qkv(B=1, H=2, N=8, dk=32, dv=64, dtype=torch.bfloat16):
    return (torch.zeros(B, H, N, dk, dtype=dtype), torch.zeros(B, H, N, dk, dtype=dtype),
            torch.zeros(B, H, N, dv, dtype=dtype))


def test_host_tensors_are_refused_by_every_entry_point():
    q, k, v = _qkv()
    g = [0.9, 0.8]
    with pytest.raises(ValueError, match="device tensor"):
        ret.parallel(q, k, v, g)
    with pytest.raises(ValueError, match="device tensor"):
        ret.chunkwise(q, k, v, g, 64)
    with pytest.raises(ValueError, match="device tensor"):
        ret.chunk_states(k, v, g, 64, torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="device tensor"):
        ret.chunk_output(q, k, v, g, 64, torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="device tensor"):
        ret.chunkwise_backward(q, k, v, v.clone(), g, 64)
    with pytest.raises(ValueError, match="device tensor"):
        ret.recurrent_step(q[:, :, 0], k[:, :, 0], v[:, :, 0], g, torch.zeros(1, 2, 32, 64))


def test_non_tensors_are_refused():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="must be a tensor"):
        ret.parallel(q.tolist(), k, v, [0.9, 0.8])


@pytest.mark.parametrize("bad, match", [
    (torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, device=META), "must be on cpu"),
    (torch.zeros(1, 2, 8, 64, dtype=torch.float32), "must be torch.bfloat16"),
    (torch.zeros(1, 2, 8, 65, dtype=torch.bfloat16), "must have shape"),
    (torch.zeros(1, 2, 64, 8, dtype=torch.bfloat16).transpose(2, 3), "must be contiguous"),
    ([0.0] * 4, "must be a tensor"),
])
def test_require_checks_device_dtype_shape_and_contiguity(bad, match):
    with pytest.raises(ValueError, match=match):
        ret._require(bad, "out", (1, 2, 8, 64), torch.bfloat16, CPU)


def test_require_accepts_a_matching_tensor():
    t = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    assert ret._require(t, "out", (1, 2, 8, 64), torch.bfloat16, CPU) is t


def test_state_must_be_fp32_bhdkdv():
    assert ret._state(None, "state_in", 1, 2, 32, 64, CPU) is None
    with pytest.raises(ValueError, match="torch.float32"):
        ret._state(torch.zeros(1, 2, 32, 64, dtype=torch.bfloat16), "state_in", 1, 2, 32, 64, CPU)
    with pytest.raises(ValueError, match="shape"):
        ret._state(torch.zeros(1, 2, 64, 32), "state_in", 1, 2, 32, 64, CPU)


def test_workspace_size_device_and_layout():
    ws = torch.zeros(100, dtype=torch.uint8)
    assert ret._require_workspace(ws, "workspace", 100, CPU) is ws
    # Counted in bytes, whatever the element type.
    assert ret._require_workspace(torch.zeros(25, dtype=torch.float32), "workspace", 100, CPU) is not None
    with pytest.raises(ValueError, match="holds 100 bytes, 101"):
        ret._require_workspace(ws, "workspace", 101, CPU)
    with pytest.raises(ValueError, match="must be on"):
        ret._require_workspace(torch.zeros(100, dtype=torch.uint8, device=META), "workspace", 1, CPU)
    with pytest.raises(ValueError, match="contiguous"):
        ret._require_workspace(torch.zeros(10, 20, dtype=torch.uint8).t(), "workspace", 1, CPU)


def test_outputs_must_not_overlap_inputs():
    base = torch.zeros(1024)
    a, b = base[:512], base[256:768]
    with pytest.raises(ValueError, match="overlap"):
        ret._no_overlap(a, "out", b)
    ret._no_overlap(base[:256], "out", base[256:512], None)  # adjacent is fine


def test_unsupported_dtype_is_a_type_error():
    with pytest.raises(TypeError, match="unsupported dtype"):
        ret._dtype_code(torch.zeros(4, dtype=torch.float16))
