"""The Python binding on a host without a GPU: no CPU fallback exists.  A missing library makes every
entry point raise, and host tensors are rejected before any library call."""

import pytest
import torch

import exact_tiled_attention_22_amd as fa
from exact_tiled_attention_22_amd import binding


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "libfa.so"))
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()
    with pytest.raises(RuntimeError, match="missing"):
        fa.decode_workspace_bytes(1, 1, 1, 64, 128)
    with pytest.raises(RuntimeError, match="missing"):
        fa.naive_row_stride(100)
    with pytest.raises(RuntimeError, match="missing"):
        fa.split_workspace_bytes(1, 1, 8, 64, 2)


@pytest.mark.parametrize("entry", ["fwd", "fwd_naive"])
def test_host_tensors_rejected(entry):
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        getattr(fa, entry)(q, q, q)


def test_host_tensors_rejected_decode_and_bwd():
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fwd_decode(q, q, q)
    with pytest.raises(ValueError, match="GPU"):
        fa.fwd_rect(q, q, q)
    with pytest.raises(ValueError, match="GPU"):
        fa.fwd_split(q, q, q, nsplit=2)
    lse = torch.zeros(1, 1, 8)
    with pytest.raises(ValueError):
        fa.bwd(q, q, q, q, lse, q)
