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


def test_library_of_another_abi_version_is_refused(monkeypatch, tmp_path):
    import subprocess

    src = tmp_path / "fake.c"
    src.write_text("int fa_abi_version(void) { return 99; }\n")
    so = tmp_path / "libfa.so"
    subprocess.run(["gcc", "-shared", "-fPIC", str(src), "-o", str(so)], check=True)
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(so))
    with pytest.raises(RuntimeError, match="ABI version 99"):
        binding.lib()


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


class _NoLaunch:
    """Stands in for libfa.so: any attribute access means an entry point would have been called."""

    def __getattr__(self, name):
        raise AssertionError(f"{name} was reached although the arguments are invalid")


@pytest.fixture
def no_launch(monkeypatch):
    # host tensors stand in for device tensors: only the checks that follow the device check run
    monkeypatch.setattr(binding, "_lib", _NoLaunch())
    monkeypatch.setattr(binding, "_check_qkv", lambda q, k, v: None)


def _fp8_qkv(B=1, H=2, N=130, d=64):
    x = torch.zeros(B, H, N, d, dtype=torch.float8_e4m3fn)
    return x, x.clone(), x.clone()


def test_fp8_scales_shape_checked(no_launch):
    q, k, v = _fp8_qkv()
    good = torch.ones(1, 2, 3)  # ceil(130 / 64) = 3 blocks
    # scales written for another block size (block 128 -> 2 blocks) would be read past their end
    short = torch.ones(1, 2, 2)
    with pytest.raises(ValueError, match="shape"):
        fa.fwd(q, k, v, fp8_scales=(good, good, short))
    # scales of 64-row blocks announced as 128-row blocks
    with pytest.raises(ValueError, match="shape"):
        fa.fwd(q, k, v, fp8_scales=(good, good, good), block=128)


def test_fp8_scales_dtype_device_contiguity_checked(no_launch):
    q, k, v = _fp8_qkv()
    good = torch.ones(1, 2, 3)
    with pytest.raises(ValueError, match="float32"):
        fa.fwd(q, k, v, fp8_scales=(good, good.half(), good))
    with pytest.raises(ValueError, match="float32"):
        fa.fwd(q, k, v, fp8_scales=(good, good, torch.ones(1, 2, 3, device="meta")))
    strided = torch.ones(1, 2, 6)[..., ::2]
    with pytest.raises(ValueError, match="contiguous"):
        fa.fwd(q, k, v, fp8_scales=(strided, good, good))
    with pytest.raises(ValueError, match="triple"):
        fa.fwd(q, k, v, fp8_scales=(good, good))
    with pytest.raises(ValueError, match="positive"):
        fa.fwd(q, k, v, fp8_scales=(good, good, good), block=0)


def test_fp8_scales_rejected_for_16bit(no_launch):
    q = torch.zeros(1, 2, 130, 64, dtype=torch.bfloat16)
    good = torch.ones(1, 2, 3)
    with pytest.raises(ValueError, match="float8_e4m3fn"):
        fa.fwd(q, q, q, fp8_scales=(good, good, good))


def test_bwd_lse_device_checked(no_launch):
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 8, device="meta")
    with pytest.raises(ValueError, match="lse"):
        fa.bwd(q, q, q, q, lse, q)


def test_fp8_prep_signs_checked():
    x = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="d = 64"):
        binding._sign_buffer([1] * 32, 64)
    with pytest.raises(ValueError, match="\\+1 or -1"):
        binding._sign_buffer([1] * 63 + [2], 64)
    buf = binding._sign_buffer([1, -1] * 32, 64)
    assert len(buf) == 64 and buf[1] == -1
    with pytest.raises(ValueError):
        fa.fp8_prep(x, [1] * 32)  # a host tensor, and too few signs: rejected before any call
