"""Argument checks of the torch-level binding that run before any launch
(no GPU needed): wrong devices, dtypes and formats are refused in Python."""
import pytest

torch = pytest.importorskip("torch")
taco = pytest.importorskip("gradients_taco_compress_amd")


def test_stream_refuses_tensors_on_two_devices():
    a = torch.empty(4)
    b = torch.empty(4, device="meta")
    with pytest.raises(ValueError, match="different devices"):
        taco._stream(None, a, [(b, None)])


def test_host_tensors_are_refused():
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="CUDA/HIP"):
        taco.compress(x, block=128)
    with pytest.raises(TypeError, match="CUDA/HIP"):
        taco.decompress(torch.zeros(512, dtype=torch.uint8), torch.zeros(4), torch.zeros(4),
                        block=128)


def test_unknown_format_and_variant_are_refused():
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="unknown code format"):
        taco.compress(x, block=128, fmt="e3m4")
    with pytest.raises(ValueError, match="unknown variant"):
        taco.roundtrip(x, block=128, variant="none")
