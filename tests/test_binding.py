"""The Python binding's own argument checks (CPU only). What the C call cannot
see from plain pointers -- device memory, contiguity, dtype, size -- is
checked before any library call; shape errors are left to the library."""
import pytest
import torch

from quantized_decode_q4_amd import q4k


class FakeDeviceTensor:
    """Stands in for a device tensor on a machine without a GPU."""

    def __init__(self, numel, dtype=torch.float32, contiguous=True, ptr=0x7F0000000000):
        self._n, self.dtype, self._c, self._p = numel, dtype, contiguous, ptr
        self.is_cuda = True

    def numel(self):
        return self._n

    def element_size(self):
        return torch.empty(0, dtype=self.dtype).element_size()

    def is_contiguous(self):
        return self._c

    def data_ptr(self):
        return self._p


def test_arg_accepts_a_big_enough_device_tensor_and_raw_pointers():
    assert q4k._arg(FakeDeviceTensor(256), "x", 1024, torch.float32) == 0x7F0000000000
    assert q4k._arg(12345, "x", 1 << 40, torch.float32) == 12345     # raw pointer: unchecked
    assert q4k._arg(None, "delta", 1024, torch.float32, optional=True) is None


@pytest.mark.parametrize("t,why", [
    (FakeDeviceTensor(255), "holds 1020 bytes"),
    (FakeDeviceTensor(256, dtype=torch.float16), "must be torch.float32"),
    (FakeDeviceTensor(256, contiguous=False), "contiguous"),
    (torch.zeros(256), "device"),
    (None, "required"),
])
def test_arg_rejects(t, why):
    with pytest.raises(ValueError, match=why):
        q4k._arg(t, "x", 1024, torch.float32)


def test_calls_reject_host_tensors_before_the_library():
    W = torch.zeros(10 * 144, dtype=torch.uint8)
    x, y = torch.zeros(256), torch.zeros(10)
    with pytest.raises(ValueError, match="device"):
        q4k.q4k_matvec(W, x, y, 10, 256)
    with pytest.raises(ValueError, match="device"):
        q4k.q6k_matvec(torch.zeros(2100, dtype=torch.uint8), x, y, 10, 256)


def test_sizes_follow_the_shapes():
    assert q4k._wq4(10, 2560) == 10 * 10 * 144
    assert q4k._wq6(10, 2560) == 10 * 10 * 210
    assert q4k._colv(2560) == 10240 and q4k._colv(300) == 0 and q4k._colv(0) == 0
    assert q4k._f32(-3) == 0
