"""The Python binding's own checks, without a GPU: a tensor whose shape, dtype or device
differs from what the C ABI will assume is refused before any pointer is passed on."""
import pytest
import torch

from selective_state_space_76_amd import _lib as L


def test_expect_shape_dtype_device():
    t = torch.zeros(2, 3, dtype=torch.float32)
    L._expect(t, (2, 3), torch.float32, "t", t.device)
    L._expect(None, (9,), torch.float32, "absent")
    with pytest.raises(ValueError, match="shape"):
        L._expect(t, (3, 2), torch.float32, "t")
    with pytest.raises(TypeError, match="expected torch.bfloat16"):
        L._expect(t, (2, 3), torch.bfloat16, "t")
    with pytest.raises(ValueError, match="expected a tensor on meta"):
        L._expect(t, (2, 3), torch.float32, "t", torch.device("meta"))


def test_stream_dtypes_and_flags():
    assert L._io_dtype(torch.zeros(1, dtype=torch.float32)) == L.SSM_F32
    assert L._io_dtype(torch.zeros(1, dtype=torch.bfloat16)) == L.SSM_BF16
    with pytest.raises(TypeError):
        L._io_dtype(torch.zeros(1, dtype=torch.float16))
    sh = L.make_shape(2, 3, 4, 5, L.SSM_BF16, zoh=True, reverse=True)
    assert (sh.batch, sh.dim, sh.dstate, sh.seqlen, sh.io_dtype, sh.flags) == (2, 3, 4, 5, 1, 3)


def test_ptr_refuses_host_and_strided_tensors():
    with pytest.raises(ValueError, match="GPU"):
        L._ptr(torch.zeros(4))
    assert L._ptr(None) is None
