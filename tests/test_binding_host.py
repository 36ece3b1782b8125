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


EMPTY_CASES = [(w, e) for w in ("scan", "bwd", "step", "conv", "conv_update") for e in ("batch", "dim", "seqlen")
               if not (w in ("step", "conv_update") and e == "seqlen")]  # decode calls have no length


@pytest.mark.parametrize("which,empty", EMPTY_CASES)
def test_empty_inputs_refused_by_name(which, empty):
    """An empty tensor is refused, naming the empty size, before any pointer is taken."""
    from selective_state_space_76_amd import conv1d_fwd, conv1d_update, scan_bwd, scan_fwd, state_update
    sz = dict(batch=2, dim=3, seqlen=5)
    sz[empty] = 0
    Bsz, Dm, Ln, N = sz["batch"], sz["dim"], sz["seqlen"], 4
    f = torch.float32
    u = torch.zeros(Bsz, Dm, Ln, dtype=f)
    A = torch.zeros(Dm, N, dtype=f)
    Bc = torch.zeros(Bsz, N, Ln, dtype=f)
    with pytest.raises(ValueError, match="empty input.*%s=0" % empty):
        if which == "scan":
            scan_fwd(u, u, A, Bc, Bc)
        elif which == "bwd":
            scan_bwd(u, u, A, Bc, Bc, dout=u)
        elif which == "step":
            state_update(torch.zeros(Bsz, Dm, N), u[:, :, 0], u[:, :, 0], A, Bc[:, :, 0], Bc[:, :, 0])
        elif which == "conv":
            conv1d_fwd(u, torch.zeros(Dm, 4))
        else:
            conv1d_update(torch.zeros(Bsz, Dm, 3), u[:, :, 0], torch.zeros(Dm, 4))
