"""The bandwidth probe's copy is exact and its read writes nothing.

cpattn_stream_probe is a measurement helper (the bandwidth ceiling that the
HBM-bound merge and sink kernels are compared with), not a step of the
attention path; these checks make sure the bytes it is timed on are really
moved."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_blockwise_attention_amd as cpattn
    cpattn.lib()
    return cpattn


@pytest.mark.parametrize("n_floats,grid", [(4, 0), (1000, 0), (1 << 20, 0), (1 << 20, 7), (3 << 20, 1024)])
def test_copy_is_exact(cp, n_floats, grid):
    g = torch.Generator(device="cpu").manual_seed(n_floats + grid)
    src = torch.randn(n_floats, generator=g).cuda()
    dst = torch.full((n_floats + 4,), 7.0, device="cuda")
    cp.stream_probe("copy", src, dst, grid=grid)
    torch.cuda.synchronize()
    assert torch.equal(dst[:n_floats], src)
    assert torch.all(dst[n_floats:] == 7.0)     # nothing past the end


@pytest.mark.parametrize("grid", [0, 1024])
def test_read_leaves_dst(cp, grid):
    src = torch.randn(1 << 20, generator=torch.Generator(device="cpu").manual_seed(1)).cuda()
    dst = torch.full((4,), 7.0, device="cuda")
    cp.stream_probe("read", src, dst, grid=grid)
    torch.cuda.synchronize()
    assert torch.all(dst == 7.0)
