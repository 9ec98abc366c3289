"""The measurement helper pkv_stream_copy copies bytes exactly (it is the
benchmark's bandwidth reference, so it must move what it claims to)."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (1 << 20, 7), ((1 << 24) + 48, 4096)])
def test_stream_copy_exact(nbytes, blocks):
    import paged_kv_cache_wavefront_amd as pkv
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    pkv.pkv_stream_copy(dst, src, blocks)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert not bool(dst[nbytes:].any())
