"""The measurement helper pkv_stream_copy copies bytes exactly (it is the
benchmark's bandwidth reference, so it must move what it claims to)."""
import numpy as np
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


def _mix_reference(src: np.ndarray, R: int, W: int, blocks: int) -> np.ndarray:
    """What pkv_stream_mix writes (16-byte pieces as rows of 4 uint32), from
    its stated schedule: waves take chunks of 256 pieces grid-stride, lane l
    of a wave takes pieces 64k + l of its chunk (k = 0..3); iteration i moves
    piece i of the longer stream, and piece m(i) = (i * ratio) >> 32 of the
    shorter one when m moves on (ratio = ceil(shorter * 2^32 / longer)); a
    written piece is the XOR of the pieces its thread read since its previous
    write."""
    out = np.zeros((W, 4), np.uint32)
    N = max(R, W)
    lo, hi = min(R, W), max(R, W)
    ratio = -(-(lo << 32) // hi) if hi else 0
    waves = 4 * blocks
    chunks = -(-N // 256)
    for w in range(waves):
        for lane in range(64):
            acc = np.zeros(4, np.uint32)
            for c in range(w, chunks, waves):
                for k in range(4):
                    i = c * 256 + 64 * k + lane
                    if R >= W:
                        if i < R:
                            acc = acc ^ src[i]
                            m = (i * ratio) >> 32
                            if ((i + 1) * ratio) >> 32 != m and m < W:
                                out[m] = acc
                                acc = np.zeros(4, np.uint32)
                    elif i < W:
                        m = (i * ratio) >> 32
                        if R and (i == 0 or ((i - 1) * ratio) >> 32 != m) and m < R:
                            acc = acc ^ src[m]
                        out[i] = acc
                        acc = np.zeros(4, np.uint32)
    return out


@pytest.mark.parametrize("R,W,blocks", [(1000, 1000, 1), (1000, 500, 1), (999, 333, 2),
                                        (500, 1000, 1), (7, 300, 1), (640, 0, 1), (0, 96, 1),
                                        (3001, 2999, 1), (2999, 3001, 3)])
def test_stream_mix_schedule(R, W, blocks):
    """pkv_stream_mix reads and writes the pieces its schedule names, and
    nothing past write_bytes."""
    import paged_kv_cache_wavefront_amd as pkv
    g = torch.Generator(device="cpu").manual_seed(R * 7 + W)
    src_h = torch.randint(-2**31, 2**31 - 1, (max(R, 1), 4), dtype=torch.int64,
                          generator=g).to(torch.int32)
    src = src_h.cuda()
    dst = torch.zeros((W + 8, 4), dtype=torch.int32, device="cuda")
    pkv.pkv_stream_mix(dst, src, 16 * R, 16 * W, blocks)
    torch.cuda.synchronize()
    want = _mix_reference(src_h.numpy().view(np.uint32), R, W, blocks)
    got = dst.cpu().numpy().view(np.uint32)
    assert np.array_equal(got[:W], want)
    assert not got[W:].any()


def test_stream_mix_in_place():
    """In place (dst is src), every piece is read and written back unchanged."""
    import paged_kv_cache_wavefront_amd as pkv
    g = torch.Generator(device="cpu").manual_seed(5)
    buf_h = torch.randint(0, 256, ((1 << 20) + 64,), dtype=torch.uint8, generator=g)
    buf = buf_h.cuda()
    pkv.pkv_stream_mix(buf, buf, 1 << 20, 1 << 20, 64)
    torch.cuda.synchronize()
    assert torch.equal(buf.cpu(), buf_h)
