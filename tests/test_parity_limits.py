"""GPU parity at the edges of the input space, through the C ABI: batches of
more than 256 requests (the request lookup's loop path), caches whose layer
and page offsets lie beyond 4 GiB (64-bit addressing), and positions on the
last row of the freqs table."""
import numpy as np
import pytest
import torch

import gpu_helpers as gh
import oracle_pins
import workloads

pytestmark = pytest.mark.gpu

FOUR_GIB = 1 << 32


def _say(*a):
    print(*a, flush=True)


# -- more than 256 requests ----------------------------------------------------------------

@pytest.mark.parametrize("B,H,mode", [(300, 16, "per_token"), (700, 128, "per_tensor")])
def test_mla_many_requests(orc, B, H, mode):
    rng = workloads.make_rng(8000 + B)
    new = rng.integers(0, 3, size=B, endpoint=True)
    prior = rng.integers(0, 300, size=B, endpoint=True)
    case = workloads.build_mla(f"mla_b{B}", 8000 + B, new, prior, H=H, page_size=16,
                               max_seq_len=512, spare_pages=8, scale_mode=mode,
                               tensor_scale=0.05, rng=rng)
    _say(f"[limits] mla B={B} T={case.T} H={H} {mode}")
    dev = gh.MlaDevice(case)
    dev.run()
    gpu = dev.results()
    assert gpu[3] == 0
    _say(f"[limits] {gh.compare_mla(case, gpu, gh.oracle_mla(orc, case))}")


def _qk_many(B):
    rng = workloads.make_rng(8100 + B)
    new = rng.integers(0, 4, size=B, endpoint=True)
    prior = rng.integers(0, 200, size=B, endpoint=True)
    return workloads.build_qk(f"qk_b{B}", 8100 + B, new, prior, Hq=8, Hkv=2, D=128,
                              page_size=16, max_seq_len=4096, theta=10000.0,
                              interleaved=False, with_position_ids=False, norm_cols=128,
                              rng=rng)


def test_qk_many_requests(orc):
    case = _qk_many(300)
    _say(f"[limits] qk B=300 T={case.T}")
    dev = gh.QkDevice(case)
    dev.rope(True)
    q = gh.host_bf16(dev.q_out)
    k, _ = dev.k_host()
    assert int(dev.error_count.item()) == 0
    q_o = np.zeros_like(case.q)
    k_o = case.k_cache.copy()
    orc.qk_rope_paged_ragged(q_o, case.q, case.row_offsets, case.cache_lengths, case.page_table,
                             k_o, case.layer_idx, case.freqs, case.position_ids,
                             case.interleaved, case.gamma, case.epsilon)
    from test_parity_qk import check_k_rows
    gh.check_bf16(q, q_o, "q")
    _say(f"[limits] {check_k_rows(case, k, k_o, 'k', case.gamma.size)}")


def test_kv_norm_many_requests(orc):
    case = _qk_many(300)
    dev = gh.QkDevice(case)
    dev.kv_norm(dev.gamma, 0.0, case.T, True)
    k, _ = dev.k_host()
    assert int(dev.error_count.item()) == 0
    k_o = case.k_cache.copy()
    orc.rms_norm_kv_cache_paged(k_o, case.layer_idx, case.row_offsets, case.cache_lengths,
                                case.page_table, case.gamma, case.epsilon, 0.0, case.T, True)
    rows = gh.written_k_rows(case)
    assert np.array_equal(k[~rows], case.k_cache[~rows])
    gh.check_bf16(k[rows], k_o[rows], "kv norm B=300")


def test_gather_many_requests(orc):
    import paged_kv_cache_wavefront_amd as pkv
    B = 300
    rng = workloads.make_rng(8200)
    new = rng.integers(0, 2, size=B, endpoint=True)
    prior = rng.integers(0, 40, size=B, endpoint=True)
    case = workloads.build_mla("gather_b300", 8200, new, prior, H=1, page_size=8,
                               max_seq_len=64, spare_pages=4, scale_mode="per_tensor",
                               tensor_scale=0.05, rng=rng)
    case.cache[(case.cache & 0x7F) == 0x7F] ^= 0x01        # finite codes only
    ctx = case.cache_lengths.astype(np.int64) + np.diff(case.row_offsets.astype(np.int64))
    kvo = np.zeros(B + 1, np.uint32)
    kvo[1:] = np.cumsum(ctx)
    rows = int(kvo[-1])
    _say(f"[limits] gather B={B} rows={rows}")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    desc = pkv.paged_cache(gh.dev_u8(case.cache), None, gh.dev_u32(case.page_table),
                           pkv.PKV_SCALE_PER_TENSOR,
                           gh.dev_f32(np.array([case.tensor_scale], np.float32)), err)
    out = torch.zeros((rows, 576), dtype=torch.bfloat16, device="cuda")
    pkv.mla_gather_latent_paged(out, gh.dev_u32(kvo), desc, case.layer_idx)
    got = gh.host_bf16(out)
    assert int(err.item()) == 0
    want = np.zeros((rows, 576), np.uint16)
    orc.mla_gather_latent_paged(want, kvo, case.page_table, case.cache, case.layer_idx,
                                "per_tensor", np.array([case.tensor_scale], np.float32), None)
    gh.check_bf16(got, want, "gather B=300")


# -- caches beyond 4 GiB -------------------------------------------------------------------

def _big_pool_pages(page_bytes: int, P: int) -> int:
    """Pages per layer such that layer 1 starts past 4 GiB and the case's P
    pages, placed at the top of the layer, lie past 4 GiB inside it too."""
    return FOUR_GIB // page_bytes + P + 1


def test_mla_cache_beyond_4gib(orc):
    """The small per-token case's pool placed at the top of a 2-layer pool of
    more than 8 GiB: layer offset and page offsets both exceed 32 bits."""
    import paged_kv_cache_wavefront_amd as pkv
    case = list(oracle_pins.small_mla_cases())[3]
    assert case.scale_mode == "per_token"
    L, P, S = case.cache.shape[:3]
    W = case.cache.shape[-1]
    big_p = _big_pool_pages(S * W, P)
    shift = big_p - P
    _say(f"[limits] mla pool {L} x {big_p} pages x {S} x {W} B = {L * big_p * S * W / 2**30:.1f} GiB")
    dev = gh.MlaDevice(case)
    big = torch.zeros((L, big_p, S, 1, W), dtype=torch.uint8, device="cuda")
    big[:, shift:] = gh.dev_u8(case.cache)
    scales = torch.zeros((L, big_p, S, 1), dtype=torch.float32, device="cuda")
    scales[:, shift:] = gh.dev_f32(case.token_scales)
    pt = case.page_table.copy()
    pt[pt != workloads.UNUSED_PAGE] += np.uint32(shift)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    desc = pkv.paged_cache(big, dev.cache_lengths, gh.dev_u32(pt), pkv.PKV_SCALE_PER_TOKEN,
                           scales, err)
    pkv.mla_rope_rmsnorm_quant(dev.q_out, dev.q_in, dev.latent, dev.offsets, dev.freqs, dev.gamma,
                               case.epsilon, desc, case.layer_idx)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert not bool(big[:, :shift].any()), "bytes below the placed pool changed"
    assert not bool(scales[:, :shift].any()), "scales below the placed pool changed"
    got = (gh.host_bf16(dev.q_out), big[:, shift:].cpu().numpy(),
           scales[:, shift:].cpu().numpy(), 0)
    del big, scales
    torch.cuda.empty_cache()
    _say(f"[limits] {gh.compare_mla(case, got, gh.oracle_mla(orc, case))}")


def test_qk_and_kv_norm_cache_beyond_4gib(orc):
    """Q/K RoPE with the fused K norm, and (on a fresh copy) the K-cache norm,
    on a bf16 K pool of more than 8 GiB (the small interleaved case's pages at
    the top)."""
    import paged_kv_cache_wavefront_amd as pkv
    from test_parity_qk import check_k_rows
    case = list(oracle_pins.small_qk_cases())[0]
    L, P, S, Hkv, D = case.k_cache.shape
    big_p = _big_pool_pages(S * Hkv * D * 2, P)
    shift = big_p - P
    _say(f"[limits] K pool {L} x {big_p} pages = {L * big_p * S * Hkv * D * 2 / 2**30:.1f} GiB")
    dev = gh.QkDevice(case)
    big = torch.zeros((L, big_p, S, Hkv, D), dtype=torch.bfloat16, device="cuda")
    pool = gh.dev_bf16(case.k_cache)
    pt = case.page_table.copy()
    pt[pt != workloads.UNUSED_PAGE] += np.uint32(shift)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    desc = pkv.paged_cache(big, dev.cache_lengths, gh.dev_u32(pt), pkv.PKV_SCALE_NONE, None, err)
    results = {}
    for step in ("rope", "norm"):
        big[:, shift:] = pool
        if step == "rope":
            pkv.qk_rope_paged_ragged(dev.q_out, dev.q_in, dev.offsets, desc, case.layer_idx,
                                     dev.freqs, dev.pos, case.interleaved, dev.gamma,
                                     case.epsilon)
        else:
            pkv.rms_norm_kv_cache_paged(desc, case.layer_idx, dev.gamma, case.epsilon, 0.0,
                                        case.T, dev.offsets, True, True)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert not bool(big[:, :shift].view(torch.int16).any()), "K below the pool changed"
        results[step] = gh.host_bf16(big[:, shift:])
    q = gh.host_bf16(dev.q_out)
    del big
    torch.cuda.empty_cache()
    q_o = np.zeros_like(case.q)
    k_rope = case.k_cache.copy()
    orc.qk_rope_paged_ragged(q_o, case.q, case.row_offsets, case.cache_lengths, case.page_table,
                             k_rope, case.layer_idx, case.freqs, case.position_ids,
                             case.interleaved, case.gamma, case.epsilon)
    k_norm = case.k_cache.copy()
    orc.rms_norm_kv_cache_paged(k_norm, case.layer_idx, case.row_offsets, case.cache_lengths,
                                case.page_table, case.gamma, case.epsilon, 0.0, case.T, True)
    gh.check_bf16(q, q_o, "q")
    _say(f"[limits] rope K {check_k_rows(case, results['rope'], k_rope, 'k', case.gamma.size)}")
    rows = gh.written_k_rows(case)
    assert np.array_equal(results["norm"][~rows], case.k_cache[~rows])
    _say(f"[limits] norm K {gh.check_bf16(results['norm'][rows], k_norm[rows], 'k norm')}")


def test_gather_cache_beyond_4gib(orc):
    import paged_kv_cache_wavefront_amd as pkv
    case, kvo = oracle_pins.gather_case("fp8_token")
    L, P, S = case.cache.shape[:3]
    W = case.cache.shape[-1]
    big_p = _big_pool_pages(S * W, P)
    shift = big_p - P
    big = torch.zeros((L, big_p, S, 1, W), dtype=torch.uint8, device="cuda")
    big[:, shift:] = gh.dev_u8(case.cache)
    scales = torch.zeros((L, big_p, S, 1), dtype=torch.float32, device="cuda")
    scales[:, shift:] = gh.dev_f32(case.token_scales)
    pt = case.page_table.copy()
    pt[pt != workloads.UNUSED_PAGE] += np.uint32(shift)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    desc = pkv.paged_cache(big, None, gh.dev_u32(pt), pkv.PKV_SCALE_PER_TOKEN, scales, err)
    rows = int(kvo[-1])
    out = torch.zeros((rows, W), dtype=torch.bfloat16, device="cuda")
    pkv.mla_gather_latent_paged(out, gh.dev_u32(kvo), desc, case.layer_idx)
    got = gh.host_bf16(out)
    assert int(err.item()) == 0
    del big, scales
    torch.cuda.empty_cache()
    want = np.zeros((rows, W), np.uint16)
    orc.mla_gather_latent_paged(want, kvo, case.page_table, case.cache, case.layer_idx,
                                "per_token", case.token_scales, None)
    gh.check_bf16(got, want, "gather beyond 4 GiB")


# -- the last freqs row ------------------------------------------------------------------------

def test_mla_last_position(orc):
    """Every new token of a request sits on the last rows of the freqs table
    (positions max_seq_len - 4 .. max_seq_len - 1)."""
    case = workloads.build_mla("mla_last_pos", 8300, [4, 1], [60, 63], H=8, page_size=16,
                               max_seq_len=64, spare_pages=2, scale_mode="per_tensor",
                               tensor_scale=0.05)
    dev = gh.MlaDevice(case)
    dev.run()
    gpu = dev.results()
    assert gpu[3] == 0
    gh.compare_mla(case, gpu, gh.oracle_mla(orc, case))
