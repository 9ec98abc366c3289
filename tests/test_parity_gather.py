"""GPU parity of mla_gather_latent_paged against the oracle, through the C ABI:
fp8 -> fp8 (with per-token scales), fp8 -> bf16 (per-tensor and per-token),
bf16 -> bf16 and bf16 -> fp8, on small ragged contexts and on long contexts
taken from the decode workload's pool."""
import numpy as np
import pytest
import torch

import gpu_helpers as gh
import oracle_pins
import workloads

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def finite_pool(case, seed):
    """Make the pool's values finite (fp8: no NaN codes; per-token scales
    finite and positive) so that every output has a numeric value."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if case.cache.dtype == np.uint8:
        nan = (case.cache & 0x7F) == 0x7F
        case.cache[nan] ^= 0x01
    else:
        case.cache[...] = workloads.bf16_bits(
            rng.standard_normal(case.cache.shape).astype(np.float32) * 3)
    if case.token_scales is not None:
        case.token_scales[...] = rng.uniform(1e-3, 2.0, case.token_scales.shape).astype(np.float32)


def check_dequant(case, kvo, got, want):
    """fp8 -> bf16: the kernel forms code x scale in fp32 (relative error at
    most 2^-24; the exact product has up to 28 significant bits) and rounds
    that to bf16, so it may differ from the oracle's once-rounded exact
    product by one bf16 step, and only where the exact product lies within
    2^-24 of its magnitude of a bf16 midpoint.  Everything else is
    bit-exact."""
    owners = oracle_pins.gather_owners(case, kvo)
    rows, W = got.shape
    exact = np.zeros((rows, W))
    L = case.layer_idx
    for (page, off), r in owners.items():
        s = (case.token_scales[L, page, off, 0] if case.scale_mode == "per_token"
             else case.tensor_scale)
        exact[r] = oracle_pins.fp8_to_f64(case.cache[L, page, off, 0]) * float(np.float32(s))
    # distance to the nearest bf16 midpoint: the midpoint above the bf16 value
    # nearest to the exact product, or the one below
    near = oracle_pins.bf16_to_f64(want)
    ulp = oracle_pins.ulp_bf16(exact)
    dist = np.minimum(np.abs(exact - (near + ulp / 2)), np.abs(exact - (near - ulp / 2)))
    tie_zone = dist <= 2.0 ** -24 * np.abs(exact)
    d = gh.bf16_ulp_diff(got, want)
    assert np.all(d[~tie_zone] == 0), "fp8 -> bf16 differs away from a bf16 midpoint"
    assert int(d.max(initial=0)) <= 1, "fp8 -> bf16 differs by more than one step"
    return {"max_ulp": int(d.max(initial=0)), "near_midpoint": int(tie_zone.sum()),
            "diff": int((d != 0).sum()), "n": d.size}


def run_gather(orc, case, kvo, out_fp8, out_scale=0.25, subset=None):
    import paged_kv_cache_wavefront_amd as pkv
    rows = int(kvo[-1])
    W = case.cache.shape[-1]
    _say(f"[gather] case={case.name} rows={rows} in={case.cache.dtype} out_fp8={out_fp8} "
         f"scale={case.scale_mode}")
    cache = gh.dev_bf16(case.cache) if case.cache.dtype == np.uint16 else gh.dev_u8(case.cache)
    pt = gh.dev_u32(case.page_table)
    kv = gh.dev_u32(kvo)
    if case.cache.dtype == np.uint16:
        mode, scales = pkv.PKV_SCALE_NONE, None
    elif case.scale_mode == "per_token":
        mode, scales = pkv.PKV_SCALE_PER_TOKEN, gh.dev_f32(case.token_scales)
    else:
        mode, scales = pkv.PKV_SCALE_PER_TENSOR, gh.dev_f32(np.array([case.tensor_scale], np.float32))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    desc = pkv.paged_cache(cache, None, pt, mode, scales, err)
    out = torch.full((rows, W), 0x55 if out_fp8 else 0x5555, device="cuda",
                     dtype=torch.uint8 if out_fp8 else torch.int16)
    if not out_fp8:
        out = out.view(torch.bfloat16)
    osc = torch.full((max(rows, 1),), -7.0, device="cuda")
    oscale = gh.dev_f32(np.array([out_scale], np.float32))
    pkv.mla_gather_latent_paged(out, kv, desc, case.layer_idx, osc, oscale)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = gh.host_u8(out) if out_fp8 else gh.host_bf16(out)
    got_sc = gh.host_f32(osc)
    want = np.zeros((rows, W), np.uint8 if out_fp8 else np.uint16)
    want_sc = np.full(max(rows, 1), -7.0, np.float32)
    sc_host = (case.token_scales if case.scale_mode == "per_token" else
               np.array([case.tensor_scale], np.float32))
    import contextlib
    with (orc.fp8_probe(want) if out_fp8 else contextlib.nullcontext()) as pre:
        orc.mla_gather_latent_paged(want, kvo, case.page_table, case.cache, case.layer_idx,
                                    case.scale_mode if case.cache.dtype == np.uint8 else "none",
                                    sc_host if case.cache.dtype == np.uint8 else None,
                                    want_sc, out_tensor_scale=out_scale)
    if out_fp8:
        if case.cache.dtype == np.uint8:
            assert np.array_equal(got, want), "fp8 copy must be exact"
        stats = gh.check_fp8(got, want, pre, "gather fp8")
        if case.scale_mode == "per_token" and case.cache.dtype == np.uint8:
            assert np.array_equal(got_sc[:rows].view(np.uint32), want_sc[:rows].view(np.uint32))
    else:
        if case.cache.dtype == np.uint16:
            assert np.array_equal(got, want), "bf16 copy must be exact"
            stats = gh.check_bf16(got, want, "gather bf16")
        else:
            stats = check_dequant(case, kvo, got, want)
    _say(f"[gather] {case.name}: {stats}")


@pytest.mark.parametrize("kind", ["fp8_tensor", "fp8_token", "bf16"])
@pytest.mark.parametrize("out_fp8", [True, False])
def test_small_contexts(orc, kind, out_fp8):
    case, kvo = oracle_pins.gather_case(kind)
    run_gather(orc, case, kvo, out_fp8)


@pytest.mark.parametrize("out_fp8", [True, False])
def test_long_contexts(orc, out_fp8):
    """16 requests of the decode workload's pool, each gathered over its whole
    prior context plus the new token (page size 128, per-tensor scale 0.05)."""
    case = workloads.mla_decode()
    finite_pool(case, 7001)
    n = 16
    ctx = case.cache_lengths[:n].astype(np.int64) + 1
    kvo = np.zeros(n + 1, np.uint32)
    kvo[1:] = np.cumsum(ctx)
    case.page_table = np.ascontiguousarray(case.page_table[:n])
    run_gather(orc, case, kvo, out_fp8)


def test_mixed_per_token(orc):
    case = workloads.mla_mixed()
    finite_pool(case, 7002)
    n = 6
    sel = np.r_[0:2, 64:68]      # two decode rows (long contexts) + the 4 prefill requests
    ctx = case.cache_lengths[sel].astype(np.int64) + np.diff(case.row_offsets.astype(np.int64))[sel]
    kvo = np.zeros(n + 1, np.uint32)
    kvo[1:] = np.cumsum(ctx)
    case.page_table = np.ascontiguousarray(case.page_table[sel])
    run_gather(orc, case, kvo, out_fp8=False)
    run_gather(orc, case, kvo, out_fp8=True)


@pytest.mark.parametrize("out_bf16", [False, True])
def test_bad_page_rows_skipped(orc, out_bf16):
    """A row whose page id lies past the pool is skipped (not written) and
    counted; the other rows are exact (fp8 copy) or the oracle's (fp8 -> bf16,
    the LDS-staged path, where a skipped row is neither staged nor stored)."""
    import paged_kv_cache_wavefront_amd as pkv
    case, kvo = oracle_pins.gather_case("fp8_tensor")
    good_table = case.page_table.copy()
    case.page_table[2, 0] = case.meta["num_pages"] + 1     # request 2: its first page
    cache = gh.dev_u8(case.cache)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    desc = pkv.paged_cache(cache, None, gh.dev_u32(case.page_table), pkv.PKV_SCALE_PER_TENSOR,
                           gh.dev_f32(np.array([case.tensor_scale], np.float32)), err)
    rows = int(kvo[-1])
    if out_bf16:
        out = torch.full((rows, 576), 0x5555, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    else:
        out = torch.full((rows, 576), 0x55, dtype=torch.uint8, device="cuda")
    pkv.mla_gather_latent_paged(out, gh.dev_u32(kvo), desc, case.layer_idx)
    torch.cuda.synchronize()
    got = gh.host_bf16(out) if out_bf16 else gh.host_u8(out)
    r2 = range(int(kvo[2]), int(kvo[3]))
    bad = [r for r in r2 if (r - int(kvo[2])) < case.meta["page_size"]]
    assert int(err.item()) == len(bad)
    assert np.all(got[bad] == (0x5555 if out_bf16 else 0x55))
    want = np.zeros_like(got)
    orc.mla_gather_latent_paged(want, kvo, good_table, case.cache, case.layer_idx, "per_tensor",
                                np.array([case.tensor_scale], np.float32))
    keep = np.ones(rows, bool)
    keep[bad] = False
    if out_bf16:
        assert int(gh.bf16_ulp_diff(got[keep], want[keep]).max()) <= 1
    else:
        assert np.array_equal(got[keep], want[keep])


@pytest.mark.parametrize("W", [80, 208, 1024])
@pytest.mark.parametrize("kind", ["fp8_tensor", "fp8_token", "bf16"])
@pytest.mark.parametrize("out_fp8", [True, False])
def test_row_widths(orc, W, kind, out_fp8):
    """Rows other than the MLA latent's 576: narrower (80, 208) and up to the
    widest supported (1024 elements, the second launch shape; for fp8 -> bf16
    the LDS staging area then takes 48 KiB per block)."""
    mode = {"fp8_tensor": "per_tensor", "fp8_token": "per_token", "bf16": "none"}[kind]
    seed = 7100 + W
    case = workloads.build_mla(f"gather_w{W}_{kind}", seed, [3, 0, 9, 1, 20], [13, 5, 0, 30, 2],
                               H=1, R=64, Dn=W - 64, page_size=8, max_seq_len=64,
                               spare_pages=3, scale_mode=mode, tensor_scale=0.05,
                               cache_dtype="bf16" if kind == "bf16" else "fp8")
    finite_pool(case, seed)
    ctx = case.cache_lengths.astype(np.int64) + np.diff(case.row_offsets.astype(np.int64))
    kvo = np.zeros(ctx.size + 1, np.uint32)
    kvo[1:] = np.cumsum(ctx)
    run_gather(orc, case, kvo, out_fp8)
