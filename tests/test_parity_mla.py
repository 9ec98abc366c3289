"""GPU parity of mla_rope_rmsnorm_quant (and of its in-place form,
mla_rope_rmsnorm_inplace) against the CPU oracle, through the C ABI (binding
-> libpkv.so), on the four MLA workloads at full size, small ragged cases, q
layouts, degenerate inputs, the E4M3FN codec over every bf16 value, and
determinism."""
import numpy as np
import pytest
import torch

import gpu_helpers as gh
import oracle_pins
import workloads

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _run_and_compare(orc, case, q_layout="dense", q_f32=False):
    _say(f"[mla] case={case.name} seed={case.seed} T={case.T} B={case.B} H={case.H} "
         f"scale={case.scale_mode} layout={q_layout} q_f32={q_f32}")
    dev = gh.MlaDevice(case, q_layout, q_f32)
    dev.run()
    gpu = dev.results()
    assert gpu[3] == 0, f"{gpu[3]} tokens skipped"
    stats = gh.compare_mla(case, gpu, gh.oracle_mla(orc, case, q_f32))
    _say(f"[mla] {case.name}: {stats}")
    return stats


@pytest.mark.parametrize("name", ["mla_tiny", "mla_decode", "mla_prefill", "mla_mixed"])
def test_named_workload(orc, name):
    _run_and_compare(orc, workloads.NAMED[name]())


@pytest.mark.parametrize("name", ["mla_tiny", "mla_decode", "mla_mixed"])
def test_fp32_q_output(orc, name):
    """q_rope_output in float32 (the pages' out_rope_dtype): every value within
    2 fp32 ulps of the oracle's once-rounded result; cache rows as for bf16."""
    _run_and_compare(orc, workloads.NAMED[name](), q_f32=True)


def test_fp32_q_output_h40(orc):
    case = workloads.build_mla("mla_h40_f32", 4005, [5, 0, 77, 1, 300], [0, 3, 9, 200, 1],
                               H=40, page_size=16, max_seq_len=1024, spare_pages=3,
                               scale_mode="per_token")
    _run_and_compare(orc, case, q_f32=True)


def test_fp32_q_output_strided(orc):
    """fp32 q_rope_output written into a view of a wider buffer (token stride
    H*R + 4 floats, head stride 2*R: the rope slice of a [T, H, 2R] tensor)
    from a strided bf16 q; every float outside the view keeps its sentinel."""
    import paged_kv_cache_wavefront_amd as pkv
    case = workloads.build_mla("mla_f32_strided", 4006, [3, 9, 0, 14], [5, 0, 2, 30], H=20,
                               page_size=8, max_seq_len=64, spare_pages=3,
                               scale_mode="per_tensor", tensor_scale=0.05)
    T, H, R = case.q.shape
    dev = gh.MlaDevice(case, "strided")
    big = torch.full((T, 2 * H * R + 4), -3.0, dtype=torch.float32, device="cuda")
    view = big[:, : 2 * H * R].view(T, H, 2 * R)[:, :, R:]
    pkv.mla_rope_rmsnorm_quant(view, dev.q_in, dev.latent, dev.offsets, dev.freqs, dev.gamma,
                               case.epsilon, dev.desc, case.layer_idx)
    torch.cuda.synchronize()
    host = big.cpu().numpy()
    got = host[:, : 2 * H * R].reshape(T, H, 2 * R)[:, :, R:]
    rest = np.concatenate([host[:, : 2 * H * R].reshape(T, H, 2 * R)[:, :, :R].ravel(),
                           host[:, 2 * H * R:].ravel()])
    assert np.all(rest == -3.0), "floats outside the output view changed"
    q_o, cache_o, _, pre = gh.oracle_mla(orc, case, q_f32=True)
    d = gh.f32_ulp_diff(np.ascontiguousarray(got), q_o)
    assert int(d.max(initial=0)) <= gh.F32_MAX_ULP
    _, cache_g, _, skipped = dev.results()
    assert skipped == 0
    rows = gh.written_rows(case)
    assert np.array_equal(cache_g[~rows], case.cache[~rows])
    gh.check_fp8(cache_g[rows], cache_o[rows], pre[rows], "cache rows", max_frac=1e-3)


@pytest.mark.parametrize("idx", range(5))
def test_small_cases(orc, idx):
    case = list(oracle_pins.small_mla_cases())[idx]
    _run_and_compare(orc, case)


@pytest.mark.parametrize("layout", ["strided", "inplace"])
def test_q_layouts(orc, layout):
    case = workloads.build_mla("mla_layout", 4001, [7, 0, 13, 1, 20], [3, 9, 0, 30, 2], H=24,
                               page_size=8, max_seq_len=64, spare_pages=5,
                               scale_mode="per_tensor", tensor_scale=0.05)
    _run_and_compare(orc, case, layout)


def test_heads_not_multiple_of_16(orc):
    # 4100 tokens x 40 heads: wide-chunk kernel with masked head lanes
    rng = workloads.make_rng(4002)
    new = rng.integers(1, 300, size=30, endpoint=True)
    new = np.append(new, 4100 - new.sum()) if new.sum() < 4100 else new
    case = workloads.build_mla("mla_h40", 4002, new, rng.integers(0, 100, size=new.size), H=40,
                               page_size=32, max_seq_len=8192, spare_pages=4,
                               scale_mode="per_token", rng=rng)
    _run_and_compare(orc, case)


# (rope_dim, kv_norm_dim): 4, 8 and 16 lanes per head (quad, half-row and
# row mirrors), non-rope parts of 16 to 512 values (lanes past kv_norm_dim / 8
# idle in the statistic, the max and the store)
OTHER_DIMS = [(32, 256), (32, 512), (64, 256), (128, 512), (128, 128), (64, 16)]


@pytest.mark.parametrize("R,Dn", OTHER_DIMS)
@pytest.mark.parametrize("mode", ["per_tensor", "per_token", "bf16"])
def test_other_dims(orc, R, Dn, mode):
    """MLA rows of Dn + R values other than 512 + 64, every cache encoding,
    a ragged batch with prior lengths and page crossings, 40 heads (a masked
    head chunk at every rope_dim)."""
    rng = workloads.make_rng(4200 + R + Dn)
    new = rng.integers(0, 150, size=9, endpoint=True)
    prior = rng.integers(0, 300, size=9, endpoint=True)
    case = workloads.build_mla(f"mla_r{R}_d{Dn}_{mode}", 4200 + R + Dn, new, prior, H=40, R=R,
                               Dn=Dn, page_size=16, max_seq_len=512, spare_pages=5,
                               scale_mode="per_token" if mode == "per_token" else "per_tensor",
                               tensor_scale=0.05, cache_dtype="bf16" if mode == "bf16" else "fp8",
                               outlier_p=0.01, rng=rng)
    _run_and_compare(orc, case)


@pytest.mark.parametrize("R,Dn,H", [(32, 256, 128), (128, 512, 16)])
def test_other_dims_prefill_shape(orc, R, Dn, H):
    """A prefill-shaped batch (8 requests of U{512..4096} tokens, about 17k
    tokens) at other widths: a grid of many thousand waves at rope_dim 32
    (two head chunks per token) and 128."""
    rng = workloads.make_rng(4300 + R)
    new = rng.integers(512, 4096, size=8, endpoint=True)
    case = workloads.build_mla(f"mla_prefill_r{R}_d{Dn}", 4300 + R, new, np.zeros(8, np.int64),
                               H=H, R=R, Dn=Dn, page_size=128, max_seq_len=4096, spare_pages=8,
                               latent_sigma=2.0, scale_mode="per_tensor", tensor_scale=0.05,
                               rng=rng)
    _run_and_compare(orc, case)


@pytest.mark.parametrize("R,Dn", [(32, 256), (128, 512)])
def test_other_dims_inplace_and_planned(orc, R, Dn):
    """The in-place form on a bf16 cache and the planned form at other widths."""
    import paged_kv_cache_wavefront_amd as pkv
    rng = workloads.make_rng(4400 + R)
    new = rng.integers(1, 90, size=7, endpoint=True)
    prior = rng.integers(0, 200, size=7, endpoint=True)
    case = workloads.build_mla(f"mla_inplace_r{R}", 4400 + R, new, prior, H=24, R=R, Dn=Dn,
                               page_size=16, max_seq_len=512, spare_pages=4, cache_dtype="bf16",
                               rng=rng)
    dev = gh.MlaDevice(case)
    dev.place_rows()
    dev.run_inplace()
    gh.compare_mla(case, dev.results(), gh.oracle_mla_inplace(orc, case))
    fcase = workloads.build_mla(f"mla_planned_r{R}", 4400 + R, new, prior, H=24, R=R, Dn=Dn,
                                page_size=16, max_seq_len=512, spare_pages=4,
                                scale_mode="per_token", rng=workloads.make_rng(4500 + R))
    fdev = gh.MlaDevice(fcase)
    plan = torch.empty((fcase.T, 4), dtype=torch.int32, device="cuda")
    pkv.pkv_token_plan(plan, fdev.offsets, fdev.desc)
    pkv.mla_rope_rmsnorm_quant_planned(fdev.q_out, fdev.q_in, fdev.latent, plan, fdev.freqs,
                                       fdev.gamma, fcase.epsilon, fdev.desc, fcase.layer_idx)
    _say(f"[dims] planned r{R}: "
         f"{gh.compare_mla(fcase, fdev.results(), gh.oracle_mla(orc, fcase))}")


def test_three_head_chunks_per_token(orc):
    """Three head chunks per token (80 heads of 64: 32 + 32 + a masked 16),
    over more than 4096 work items: every (token, chunk) item is written once
    and only chunk 0 stores the latent row."""
    rng = workloads.make_rng(4600)
    new = rng.integers(200, 700, size=6, endpoint=True)
    prior = rng.integers(0, 100, size=6, endpoint=True)
    case = workloads.build_mla("mla_h80", 4600, new, prior, H=80, page_size=64,
                               max_seq_len=1024, spare_pages=4, scale_mode="per_token", rng=rng)
    assert case.T * 3 > 4096
    _run_and_compare(orc, case)


def test_empty_batch(orc):
    import paged_kv_cache_wavefront_amd as pkv
    case = workloads.build_mla("mla_empty", 4003, [0, 0], [5, 0], H=4, page_size=16,
                               max_seq_len=64, spare_pages=2)
    assert case.T == 0
    dev = gh.MlaDevice(case)
    dev.run()
    q, cache, _, skipped = dev.results()
    assert skipped == 0 and q.size == 0
    assert np.array_equal(cache, case.cache)
    _ = pkv


def test_codec_every_bf16_value(orc):
    """Every bf16 pattern goes through the rope tail at position 0 (cos 1,
    sin 0: a finite value is passed through exactly) and is quantised with
    scale 1 and with scale 1/8: the fp8 codes must equal the oracle's (+-0
    equal) -- this pins the hardware conversion (rounding, ties, subnormals,
    saturation).  Infinities saturate to +-448; a NaN, and every value whose
    rotation partner is infinite or NaN (0 x inf), becomes the NaN code, as
    in the oracle (the NaN code's sign is not compared)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rows = -(-bits.size // 64)
    tail = np.zeros(rows * 64, np.uint16)
    tail[: bits.size] = bits
    for scale in (1.0, 0.125):
        case = workloads.build_mla("mla_codec", 4004, [1] * rows, [0] * rows, H=1,
                                   page_size=4, max_seq_len=1, spare_pages=3,
                                   scale_mode="per_tensor", tensor_scale=scale)
        case.latent[:, case.Dn:] = tail.reshape(rows, 64)
        dev = gh.MlaDevice(case)
        dev.run()
        q, cache, _, skipped = dev.results()
        assert skipped == 0
        _, cache_o, _, _ = gh.oracle_mla(orc, case)
        rows_mask = gh.written_rows(case)
        got = cache[rows_mask][:, 0, case.Dn:]
        want = cache_o[rows_mask][:, 0, case.Dn:]
        d = gh.fp8_ulp_diff(got, want)
        nan = (want & 0x7F) == 0x7F
        _say(f"[codec] scale={scale}: {int((d != 0).sum())} of {d.size} tail codes differ; "
             f"{int(nan.sum())} NaN codes")
        assert int(d.max()) == 0
        # 254 NaN patterns, each with its rotation partner (and the infinities'
        # partners) in the same 64-value tail: four whole tails of NaN codes
        assert int(nan.sum()) == 256, "a NaN input gives the NaN code"
        stats = gh.compare_mla(case, (q, cache, None, 0), gh.oracle_mla(orc, case))
        _say(f"[codec] scale={scale}: {stats}")


@pytest.mark.parametrize("H", [4, 40])
def test_non_finite_q_values(orc, H):
    """+-inf and NaN in q: a rotated value whose pair holds an infinity is
    +-inf, or NaN where the two products are opposite infinities or an
    infinity meets a zero cos/sin (position 0: sin 0); a NaN spreads to its
    pair.  Every q output as the oracle's: NaN where it is NaN, every other
    value within the usual bar (infinities equal).  16 and 32 heads per wave."""
    rng = workloads.make_rng(4500 + H)
    case = workloads.build_mla(f"mla_q_nonfinite_h{H}", 4500 + H, [9, 7], [0, 40], H=H,
                               page_size=16, max_seq_len=128, spare_pages=2,
                               scale_mode="per_tensor", tensor_scale=0.05, rng=rng)
    pinf, ninf, nan = np.uint16(0x7F80), np.uint16(0xFF80), np.uint16(0x7FC0)
    q = case.q                                  # [T, H, R] bf16 patterns
    q[0, 0, 3] = pinf                           # token 0 sits at position 0
    q[1, 1, 5] = ninf
    q[2, 2, 40] = nan
    q[3, 3, 0], q[3, 3, 32] = pinf, pinf        # both members of one pair
    q[4, 0, 10], q[4, 0, 42] = pinf, ninf
    q[5, H - 1, 63] = nan
    q[10, 1, 1] = pinf                          # second request, position 40
    dev = gh.MlaDevice(case)
    dev.run()
    gpu = dev.results()
    assert gpu[3] == 0
    want = gh.oracle_mla(orc, case)
    g, w = gpu[0], want[0]
    gnan = (g & 0x7FFF) > 0x7F80
    wnan = (w & 0x7FFF) > 0x7F80
    assert np.array_equal(gnan, wnan), "NaN positions differ"
    assert wnan.sum() >= 2
    d = gh.bf16_ulp_diff(g[~wnan], w[~wnan])
    assert int(d.max(initial=0)) <= gh.BF16_MAX_ULP
    inf_w = (w[~wnan] & 0x7FFF) == 0x7F80
    assert inf_w.sum() >= 4 and np.array_equal(g[~wnan][inf_w], w[~wnan][inf_w])
    # the cache rows are untouched by q: as the oracle's
    stats = gh.compare_mla(case, (np.where(wnan, w, g), gpu[1], gpu[2], 0), want)
    _say(f"[q-nonfinite] H={H}: {int(wnan.sum())} NaN, {int(inf_w.sum())} inf; {stats}")


@pytest.mark.parametrize("scale_mode", ["per_tensor", "per_token"])
def test_non_finite_latent_values(orc, scale_mode):
    """A NaN or an infinity in the latent row's non-rope part reaches the
    statistic: a NaN makes every normalised value NaN; an infinity makes r = 0,
    so the infinite value becomes NaN (inf x 0) and the others +-0.  The rope
    tail is rotated as usual.  Codes (NaN codes by NaN-ness), and per-token
    scales (which ignore NaN values, as a max over the row does), match the
    oracle."""
    case = workloads.build_mla(f"mla_nonfinite_{scale_mode}", 4010, [3, 5], [2, 7], H=4,
                               page_size=8, max_seq_len=64, spare_pages=2,
                               scale_mode=scale_mode, tensor_scale=0.05)
    nan, inf, ninf = np.uint16(0x7FC0), np.uint16(0x7F80), np.uint16(0xFF80)
    case.latent[0, 17] = nan                 # NaN in the normalised part
    case.latent[1, 300] = inf                # +inf in the normalised part
    case.latent[2, 5] = ninf                 # -inf in the normalised part
    case.latent[3, case.Dn + 3] = nan        # NaN in the rope tail
    case.latent[4, case.Dn + 40] = inf       # +inf in the rope tail
    case.latent[5, :case.Dn] = nan           # every normalised value NaN
    dev = gh.MlaDevice(case)
    dev.run()
    res = dev.results()
    assert res[3] == 0
    stats = gh.compare_mla(case, res, gh.oracle_mla(orc, case), small_case_floor=3)
    _say(f"[nonfinite] {scale_mode}: {stats}")
    rows = gh.written_rows(case)
    codes = res[1][rows][:, 0]
    assert ((codes & 0x7F) == 0x7F).any(axis=1).sum() >= 5


def test_skipped_tokens_are_counted(orc):
    """Device data that breaks the rules (a page id beyond the pool, slots past
    the page table / positions past the freqs table) makes the kernel skip those
    tokens, leave their outputs alone and count them; the other tokens are
    unaffected."""
    def make():
        return workloads.build_mla("mla_bad", 4005, [3, 4, 5], [0, 10, 2], H=8, page_size=8,
                                   max_seq_len=16, spare_pages=2)
    good, case = make(), make()
    case.page_table[0, 0] = case.meta["num_pages"] + 3   # request 0: page beyond the pool
    case.cache_lengths[1] = 14                            # request 1: slots 14..17; 16, 17 break
    dev = gh.MlaDevice(case)
    dev.q_out.zero_()
    dev.run()
    q, cache, _, skipped = dev.results()
    assert skipped == 5, skipped
    assert not q[[0, 1, 2, 5, 6]].any(), "skipped tokens wrote q"
    q_o, cache_o, _, pre = gh.oracle_mla(orc, good)
    assert gh.bf16_ulp_diff(q[7:], q_o[7:]).max() <= 1       # request 2 unaffected
    owners = oracle_pins.slot_owners(good.row_offsets, good.cache_lengths, good.page_table, 8)
    L = good.layer_idx
    for (page, off), (t, slot) in owners.items():
        if t >= 7:
            gh.check_fp8(cache[L, page, off], cache_o[L, page, off], pre[L, page, off], "row")
        elif t < 3:
            assert np.array_equal(cache[L, page, off], good.cache[L, page, off])


def test_deterministic(orc):
    case = workloads.mla_prefill()
    a = gh.MlaDevice(case)
    a.run()
    ra = a.results()
    b = gh.MlaDevice(case)
    b.run()
    rb = b.results()
    assert np.array_equal(ra[0], rb[0]) and np.array_equal(ra[1], rb[1])


def test_stream_ordering(orc):
    """A launch on a side stream is ordered on that stream only."""
    case = workloads.mla_tiny()
    dev = gh.MlaDevice(case)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dev.run(stream=s)
    s.synchronize()
    gh.compare_mla(case, dev.results(), gh.oracle_mla(orc, case))


# -- in-place form on a bf16 cache that already holds the rows --------------------------


def _run_inplace(orc, case, q_f32=False):
    _say(f"[mla-inplace] case={case.name} seed={case.seed} T={case.T} B={case.B} H={case.H} "
         f"q_f32={q_f32}")
    dev = gh.MlaDevice(case, "dense", q_f32)
    dev.place_rows()
    dev.run_inplace()
    gpu = dev.results()
    assert gpu[3] == 0, f"{gpu[3]} tokens skipped"
    stats = gh.compare_mla(case, gpu, gh.oracle_mla_inplace(orc, case, q_f32))
    _say(f"[mla-inplace] {case.name}: {stats}")
    return gpu


@pytest.mark.parametrize("idx", range(3))
@pytest.mark.parametrize("q_f32", [False, True])
def test_inplace_small_cases(orc, idx, q_f32):
    _run_inplace(orc, list(oracle_pins.small_mla_inplace_cases())[idx], q_f32)


def _inplace_big():
    rng = workloads.make_rng(4101)
    new = rng.integers(1, 600, size=12, endpoint=True)
    return workloads.build_mla("mla_inplace_big", 4101, new, rng.integers(0, 3000, size=12),
                               H=128, page_size=128, max_seq_len=4096, spare_pages=4,
                               latent_sigma=2.0, scale_mode="none", cache_dtype="bf16", rng=rng)


def test_inplace_prefill_shaped(orc):
    """128 heads, 12 ragged requests, page size 128, bf16 cache."""
    _run_inplace(orc, _inplace_big())


def test_inplace_equals_buffer_form(orc):
    """The in-place form is the buffer form with the row read from the cache:
    bit-identical q and cache to a buffer-form launch into a bf16 cache."""
    case = _inplace_big()
    a = gh.MlaDevice(case)
    a.place_rows()
    a.run_inplace()
    ra = a.results()
    b = gh.MlaDevice(case)
    b.run()
    rb = b.results()
    rows = gh.written_rows(case)
    assert np.array_equal(ra[0], rb[0]), "q differs"
    assert np.array_equal(ra[1][rows], rb[1][rows]), "cache rows differ"
    assert np.array_equal(ra[1][~rows], case.cache[~rows])


def test_inplace_skipped_tokens(orc):
    """A token whose page id lies beyond the pool is skipped and counted; its
    row (wherever the table points) is neither read nor written."""
    good = workloads.build_mla("mla_inplace_bad", 4102, [3, 4], [0, 10], H=8, page_size=8,
                               max_seq_len=32, spare_pages=2, scale_mode="none",
                               cache_dtype="bf16")
    dev = gh.MlaDevice(good)
    dev.place_rows()
    placed = gh.host_bf16(dev.cache).copy()
    bad_table = good.page_table.copy()
    bad_table[0, 0] = good.meta["num_pages"] + 1
    dev.page_table.copy_(gh.dev_u32(bad_table))
    dev.q_out.zero_()
    dev.run_inplace()
    q, cache, _, skipped = dev.results()
    assert skipped == 3, skipped
    assert not q[:3].any(), "skipped tokens wrote q"
    q_o, cache_o, _, _ = gh.oracle_mla_inplace(orc, good)
    assert gh.bf16_ulp_diff(q[3:], q_o[3:]).max() <= 1
    owners = oracle_pins.slot_owners(good.row_offsets, good.cache_lengths, good.page_table, 8)
    L = good.layer_idx
    for (page, off), (t, slot) in owners.items():
        if t < 3:
            assert np.array_equal(cache[L, page, off], placed[L, page, off]), "skipped row changed"
        else:
            gh.check_bf16(cache[L, page, off], cache_o[L, page, off], "row")


def test_zero_rows_per_token(orc):
    """Per-token scale on degenerate latent rows: all +0, all -0, a mix of
    signed zeros, only the rope tail non-zero, only the non-rope part
    non-zero.  A zero row stores scale 0 and zero codes (its normalised part
    keeps each value's sign); every row as the oracle."""
    case = workloads.build_mla("mla_zero_rows", 4201, [6, 5], [0, 9], H=4, page_size=8,
                               max_seq_len=32, spare_pages=2, scale_mode="per_token")
    lat = case.latent
    lat[0] = 0x0000
    lat[1] = 0x8000
    lat[2, ::2], lat[2, 1::2] = 0x0000, 0x8000
    lat[3, : case.Dn] = 0x0000                 # rope tail only
    lat[4, case.Dn:] = 0x8000                  # non-rope part only
    dev = gh.MlaDevice(case)
    dev.run()
    gpu = dev.results()
    assert gpu[3] == 0
    stats = gh.compare_mla(case, gpu, gh.oracle_mla(orc, case))
    _say(f"[mla-zero] {stats}")
    owners = oracle_pins.slot_owners(case.row_offsets, case.cache_lengths, case.page_table,
                                     case.meta["page_size"])
    L = case.layer_idx
    for (page, off), (t, slot) in owners.items():
        if t < 3:
            assert gpu[2][L, page, off, 0] == 0.0, f"token {t}: scale of a zero row"
            codes = gpu[1][L, page, off, 0]
            assert np.all((codes & 0x7F) == 0), f"token {t}: non-zero code"
            # the normalised part keeps each zero's sign (x * r * gamma); the
            # rotated tail's zero signs follow IEEE sums of signed zeros
            assert np.array_equal(codes[: case.Dn] >> 7, (lat[t, : case.Dn] >> 15).astype(np.uint8)), \
                f"token {t}: zero signs"


@pytest.mark.parametrize("mode", ["per_tensor", "per_token", "bf16"])
def test_no_heads(orc, mode):
    """num_heads = 0 (q tensors [T, 0, R], null pointers): the wave of each
    token writes its latent row alone, its q lanes read nothing from q; also
    through the token plan."""
    case = workloads.build_mla(f"mla_h0_{mode}", 4401, [7, 0, 12], [0, 5, 30], H=0,
                               page_size=16, max_seq_len=128, spare_pages=2,
                               scale_mode="per_token" if mode == "per_token" else "per_tensor",
                               cache_dtype="bf16" if mode == "bf16" else "fp8",
                               rng=workloads.make_rng(4401))
    assert case.q.shape[1] == 0
    _run_and_compare(orc, case)
    dev = gh.MlaDevice(case)
    plan = torch.empty((case.T, 4), dtype=torch.int32, device="cuda")
    import paged_kv_cache_wavefront_amd as pkv
    pkv.pkv_token_plan(plan, dev.offsets, dev.desc)
    pkv.mla_rope_rmsnorm_quant_planned(dev.q_out, dev.q_in, dev.latent, plan, dev.freqs,
                                       dev.gamma, case.epsilon, dev.desc, case.layer_idx)
    gpu = dev.results()
    assert gpu[3] == 0
    stats = gh.compare_mla(case, gpu, gh.oracle_mla(orc, case))
    _say(f"[mla-h0 planned] {stats}")


def test_launch_shape_invariance():
    """The same tokens under different wave mappings give identical bits: a
    32-head launch (32 heads per wave) against two 16-head launches over its
    head halves (16 heads per wave, one wave per token), and a 40-head launch
    (masked lanes) against the same 32 + 8 heads launched apart."""
    import paged_kv_cache_wavefront_amd as pkv
    base = workloads.build_mla("mla_shape", 4301, [37, 0, 120, 5], [3, 9, 0, 200], H=40,
                               page_size=16, max_seq_len=512, spare_pages=3,
                               scale_mode="per_token")
    full = gh.MlaDevice(base)
    full.run()
    q_full, cache_full, ts_full, _ = full.results()
    for lo, hi in ((0, 16), (16, 32), (32, 40), (0, 32)):
        dev = gh.MlaDevice(base)
        q_in = dev.q_in[:, lo:hi]
        q_out = dev.q_out[:, lo:hi]
        pkv.mla_rope_rmsnorm_quant(q_out, q_in, dev.latent, dev.offsets, dev.freqs, dev.gamma,
                                   base.epsilon, dev.desc, base.layer_idx)
        q, cache, ts, _ = dev.results()
        assert np.array_equal(q[:, lo:hi], q_full[:, lo:hi]), f"heads {lo}:{hi}"
        assert np.array_equal(cache, cache_full), f"cache with heads {lo}:{hi}"
        assert np.array_equal(ts.view(np.uint32), ts_full.view(np.uint32))
