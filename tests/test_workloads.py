"""The seeded input recipe (CPU): shapes and sizes of the named workloads,
ragged-batch and page-table construction (every new token gets a distinct
slot in a page of the pool, unused table entries marked, untouched pages
exist), the RoPE angle table against its definition, bf16 rounding of the
normal draws, and reproducibility from the seed."""
import numpy as np
import pytest

import oracle_pins
import workloads


def _check_batch(case, page_size):
    offs = case.row_offsets.astype(np.int64)
    assert offs[0] == 0 and np.all(np.diff(offs) >= 0) and offs[-1] == case.T
    owners = oracle_pins.slot_owners(case.row_offsets, case.cache_lengths, case.page_table,
                                     page_size)
    assert len(owners) == case.T                       # every token has one slot, none shared
    pages = {p for (p, _) in owners}
    num_pages = case.meta["num_pages"]
    assert max(pages) < num_pages
    used = case.page_table[case.page_table != workloads.UNUSED_PAGE]
    assert len(np.unique(used)) == used.size          # no page mapped twice
    assert used.size < num_pages                      # spare (untouched) pages exist


@pytest.mark.parametrize("name,T,H", [("mla_tiny", 16, 4), ("mla_decode", 256, 128),
                                      ("mla_prefill", 17108, 128), ("mla_mixed", 8256, 16),
                                      ("mla_prefill_inplace", 17108, 128)])
def test_mla_workloads(name, T, H):
    case = workloads.NAMED[name]()
    assert case.T == T and case.q.shape == (T, H, 64) and case.latent.shape == (T, 576)
    assert case.q.dtype == np.uint16 and case.latent.dtype == np.uint16
    assert case.cache.shape[0] == 2 and case.layer_idx == 1
    _check_batch(case, case.meta["page_size"])
    if name in ("mla_prefill", "mla_prefill_inplace"):
        assert case.B == 8 and np.all(case.cache_lengths == 0)
        new = np.diff(case.row_offsets.astype(np.int64))
        assert new.min() >= 512 and new.max() <= 4096
    if name == "mla_decode":
        assert case.B == 256 and np.all(np.diff(case.row_offsets.astype(np.int64)) == 1)
    # the two prefill workloads draw the same batch and values
    if name == "mla_prefill_inplace":
        ref = workloads.mla_prefill()
        assert np.array_equal(case.q, ref.q) and np.array_equal(case.latent, ref.latent)
        assert case.cache.dtype == np.uint16 and case.scale_mode == "none"


def test_qk_workload():
    case = workloads.qk_generic()
    assert case.q.shape[1:] == (32, 128) and case.k_cache.shape[3:] == (8, 128)
    assert case.interleaved and case.position_ids is not None
    assert int(case.position_ids.max()) < 131072
    _check_batch(case, case.meta["page_size"])


def test_freqs_table_definition():
    """Column 2i is cos and 2i+1 is sin of p * theta^(-2i/dim), each the fp32
    rounding of the binary64 value (checked at scattered rows against
    math.cos / math.sin)."""
    import math
    for dim, theta, rows in ((64, 10000.0, 16384), (128, 500000.0, 4096)):
        t = workloads.freqs_table(rows, dim, theta)
        assert t.shape == (rows, dim) and t.dtype == np.float32
        for p in (0, 1, 7, rows // 3, rows - 1):
            for i in (0, 1, dim // 4, dim // 2 - 1):
                a = p * theta ** (-2.0 * i / dim)
                assert t[p, 2 * i] == np.float32(math.cos(a))
                assert t[p, 2 * i + 1] == np.float32(math.sin(a))
        assert np.all(t[0, 0::2] == 1.0) and np.all(t[0, 1::2] == 0.0)


def test_normal_draws_are_bf16_roundings():
    """Inputs are fp32 normal draws rounded once to bf16 (nearest, ties to
    even): re-rounding the bf16 values changes nothing, and the sample moments
    fit N(0, sigma) for the prefill latent (sigma 2)."""
    case = workloads.mla_prefill()
    x = oracle_pins.bf16_to_f64(case.latent)
    assert np.array_equal(workloads.bf16_bits(x.astype(np.float32)), case.latent)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 2.0) < 0.01


def test_seeded_reproducibility():
    a, b = workloads.mla_mixed(), workloads.mla_mixed()
    for f in ("row_offsets", "cache_lengths", "page_table", "q", "latent", "gamma", "cache",
              "token_scales"):
        # as bytes: the sentinel scales are random bits, NaNs among them
        assert np.array_equal(getattr(a, f).view(np.uint8), getattr(b, f).view(np.uint8)), f
    c = workloads.mla_mixed(seed=1234)
    assert not np.array_equal(a.q, c.q)
