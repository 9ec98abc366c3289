"""The committed oracle against its pins (closed forms, invariants, brute
force, library special cases, format landmarks)."""
import pytest

import exact_pins
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


@pytest.mark.parametrize("pin", exact_pins.ALL_EXACT_PINS, ids=lambda f: f.__name__)
def test_exact_pin(orc, pin):
    """Every output of the entry points on tiny cases equals the exact value
    (120-digit decimal arithmetic) rounded once, exact ties to even."""
    pin(orc)


def test_exact_rounding_helpers(orc):
    """The decimal rounding helpers themselves: format landmarks, exact ties
    to even, saturation, signed zero, and agreement with the oracle's own
    (separately pinned) encoders away from ties."""
    from decimal import Decimal
    import numpy as np
    E = exact_pins
    assert E.round_fp8(Decimal(448))[0] == 0x7E and E.round_fp8(Decimal(10 ** 6))[0] == 0x7E
    assert E.round_fp8(Decimal(-464))[0] == 0xFE
    assert E.round_fp8(Decimal(2) ** -10) == (0x00, E.TIE)      # halfway to the first subnormal
    assert E.round_fp8(Decimal(3) * Decimal(2) ** -10) == (0x02, E.TIE)
    assert E.round_fp8(Decimal("-0"))[0] == 0x80
    assert E.round_fp8(Decimal(17))[0] == 0x58                    # 17 between 16 and 18: even 16
    assert E.round_bf16(Decimal(1) + Decimal(2) ** -8) == (0x3F80, E.TIE)
    assert E.round_bf16(Decimal(1) + Decimal(3) * Decimal(2) ** -8) == (0x3F82, E.TIE)
    assert E.round_bf16(Decimal(1) + Decimal(2) ** -8 + Decimal(2) ** -60) == (0x3F81, E.NEAR_TIE)
    assert E.round_f32(Decimal(1) + Decimal(2) ** -24) == (0x3F800000, E.TIE)
    assert E.round_f32(Decimal(-1) - Decimal(2) ** -23) == (0xBF800001, E.OK)
    assert E.fp8_value(0x80).is_signed() and E.fp8_value(0x7E) == 448
    assert E.round_f16(Decimal(1) + Decimal(2) ** -11) == (0x3C00, E.TIE)
    assert E.round_f16(Decimal(1) + Decimal(3) * Decimal(2) ** -11) == (0x3C02, E.TIE)
    assert E.round_f16(Decimal(-1) - Decimal(2) ** -10) == (0xBC01, E.OK)
    assert E.round_f16(Decimal(2) ** -25) == (0x0000, E.TIE)      # halfway to 2^-24
    rng = np.random.default_rng(5)
    for v in rng.standard_normal(300) * 50:
        d = Decimal(float(v))
        assert E.round_bf16(d)[0] == orc.bf16_encode(float(v))
        assert E.round_fp8(d)[0] == orc.e4m3fn_encode(float(v))


def test_fp8_midpoint_distance():
    """The near-tie measure used by the fp8 parity bar: zero at midpoints,
    exact relative distances elsewhere, no midpoint past saturation."""
    import numpy as np
    rel = oracle_pins.fp8_midpoint_rel(np.array([152.0, -152.0, 151.0, 2.0 ** -10, 1.0,
                                                 1.0625, 449.0, 464.0, np.nan]))
    assert rel[0] == 0 and rel[1] == 0
    assert rel[2] == 1.0 / 152.0
    assert rel[3] == 0                        # between +0 and the first subnormal
    assert rel[4] == 0.03125 / 0.96875        # 1.0 sits on a code; midpoints 0.96875, 1.0625
    assert rel[5] == 0
    assert np.isinf(rel[6]) and np.isinf(rel[7]) and np.isnan(rel[8])


def test_fp8_probe_records_rounded_values(orc):
    """The oracle's fp8 probe: every code an entry point encodes has the
    binary64 value it came from, an exhaustive nearest-code search over that
    value gives the code, bytes not encoded stay NaN, and the outputs equal
    those of an unprobed call.  (torch's cast from float64 is not used here:
    it rounds through float32 first, and these values sit on near-ties often
    enough for that double rounding to show.)"""
    import numpy as np

    def nearest_codes(v):
        return oracle_pins.fp8_encode_bruteforce(v).reshape(v.shape)

    import gpu_helpers as gh
    for case in list(oracle_pins.small_mla_cases())[1:4]:
        if case.cache.dtype != np.uint8:
            continue
        _, plain, plain_ts, _ = gh.oracle_mla(orc, case)   # probed
        cache = case.cache.copy()
        ts = None if case.token_scales is None else case.token_scales.copy()
        orc.mla_rope_rmsnorm_quant(np.zeros_like(case.q), case.q, case.latent, case.row_offsets,
                                   case.cache_lengths, case.page_table, case.freqs, case.gamma,
                                   case.epsilon, cache, case.layer_idx, case.scale_mode,
                                   case.tensor_scale, ts)
        assert np.array_equal(cache, plain)
        with orc.fp8_probe(cache.copy()) as _:
            pass
        cache = case.cache.copy()
        with orc.fp8_probe(cache) as pre:
            orc.mla_rope_rmsnorm_quant(np.zeros_like(case.q), case.q, case.latent,
                                       case.row_offsets, case.cache_lengths, case.page_table,
                                       case.freqs, case.gamma, case.epsilon, cache,
                                       case.layer_idx, case.scale_mode, case.tensor_scale,
                                       None if ts is None else case.token_scales.copy())
        rows = gh.written_rows(case)
        assert np.all(np.isfinite(pre[rows])), case.name
        assert np.all(np.isnan(pre[~rows])), case.name
        assert np.array_equal(nearest_codes(pre[rows]), cache[rows]), case.name
    # after the context the probe is off: a call records nothing
    dummy = np.zeros(4, np.uint8)
    with orc.fp8_probe(dummy) as pre:
        pass
    case = list(oracle_pins.small_mla_cases())[1]
    gh.oracle_mla(orc, case)
    assert np.all(np.isnan(pre))
