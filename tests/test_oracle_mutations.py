"""The pins must catch plausible mistakes in the oracle.

Each mutant is the committed oracle source with one small, plausible error
planted in it (a flipped sign, a swapped operand or index, a dropped term, a
wrong rounding rule, a wrong address).  The mutant is compiled with gcc into
a temporary directory and every pin is run against it in a child process; the
child must fail (an assertion, or a crash of the mutant).  Everything here
runs on the CPU; the HIP library is not involved.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pkv_oracle.c")

# (name, text in the committed source, replacement)
MUTANTS = [
    ("rope_first_sign", "out[ia] = a * cs - b * sn;", "out[ia] = a * cs + b * sn;"),
    ("rope_second_sign", "out[ib] = b * cs + a * sn;", "out[ib] = b * cs - a * sn;"),
    ("rope_swapped_operand", "out[ib] = b * cs + a * sn;", "out[ib] = a * cs + b * sn;"),
    ("rope_cos_sin_columns", "double cs = (double)freqs_row[2 * i];",
     "double cs = (double)freqs_row[2 * i + 1];"),
    ("rope_split_table", "double sn = (double)freqs_row[2 * i + 1];",
     "double sn = (double)freqs_row[half + i];"),
    ("rope_half_pairing", "int64_t ib = interleaved ? 2 * i + 1 : i + half;",
     "int64_t ib = interleaved ? 2 * i + 1 : half - 1 - i;"),
    ("rope_interleaved_pairing", "int64_t ia = interleaved ? 2 * i : i;",
     "int64_t ia = interleaved ? i : i;"),
    ("rms_dropped_eps", "return 1.0 / sqrt(ss / (double)n + eps);",
     "return 1.0 / sqrt(ss / (double)n);"),
    ("rms_eps_outside_root", "return 1.0 / sqrt(ss / (double)n + eps);",
     "return 1.0 / (sqrt(ss / (double)n) + eps);"),
    ("rms_sum_not_mean", "return 1.0 / sqrt(ss / (double)n + eps);",
     "return 1.0 / sqrt(ss + eps);"),
    ("rms_dropped_gamma", "for (int64_t k = 0; k < n; ++k) y[k] = x[k] * r * g[k];",
     "for (int64_t k = 0; k < n; ++k) y[k] = x[k] * r;"),
    ("mla_position_ignores_prior", "const int64_t pos = (int64_t)cache_lengths[b] + j;",
     "const int64_t pos = j;"),
    ("mla_rope_tail_normalised", "oracle_rope_row(x + Dn, y + Dn, R, fr, 0);",
     "oracle_rope_row(y + Dn, x + Dn, R, fr, 0); memcpy(y + Dn, x + Dn, R * sizeof(double));"),
    ("mla_scale_multiplied", "put_fp8(&dst[k], y[k] / s);",
     "put_fp8(&dst[k], y[k] * s);"),
    ("mla_amax_nope_only", "for (int64_t k = 0; k < W; ++k)\n      if (fabs(y[k]) > amax)",
     "for (int64_t k = 0; k < Dn; ++k)\n      if (fabs(y[k]) > amax)"),
    ("mla_token_scale_448", "const float st = (float)(amax / 448.0); /* stored fp32",
     "const float st = (float)(amax / 240.0); /* stored fp32"),
    ("page_offset", "const int64_t off = slot % page_size;\n      const int64_t row = ((layer_idx",
     "const int64_t off = (slot + 1) % page_size;\n      const int64_t row = ((layer_idx"),
    ("page_table_column", "int64_t col = slot / page_size;", "int64_t col = slot / page_size + 1;"),
    ("wrong_layer", "const int64_t row = ((layer_idx * num_pages + page) * page_size + off);",
     "const int64_t row = (((layer_idx - 1) * num_pages + page) * page_size + off);"),
    ("fp8_ties_away", "double n = nearbyint(ldexp(a, -qexp));\n  double r = ldexp(n, qexp);    /* rounded magnitude",
     "double n = round(ldexp(a, -qexp));\n  double r = ldexp(n, qexp);    /* rounded magnitude"),
    ("fp8_no_saturation", "if (a > 448.0) a = 448.0;", "if (a > 480.0) a = 480.0;"),
    ("fp8_flush_subnormals", "if (qexp < -9) qexp = -9;     /* subnormal quantum 2^-9 */",
     "if (qexp < -6) qexp = -6;"),
    ("fp8_bias", "return (uint8_t)(sign | ((E + 7) << 3) | m);",
     "return (uint8_t)(sign | ((E + 8) << 3) | m);"),
    ("fp8_decode_subnormal", "mag = ldexp((double)m, -9);", "mag = ldexp((double)m, -10);"),
    ("bf16_truncate", "double n = nearbyint(ldexp(a, -qexp)); /* default mode: ties to even */",
     "double n = trunc(ldexp(a, -qexp));"),
    ("bf16_precision", "int qexp = e - 8;             /* keep 8 significant bits */",
     "int qexp = e - 9;"),
    ("qk_ignores_position_ids",
     "const int64_t pos = position_ids ? (int64_t)position_ids[t] : slot;",
     "const int64_t pos = slot;"),
    ("qk_norm_skips_gamma",
     "if (i < k_norm_cols) a[i] = both[i] ? a[i] * g[i] : a[i] * inv * g[i];",
     "if (i < k_norm_cols) a[i] = both[i] ? a[i] : a[i] * inv;"),
    ("qk_norm_all_columns", "const double inv = oracle_inv_rms(a, k_norm_cols, eps);",
     "const double inv = oracle_inv_rms(a, D, eps);"),
    ("qk_norm_inv_not_applied_after", "if (both[i]) r[i] *= inv;", "if (both[i]) r[i] *= 1.0;"),
    ("qk_norm_mixed_pair_unnormalised",
     "if (i < k_norm_cols) a[i] = both[i] ? a[i] * g[i] : a[i] * inv * g[i];",
     "if (i < k_norm_cols) a[i] = a[i] * g[i];"),
    # the per-member order before the rotation: a binary64 residue where a
    # pair cancels exactly (only the exact-cancellation pin sees it)
    ("qk_norm_inv_before_rotation",
     "if (i < k_norm_cols) a[i] = both[i] ? a[i] * g[i] : a[i] * inv * g[i];\n"
     "          }\n          oracle_rope_row(a, r, D, fr, interleaved);\n"
     "          for (int64_t i = 0; i < D; ++i)\n            if (both[i]) r[i] *= inv;",
     "if (i < k_norm_cols) a[i] = a[i] * inv * g[i];\n"
     "          }\n          oracle_rope_row(a, r, D, fr, interleaved);"),
    ("kvnorm_no_offset", "g[k] = elem(gamma, k, gamma_type) + (double)weight_offset;",
     "g[k] = elem(gamma, k, gamma_type);"),
    ("kvnorm_cast_order", "if (multiply_before_cast) {", "if (!multiply_before_cast) {"),
    ("kvnorm_ignores_total", "if (t >= total_seq_len) break;", "(void)total_seq_len;"),
    ("gather_slot_shift", "const int64_t slot = row - (int64_t)kv_row_offsets[b];",
     "const int64_t slot = row - (int64_t)kv_row_offsets[b] + (b > 0);"),
    ("gather_tensor_scale_only",
     "scale = (double)(scale_mode == ORACLE_SCALE_PER_TOKEN ? cache_scales[src_row]",
     "scale = (double)(scale_mode == ORACLE_SCALE_PER_TENSOR ? cache_scales[src_row]"),
    ("k_fp8_ignores_scale",
     ": oracle_e4m3fn_decode(((const uint8_t*)k_cache)[elem + i]) * scale;",
     ": oracle_e4m3fn_decode(((const uint8_t*)k_cache)[elem + i]);"),
    ("k_fp8_token_scale_stale", "    *token_scale = st;\n    s = (double)st;",
     "    *token_scale = st;"),
    ("mla_f32_q_truncated", "for (int64_t i = 0; i < R; ++i) dst[i] = (float)qb[i];  /* RNE */",
     "for (int64_t i = 0; i < R; ++i) dst[i] = (float)(qb[i] * (1 - 1e-7));"),
    ("token_norm_per_head_count", "token_inv = 1.0 / sqrt(ss / (double)(Hkv * gamma_len) + eps);",
     "token_inv = 1.0 / sqrt(ss / (double)(gamma_len) + eps);"),
    ("mrope_section_boundary", "const int64_t k = i < mrope_section[0] ? 0",
     "const int64_t k = i <= mrope_section[0] ? 0"),
    ("mrope_row_layout", "const int64_t pk = (int64_t)position_ids[k * T + t];",
     "const int64_t pk = (int64_t)position_ids[t * 3 + k];"),
    ("gather_quant_multiplies", "oracle_bf16_decode(bits) / (double)out_tensor_scale);",
     "oracle_bf16_decode(bits) * (double)out_tensor_scale);"),
    ("inplace_reads_next_slot",
     "const uint16_t* src = latent ? latent + t * W : (const uint16_t*)cache + row * W;",
     "const uint16_t* src = latent ? latent + t * W : (const uint16_t*)cache + (row + 1) * W;"),
    # rounding-rule slips only the exact-arithmetic pins see: a per-token
    # scale rounded twice, and exact ties broken upwards
    ("mla_token_scale_two_roundings", "const float st = (float)(amax / 448.0); /* stored fp32",
     "const float st = (float)amax / 448.0f; /* stored fp32"),
    ("k_token_scale_two_roundings", "const float st = (float)(amax / 448.0);\n    *token_scale = st;",
     "const float st = (float)amax / 448.0f;\n    *token_scale = st;"),
    ("mla_f32_q_ties_up", "dst[i] = (float)qb[i];  /* RNE */",
     "dst[i] = (float)(qb[i] * (1 + 0x1p-40));  /* RNE */"),
    ("kvnorm_unrounded_ties_up",
     "a[i] = oracle_bf16_decode(oracle_bf16_encode(a[i] * inv)) * g[i];",
     "a[i] = oracle_bf16_decode(oracle_bf16_encode(a[i] * inv)) * g[i] * (1 + 0x1p-40);"),
    # the token plan and the step placed by it
    ("plan_offset", "plan[4 * t + 1] = (uint32_t)(slot % page_size);",
     "plan[4 * t + 1] = (uint32_t)((slot + 1) % page_size);"),
    ("plan_position", "plan[4 * t + 2] = (uint32_t)slot;", "plan[4 * t + 2] = (uint32_t)slot + 1;"),
    ("planned_ignores_flag", "return !(e[3] == 0 || (int64_t)e[0] >= num_pages",
     "return !((int64_t)e[0] >= num_pages"),
    ("planned_kvnorm_drops_last", "for (int64_t t = 0; t < total_seq_len; ++t) {",
     "for (int64_t t = 0; t + 1 < total_seq_len; ++t) {"),
    ("planned_kvnorm_next_slot", "layer_idx, (int64_t)e[0], (int64_t)e[1], g, gamma_len, eps,",
     "layer_idx, (int64_t)e[0], (int64_t)(e[1] ^ 1u), g, gamma_len, eps,"),
    # the element types: binary16 codec, typed reads and writes, freqs and gamma types
    ("f16_decode_subnormal", "else if (e == 0) mag = ldexp((double)m, -24);",
     "else if (e == 0) mag = ldexp((double)m, -25);"),
    ("f16_bias", "return (uint16_t)(sign | ((E + 15) << 10) | m);",
     "return (uint16_t)(sign | ((E + 16) << 10) | m);"),
    ("f16_precision", "int qexp = e - 11;            /* keep 11 significant bits */",
     "int qexp = e - 10;"),
    ("f16_ties_away", "double n = nearbyint(ldexp(a, -qexp));\n  double r = ldexp(n, qexp);\n  if (r > 65504.0)",
     "double n = round(ldexp(a, -qexp));\n  double r = ldexp(n, qexp);\n  if (r > 65504.0)"),
    ("elem_f16_read_as_bf16",
     "return type == ORACLE_F16 ? oracle_f16_decode(bits) : oracle_bf16_decode(bits);",
     "return oracle_bf16_decode(bits);"),
    ("elem_f16_written_as_bf16",
     "else if (type == ORACLE_F16) ((uint16_t*)base)[i] = oracle_f16_encode(v);",
     "else if (type == ORACLE_F16) ((uint16_t*)base)[i] = oracle_bf16_encode(v);"),
    ("freqs_type_ignored", "buf[i] = (float)elem(freqs, p * dim + i, type);",
     "buf[i] = (float)elem(freqs, p * dim + i, ORACLE_BF16);"),
    ("mla_gamma_type_ignored",
     "g[k] = elem(gamma, k, gamma_type);\n  const double eps = (double)epsilon; /* the fp32",
     "g[k] = elem(gamma, k, ORACLE_BF16);\n  const double eps = (double)epsilon; /* the fp32"),
    ("planned_offset_as_position",
     "mla_token(q_out, q_out_type, q_in, q_in_type, latent, t, (int64_t)e[2], row,",
     "mla_token(q_out, q_out_type, q_in, q_in_type, latent, t, (int64_t)e[1], row,"),
]

RUNNER = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, oracle_pins, exact_pins
orc = oracle.Oracle({lib!r})
for pin in oracle_pins.ALL_PINS + exact_pins.ALL_EXACT_PINS:
    try:
        pin(orc)
    except Exception as e:
        print("CAUGHT by", pin.__name__, ":", str(e)[:200])
        sys.exit(1)
print("SURVIVED")
"""


def _run_mutant(name, old, new, tmp):
    src = open(SRC).read()
    assert src.count(old) == 1, f"{name}: anchor text must occur once"
    path = os.path.join(tmp, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(tmp, f"lib_{name}.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-ffp-contract=off", "-shared",
                    "-I", os.path.dirname(SRC), "-o", lib, path, "-lm"], check=True,
                   capture_output=True)
    code = RUNNER.format(root=ROOT, tests=os.path.dirname(os.path.abspath(__file__)), lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=600)
    return name, r.returncode, (r.stdout + r.stderr)[-400:]


@pytest.mark.slow
def test_every_mutant_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=6) as ex:
            results = list(ex.map(lambda m: _run_mutant(*m, tmp), MUTANTS))
    survived = [(n, out) for n, rc, out in results if rc == 0]
    assert not survived, f"mutants not caught by any pin: {survived}"


def test_committed_oracle_passes_runner():
    """The same runner reports no failure on the committed oracle."""
    import oracle
    code = RUNNER.format(root=ROOT, tests=os.path.dirname(os.path.abspath(__file__)),
                         lib=oracle.LIB_PATH)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0 and "SURVIVED" in r.stdout, r.stdout + r.stderr
