"""Seeded synthetic inputs for the paged-KV pre-attention path.

This module only draws inputs: random values, ragged batch structure, page
tables, the RoPE frequency table and sentinel-filled cache pools.  It holds
none of the method's arithmetic and is shared, as plain numpy arrays, by the
tests, the benchmark and the oracle checks; neither the HIP library nor the
oracle imports it.

Every generator is deterministic in its seed (numpy PCG64).  Normal draws are
made in float32 and rounded once to bfloat16 by torch's CPU conversion
(round-to-nearest-even).  The workloads mirror the shapes of a DeepSeek-V3
style MLA layer (128 heads, kv_lora_rank 512, rope 64) and of a Llama-style
GQA layer (32 query heads, 8 KV heads, head size 128); no dataset or trained
weight is involved.

Structure shared by every case:
* ``row_offsets`` u32 [B+1]: prefix sums of the new-token counts;
* ``cache_lengths`` u32 [B]: tokens already in each request's cache;
* ``page_table`` u32 [B, stride]: each request gets ceil((prior + new) /
  page_size) pages drawn without replacement from a random permutation of the
  pool; entries past a request's last page hold 0xFFFFFFFF;
* the pool holds ``num_layers`` (2) layers and spare pages nobody owns, and
  every byte of it starts as seeded random data, so that any byte the method
  must not touch can be compared against its starting value.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

UNUSED_PAGE = 0xFFFFFFFF


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (torch CPU cast) and return the bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def as_elem(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values in an element type: "bf16" (bits as uint16, torch's
    round-to-nearest-even cast), "f16" (numpy float16, round-to-nearest-even)
    or "f32" (unchanged)."""
    x = np.ascontiguousarray(x, np.float32)
    if dtype == "bf16":
        return bf16_bits(x)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


def freqs_table(max_seq_len: int, dim: int, theta: float, dtype: str = "f32") -> np.ndarray:
    """RoPE table [max_seq_len, dim]: column 2i = cos, 2i+1 = sin of
    position * theta^(-2i/dim), computed in float64 and rounded once to fp32
    (and from there to bf16 or fp16 for those dtypes)."""
    i = np.arange(dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / dim)
    ang = np.arange(max_seq_len, dtype=np.float64)[:, None] * inv_freq[None, :]
    out = np.empty((max_seq_len, dim), np.float64)
    out[:, 0::2] = np.cos(ang)
    out[:, 1::2] = np.sin(ang)
    return as_elem(out.astype(np.float32), dtype)


def _normal_bf16(rng, shape, sigma=1.0, outlier_p=0.0, outlier_mult=50.0, dtype="bf16"):
    x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)
    if outlier_p > 0.0:
        hit = rng.random(size=shape) < outlier_p
        x = np.where(hit, x * np.float32(outlier_mult), x)
    return as_elem(x, dtype)


def _uniform_bf16(rng, shape, lo, hi, dtype="bf16"):
    return as_elem(rng.uniform(lo, hi, size=shape).astype(np.float32), dtype)


_SENTINEL_PERIOD = (16 << 20) + 7  # odd period: no two pages see the same bytes


def _random_bytes(rng, nbytes: int) -> np.ndarray:
    """Seeded sentinel bytes.  Pools of a gigabyte would take seconds per
    draw, so long buffers repeat one random block with an odd period."""
    if nbytes <= _SENTINEL_PERIOD:
        return np.frombuffer(rng.bytes(nbytes), dtype=np.uint8).copy()
    block = np.frombuffer(rng.bytes(_SENTINEL_PERIOD), dtype=np.uint8)
    return np.resize(block, nbytes)


def ragged_batch(new_lens, prior_lens, page_size, spare_pages, rng):
    """Offsets, cache lengths, a permuted page table and the pool size."""
    new_lens = np.asarray(new_lens, np.int64)
    prior_lens = np.asarray(prior_lens, np.int64)
    B = new_lens.size
    offsets = np.zeros(B + 1, np.uint32)
    offsets[1:] = np.cumsum(new_lens).astype(np.uint32)
    need = -(-(prior_lens + new_lens) // page_size)  # ceil
    total = int(need.sum())
    num_pages = total + int(spare_pages)
    perm = rng.permutation(num_pages).astype(np.uint32)
    stride = max(1, int(need.max()) if B else 1)
    pt = np.full((B, stride), UNUSED_PAGE, np.uint32)
    cur = 0
    for b in range(B):
        pt[b, : need[b]] = perm[cur: cur + need[b]]
        cur += int(need[b])
    return offsets, prior_lens.astype(np.uint32), pt, num_pages


@dataclass
class MlaCase:
    """Inputs of one fused MLA pre-attention call (host arrays)."""

    name: str
    seed: int
    row_offsets: np.ndarray      # u32 [B+1]
    cache_lengths: np.ndarray    # u32 [B]
    page_table: np.ndarray       # u32 [B, stride]
    q: np.ndarray                # bf16 bits [T, H, R] (or float16)
    latent: np.ndarray           # bf16 bits [T, Dn + R]
    gamma: np.ndarray            # bf16 bits [Dn] (or float16, float32)
    freqs: np.ndarray            # f32 [max_seq_len, R] (or bf16 bits, float16)
    epsilon: float
    cache: np.ndarray            # u8 [L, P, S, 1, Dn + R] (fp8) or u16 (bf16)
    layer_idx: int
    scale_mode: str              # "per_tensor" | "per_token" | "none"
    tensor_scale: float
    token_scales: np.ndarray | None  # f32 [L, P, S, 1] (per_token only)
    meta: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def B(self) -> int:
        return int(self.row_offsets.size - 1)

    @property
    def H(self) -> int:
        return int(self.q.shape[1])

    @property
    def R(self) -> int:
        return int(self.q.shape[2])

    @property
    def Dn(self) -> int:
        return int(self.latent.shape[1] - self.q.shape[2])


def make_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def build_mla(name, seed, new_lens, prior_lens, H, R=64, Dn=512, *,
              page_size, max_seq_len, theta=10000.0, spare_pages=16,
              q_sigma=1.0, latent_sigma=1.0, outlier_p=0.0, eps=1e-6,
              scale_mode="per_tensor", tensor_scale=1.0, cache_dtype="fp8",
              num_layers=2, layer_idx=1, rng=None, q_dtype="bf16", freq_dtype="f32",
              gamma_dtype="bf16"):
    """Generic MLA case; ``rng`` continues a preset's stream if given.
    q_dtype ("bf16" | "f16"), freq_dtype ("f32" | "bf16" | "f16") and
    gamma_dtype ("bf16" | "f16" | "f32") pick the element types of q_rope,
    freqs_cis and gamma (the same draws, rounded into that type)."""
    rng = make_rng(seed) if rng is None else rng
    offsets, clens, pt, P = ragged_batch(new_lens, prior_lens, page_size,
                                         spare_pages, rng)
    T = int(offsets[-1])
    W = Dn + R
    q = _normal_bf16(rng, (T, H, R), q_sigma, outlier_p, dtype=q_dtype)
    latent = _normal_bf16(rng, (T, W), latent_sigma, outlier_p)
    gamma = _uniform_bf16(rng, (Dn,), 0.5, 1.5, dtype=gamma_dtype)
    freqs = freqs_table(max_seq_len, R, theta, freq_dtype)
    if cache_dtype == "fp8":
        cache = _random_bytes(rng, num_layers * P * page_size * W).reshape(
            num_layers, P, page_size, 1, W)
    elif cache_dtype == "bf16":
        cache = _random_bytes(rng, num_layers * P * page_size * W * 2).view(
            np.uint16).reshape(num_layers, P, page_size, 1, W)
    else:
        raise ValueError(cache_dtype)
    token_scales = None
    if scale_mode == "per_token":
        token_scales = _random_bytes(rng, num_layers * P * page_size * 4).view(
            np.float32).reshape(num_layers, P, page_size, 1)
    return MlaCase(name=name, seed=seed, row_offsets=offsets, cache_lengths=clens,
                   page_table=pt, q=q, latent=latent, gamma=gamma, freqs=freqs,
                   epsilon=float(np.float32(eps)), cache=cache, layer_idx=layer_idx,
                   scale_mode=scale_mode, tensor_scale=float(np.float32(tensor_scale)),
                   token_scales=token_scales,
                   meta=dict(page_size=page_size, num_pages=P, theta=theta,
                             max_seq_len=max_seq_len, q_sigma=q_sigma,
                             latent_sigma=latent_sigma, outlier_p=outlier_p))


# -- the five named workloads --------------------------------------------------

def mla_tiny(seed: int = 1001) -> MlaCase:
    """Tiny ragged MLA batch: 2 requests, new [5, 11], prior [0, 3], 4 heads,
    freqs [64, 64], page size 16, 8-page shuffled pool, per-tensor scale 1."""
    return build_mla("mla_tiny", seed, [5, 11], [0, 3], H=4, page_size=16,
                     max_seq_len=64, spare_pages=6, scale_mode="per_tensor",
                     tensor_scale=1.0)


def mla_decode(seed: int = 1002) -> MlaCase:
    """DeepSeek-V3-shaped decode: 256 requests x 1 new token, prior lengths
    U{0..8191}, 128 heads, freqs [16384, 64], page size 128, 64 spare pages,
    per-tensor scale 0.05."""
    rng = make_rng(seed)
    prior = rng.integers(0, 8191, size=256, endpoint=True)
    return build_mla("mla_decode", seed, np.ones(256, np.int64), prior, H=128,
                     page_size=128, max_seq_len=16384, spare_pages=64,
                     scale_mode="per_tensor", tensor_scale=0.05, rng=rng)


def mla_prefill(seed: int = 1003) -> MlaCase:
    """DeepSeek-V3-shaped prefill: 8 requests with new lengths U{512..4096},
    prior 0, 128 heads, latent ~N(0, sigma=2), freqs [16384, 64], page size
    128, per-tensor scale 0.05."""
    rng = make_rng(seed)
    new = rng.integers(512, 4096, size=8, endpoint=True)
    return build_mla("mla_prefill", seed, new, np.zeros(8, np.int64), H=128,
                     page_size=128, max_seq_len=16384, spare_pages=16,
                     latent_sigma=2.0, scale_mode="per_tensor", tensor_scale=0.05,
                     rng=rng)


def mla_prefill_f16(seed: int = 1003) -> MlaCase:
    """The prefill batch of :func:`mla_prefill` (same lengths and latent
    draws) with fp16 q (q_rope and q_rope_output), bf16 freqs_cis and fp32
    gamma: the element-type variants the MLA page parameterises."""
    rng = make_rng(seed)
    new = rng.integers(512, 4096, size=8, endpoint=True)
    return build_mla("mla_prefill_f16", seed, new, np.zeros(8, np.int64), H=128,
                     page_size=128, max_seq_len=16384, spare_pages=16,
                     latent_sigma=2.0, scale_mode="per_tensor", tensor_scale=0.05,
                     rng=rng, q_dtype="f16", freq_dtype="bf16", gamma_dtype="f32")


def mla_prefill_inplace(seed: int = 1003) -> MlaCase:
    """The DeepSeek-V3-shaped prefill batch of :func:`mla_prefill` over a bf16
    latent cache, for the in-place form (the rows are placed at their slots
    before the step)."""
    rng = make_rng(seed)
    new = rng.integers(512, 4096, size=8, endpoint=True)
    return build_mla("mla_prefill_inplace", seed, new, np.zeros(8, np.int64), H=128,
                     page_size=128, max_seq_len=16384, spare_pages=16,
                     latent_sigma=2.0, scale_mode="none", cache_dtype="bf16", rng=rng)


def mla_mixed(seed: int = 1004) -> MlaCase:
    """Mixed ragged batch: 64 decode rows (prior U{0..32767}) then 4 prefill
    requests of 2048 tokens; 16 heads (128 heads split 8 ways); inputs ~N(0,1)
    with each element x50 with probability 1%; page size 64; freqs
    [32768, 64]; per-token dynamic scale amax/448 stored as fp32."""
    rng = make_rng(seed)
    prior = np.concatenate([rng.integers(0, 32767, size=64, endpoint=True),
                            np.zeros(4, np.int64)])
    new = np.concatenate([np.ones(64, np.int64), np.full(4, 2048, np.int64)])
    return build_mla("mla_mixed", seed, new, prior, H=16, page_size=64,
                     max_seq_len=32768, spare_pages=64, outlier_p=0.01,
                     scale_mode="per_token", rng=rng)


@dataclass
class QkCase:
    """Inputs of one paged-ragged Q/K RoPE call (host arrays)."""

    name: str
    seed: int
    row_offsets: np.ndarray      # u32 [B+1]
    cache_lengths: np.ndarray    # u32 [B]
    page_table: np.ndarray       # u32 [B, stride]
    q: np.ndarray                # bf16 bits [T, Hq, D]
    k_cache: np.ndarray          # bf16 bits [L, P, S, Hkv, D]
    freqs: np.ndarray            # f32 [max_seq_len, D]
    position_ids: np.ndarray | None  # u32 [T]
    interleaved: bool
    gamma: np.ndarray | None     # bf16 bits [C]
    epsilon: float
    layer_idx: int
    meta: dict = field(default_factory=dict)
    k_scale_mode: str = "none"   # fp8 K cache: "per_tensor" | "per_token"
    k_scales: np.ndarray | None = None  # f32 [1] or [L, P, S, Hkv]
    mrope_section: tuple | None = None  # (temporal, height, width) pair counts

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def B(self) -> int:
        return int(self.row_offsets.size - 1)


def fp8_codes(x: np.ndarray) -> np.ndarray:
    """E4M3FN codes of float32 values by torch's cast (inputs within +-448)."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def build_qk(name, seed, new_lens, prior_lens, Hq, Hkv, D, *, page_size,
             max_seq_len, theta, interleaved, with_position_ids,
             norm_cols=None, eps=1e-6, spare_pages=64, num_layers=2, layer_idx=1,
             rng=None, k_dtype="bf16", k_scale_mode="per_tensor", k_scale=0.05,
             mrope_section=None, q_dtype="bf16", freq_dtype="f32"):
    """Generic Q/K RoPE case; ``rng`` continues a preset's stream if given.
    k_dtype "fp8": the K pool holds E4M3FN codes of N(0,1) values divided by
    the scale -- one tensor scale, or per (slot, head) scales ~U(0.5, 1.5) x
    k_scale (k_scale_mode "per_token").  q_dtype ("bf16" | "f16") and
    freq_dtype ("f32" | "bf16" | "f16") pick the element types of Q and of
    freqs_cis."""
    rng = make_rng(seed) if rng is None else rng
    offsets, clens, pt, P = ragged_batch(new_lens, prior_lens, page_size,
                                         spare_pages, rng)
    T = int(offsets[-1])
    q = _normal_bf16(rng, (T, Hq, D), dtype=q_dtype)
    # The whole pool holds N(0,1) bf16 values, so the new K rows (written by a
    # preceding projection) are normal draws wherever they sit, and every other
    # slot is a finite value whose bits must survive the call unchanged.
    k_shape = (num_layers, P, page_size, Hkv, D)
    k_scales = None
    if k_dtype == "bf16":
        k_cache = _normal_bf16(rng, k_shape)
        k_scale_mode = "none"
    else:
        x = rng.standard_normal(size=k_shape, dtype=np.float32)
        if k_scale_mode == "per_token":
            k_scales = (rng.uniform(0.5, 1.5, size=k_shape[:4]) * k_scale).astype(np.float32)
            k_cache = fp8_codes(x / k_scales[..., None])
        else:
            k_scales = np.array([k_scale], np.float32)
            k_cache = fp8_codes(x / k_scales[0])
    freqs = freqs_table(max_seq_len, D, theta, freq_dtype)
    pos = None
    if mrope_section is not None:
        pos = rng.integers(0, max_seq_len - 1, size=(3, T), endpoint=True).astype(np.uint32)
    elif with_position_ids:
        pos = rng.integers(0, max_seq_len - 1, size=T, endpoint=True).astype(np.uint32)
    gamma = None
    if norm_cols is not None:
        gamma = _uniform_bf16(rng, (norm_cols,), 0.5, 1.5)
    return QkCase(name=name, seed=seed, row_offsets=offsets, cache_lengths=clens,
                  page_table=pt, q=q, k_cache=k_cache, freqs=freqs,
                  position_ids=pos, interleaved=interleaved, gamma=gamma,
                  epsilon=float(np.float32(eps)), layer_idx=layer_idx,
                  meta=dict(page_size=page_size, num_pages=P, theta=theta,
                            max_seq_len=max_seq_len),
                  k_scale_mode=k_scale_mode, k_scales=k_scales,
                  mrope_section=None if mrope_section is None else tuple(mrope_section))


def qk_generic(seed: int = 1005) -> QkCase:
    """Llama-style paged-ragged Q/K RoPE: 32 requests with new lengths
    U{1..1024} and prior lengths U{0..1023}; Q [T, 32, 128]; K cache with 8 KV
    heads x 128, page size 16; interleaved RoPE with random position ids below
    131072 and theta 5e5; per-head K RMSNorm over all 128 columns with gamma
    ~U(0.5, 1.5)."""
    rng = make_rng(seed)
    new = rng.integers(1, 1024, size=32, endpoint=True)
    prior = rng.integers(0, 1023, size=32, endpoint=True)
    return build_qk("qk_generic", seed, new, prior, Hq=32, Hkv=8, D=128,
                    page_size=16, max_seq_len=131072, theta=500000.0,
                    interleaved=True, with_position_ids=True, norm_cols=128,
                    rng=rng)


def qk_generic_f16(seed: int = 1005) -> QkCase:
    """The Llama-style batch of :func:`qk_generic` (same lengths, positions and
    K pool) with fp16 Q and bf16 freqs_cis."""
    rng = make_rng(seed)
    new = rng.integers(1, 1024, size=32, endpoint=True)
    prior = rng.integers(0, 1023, size=32, endpoint=True)
    return build_qk("qk_generic_f16", seed, new, prior, Hq=32, Hkv=8, D=128,
                    page_size=16, max_seq_len=131072, theta=500000.0,
                    interleaved=True, with_position_ids=True, norm_cols=128,
                    rng=rng, q_dtype="f16", freq_dtype="bf16")


NAMED = {
    "mla_tiny": mla_tiny,
    "mla_decode": mla_decode,
    "mla_prefill": mla_prefill,
    "mla_mixed": mla_mixed,
    "mla_prefill_inplace": mla_prefill_inplace,
    "mla_prefill_f16": mla_prefill_f16,
    "qk_generic": qk_generic,
    "qk_generic_f16": qk_generic_f16,
}
