"""Seeded synthetic inputs for the Palu decode-attention workloads.

This module is shared by the fp64 oracle side (tests, CPU baseline) and the
HIP side (tests, bench, smoke).  It only draws random numbers and converts
them to the stored number formats; it holds none of the method's arithmetic
(no projection, reconstruction, RoPE, softmax or quantisation).

Workloads follow the shapes named for the method's hot path: a tiny fp32
layer, a Llama-2-7B-shaped layer, long-context ragged batches, a GQA
Llama-3-8B-shaped layer pair (RoPE / no-RoPE) and an int4 layer with its
prefill chunk.  Distributions (the pages give none; one plain reading):

* factor matrices A (d_model x r) and B (r x w) are Gaussian with standard
  deviation 1/sqrt(fan_in) (fan_in = d_model for A, r for B);
* the cached latents z = x.A are drawn directly as N(0, 1): with x ~ N(0, 1)
  and A as above every entry of x.A is a sum of d_model products with
  variance 1/d_model each, so N(0, 1) is its distribution; drawing it
  directly keeps multi-terabyte-flop fp64 projections out of the test budget;
* queries q ~ N(0, 1); prefill activations x ~ N(0, 1);
* stored int4 latents (the decode's input for 'i4' workloads) are drawn as
  codes and scales directly: codes binomial(14, 1/2) - 7 (integers in
  [-7, 7] peaked at 0, the shape that quantising normal rows to amax/7
  steps gives), one binary16 scale per 32 elements uniform in [0.28, 0.45]
  (amax/7 of 32 standard normal draws lies there in most chunks); pad
  nibbles past the rank are zero.  Packing them into the documented byte
  layout is data placement, not quantisation.

Every array comes from its own counter-style stream
``PCG64(SeedSequence([seed, stream_tag, *indices]))`` so that any (sequence,
group) block can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "scaled",
    "to_f16", "to_bf16_bits", "to_format",
    "ranks", "lengths", "factor", "latent", "latent_f32", "latent_int4", "query", "query_chunk", "prefill_x",
    "prefill_A",
]

# stream tags (stable: changing them changes every generated array)
_T_RANK, _T_LEN, _T_BK, _T_BV, _T_AK, _T_AV, _T_ZK, _T_ZV, _T_Q, _T_X, _T_QK4, _T_QV4, _T_QC = range(1, 14)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_groups: int
    max_len: int
    latent: str            # 'f32' | 'f16' | 'bf16' | 'i4'
    act: str               # 'f32' | 'f16' | 'bf16'  (q, B_k, B_v, out)
    use_rope: bool = True
    rope_base: float = 10000.0
    rank: Optional[int] = None                 # uniform rank per group
    rank_choices: Optional[Sequence[int]] = None  # per-group rank drawn from this set
    ragged: bool = False   # lengths ~ U[max_len/2, max_len] (inclusive)
    fixed_lengths: Optional[Sequence[int]] = None
    layer: int = 0         # selects independent factor / latent streams
    n_tok: int = 0         # prefill chunk length (palu_project workloads)

    @property
    def kv_per_group(self) -> int:
        return self.n_kv_heads // self.n_groups

    @property
    def group_width(self) -> int:
        return self.kv_per_group * self.head_dim

    @property
    def q_per_kv(self) -> int:
        return self.n_q_heads // self.n_kv_heads


WORKLOADS: Dict[str, Workload] = {
    # 1 layer, batch 1, d_model 512, 8 heads of 64, 2 groups of 4 heads, rank 128, L 512, fp32
    "tiny": Workload("tiny", 1, 1, 512, 8, 8, 64, 2, 512, "f32", "f32", rank=128),
    # Llama-2-7B-shaped layer: 32 heads of 128, 8 groups of 4, rank 256, batch 16, L 4096, fp16
    "llama2_7b": Workload("llama2_7b", 2, 16, 4096, 32, 32, 128, 8, 4096, "f16", "f16", rank=256),
    # long context, ragged lengths in [L/2, L], bf16
    "long_b1": Workload("long_b1", 3, 1, 4096, 32, 32, 128, 8, 65536, "bf16", "bf16", rank=256,
                        ragged=True),
    "long_b4": Workload("long_b4", 3, 4, 4096, 32, 32, 128, 8, 32768, "bf16", "bf16", rank=256,
                        ragged=True, layer=1),
    # GQA Llama-3-8B-shaped layer pair: 32 q heads over 8 kv heads, groups of 2 kv heads,
    # per-group ranks from {128, 192, 256, 320}; layer 0 with RoPE, layer 1 without
    "gqa_rope": Workload("gqa_rope", 4, 32, 4096, 32, 8, 128, 4, 8192, "bf16", "bf16",
                         rank_choices=(128, 192, 256, 320), layer=0),
    "gqa_norope": Workload("gqa_norope", 4, 32, 4096, 32, 8, 128, 4, 8192, "bf16", "bf16",
                           use_rope=False, rank_choices=(128, 192, 256, 320), layer=1),
    # int4 latents (one fp16 scale per 32 elements per token), rank 154, batch 8, L 16384
    "int4": Workload("int4", 5, 8, 4096, 32, 32, 128, 8, 16384, "i4", "f16", rank=154),
    # prefill chunk for palu_project: 8192 tokens x 4096, bf16, writes int4 latents of rank 154
    "int4_prefill": Workload("int4_prefill", 5, 1, 4096, 32, 32, 128, 8, 8192, "i4", "bf16",
                             rank=154, n_tok=8192, layer=2),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(base: str | Workload, **over) -> Workload:
    """A smaller (or otherwise modified) copy of a workload, e.g. for parity
    tests that must finish in seconds: ``scaled('llama2_7b', batch=2, max_len=300)``."""
    wl = WORKLOADS[base] if isinstance(base, str) else base
    over.setdefault("name", wl.name + "_scaled")
    return dataclasses.replace(wl, **over)


# ---------------------------------------------------------------- formats
def to_f16(x: np.ndarray) -> np.ndarray:
    """fp32 -> IEEE binary16, round to nearest even."""
    return np.asarray(x, dtype=np.float32).astype(np.float16)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest even.
    Inputs here are finite draws, so NaN handling is not needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def to_format(x: np.ndarray, fmt: str) -> np.ndarray:
    """Round fp32 draws to a stored format: 'f32' float32, 'f16' float16,
    'bf16' uint16 bit patterns.  ('i4' latents stay fp32; quantising them is
    part of the method and is done by the consumer.)"""
    if fmt in ("f32", "i4"):
        return np.ascontiguousarray(x, dtype=np.float32)
    if fmt == "f16":
        return to_f16(x)
    if fmt == "bf16":
        return to_bf16_bits(x)
    raise ValueError(fmt)


def _rng(wl: Workload, tag: int, *idx: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, tag, wl.layer, *idx])))


# ---------------------------------------------------------------- draws
def ranks(wl: Workload) -> np.ndarray:
    """Rank of each head-group (same rank for keys and values)."""
    if wl.rank is not None:
        return np.full(wl.n_groups, wl.rank, dtype=np.int32)
    choices = np.asarray(wl.rank_choices, dtype=np.int32)
    return choices[_rng(wl, _T_RANK).integers(0, len(choices), size=wl.n_groups)]


def lengths(wl: Workload) -> np.ndarray:
    """Per-sequence history lengths (int32)."""
    if wl.fixed_lengths is not None:
        return np.asarray(wl.fixed_lengths, dtype=np.int32)
    if not wl.ragged:
        return np.full(wl.batch, wl.max_len, dtype=np.int32)
    lo = wl.max_len // 2
    return _rng(wl, _T_LEN).integers(lo, wl.max_len, size=wl.batch, endpoint=True).astype(np.int32)


def factor(wl: Workload, which: str, g: int) -> np.ndarray:
    """Factor matrix of group g in the activation format.
    which: 'Bk' / 'Bv' -> [r_g][w] (std 1/sqrt(r_g));
           'Ak' / 'Av' -> [d_model][r_g] (std 1/sqrt(d_model))."""
    r = int(ranks(wl)[g])
    tag = {"Bk": _T_BK, "Bv": _T_BV, "Ak": _T_AK, "Av": _T_AV}[which]
    if which in ("Bk", "Bv"):
        shape, fan_in = (r, wl.group_width), r
    else:
        shape, fan_in = (wl.d_model, r), wl.d_model
    x = _rng(wl, tag, g).standard_normal(shape, dtype=np.float32) * np.float32(1.0 / np.sqrt(fan_in))
    return to_format(x, wl.act)


def latent_f32(wl: Workload, which: str, b: int, g: int, n: Optional[int] = None) -> np.ndarray:
    """fp32 N(0,1) draws for the cached latent of (sequence b, group g):
    [n][r_g] with n = max_len by default (rows past the sequence length are
    valid memory that the method never reads)."""
    r = int(ranks(wl)[g])
    n = wl.max_len if n is None else n
    tag = _T_ZK if which == "k" else _T_ZV
    return _rng(wl, tag, b, g).standard_normal((n, r), dtype=np.float32)


def latent(wl: Workload, which: str, b: int, g: int, n: Optional[int] = None) -> np.ndarray:
    """Cached latent of (b, g) in its stored format ('i4' workloads return the
    fp32 values that are to be quantised)."""
    return to_format(latent_f32(wl, which, b, g, n), wl.latent)


def latent_int4(wl: Workload, which: str, b: int, g: int, n: Optional[int] = None):
    """Stored int4 latent of (sequence b, group g): (codes, scales) with codes
    uint8 [n][16 * ceil(r_g/32)] (4-bit two's complement, element 2i in the
    low nibble of byte i, zero nibbles past the rank) and scales float16
    [n][ceil(r_g/32)]; n = max_len by default.  Drawn directly (no
    quantisation): see the module docstring."""
    r = int(ranks(wl)[g])
    n = wl.max_len if n is None else n
    nc = (r + 31) // 32
    rng = _rng(wl, _T_QK4 if which == "k" else _T_QV4, b, g)
    codes = rng.binomial(14, 0.5, size=(n, r)).astype(np.int16) - 7
    scales = to_f16(rng.uniform(0.28, 0.45, size=(n, nc)).astype(np.float32))
    nib = np.zeros((n, 32 * nc), dtype=np.uint8)
    nib[:, :r] = (codes & 0xF).astype(np.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales


def query(wl: Workload) -> np.ndarray:
    """Decode queries [batch][n_q_heads][head_dim] in the activation format."""
    x = _rng(wl, _T_Q).standard_normal((wl.batch, wl.n_q_heads, wl.head_dim), dtype=np.float32)
    return to_format(x, wl.act)


def query_chunk(wl: Workload, q_len: int) -> np.ndarray:
    """Queries of a chunk of q_len tokens per sequence [batch][q_len][n_q_heads][head_dim]."""
    x = _rng(wl, _T_QC, q_len).standard_normal((wl.batch, q_len, wl.n_q_heads, wl.head_dim), dtype=np.float32)
    return to_format(x, wl.act)


def prefill_x(wl: Workload, n_tok: Optional[int] = None) -> np.ndarray:
    """Prefill activations [n_tok][d_model] in the activation format."""
    n = wl.n_tok if n_tok is None else n_tok
    x = _rng(wl, _T_X).standard_normal((n, wl.d_model), dtype=np.float32)
    return to_format(x, wl.act)


def prefill_A(wl: Workload) -> List[np.ndarray]:
    """[A_k^0 .. A_k^{G-1}, A_v^0 .. A_v^{G-1}], each [d_model][r_g]."""
    return [factor(wl, "Ak", g) for g in range(wl.n_groups)] + \
           [factor(wl, "Av", g) for g in range(wl.n_groups)]
