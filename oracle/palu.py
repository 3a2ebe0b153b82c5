"""fp64 CPU oracle for Palu decode attention over a low-rank latent KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product imports this module; only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP library.

Sources (the method's pages; section names are English glosses):

* "Palu low-rank projection explainer", section "Low-rank projection
  decomposition", formula block: W_k ~ A_k B_k, W_v ~ A_v B_v with
  A in R^{d_model x r}, B in R^{r x d}; the cache holds z_k = x A_k and
  z_v = x A_v; keys and values are rebuilt as K = z_k B_k, V = z_v B_v.
* same page, section "Inference flow": prefill stores the latents (steps 3-4);
  a decode step reads the latents, rebuilds K/V through B (or fuses the
  rebuild into the attention kernel) and attends over the history (steps 1-3).
* "Palu: Compressing KV-Cache with Low-Rank Projection" abstract
  (arXiv 2407.21118v2): keys and values are reconstructed on the fly; the
  speedups are reported on RoPE-based attention; quantization composes.

What is computed here is the plain definition: rebuild full K and V in fp64,
apply RoPE to the rebuilt keys and to the query, run naive softmax attention.
Fusion on the GPU is a speed claim only and must not change this result.

Readings where the pages are silent:

* RoPE: theta_i = base^(-2i/d_h), i < d_h/2, pairs (i, i + d_h/2)
  ("half-split"); keys rotate by their cache index t, the query by its
  position p (default: history length - 1).
* score scale: sm_scale passed explicitly (1/sqrt(d_h) by default).
* GQA: query head h reads kv head h // (H / H_kv); head-group j holds the
  contiguous kv heads [j*n_g, (j+1)*n_g); B^j has n_g*d_h columns, head-major.
* empty history: output is zero.
* int4 latents: symmetric, one fp16 scale per 32 consecutive elements of a
  token's latent row; s32 = amax/7 (fp32 divide), s16 = fp16(s32) (RNE),
  q = clamp(rint(z / s16), -7, 7) in fp32 with ties to even, q = 0 when
  s16 == 0; the last chunk of a row whose rank is not a multiple of 32 is
  short; codes are 4-bit two's complement, element 2i in the low nibble of
  byte i, rows padded with zero nibbles to a 16-byte multiple.
* int4 decode: the attention consumes the dequantised latent
  z_hat = code * scale exactly (a 4-bit integer times a binary16 scale has at
  most 14 significant bits, so the product is exact in fp64 and in fp32);
  everything after that is the plain definition above.  The 16-bit rows of
  the library's stand-alone expansion call are that product rounded once, to
  nearest even, into fp16 or bf16 (int4_rows16); the decode never reads
  them.

* low-rank-aware int4 (rotated chunks): before quantisation every full
  32-element chunk of a latent row is rotated by the Sylvester Hadamard
  matrix H (entries +-1, H H^T = 32 I): z' = z H; a trailing partial chunk
  is left as is.  The rotation is folded into the factors, A' = A H and
  B' = H B / 32, so that z' B' = z B and the decode is the plain definition
  over z' and B'.  The quantiser decides codes on z' formed in binary32 by
  the fast Walsh-Hadamard butterflies (stages h = 1, 2, 4, 8, 16; pairs
  (i, i + h) become (a + b, a - b)), the precision the kernel uses.

Pins (tests/test_oracle_pins.py): standard attention through
torch.nn.functional.scaled_dot_product_attention (float64, CPU) in the
identity case A = W, B = I; the absorbed-query and fused-value forms for
no-RoPE heads; an mpmath scalar brute force on tiny shapes; RoPE as complex
multiplication and its group laws; closed forms of softmax attention;
split-history merges; int4 bounds and hand-worked codes; the golden fixtures
under tests/golden/.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "upcast", "rope_theta", "rope", "reconstruct", "attend", "attend_partial", "merge_partials",
    "decode_attention", "project", "quant_int4", "pack_int4", "unpack_int4", "dequant_int4",
    "chunks_per_row", "round_to", "int4_latent", "int4_rows16", "chunk_attention",
    "hadamard", "rotate_chunks", "rotate_chunks_f32", "fold_rotation", "quant_int4_rotated",
]

QUANT_GROUP = 32


# ------------------------------------------------------------------ formats
def upcast(a: np.ndarray, fmt: str) -> np.ndarray:
    """Exact widening of a stored array to fp64.  'bf16' arrays are uint16 bit
    patterns (the upper half of an IEEE binary32)."""
    if fmt == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(a).astype(np.float64)


_SIG_BITS = {"f16": 11, "bf16": 8}


def round_to(x: np.ndarray, fmt: str) -> np.ndarray:
    """Round fp64 values to nearest (ties to even) at the precision of 'f16'
    or 'bf16', returned in fp64.  Written from the definition: with
    x = m * 2^e (0.5 <= |m| < 1), keep rint(m * 2^p) * 2^(e - p) for p
    significant bits; below the smallest normal (binary16: 2^-14) the
    quantum stays that of the smallest binade (2^-24), as IEEE gradual
    underflow has it.  Values that would overflow are rejected (none occur
    here); bf16 is only used in its normal range."""
    x = np.asarray(x, dtype=np.float64)
    p = _SIG_BITS[fmt]
    nz = x != 0
    if fmt == "f16":
        assert np.all(np.abs(x) <= 65504.0), "round_to: binary16 overflow"
    else:
        assert np.all(np.abs(x[nz]) >= 2.0 ** -126) and np.all(np.abs(x) <= 3.0e38), "round_to: outside bf16 normals"
    m, e = np.frexp(x)
    if fmt == "f16":
        e = np.maximum(e, -13)          # x = m' * 2^-13 with |m'| < 0.5 below 2^-14
        m = np.ldexp(x, -e)
    return np.ldexp(np.rint(np.ldexp(m, p)), e - p)


def int4_latent(packed: np.ndarray, scales: np.ndarray, r: int) -> np.ndarray:
    """Latent rows a decode step attends over when the cache holds int4
    codes: unpack, then z_hat = code * scale, exact in fp64 (the reading
    stated in the module docstring)."""
    return dequant_int4(unpack_int4(packed, r), scales)


def int4_rows16(packed: np.ndarray, scales: np.ndarray, r: int, fmt: str) -> np.ndarray:
    """16-bit rows of the stand-alone int4 expansion: the exact z_hat rounded
    once, to nearest even, into fmt ('f16' or 'bf16')."""
    return round_to(int4_latent(packed, scales, r), fmt)


# ------------------------------------------------------------------ RoPE
def rope_theta(head_dim: int, base: float) -> np.ndarray:
    """Rotation frequencies theta_i = base^(-2i/d_h), i = 0 .. d_h/2 - 1 (fp64)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return base ** (-2.0 * i / head_dim)


def rope(u: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate the half-split pairs (u_i, u_{i+d/2}) of the last axis by pos*theta_i.
    ``pos`` broadcasts against u's leading axes."""
    d = u.shape[-1]
    h = d // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_theta(d, base)
    c, s = np.cos(ang), np.sin(ang)
    x, y = u[..., :h], u[..., h:]
    return np.concatenate([x * c - y * s, x * s + y * c], axis=-1)


# ------------------------------------------------------------------ core steps
def reconstruct(z: np.ndarray, B: np.ndarray) -> np.ndarray:
    """K = z_k B_k (or V = z_v B_v): rebuild full rows from the cached latents."""
    return z @ B


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """Naive softmax attention of one query over all L rows of K/V."""
    s = sm_scale * (K @ q)
    p = np.exp(s - s.max())
    p /= p.sum()
    return p @ V


def attend_partial(q, K, V, sm_scale) -> Tuple[float, float, np.ndarray]:
    """Unnormalised attention over a slice of the history: (m, l, acc) with
    m = max score, l = sum exp(s - m), acc = sum exp(s - m) V.  Used to state
    what split-history partial results mean."""
    s = sm_scale * (K @ q)
    m = float(s.max())
    p = np.exp(s - m)
    return m, float(p.sum()), p @ V


def merge_partials(parts: Sequence[Tuple[float, float, np.ndarray]]) -> np.ndarray:
    """Combine partials of disjoint history slices into the attention output."""
    m = max(p[0] for p in parts)
    l = sum(p[1] * math.exp(p[0] - m) for p in parts)
    acc = sum(p[2] * math.exp(p[0] - m) for p in parts)
    return acc / l


def decode_attention(q: np.ndarray, zk: Sequence[np.ndarray], zv: Sequence[np.ndarray],
                     Bk: Sequence[np.ndarray], Bv: Sequence[np.ndarray],
                     seq_lens: Sequence[int], q_pos: Optional[Sequence[int]] = None, *,
                     n_kv_heads: int, use_rope: bool = True, rope_base: float = 10000.0,
                     sm_scale: Optional[float] = None,
                     heads: Optional[Sequence[Tuple[int, int]]] = None) -> np.ndarray:
    """One decode step over the latent cache, all in fp64.

    q      [batch][H][d_h]
    zk[j]  [batch][>= L_b][r_k,j]   cached key latents of head-group j
    zv[j]  [batch][>= L_b][r_v,j]
    Bk[j]  [r_k,j][n_g*d_h], Bv[j] [r_v,j][n_g*d_h]
    returns out [batch][H][d_h] (fp64).  ``heads``: optional list of (b, h)
    pairs; only those outputs are computed (others stay zero).
    """
    q = np.asarray(q, dtype=np.float64)
    batch, H, d_h = q.shape
    G = len(Bk)
    n_g = n_kv_heads // G
    q_per_kv = H // n_kv_heads
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d_h)
    out = np.zeros((batch, H, d_h))
    wanted = None if heads is None else {(int(b), int(h)) for b, h in heads}
    for b in range(batch):
        L = int(seq_lens[b])
        if L == 0:
            continue
        p = L - 1 if q_pos is None else int(q_pos[b])
        for j in range(G):
            hs = [h for h in range(H) if (h // q_per_kv) // n_g == j
                  and (wanted is None or (b, h) in wanted)]
            if not hs:
                continue
            K = reconstruct(np.asarray(zk[j][b][:L], dtype=np.float64), np.asarray(Bk[j], dtype=np.float64))
            V = reconstruct(np.asarray(zv[j][b][:L], dtype=np.float64), np.asarray(Bv[j], dtype=np.float64))
            for h in hs:
                c = (h // q_per_kv) % n_g
                Kc = K[:, c * d_h:(c + 1) * d_h]
                Vc = V[:, c * d_h:(c + 1) * d_h]
                qh = q[b, h]
                if use_rope:
                    Kc = rope(Kc, np.arange(L), rope_base)
                    qh = rope(qh, p, rope_base)
                out[b, h] = attend(qh, Kc, Vc, sm_scale)
    return out


# ------------------------------------------------------------------ prefill
def chunk_attention(q: np.ndarray, zk, zv, Bk, Bv, seq_lens: Sequence[int], *, n_kv_heads: int,
                    use_rope: bool = True, rope_base: float = 10000.0,
                    sm_scale: Optional[float] = None) -> np.ndarray:
    """Attention of a chunk of q_len new tokens per sequence, causal within
    the chunk (reading of the pages' prefill/decode flow for several new
    tokens: every new token attends to the history up to and including
    itself).  q [batch][q_len][H][d_h]; the chunk's latents are the last
    q_len of the L_b cached rows, so query i sits at p = L_b - q_len + i and
    sees rows 0..p; p < 0 gives zeros.  Returns [batch][q_len][H][d_h]."""
    q = np.asarray(q, dtype=np.float64)
    batch, q_len = q.shape[:2]
    out = np.zeros(q.shape)
    for i in range(q_len):
        pos = [int(seq_lens[b]) - q_len + i for b in range(batch)]
        lens = [p + 1 if p >= 0 else 0 for p in pos]
        out[:, i] = decode_attention(q[:, i], zk, zv, Bk, Bv, lens, [max(p, 0) for p in pos], n_kv_heads=n_kv_heads,
                                     use_rope=use_rope, rope_base=rope_base, sm_scale=sm_scale)
    return out


def project(x: np.ndarray, A: np.ndarray) -> np.ndarray:
    """Prefill latents z = x A (fp64)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(A, dtype=np.float64)


# ------------------------------------------------------------------ int4
def chunks_per_row(r: int) -> int:
    return -(-r // QUANT_GROUP)


def quant_int4(z: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric int4 quantisation of rows of fp32 latents.

    z [..., r] (converted to fp32 first).  Returns (codes int8 [..., r],
    scales float16 [..., ceil(r/32)]).  All arithmetic in fp32, as read above.
    """
    z = np.asarray(z, dtype=np.float32)
    r = z.shape[-1]
    nc = chunks_per_row(r)
    codes = np.zeros(z.shape, dtype=np.int8)
    scales = np.zeros(z.shape[:-1] + (nc,), dtype=np.float16)
    for c in range(nc):
        seg = z[..., c * QUANT_GROUP:min(r, (c + 1) * QUANT_GROUP)]
        amax = np.abs(seg).max(axis=-1)
        s32 = (amax / np.float32(7.0)).astype(np.float32)
        s16 = s32.astype(np.float16)
        sf = s16.astype(np.float32)[..., None]
        with np.errstate(divide="ignore", invalid="ignore"):
            qf = np.where(sf == 0, np.float32(0), np.rint(seg / np.where(sf == 0, np.float32(1), sf)))
        codes[..., c * QUANT_GROUP:min(r, (c + 1) * QUANT_GROUP)] = np.clip(qf, -7, 7).astype(np.int8)
        scales[..., c] = s16
    return codes, scales


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """int8 codes [..., r] -> bytes [..., 16*ceil(r/32)]; element 2i in the low
    nibble of byte i, 4-bit two's complement, zero padding."""
    r = codes.shape[-1]
    nbytes = 16 * chunks_per_row(r)
    padded = np.zeros(codes.shape[:-1] + (2 * nbytes,), dtype=np.int16)
    padded[..., :r] = codes
    nib = (padded & 0xF).astype(np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray, r: int) -> np.ndarray:
    """Inverse of pack_int4: bytes -> int8 codes [..., r]."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    nib = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int16)
    nib[..., 0::2] = lo
    nib[..., 1::2] = hi
    nib = np.where(nib >= 8, nib - 16, nib)
    return nib[..., :r].astype(np.int8)


def dequant_int4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """z_hat = q * s per 32-element chunk, exact in fp64 (and in fp32)."""
    codes = np.asarray(codes)
    r = codes.shape[-1]
    s = np.repeat(np.asarray(scales, dtype=np.float64), QUANT_GROUP, axis=-1)[..., :r]
    return codes.astype(np.float64) * s


# ------------------------------------------------------------------ low-rank-aware int4 (rotated chunks)
def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), entries +-1:
    H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]."""
    assert n >= 1 and n & (n - 1) == 0, "order must be a power of two"
    H = np.ones((1, 1))
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def _full_chunks(r: int) -> int:
    return r // QUANT_GROUP


def rotate_chunks(z: np.ndarray) -> np.ndarray:
    """z' = z H on every full 32-element chunk of the last axis (a trailing
    partial chunk is left as is), in fp64."""
    z = np.asarray(z, dtype=np.float64)
    out = z.copy()
    H = hadamard(QUANT_GROUP)
    for c in range(_full_chunks(z.shape[-1])):
        sl = slice(c * QUANT_GROUP, (c + 1) * QUANT_GROUP)
        out[..., sl] = z[..., sl] @ H
    return out


def rotate_chunks_f32(z: np.ndarray) -> np.ndarray:
    """The same rotation formed in binary32 by the fast Walsh-Hadamard
    butterflies: for h = 1, 2, 4, 8, 16, within blocks of 2h elements the pair
    (i, i + h) becomes (a + b, a - b), every sum rounded to binary32."""
    x = np.array(z, dtype=np.float32)
    for c in range(_full_chunks(x.shape[-1])):
        base = c * QUANT_GROUP
        h = 1
        while h < QUANT_GROUP:
            for start in range(base, base + QUANT_GROUP, 2 * h):
                a = x[..., start:start + h].copy()
                b = x[..., start + h:start + 2 * h].copy()
                x[..., start:start + h] = a + b
                x[..., start + h:start + 2 * h] = a - b
            h *= 2
    return x


def fold_rotation(A: np.ndarray, B: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Factors for rotated latents: A' = A Hbd, B' = Hbd B / 32 (Hbd: H on
    each full 32-row block, identity on a trailing partial block), so that
    (x A') B' = x A B; fp64."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    r = A.shape[1]
    assert B.shape[0] == r
    H = hadamard(QUANT_GROUP)
    A2, B2 = A.copy(), B.copy()
    for c in range(_full_chunks(r)):
        sl = slice(c * QUANT_GROUP, (c + 1) * QUANT_GROUP)
        A2[:, sl] = A[:, sl] @ H
        B2[sl] = H @ B[sl] / QUANT_GROUP
    return A2, B2


def quant_int4_rotated(z: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Low-rank-aware int4: rotate the full chunks in binary32, then the
    plain symmetric int4 quantisation of the rotated row."""
    return quant_int4(rotate_chunks_f32(z))
