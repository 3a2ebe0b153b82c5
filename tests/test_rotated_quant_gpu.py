"""GPU: the low-rank-aware int4 variant (rotated chunks) through the C ABI.

palu_quant_latent_rotated against the oracle's quant_int4_rotated: codes and
scales bit for bit (the butterflies are binary32 on both sides, in the same
order), on fp32 / fp16 / bf16 rows, with and without a partial last chunk,
exact ties, zero and one-hot rows.  End to end: latents with unequal channel
energy are quantised rotated on the GPU, palu_decode_attn attends over the
int4 cache with the folded factors B' = H B / 32, and the result matches the
oracle's decode over the exact dequantised rotated latents with the same B'.
"""
import math

import numpy as np
import pytest

import oracle
import palu_inputs as PI
from palu_cases import compare, from_device, to_device
from rank_decode_attention_amd import factorize as F

pytestmark = pytest.mark.gpu


def _rows(fmt, n_rows, r, seed):
    rng = np.random.default_rng(seed)
    # channel std decaying along the rank (latents of an SVD-style factorisation)
    z = rng.standard_normal((n_rows, r)).astype(np.float32) * np.exp(-np.arange(r) / 40.0).astype(np.float32)
    z[0] = 0.0
    if n_rows > 1:
        z[1] = 0.0
        z[1, min(5, r - 1)] = 8.0                      # one-hot: rotates to +-8 everywhere in the chunk
    if n_rows > 2:
        z[2] = np.round(z[2] * 4) / 4                  # quarter-integers: many exact ties
    return PI.to_format(z, fmt)


def _quant_gpu(stored, fmt, r, stride, rotated=True, off=0):
    import torch
    import rank_decode_attention_amd as R
    n = stored.shape[0]
    flat = np.zeros(n * stride + off, dtype=stored.dtype)
    for i in range(n):
        flat[off + i * stride: off + i * stride + r] = stored[i]
    z = to_device(flat, fmt)[off:off + n * stride].view(n, stride)
    nc = oracle.chunks_per_row(r)
    codes = torch.full((n, 16 * nc), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((n, nc), -1, dtype=torch.int16, device="cuda")
    fn = R.palu_quant_latent_rotated if rotated else R.palu_quant_latent
    fn(z, r, stride, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("fmt,r,stride,off", [("f32", 154, 160, 0), ("f16", 154, 154, 0), ("bf16", 64, 64, 0),
                                               ("f16", 320, 328, 0), ("bf16", 7, 8, 0), ("f32", 96, 97, 0),
                                               ("bf16", 154, 157, 3), ("f32", 1100, 1100, 1)])
def test_rotated_quant_bit_exact(fmt, r, stride, off):
    """(off: the first row starts that many elements past a 256-byte boundary,
    so lanes' pieces straddle aligned 16-byte blocks; rows over 4 KB put a
    wave's 64 chunks within one or two rows)"""
    stored = _rows(fmt, 1200 if r < 1000 else 300, r, seed=r + stride)
    codes, scales = _quant_gpu(stored, fmt, r, stride, off=off)
    ref_codes, ref_scales = oracle.quant_int4_rotated(oracle.upcast(stored, fmt).astype(np.float32))
    assert np.array_equal(scales, ref_scales.view(np.uint16)), "scales differ"
    ref_packed = oracle.pack_int4(ref_codes)
    assert np.array_equal(codes, ref_packed), f"codes differ in {int((codes != ref_packed).sum())} bytes"
    if r >= 32:
        # the one-hot row: |z H| = 8 everywhere in chunk 0, so scale 8/7 and codes +-7
        assert np.all(np.abs(oracle.unpack_int4(codes[1:2], r)[0, :32]) == 7)


@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_rotated_int4_decode(act):
    """Rotated int4 cache + folded factors through palu_decode_attn (MHA
    head-group kernel, rank 154), against the oracle on the same rotated
    latents and folded factors."""
    import torch
    import rank_decode_attention_amd as R
    batch, L, G, H, d_h, r = 2, 200, 2, 8, 128, 154
    w = 4 * d_h
    lens = [200, 71]
    rng = np.random.default_rng(17)
    decay = np.exp(-np.arange(r) / 40.0)
    zk = [[(rng.standard_normal((L, r)) * decay).astype(np.float32) for _ in range(batch)] for _ in range(G)]
    zv = [[(rng.standard_normal((L, r)) * decay).astype(np.float32) for _ in range(batch)] for _ in range(G)]
    Bk = [rng.standard_normal((r, w)) / math.sqrt(r) / decay[:, None] / 2 for _ in range(G)]
    Bv = [rng.standard_normal((r, w)) / math.sqrt(r) / decay[:, None] / 2 for _ in range(G)]
    dummyA = np.zeros((1, r))
    Bk2 = [F.fold_rotation(dummyA, b)[1] for b in Bk]
    Bv2 = [F.fold_rotation(dummyA, b)[1] for b in Bv]
    for a, b in zip(Bk2 + Bv2, [oracle.fold_rotation(dummyA, b)[1] for b in Bk + Bv]):
        assert np.array_equal(a, b)                    # the library's fold is the oracle's reading
    Bk2 = [PI.to_format(b.astype(np.float32), act) for b in Bk2]
    Bv2 = [PI.to_format(b.astype(np.float32), act) for b in Bv2]
    q = PI.to_format(rng.standard_normal((batch, H, d_h)).astype(np.float32), act)

    desc = R.AttnDesc(H, H, d_h, G, [r] * G, use_rope=True, latent_dtype="i4", act_dtype=act)
    nc = oracle.chunks_per_row(r)
    ref_lat = {}

    def rows(which, b, j):
        z = (zk if which == 0 else zv)[j][b]
        codes, scales = _quant_gpu(PI.to_format(z, "f32"), "f32", r, r)
        ref_lat[(which, b, j)] = oracle.quant_int4_rotated(z)
        return codes[:, :16 * nc], scales.view(np.float16)

    cache = R.fill_cache(desc, batch, L, rows)
    for (which, b, j), (c, s) in ref_lat.items():
        ref_lat[(which, b, j)] = oracle.dequant_int4(c, s)     # exact code * scale of the rotated latents
    cat = lambda Bs: to_device(np.concatenate([m.reshape(-1) for m in Bs]), act)
    ws = torch.empty(R.decode_workspace_bytes(desc, batch, L), dtype=torch.uint8, device="cuda")
    out = torch.empty((batch, H, d_h), dtype=torch.float16 if act == "f16" else torch.bfloat16, device="cuda")
    sm = 1.0 / math.sqrt(d_h)
    R.palu_decode_attn(desc, to_device(q, act), cache, cat(Bk2), cat(Bv2),
                       torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda(), None, sm, out, ws)
    torch.cuda.synchronize()
    up = lambda a: oracle.upcast(a, act)
    zk_or = [[ref_lat[(0, b, j)] for b in range(batch)] for j in range(G)]
    zv_or = [[ref_lat[(1, b, j)] for b in range(batch)] for j in range(G)]
    ref = oracle.decode_attention(up(q), zk_or, zv_or, [up(b) for b in Bk2], [up(b) for b in Bv2], lens,
                                  n_kv_heads=H, use_rope=True, sm_scale=sm)
    compare(from_device(out), ref, act, f"rotated int4 decode {act}")
