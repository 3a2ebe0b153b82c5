"""GPU parity of palu_quant_latent and palu_project against the oracle,
through the C ABI.

palu_quant_latent: bit-exact codes and scales (int4 quantisation is integer
work decided in binary32 on both sides), including chunks that hit exact
rounding ties, all-zero chunks, short last chunks and strided rows.

palu_project: latents z = x A.  With 16-bit or fp32 latents the GPU rounds
its binary32 accumulation once; the oracle rounds the exact fp64 product
once, so they differ only where the binary32 accumulation error moves the
value across a rounding boundary (bar: every element within half an ulp of
the format plus the binary32 accumulation bound of a d_model-term dot
product, and 16-bit results correctly rounded for all but a rare few).  With int4 latents
the quantisation is fused: codes may differ by one step where the binary32
and fp64 values of z straddle a rounding boundary (bar: |dq| <= 1, rare,
and every dequantised value within half a step of the exact z).
"""
import numpy as np
import pytest

import oracle
import palu_inputs as PI
from palu_cases import to_device

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ quantisation
def _quant_rows(fmt: str, n_rows: int, r: int, seed: int) -> np.ndarray:
    """fp32 rows with special chunks: exact ties, zeros, one non-zero, large range."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((n_rows, r), dtype=np.float32) * np.float32(3.0)
    z[0] = 0.0                                        # all-zero row: scale 0, codes 0
    if n_rows > 1:
        z[1] = 0.0
        z[1, min(5, r - 1)] = -2.5                    # one non-zero element per row
    if n_rows > 2 and r >= 4:
        # chunk 0 of row 2: amax 3.5 -> s = 0.5 exactly; k/2 + 1/4 give exact ties
        z[2, :] = 0.0
        ties = np.array([3.5, 0.25, 0.75, 1.25, -0.25, -0.75, -1.25, 1.75], dtype=np.float32)
        z[2, :min(r, 8)] = ties[:min(r, 8)]
    if n_rows > 3:
        z[3] *= np.float32(1e3)                       # large magnitudes (finite in fp16)
    if n_rows > 4:
        z[4] *= np.float32(1e-5)                      # tiny magnitudes (fp16 subnormal scales)
    # round through the stored format so the GPU and the oracle see the same values
    stored = PI.to_format(z, fmt)
    return stored


@pytest.mark.parametrize("fmt,r,stride", [("f32", 154, 160), ("f16", 154, 154), ("bf16", 154, 200),
                                           ("f16", 32, 32), ("f32", 7, 9), ("bf16", 320, 320),
                                           ("f16", 33, 40)])
def test_quant_bit_exact(fmt, r, stride):
    import torch
    import rank_decode_attention_amd as R
    n_rows = 1500
    stored = _quant_rows(fmt, n_rows, r, seed=r * 7 + stride)
    buf = np.zeros((n_rows, stride), dtype=stored.dtype)
    buf[:, :r] = stored
    z = to_device(buf, fmt)
    nb = 16 * oracle.chunks_per_row(r)
    ns = oracle.chunks_per_row(r)
    codes = torch.full((n_rows, nb), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((n_rows, ns), -1, dtype=torch.int16, device="cuda")
    R.palu_quant_latent(z, r, stride, codes, scales)
    torch.cuda.synchronize()
    ref_codes, ref_scales = oracle.quant_int4(oracle.upcast(stored, fmt).astype(np.float32))
    ref_packed = oracle.pack_int4(ref_codes)
    got_codes = codes.cpu().numpy()
    got_scales = scales.cpu().numpy().view(np.float16)
    assert np.array_equal(got_scales.view(np.uint16), ref_scales.view(np.uint16)), "scales differ"
    assert np.array_equal(got_codes, ref_packed), \
        f"codes differ in {int((got_codes != ref_packed).sum())} bytes"
    # the tie row: 0.25/0.5 = 0.5 -> 0, 0.75/0.5 = 1.5 -> 2, 1.25/0.5 = 2.5 -> 2 (ties to even)
    if r >= 8:
        assert oracle.unpack_int4(got_codes[2:3], r)[0, :8].tolist() == [7, 0, 2, 2, 0, -2, -2, 4]


@pytest.mark.parametrize("fmt,r,stride,off", [("f16", 154, 154, 1), ("bf16", 154, 157, 3), ("f32", 154, 155, 1),
                                               ("bf16", 40, 41, 5), ("f16", 2100, 2100, 1), ("f32", 1100, 1103, 2)])
def test_quant_unaligned_and_long_rows(fmt, r, stride, off):
    """Rows starting at every alignment (the first row `off` elements past a
    256-byte boundary, odd strides: a lane's 8 elements straddle two aligned
    16-byte blocks, or three for binary32), and rows of more than 4 KB (a
    wave's 64 chunks within one or two rows)."""
    import torch
    import rank_decode_attention_amd as R
    n_rows = 1500 if r * stride < 200000 else 300
    stored = _quant_rows(fmt, n_rows, r, seed=r * 3 + stride + off)
    flat = np.zeros(n_rows * stride + off, dtype=stored.dtype)
    for i in range(n_rows):
        flat[off + i * stride: off + i * stride + r] = stored[i]
    dev = to_device(flat, fmt)
    z = dev[off:off + n_rows * stride].view(n_rows, stride)
    nc = oracle.chunks_per_row(r)
    codes = torch.full((n_rows, 16 * nc), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((n_rows, nc), -1, dtype=torch.int16, device="cuda")
    R.palu_quant_latent(z, r, stride, codes, scales)
    torch.cuda.synchronize()
    ref_codes, ref_scales = oracle.quant_int4(oracle.upcast(stored, fmt).astype(np.float32))
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), ref_scales.view(np.uint16)), "scales differ"
    got = codes.cpu().numpy()
    ref = oracle.pack_int4(ref_codes)
    assert np.array_equal(got, ref), f"codes differ in {int((got != ref).sum())} bytes"


@pytest.mark.parametrize("r", [7, 154])
def test_quant_rows_at_the_largest_stride(r):
    """fp16 rows 64 MiB apart, the largest row distance palu_quant_latent
    takes (its loads address a wave's rows by 32-bit offsets from one row
    base: with r = 7 a wave's 32 chunks span 32 rows, offsets near 2 GiB)."""
    import torch
    import rank_decode_attention_amd as R
    n_rows, stride = 40, 1 << 25
    stored = _quant_rows("f16", n_rows, r, seed=r + 11)
    z = torch.zeros((n_rows, stride), dtype=torch.float16, device="cuda")
    z[:, :r] = to_device(stored, "f16")
    nc = oracle.chunks_per_row(r)
    codes = torch.full((n_rows, 16 * nc), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((n_rows, nc), -1, dtype=torch.int16, device="cuda")
    R.palu_quant_latent(z, r, stride, codes, scales)
    torch.cuda.synchronize()
    del z
    ref_codes, ref_scales = oracle.quant_int4(oracle.upcast(stored, "f16").astype(np.float32))
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), ref_scales.view(np.uint16)), "scales differ"
    got = codes.cpu().numpy()
    ref = oracle.pack_int4(ref_codes)
    assert np.array_equal(got, ref), f"codes differ in {int((got != ref).sum())} bytes"


def test_quant_empty_is_noop():
    import torch
    import rank_decode_attention_amd as R
    z = torch.zeros((0, 32), dtype=torch.float16, device="cuda")
    codes = torch.zeros((1, 16), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((1, 1), dtype=torch.int16, device="cuda")
    R.palu_quant_latent(z, 32, 32, codes, scales)
    torch.cuda.synchronize()
    assert int(codes.sum()) == 0


# ------------------------------------------------------------------ projection
def _project_case(wl, n_tok: int, seq: int, pos0: int):
    """Device x, A_kv ([n_lat][d_model], Linear layout) and a sentinel-filled cache."""
    import torch
    import rank_decode_attention_amd as R
    from palu_cases import desc_of
    desc = desc_of(wl)
    x = PI.prefill_x(wl, n_tok)
    As = PI.prefill_A(wl)                                  # each [d_model][r]
    A_kv = np.concatenate([a.T for a in As], axis=0)       # [sum r][d_model]
    cache = R.alloc_cache(desc, wl.batch, wl.max_len)
    for t in (cache.zk, cache.zv, cache.sk, cache.sv):
        if t is not None:
            t.fill_(0x5A)
    R.palu_project(desc, to_device(x, wl.act), to_device(np.ascontiguousarray(A_kv), wl.act), cache, seq, pos0)
    torch.cuda.synchronize()
    host = {k: (None if t is None else t.cpu().numpy()) for k, t in
            (("zk", cache.zk), ("zv", cache.zv), ("sk", cache.sk), ("sv", cache.sv))}
    return desc, x, As, host


def _rows_of(desc, host, wl, which, j, seq, t0, n, scales=False):
    import rank_decode_attention_amd as R
    r = (desc.rank_k if which == 0 else desc.rank_v)[j]
    pitch = R.scale_pitch(r) if scales else R.row_pitch(desc.latent_dtype, r)
    buf = host[("sk" if which == 0 else "sv") if scales else ("zk" if which == 0 else "zv")]
    off = R.latent_offset(desc, wl.max_len, which, scales, seq, j, t0)
    return buf[off:off + n * pitch].reshape(n, pitch)


def _ulp(v: np.ndarray, fmt: str) -> np.ndarray:
    bits = {"f32": 23, "f16": 10, "bf16": 7}[fmt]
    mag = np.maximum(np.abs(v), {"f32": 2.0 ** -126, "f16": 2.0 ** -14, "bf16": 2.0 ** -126}[fmt])
    return 2.0 ** (np.floor(np.log2(mag)) - bits)


PROJ = [
    # (name, workload, n_tok, seq, pos0, sampled token rows or None for all)
    ("bf16_small", PI.scaled("int4_prefill", latent="bf16", d_model=512, batch=2, max_len=400, n_tok=300), 300, 1, 50,
     None),
    ("f16_ragged", PI.scaled("int4_prefill", latent="f16", act="f16", d_model=256, batch=1, max_len=300, n_tok=257,
                             rank=100), 257, 0, 43, None),
    ("f32_small", PI.scaled("tiny", n_tok=130, latent="f32", act="f32"), 130, 0, 7, None),
    ("bf16_full_size", PI.scaled("int4_prefill", latent="bf16"), 8192, 0, 0, [0, 1, 255, 256, 4097, 8190, 8191]),
]


@pytest.mark.parametrize("name,wl,n_tok,seq,pos0,sample", PROJ, ids=[p[0] for p in PROJ])
def test_project_parity(name, wl, n_tok, seq, pos0, sample):
    import rank_decode_attention_amd as R
    desc, x, As, host = _project_case(wl, n_tok, seq, pos0)
    fmt = wl.latent
    esz = 4 if fmt == "f32" else 2
    G = wl.n_groups
    xs = oracle.upcast(x, wl.act)
    rows = np.arange(n_tok) if sample is None else np.asarray(sample)
    for which in (0, 1):
        for j in range(G):
            r = (desc.rank_k if which == 0 else desc.rank_v)[j]
            ref = oracle.project(xs[rows], oracle.upcast(As[which * G + j], wl.act))   # fp64 [n][r]
            got_b = _rows_of(desc, host, wl, which, j, seq, pos0, n_tok)
            pitch_e = got_b.shape[1] // esz
            dt = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[fmt]
            got_e = got_b.view(dt).reshape(n_tok, pitch_e)
            got = oracle.upcast(got_e[:, :r], fmt)[rows]
            if pitch_e > r:                                  # row padding is written as zero
                assert np.all(got_e[:, r:].view(np.uint8) == 0), f"{name}: padding not zero"
            # bar: half an ulp of the stored format plus the binary32 accumulation
            # bound gamma_n * sum |x_i a_i| (n = d_model)
            err = np.abs(got - ref)
            n = wl.d_model
            gamma = n * 2.0 ** -24 / (1 - n * 2.0 ** -24)
            bound = gamma * (np.abs(xs[rows]) @ np.abs(oracle.upcast(As[which * G + j], wl.act)))
            assert np.all(err <= 0.5 * _ulp(ref, fmt) + bound), \
                f"{name} {which}/{j}: beyond rounding + accumulation bound (max err {err.max():.3e})"
            if fmt != "f32":
                # a 16-bit result differs from the correctly rounded one only where
                # the exact value lies within the accumulation error of a boundary
                rounded = oracle.upcast(PI.to_format(ref.astype(np.float32), fmt), fmt)
                frac = float(np.mean(got != rounded))
                assert frac <= 2e-3, f"{name} {which}/{j}: {frac:.2%} not correctly rounded"
    # rows outside [pos0, pos0 + n_tok) and other sequences are untouched (sentinel 0x5A)
    if sample is None:
        for which in (0, 1):
            buf = host["zk" if which == 0 else "zv"]
            for j in range(G):
                for b in range(wl.batch):
                    full = _rows_of(desc, host, wl, which, j, b, 0, wl.max_len)
                    keep = np.ones(wl.max_len, dtype=bool)
                    if b == seq:
                        keep[pos0:pos0 + n_tok] = False
                    assert np.all(full[keep] == 0x5A), f"{name}: rows outside the written range changed"


INT4 = [
    ("int4_small", PI.scaled("int4_prefill", d_model=512, batch=2, max_len=300, n_tok=200), 200, 1, 17, None),
    ("int4_full_size", PI.workload("int4_prefill"), 8192, 0, 0, [0, 5, 1000, 4096, 8191]),
]


@pytest.mark.parametrize("name,wl,n_tok,seq,pos0,sample", INT4, ids=[p[0] for p in INT4])
def test_project_int4_fused(name, wl, n_tok, seq, pos0, sample):
    desc, x, As, host = _project_case(wl, n_tok, seq, pos0)
    G = wl.n_groups
    xs = oracle.upcast(x, wl.act)
    rows = np.arange(n_tok) if sample is None else np.asarray(sample)
    n_code, n_total = 0, 0
    for which in (0, 1):
        for j in range(G):
            r = (desc.rank_k if which == 0 else desc.rank_v)[j]
            z = oracle.project(xs[rows], oracle.upcast(As[which * G + j], wl.act))
            ref_c, ref_s = oracle.quant_int4(z.astype(np.float32))
            got_codes = oracle.unpack_int4(_rows_of(desc, host, wl, which, j, seq, pos0, n_tok)[rows], r)
            got_s = _rows_of(desc, host, wl, which, j, seq, pos0, n_tok, scales=True)[rows].view(np.float16)
            packed = _rows_of(desc, host, wl, which, j, seq, pos0, n_tok)[rows]
            # pad nibbles are zero
            full = oracle.unpack_int4(packed, 2 * packed.shape[1])
            assert np.all(full[:, r:] == 0)
            assert np.all(np.abs(got_codes.astype(int)) <= 7)
            srel = np.abs(got_s.astype(np.float64) - ref_s.astype(np.float64)) / np.maximum(
                np.abs(ref_s.astype(np.float64)), 1e-30)
            assert np.all(srel <= 2.0 ** -10 + 1e-12), f"{name}: scales beyond one fp16 step"
            dq = np.abs(got_codes.astype(int) - ref_c.astype(int))
            assert dq.max() <= 1, f"{name}: code off by {dq.max()}"
            n_code += int((dq != 0).sum())
            n_total += dq.size
            deq = oracle.dequant_int4(got_codes, got_s)
            s_each = np.repeat(got_s.astype(np.float64), 32, axis=-1)[..., :r]
            assert np.all(np.abs(deq - z) <= s_each * (0.5 + 2.0 ** -9) + 1e-6), f"{name}: dequantised off"
    assert n_code <= max(1, n_total // 1000), f"{name}: {n_code} of {n_total} codes differ"
    print(name, "code mismatches", n_code, "of", n_total)


@pytest.mark.parametrize("fmt", ["bf16", "i4"])
def test_project_uneven_column_tiles(fmt):
    """Key and value ranks that differ, rows of several 160-channel column
    tiles with short last tiles (330 = 160 + 160 + 10, 161 = 160 + 1) and an
    odd tile count (7: the last block carries one tile), 300 tokens (a
    ragged 256-token block): every element against the oracle."""
    import torch
    import rank_decode_attention_amd as R
    rank_k, rank_v = [100, 330], [161, 40]
    d_model, n_tok, max_len, seq, pos0 = 256, 300, 320, 1, 11
    desc = R.AttnDesc(8, 8, 128, 2, rank_k, rank_v, use_rope=True, latent_dtype=fmt, act_dtype="bf16")
    rng = np.random.default_rng(2024)
    x = PI.to_format(rng.standard_normal((n_tok, d_model), dtype=np.float32), "bf16")
    As = [PI.to_format(rng.standard_normal((d_model, r), dtype=np.float32) / np.float32(np.sqrt(d_model)), "bf16")
          for r in rank_k + rank_v]
    A_kv = np.concatenate([a.T for a in As], axis=0)
    cache = R.alloc_cache(desc, 2, max_len)
    for t in (cache.zk, cache.zv, cache.sk, cache.sv):
        if t is not None:
            t.fill_(0x5A)
    R.palu_project(desc, to_device(x, "bf16"), to_device(np.ascontiguousarray(A_kv), "bf16"), cache, seq, pos0)
    torch.cuda.synchronize()
    host = {k: (None if t is None else t.cpu().numpy()) for k, t in
            (("zk", cache.zk), ("zv", cache.zv), ("sk", cache.sk), ("sv", cache.sv))}
    wl = PI.scaled("int4_prefill", max_len=max_len, batch=2, d_model=d_model)
    xs = oracle.upcast(x, "bf16")
    for which in (0, 1):
        for j in range(2):
            r = (rank_k if which == 0 else rank_v)[j]
            z = oracle.project(xs, oracle.upcast(As[which * 2 + j], "bf16"))
            rows = _rows_of(desc, host, wl, which, j, seq, pos0, n_tok)
            if fmt == "bf16":
                got = oracle.upcast(rows.view(np.uint16)[:, :r], "bf16")
                gamma = d_model * 2.0 ** -24 / (1 - d_model * 2.0 ** -24)
                bound = gamma * (np.abs(xs) @ np.abs(oracle.upcast(As[which * 2 + j], "bf16")))
                assert np.all(np.abs(got - z) <= 0.5 * _ulp(z, "bf16") + bound), f"{which}/{j}: projection off"
                assert np.all(rows.view(np.uint16)[:, r:] == 0), f"{which}/{j}: padding not zero"
            else:
                codes = oracle.unpack_int4(rows, r)
                s = _rows_of(desc, host, wl, which, j, seq, pos0, n_tok, scales=True).view(np.float16)
                ref_c, _ = oracle.quant_int4(z.astype(np.float32))
                dq = np.abs(codes.astype(int) - ref_c.astype(int))
                assert dq.max() <= 1 and (dq != 0).sum() <= max(1, dq.size // 1000), f"{which}/{j}: codes off"
                deq = oracle.dequant_int4(codes, s)
                s_each = np.repeat(s.astype(np.float64), 32, axis=-1)[..., :r]
                assert np.all(np.abs(deq - z) <= s_each * (0.5 + 2.0 ** -9) + 1e-6), f"{which}/{j}: dequantised off"
            # rows of the other sequence are untouched
            other = _rows_of(desc, host, wl, which, j, 0, 0, max_len)
            assert np.all(other == 0x5A), f"{which}/{j}: other sequence written"
