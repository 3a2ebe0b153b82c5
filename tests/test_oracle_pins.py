"""Pins of the fp64 oracle against things other than itself.

Each pin is a function ``pin_*`` that raises AssertionError when the oracle
disagrees with: a library routine (torch SDPA in float64 on the CPU), an
independent formulation (complex-multiplication RoPE, the absorbed query, the
fused value path), a scalar mpmath brute force, closed forms, or a hand-worked
fixture under tests/golden/.  ``test_planted_mistakes`` plants plausible bugs
into the oracle (on the CPU) and checks that some pin catches each one.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import oracle.palu as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _rand_case(rng, batch=2, H=4, Hkv=2, d_h=8, G=2, r=5, L=7, ragged=True):
    n_g = Hkv // G
    w = n_g * d_h
    q = rng.standard_normal((batch, H, d_h))
    zk = [rng.standard_normal((batch, L, r)) for _ in range(G)]
    zv = [rng.standard_normal((batch, L, r + 1)) for _ in range(G)]
    Bk = [rng.standard_normal((r, w)) / math.sqrt(r) for _ in range(G)]
    Bv = [rng.standard_normal((r + 1, w)) / math.sqrt(r) for _ in range(G)]
    lens = rng.integers(1, L + 1, size=batch) if ragged else np.full(batch, L)
    return q, zk, zv, Bk, Bv, lens


# ------------------------------------------------------------------ independent references
def _rope_complex(u, pos, base):
    """RoPE as complex multiplication: u_i + i*u_{i+d/2} times exp(i*pos*theta_i),
    theta_i = base^(-2i/d)."""
    d = u.shape[-1]
    h = d // 2
    theta = np.array([base ** (-(2.0 * i) / d) for i in range(h)])
    zc = (u[..., :h] + 1j * u[..., h:]) * np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None] * theta)
    return np.concatenate([zc.real, zc.imag], axis=-1)


def _sdpa(q, K, V, scale):
    import torch
    import torch.nn.functional as F
    qt = torch.from_numpy(np.ascontiguousarray(q))[None, None, None, :]
    Kt = torch.from_numpy(np.ascontiguousarray(K))[None, None]
    Vt = torch.from_numpy(np.ascontiguousarray(V))[None, None]
    return F.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)[0, 0, 0].numpy()


# ------------------------------------------------------------------ pins
def pin_identity_vs_sdpa(use_rope):
    """A = W, B = I, r = w: the method reduces to standard attention over
    K = x W_k, V = x W_v; reference: torch SDPA fp64."""
    rng = np.random.default_rng(7)
    batch, H, Hkv, d_h, G, D, L = 2, 6, 2, 8, 2, 12, 9
    n_g = Hkv // G
    w = n_g * d_h
    x = rng.standard_normal((batch, L, D))
    Wk = [rng.standard_normal((D, w)) / math.sqrt(D) for _ in range(G)]
    Wv = [rng.standard_normal((D, w)) / math.sqrt(D) for _ in range(G)]
    q = rng.standard_normal((batch, H, d_h))
    lens = np.array([L, 4])
    zk = [O.project(x.reshape(-1, D), Wk[j]).reshape(batch, L, w) for j in range(G)]
    zv = [O.project(x.reshape(-1, D), Wv[j]).reshape(batch, L, w) for j in range(G)]
    eye = [np.eye(w) for _ in range(G)]
    scale = 1.0 / math.sqrt(d_h)
    out = O.decode_attention(q, zk, zv, eye, eye, lens, n_kv_heads=Hkv, use_rope=use_rope, sm_scale=scale)
    for b in range(batch):
        Lb = lens[b]
        for h in range(H):
            kv = h // (H // Hkv)
            j, c = kv // n_g, kv % n_g
            K = (x[b, :Lb] @ Wk[j])[:, c * d_h:(c + 1) * d_h]
            V = (x[b, :Lb] @ Wv[j])[:, c * d_h:(c + 1) * d_h]
            qh = q[b, h]
            if use_rope:
                K = _rope_complex(K, np.arange(Lb), 10000.0)
                qh = _rope_complex(qh, Lb - 1, 10000.0)
            ref = _sdpa(qh, K, V, scale)
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-12)


def pin_absorbed_and_fused_value():
    """No-RoPE heads: attention through the absorbed query (q . B_k^T) against
    z_k and values through (P . z_v) . B_v equal the rebuilt-K/V result."""
    rng = np.random.default_rng(11)
    q, zk, zv, Bk, Bv, lens = _rand_case(rng, batch=3, H=8, Hkv=4, d_h=6, G=2, r=4, L=11)
    batch, H, d_h = q.shape
    Hkv, G = 4, 2
    n_g = Hkv // G
    scale = 0.37
    out = O.decode_attention(q, zk, zv, Bk, Bv, lens, n_kv_heads=Hkv, use_rope=False, sm_scale=scale)
    for b in range(batch):
        Lb = lens[b]
        for h in range(H):
            kv = h // (H // Hkv)
            j, c = kv // n_g, kv % n_g
            q_abs = Bk[j][:, c * d_h:(c + 1) * d_h] @ q[b, h]          # [r]
            s = scale * (zk[j][b, :Lb] @ q_abs)
            p = np.exp(s - s.max())
            p /= p.sum()
            o = (p @ zv[j][b, :Lb]) @ Bv[j][:, c * d_h:(c + 1) * d_h]
            np.testing.assert_allclose(out[b, h], o, rtol=0, atol=1e-12)


def pin_mpmath_bruteforce():
    """Scalar evaluation of every sum at 50 digits (mpmath) on tiny shapes
    (brute force)."""
    import mpmath as mp
    mp.mp.dps = 50
    rng = np.random.default_rng(3)
    for (d_h, r, L, G, use_rope) in [(2, 1, 3, 1, True), (4, 3, 4, 2, True), (4, 2, 2, 2, False),
                                     (2, 3, 4, 1, True)]:
        Hkv = 2 * G
        H = 2 * Hkv
        n_g = Hkv // G
        w = n_g * d_h
        q = rng.standard_normal((1, H, d_h))
        zk = [rng.standard_normal((1, L, r)) for _ in range(G)]
        zv = [rng.standard_normal((1, L, r)) for _ in range(G)]
        Bk = [rng.standard_normal((r, w)) for _ in range(G)]
        Bv = [rng.standard_normal((r, w)) for _ in range(G)]
        base, scale = 10000.0, 0.5
        out = O.decode_attention(q, zk, zv, Bk, Bv, [L], n_kv_heads=Hkv, use_rope=use_rope,
                                 rope_base=base, sm_scale=scale)
        for h in range(H):
            kv = h // (H // Hkv)
            j, c = kv // n_g, kv % n_g

            def rot(vec, pos):
                if not use_rope:
                    return vec
                hd = d_h // 2
                res = list(vec)
                for i in range(hd):
                    ang = mp.mpf(pos) * mp.power(mp.mpf(base), -mp.mpf(2 * i) / d_h)
                    a, bb = vec[i], vec[i + hd]
                    res[i] = a * mp.cos(ang) - bb * mp.sin(ang)
                    res[i + hd] = a * mp.sin(ang) + bb * mp.cos(ang)
                return res

            keys, vals = [], []
            for t in range(L):
                k = [mp.fsum(mp.mpf(zk[j][0, t, kk]) * mp.mpf(Bk[j][kk, c * d_h + d]) for kk in range(r))
                     for d in range(d_h)]
                v = [mp.fsum(mp.mpf(zv[j][0, t, kk]) * mp.mpf(Bv[j][kk, c * d_h + d]) for kk in range(r))
                     for d in range(d_h)]
                keys.append(rot(k, t))
                vals.append(v)
            qr = rot([mp.mpf(x) for x in q[0, h]], L - 1)
            s = [mp.mpf(scale) * mp.fsum(qr[d] * keys[t][d] for d in range(d_h)) for t in range(L)]
            e = [mp.exp(si) for si in s]
            z = mp.fsum(e)
            ref = [mp.fsum(e[t] * vals[t][d] for t in range(L)) / z for d in range(d_h)]
            np.testing.assert_allclose(out[0, h], np.array([float(x) for x in ref]), rtol=0, atol=1e-13)


def pin_softmax_closed_forms():
    rng = np.random.default_rng(5)
    L, d = 6, 4
    K = rng.standard_normal((L, d))
    V = rng.standard_normal((L, d))
    # L = 1: the output is the single value row
    np.testing.assert_allclose(O.attend(rng.standard_normal(d), K[:1], V[:1], 0.7), V[0], rtol=0, atol=1e-15)
    # zero query: uniform weights, output is the mean row
    np.testing.assert_allclose(O.attend(np.zeros(d), K, V, 0.7), V.mean(axis=0), rtol=0, atol=1e-14)
    # weights sum to one: with all-ones values the output is exactly ones
    np.testing.assert_allclose(O.attend(rng.standard_normal(d), K, np.ones((L, 3)), 1.3), np.ones(3),
                               rtol=0, atol=1e-14)
    # one dominant score: output tends to that row
    Kd = np.zeros((L, d))
    Kd[3, 0] = 1.0
    np.testing.assert_allclose(O.attend(np.array([800.0, 0, 0, 0]), Kd, V, 1.0), V[3], rtol=0, atol=1e-12)
    # shift invariance of the scores (adding a constant to all scores)
    q = rng.standard_normal(d)
    Kc = np.concatenate([K, np.ones((L, 1))], axis=1)
    a = O.attend(np.concatenate([q, [0.0]]), Kc, V, 1.0)
    b = O.attend(np.concatenate([q, [37.0]]), Kc, V, 1.0)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def pin_rope():
    rng = np.random.default_rng(9)
    base = 10000.0
    for d in (2, 4, 8, 128):
        u = rng.standard_normal((5, d))
        pos = rng.integers(0, 70000, size=5)
        # equals complex multiplication with theta_i = base^(-2i/d) (fixes the half-split pairing)
        np.testing.assert_allclose(O.rope(u, pos, base), _rope_complex(u, pos, base), rtol=0, atol=1e-9)
        # isometry, identity at 0, composition
        np.testing.assert_allclose(np.linalg.norm(O.rope(u, pos, base), axis=-1), np.linalg.norm(u, axis=-1),
                                   rtol=1e-13)
        np.testing.assert_array_equal(O.rope(u, np.zeros(5), base), u)
        a, b = 1234, 5678
        np.testing.assert_allclose(O.rope(O.rope(u, a, base), b, base), O.rope(u, a + b, base), rtol=0, atol=1e-10)
        # scores depend only on the relative position
        k, qv = rng.standard_normal(d), rng.standard_normal(d)
        s1 = O.rope(qv, 100, base) @ O.rope(k, 40, base)
        s2 = O.rope(qv, 1100, base) @ O.rope(k, 1040, base)
        assert abs(s1 - s2) < 1e-10 * max(1.0, abs(s1))
    # d = 2: theta_0 = 1, a plain planar rotation by t radians
    t = 3
    np.testing.assert_allclose(O.rope(np.array([1.0, 0.0]), t, base), [math.cos(t), math.sin(t)], rtol=0,
                               atol=1e-15)
    # d = 4: second pair rotates at base^(-1/2)
    th = base ** -0.5
    np.testing.assert_allclose(O.rope(np.array([0.0, 1.0, 0.0, 0.0]), 2, base),
                               [0.0, math.cos(2 * th), 0.0, math.sin(2 * th)], rtol=0, atol=1e-15)


def pin_gqa():
    """With GQA, replicating every kv head to its query heads (MHA) gives the
    same output; with H = H_kv the mapping is the identity."""
    rng = np.random.default_rng(13)
    batch, H, Hkv, d_h, G, r, L = 2, 8, 4, 4, 2, 3, 6
    n_g = Hkv // G
    q, zk, zv, Bk, Bv, lens = _rand_case(rng, batch, H, Hkv, d_h, G, r, L)
    out = O.decode_attention(q, zk, zv, Bk, Bv, lens, n_kv_heads=Hkv, use_rope=True)
    # MHA layout: group j now holds n_g * (H/Hkv) kv heads, each a copy of its source
    rep = H // Hkv
    Bk2 = [np.concatenate([Bk[j][:, (c // rep) * d_h:(c // rep + 1) * d_h] for c in range(n_g * rep)], axis=1)
           for j in range(G)]
    Bv2 = [np.concatenate([Bv[j][:, (c // rep) * d_h:(c // rep + 1) * d_h] for c in range(n_g * rep)], axis=1)
           for j in range(G)]
    out2 = O.decode_attention(q, zk, zv, Bk2, Bv2, lens, n_kv_heads=H, use_rope=True)
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-13)


def pin_split_merge():
    """Merging partials of any split of the history equals the single pass."""
    rng = np.random.default_rng(17)
    L, d = 37, 8
    q, K, V = rng.standard_normal(d), rng.standard_normal((L, d)), rng.standard_normal((L, d))
    full = O.attend(q, K, V, 0.4)
    for _ in range(10):
        cuts = sorted(set(rng.integers(1, L, size=rng.integers(1, 6)).tolist()))
        edges = [0] + cuts + [L]
        parts = [O.attend_partial(q, K[a:b], V[a:b], 0.4) for a, b in zip(edges[:-1], edges[1:])]
        np.testing.assert_allclose(O.merge_partials(parts), full, rtol=0, atol=1e-13)


def pin_golden_decode():
    with open(os.path.join(GOLDEN, "decode_worked.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        q = np.array(case["q"], dtype=np.float64)
        out = O.decode_attention(q, [np.array(case["zk"], float)], [np.array(case["zv"], float)],
                                 [np.array(case["Bk"], float)], [np.array(case["Bv"], float)],
                                 case["seq_lens"], n_kv_heads=case["n_kv_heads"], use_rope=case["use_rope"],
                                 sm_scale=case["sm_scale"])
        np.testing.assert_allclose(out, np.array(case["expected"]), rtol=0, atol=1e-14)


def pin_rope_closed_form_d2():
    """Closed form with d_h = 2 and RoPE: keys [1,0] at t=0 and 0 at t=1, query
    [ln 3, 0] at p=1: the score of key 0 is ln3*cos(1), of key 1 zero."""
    q = np.array([[[math.log(3.0), 0.0]]])
    zk = [np.array([[[1.0, 0.0], [0.0, 0.0]]])]
    zv = [np.array([[[1.0, 1.0], [0.0, 1.0]]])]
    Bk = [np.eye(2)]
    Bv = [np.array([[1.0, 2.0], [3.0, -1.0]])]
    out = O.decode_attention(q, zk, zv, Bk, Bv, [2], n_kv_heads=1, use_rope=True, sm_scale=1.0)
    p0 = 3.0 ** math.cos(1.0) / (3.0 ** math.cos(1.0) + 1.0)
    ref = p0 * np.array([4.0, 1.0]) + (1 - p0) * np.array([3.0, -1.0])
    np.testing.assert_allclose(out[0, 0], ref, rtol=0, atol=1e-14)


def pin_project():
    """z = x A against integer brute force (exact)."""
    rng = np.random.default_rng(19)
    x = rng.integers(-5, 6, size=(7, 9))
    A = rng.integers(-5, 6, size=(9, 4))
    ref = [[sum(int(x[i, k]) * int(A[k, j]) for k in range(9)) for j in range(4)] for i in range(7)]
    np.testing.assert_array_equal(O.project(x, A), np.array(ref, dtype=np.float64))


def pin_int4_golden():
    with open(os.path.join(GOLDEN, "int4_worked.json")) as f:
        fx = json.load(f)
    z = np.array(fx["z"], dtype=np.float32)
    codes, scales = O.quant_int4(z)
    np.testing.assert_array_equal(codes, np.array(fx["codes"], dtype=np.int8))
    np.testing.assert_array_equal(scales.astype(np.float64), np.array(fx["scales"]))
    packed = O.pack_int4(codes)
    assert packed.tobytes().hex() == fx["packed_hex"]
    np.testing.assert_array_equal(O.unpack_int4(packed, fx["r"]), codes)


def pin_int4_properties():
    rng = np.random.default_rng(23)
    for r in (32, 40, 154, 160):
        z = (rng.standard_normal((50, r)) * rng.uniform(0.01, 100, size=(50, 1))).astype(np.float32)
        codes, scales = O.quant_int4(z)
        assert codes.min() >= -7 and codes.max() <= 7
        assert scales.shape == (50, O.chunks_per_row(r))
        deq = O.dequant_int4(codes, scales)
        s = np.repeat(scales.astype(np.float64), 32, axis=-1)[:, :r]
        assert np.all(np.abs(z - deq) <= 0.5 * s * (1 + 1e-5))
        # every chunk reaches |code| = 7 at its largest element (scale is amax/7)
        for c in range(O.chunks_per_row(r)):
            seg = codes[:, c * 32:min(r, c * 32 + 32)]
            assert np.all(np.abs(seg).max(axis=-1) == 7)
        # dequantised values are exact in fp32: q*s has at most 3 + 11 significant bits
        np.testing.assert_array_equal(deq.astype(np.float32).astype(np.float64), deq)
        np.testing.assert_array_equal(O.unpack_int4(O.pack_int4(codes), r), codes)
    # exact round trip for z = k*s with amax = 7*s
    s = 0.25
    k = np.array([[7, -7, 0, 1, -1, 3, -3, 5] * 4], dtype=np.float32)
    codes, scales = O.quant_int4(k * s)
    np.testing.assert_array_equal(codes, k.astype(np.int8))
    assert float(scales[0, 0]) == s
    # all-zero chunk: zero scale, zero codes
    codes, scales = O.quant_int4(np.zeros((1, 32), np.float32))
    assert float(scales[0, 0]) == 0.0 and not codes.any()


def pin_upcast():
    # bf16 bit patterns: 0x3F80 = 1.0, 0xC040 = -3.0, 0x0001 = smallest subnormal 2^-133
    bits = np.array([0x3F80, 0xC040, 0x0001], dtype=np.uint16)
    np.testing.assert_array_equal(O.upcast(bits, "bf16"), [1.0, -3.0, 2.0 ** -133])
    np.testing.assert_array_equal(O.upcast(np.array([0.1], np.float16), "f16"), [float(np.float16(0.1))])


def pin_round_to():
    """round_to against the library conversions: numpy's float64 -> float16
    and torch's float32 -> bfloat16 (both round to nearest, ties to even),
    on random values and on exact ties."""
    import torch
    rng = np.random.default_rng(77)
    # normal-range values of both formats: |x| in [2^-13, 2^13)
    x = rng.choice([-1.0, 1.0], 4000) * rng.uniform(1.0, 2.0, 4000) * np.exp2(rng.integers(-13, 13, 4000))
    x = np.concatenate([x, [0.0, 1.0, -1.0]])
    ties16 = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, -(2 + 5 * 2.0 ** -10), 0.75 + 2.0 ** -12])
    got = O.round_to(np.concatenate([x, ties16]), "f16")
    want = np.concatenate([x, ties16]).astype(np.float16).astype(np.float64)
    assert np.array_equal(got, want), "f16 rounding differs from numpy"
    x32 = x.astype(np.float32).astype(np.float64)   # torch rounds from binary32
    ties_b = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(4 + 2.0 ** -6), 3 * 2.0 ** -9 + 2.0 ** -17])
    xb = np.concatenate([x32, ties_b])
    want_b = torch.from_numpy(xb.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_to(xb, "bf16"), want_b), "bf16 rounding differs from torch"
    # binary16 subnormals (quantum 2^-24) and the boundary to the normals
    sub = np.concatenate([rng.uniform(-2.0 ** -14, 2.0 ** -14, 2000), np.arange(-40, 41) * 2.0 ** -25,
                          [2.0 ** -14, -2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 2.0 ** -24, 2.0 ** -26]])
    assert np.array_equal(O.round_to(sub, "f16"), sub.astype(np.float16).astype(np.float64)), "f16 subnormals"
    # the ties go to the even neighbour
    assert O.round_to(np.array([1 + 2.0 ** -11]), "f16")[0] == 1.0
    assert O.round_to(np.array([1 + 3 * 2.0 ** -11]), "f16")[0] == 1 + 2.0 ** -9


def pin_int4_latent():
    """int4_latent is the exact product code * scale: every code against a
    sweep of binary16 scales, compared with exact rational arithmetic
    (fractions.Fraction); the byte layout against a hand-packed row (codes
    1..7, -1..-7, 0 in the documented nibble order)."""
    from fractions import Fraction
    codes = np.arange(-7, 8, dtype=np.int8)                       # 15 codes
    rng = np.random.default_rng(5)
    s = rng.uniform(0.01, 3.0, 64).astype(np.float16)
    s[:4] = [1 + 2.0 ** -10, 2.0 ** -20, 65504.0, 0.0]             # 11 significant bits, subnormal, max, zero
    full = np.zeros((64, 32), dtype=np.int8)
    full[:, :15] = np.tile(codes, 64).reshape(64, 15)
    got = O.int4_latent(O.pack_int4(full), s[:, None], 32)
    for i in range(64):
        for k in range(15):
            assert Fraction(float(got[i, k])) == Fraction(int(full[i, k])) * Fraction(float(s[i]))
    assert not got[:, 15:].any()
    # 7 * (1 + 2^-10) has 14 significant bits: kept exactly (binary16 would round it)
    assert got[0, 14] == 7 * (1 + 2.0 ** -10)
    row = bytes([0x21, 0x43, 0x65, 0xF7, 0xDE, 0xBC, 0x9A, 0x00] + [0] * 8)
    want = [1, 2, 3, 4, 5, 6, 7, -1, -2, -3, -4, -5, -6, -7, 0, 0]
    got = O.int4_latent(np.frombuffer(row, np.uint8)[None], np.array([[1.0]], np.float16), 16)
    assert got[0].tolist() == want
    # rank shorter than the chunk: only the first r elements come back
    assert O.int4_latent(np.frombuffer(row, np.uint8)[None], np.array([[0.5]], np.float16), 3).shape == (1, 3)


def pin_int4_rows16():
    """int4_rows16 (the stand-alone expansion's 16-bit rows) against the
    library conversions of the exact product: numpy float64 -> float16 and
    torch float32 -> bfloat16."""
    import torch
    rng = np.random.default_rng(6)
    full = rng.integers(-7, 8, size=(64, 32)).astype(np.int8)
    s = rng.uniform(0.01, 3.0, 64).astype(np.float16)
    exact = full.astype(np.float64) * s.astype(np.float64)[:, None]
    got16 = O.int4_rows16(O.pack_int4(full), s[:, None], 32, "f16")
    assert np.array_equal(got16, exact.astype(np.float16).astype(np.float64))
    gotb = O.int4_rows16(O.pack_int4(full), s[:, None], 32, "bf16")
    wantb = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(gotb, wantb)


def pin_int4_decode_golden():
    """A decode step over an int4 cache against its hand-worked closed form
    (tests/golden/int4_decode_worked.json); the latent 7 * (1 + 2^-10) is
    only exact when the code * scale product is not rounded to 16 bits."""
    with open(os.path.join(GOLDEN, "int4_decode_worked.json")) as f:
        fx = json.load(f)
    r = fx["rank"]

    def rows(key):
        packed = np.stack([np.frombuffer(bytes.fromhex(h), np.uint8) for h in fx[key + "_packed_hex"]])
        scales = np.array(fx[key + "_scale_bits"], dtype=np.uint16).view(np.float16)[:, None]
        return O.int4_latent(packed, scales, r)[None]          # [batch 1][L][r]
    q = np.array(fx["q"], dtype=np.float64)[None, None]
    out = O.decode_attention(q, [rows("zk")], [rows("zv")], [np.eye(2)], [np.eye(2)], [2], n_kv_heads=1,
                             use_rope=False, sm_scale=fx["sm_scale"])
    s = 1 + 2.0 ** -10
    a = 7 * s
    p0, p1 = 1.0 / (1.0 + math.exp(-a)), 1.0 / (1.0 + math.exp(a))
    want = np.array([p0 * s, -7 * s * p0 + 3.5 * p1])
    np.testing.assert_allclose(out[0, 0], want, rtol=0, atol=1e-14)


def pin_hadamard_rotation():
    """Rotated-chunk int4 (low-rank-aware reading): the Hadamard matrix against
    the library routine (scipy.linalg.hadamard), H H^T = 32 I; the binary32
    butterflies equal the matrix product exactly on integer rows (sums of
    small integers are exact in binary32) and within the binary32 bound on
    real rows; a trailing partial chunk is not rotated; the folded factors
    leave z B unchanged (fp64)."""
    import scipy.linalg
    for n in (1, 2, 4, 8, 16, 32, 64):
        assert np.array_equal(O.hadamard(n), scipy.linalg.hadamard(n).astype(np.float64))
    H = O.hadamard(32)
    assert np.array_equal(H @ H.T, 32 * np.eye(32))
    rng = np.random.default_rng(31)
    zi = rng.integers(-50, 50, size=(40, 70)).astype(np.float32)          # 2 full chunks + 6
    want = zi.astype(np.float64).copy()
    want[:, :32] = zi[:, :32] @ scipy.linalg.hadamard(32)
    want[:, 32:64] = zi[:, 32:64] @ scipy.linalg.hadamard(32)
    assert np.array_equal(O.rotate_chunks(zi), want)
    assert np.array_equal(O.rotate_chunks_f32(zi).astype(np.float64), want)
    zr = rng.standard_normal((40, 70)).astype(np.float32)
    ref = O.rotate_chunks(zr)
    bound = 5 * 2.0 ** -24 * np.repeat(np.abs(zr[:, :64]).reshape(40, 2, 32).sum(-1), 32, axis=1)
    assert np.all(np.abs(O.rotate_chunks_f32(zr)[:, :64] - ref[:, :64]) <= bound)
    assert np.array_equal(O.rotate_chunks_f32(zr)[:, 64:], zr[:, 64:])
    # fold: (x A') B' = x A B for ranks with and without a partial chunk
    for r in (64, 70, 154):
        x = rng.standard_normal((5, 48))
        A = rng.standard_normal((48, r))
        B = rng.standard_normal((r, 24))
        A2, B2 = O.fold_rotation(A, B)
        assert np.allclose((x @ A2) @ B2, (x @ A) @ B, rtol=0, atol=1e-11)
        assert np.allclose(x @ A2, O.rotate_chunks(x @ A), rtol=0, atol=1e-11)


def pin_hadamard_hand_worked():
    """Order 4 by hand: H_4 = [[1,1,1,1],[1,-1,1,-1],[1,1,-1,-1],[1,-1,-1,1]];
    the row [1, 2, 3, 4] rotates to [10, -2, -4, 0].  A 32-chunk holding a
    single 8 at position 5 rotates to 8 times row 5 of H_32 (entries +-8)."""
    assert np.array_equal(O.hadamard(4), np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]]))
    assert (np.array([1.0, 2, 3, 4]) @ O.hadamard(4)).tolist() == [10, -2, -4, 0]
    z = np.zeros((1, 32), np.float32)
    z[0, 5] = 8.0
    got = O.rotate_chunks_f32(z)[0]
    # row 5 of the Sylvester matrix: entry (5, j) = (-1)^popcount(5 & j)
    want = [8.0 * (-1) ** bin(5 & j).count("1") for j in range(32)]
    assert got.tolist() == want


def pin_chunk_attention():
    """Chunk attention: q_len = 1 is the decode step; later latents do not
    reach earlier queries; in the identity case A = W, B = I it equals
    standard attention with a causal offset mask (torch SDPA, float64)."""
    import torch
    rng = np.random.default_rng(21)
    q, zk, zv, Bk, Bv, lens = _rand_case(rng, batch=2, H=4, Hkv=2, d_h=8, G=2, r=5, L=9)
    lens = np.array([9, 6])
    q1 = q[:, None]
    a = oracle.chunk_attention(q1, zk, zv, Bk, Bv, lens, n_kv_heads=2)
    b = oracle.decode_attention(q, zk, zv, Bk, Bv, lens, n_kv_heads=2)
    assert np.allclose(a[:, 0], b, atol=1e-13)
    qc = rng.standard_normal((2, 4, 4, 8))
    base = oracle.chunk_attention(qc, zk, zv, Bk, Bv, lens, n_kv_heads=2)
    zk2 = [z.copy() for z in zk]
    zv2 = [z.copy() for z in zv]
    for z in zk2 + zv2:
        z[0, 7:] += 5.0                      # rows past query 1's position (L 9, q_len 4: p = 5, 6, 7, 8)
    moved = oracle.chunk_attention(qc, zk2, zv2, Bk, Bv, lens, n_kv_heads=2)
    assert np.allclose(moved[0, :2], base[0, :2], atol=1e-13) and not np.allclose(moved[0, 2:], base[0, 2:])
    # identity: K = z_k, V = z_v, one group of one kv head, no RoPE, mask t <= L - q_len + i
    d, L, ql = 6, 7, 3
    zk1 = [rng.standard_normal((1, L, d))]
    zv1 = [rng.standard_normal((1, L, d))]
    qq = rng.standard_normal((1, ql, 1, d))
    got = oracle.chunk_attention(qq, zk1, zv1, [np.eye(d)], [np.eye(d)], [L], n_kv_heads=1, use_rope=False)
    mask = torch.tensor([[t <= L - ql + i for t in range(L)] for i in range(ql)])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qq[:, :, 0][:, None]), torch.from_numpy(zk1[0][:, None]), torch.from_numpy(zv1[0][:, None]),
        attn_mask=mask, scale=1.0 / math.sqrt(d))
    assert np.allclose(got[:, :, 0], ref[:, 0].numpy(), atol=1e-12)


PINS = [pin_absorbed_and_fused_value, pin_mpmath_bruteforce, pin_softmax_closed_forms, pin_rope, pin_gqa,
        pin_split_merge, pin_golden_decode, pin_rope_closed_form_d2, pin_project, pin_int4_golden,
        pin_int4_properties, pin_upcast, pin_round_to, pin_int4_latent, pin_int4_rows16, pin_int4_decode_golden,
        pin_chunk_attention, pin_hadamard_rotation, pin_hadamard_hand_worked]


@pytest.mark.parametrize("use_rope", [False, True])
def test_identity_vs_sdpa(use_rope):
    pin_identity_vs_sdpa(use_rope)


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ------------------------------------------------------------------ planted mistakes
def _interleaved_rope(u, pos, base):
    d = u.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * O.rope_theta(d, base)
    c, s = np.cos(ang), np.sin(ang)
    x, y = u[..., 0::2], u[..., 1::2]
    out = np.empty_like(u)
    out[..., 0::2] = x * c - y * s
    out[..., 1::2] = x * s + y * c
    return out


def _wrong_sign_rope(u, pos, base):
    return O.__dict__["_orig_rope"](u, -np.asarray(pos), base)


def _theta_off_by_one(head_dim, base):
    i = np.arange(1, head_dim // 2 + 1, dtype=np.float64)
    return base ** (-2.0 * i / head_dim)


def _attend_no_scale(q, K, V, sm_scale):
    return O.__dict__["_orig_attend"](q, K, V, 1.0)


def _reconstruct_dropped_row(z, B):
    return z[:, 1:] @ B[1:]


def _quant_ties_away(z):
    codes, scales = O.__dict__["_orig_quant"](z)
    z = np.asarray(z, np.float32)
    s = np.repeat(scales.astype(np.float32), 32, axis=-1)[..., :z.shape[-1]]
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = np.where(s == 0, 0, np.sign(z / s) * np.floor(np.abs(z / s) + 0.5))
    return np.clip(qf, -7, 7).astype(np.int8), scales


def _merge_no_rescale(parts):
    return sum(p[2] for p in parts) / sum(p[1] for p in parts)


def _round_truncate(x, fmt):
    x = np.asarray(x, dtype=np.float64)
    p = O._SIG_BITS[fmt]
    m, e = np.frexp(x)
    return np.ldexp(np.trunc(np.ldexp(m, p)), e - p)


def _round_f16_as_bf16(x, fmt):
    return O.__dict__["_orig_round"](x, "bf16")


def _int4_latent_rounded_f16(packed, scales, r):
    return O.round_to(O.dequant_int4(O.unpack_int4(packed, r), scales), "f16")


def _butterfly_sign_swapped(z):
    x = O.__dict__["_orig_rot32"](z)
    # (b - a) instead of (a - b) in the last stage: the upper half changes sign
    x[..., 16:32] = -x[..., 16:32]
    return x


def _fold_without_scale(A, B):
    A2, B2 = O.__dict__["_orig_fold"](A, B)
    return A2, B2 * 32


def _unpack_nibbles_swapped(packed, r):
    p = np.asarray(packed, dtype=np.uint8)
    return O.__dict__["_orig_unpack"](((p << 4) | (p >> 4)).astype(np.uint8), r)


MUTANTS = [
    ("rope", _interleaved_rope),
    ("rope", _wrong_sign_rope),
    ("rope_theta", _theta_off_by_one),
    ("attend", _attend_no_scale),
    ("reconstruct", _reconstruct_dropped_row),
    ("quant_int4", _quant_ties_away),
    ("merge_partials", _merge_no_rescale),
    ("round_to", _round_truncate),
    ("round_to", _round_f16_as_bf16),
    ("unpack_int4", _unpack_nibbles_swapped),
    ("int4_latent", _int4_latent_rounded_f16),
    ("rotate_chunks_f32", _butterfly_sign_swapped),
    ("fold_rotation", _fold_without_scale),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[f"{n}:{m.__name__}" for n, m in MUTANTS])
def test_planted_mistakes(name, mutant, monkeypatch):
    """A plausible bug planted in the oracle must make at least one pin fail."""
    monkeypatch.setitem(O.__dict__, "_orig_rope", O.rope)
    monkeypatch.setitem(O.__dict__, "_orig_attend", O.attend)
    monkeypatch.setitem(O.__dict__, "_orig_quant", O.quant_int4)
    monkeypatch.setitem(O.__dict__, "_orig_round", O.round_to)
    monkeypatch.setitem(O.__dict__, "_orig_unpack", O.unpack_int4)
    monkeypatch.setitem(O.__dict__, "_orig_rot32", O.rotate_chunks_f32)
    monkeypatch.setitem(O.__dict__, "_orig_fold", O.fold_rotation)
    monkeypatch.setattr(O, name, mutant)
    caught = False
    for pin in [lambda: pin_identity_vs_sdpa(True), lambda: pin_identity_vs_sdpa(False)] + PINS:
        try:
            pin()
        except AssertionError:
            caught = True
            break
    assert caught, f"no pin caught the planted mistake in {name}"
