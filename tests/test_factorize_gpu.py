"""GPU leg of the offline factorisation helper: per-group weights W are
factorised on the host (rank_decode_attention_amd.factorize, truncated SVD
W ~ A B), the factors go through the HIP path end to end - palu_project
writes the prefill latents z = x A into the cache, palu_decode_attn attends
over them - and the output is compared with the fp64 oracle on the same
factors (oracle.project, rounded once to the latent format, then
oracle.decode_attention).  At full rank (A B = W) the no-RoPE output is also
compared with standard attention over K = x W_k, V = x W_v (torch SDPA,
float64), the formula block's W ~ A B read backwards.  Synthetic weights: a
seeded orthonormal basis with a decaying spectrum (no trained weights are
available), std 1/sqrt(d_model) overall, so z, K and V are ~N(0, 1)."""
import math

import numpy as np
import pytest

import oracle
import palu_inputs as PI
from palu_cases import compare, from_device, to_device
from rank_decode_attention_amd import factorize as F

pytestmark = pytest.mark.gpu


def _weights(d_model, w, seed, decay):
    rng = np.random.default_rng(seed)
    U, _ = np.linalg.qr(rng.standard_normal((d_model, w)))
    V, _ = np.linalg.qr(rng.standard_normal((w, w)))
    s = np.exp(-np.arange(w) / decay)
    s *= math.sqrt(w / np.sum(s * s))            # ||W||_F^2 = w: entries of x W ~ N(0, 1)
    return (U * s) @ V.T


def _run(H, H_kv, G, d_h, d_model, rank, use_rope, batch, lens, fmt="f16", seed=0, decay=64.0):
    import torch
    import rank_decode_attention_amd as R
    w = (H_kv // G) * d_h
    Wk = [_weights(d_model, w, seed + 2 * j, decay) for j in range(G)]
    Wv = [_weights(d_model, w, seed + 2 * j + 1, decay) for j in range(G)]
    fk = [F.factorize_group(W, rank) for W in Wk]
    fv = [F.factorize_group(W, rank) for W in Wv]
    # factors in the activation format (what both sides consume)
    Ak = [PI.to_format(a.astype(np.float32), fmt) for a, _, _ in fk]
    Av = [PI.to_format(a.astype(np.float32), fmt) for a, _, _ in fv]
    Bk = [PI.to_format(b.astype(np.float32), fmt) for _, b, _ in fk]
    Bv = [PI.to_format(b.astype(np.float32), fmt) for _, b, _ in fv]
    rng = np.random.default_rng(seed + 99)
    max_len = int(max(lens))
    x = [PI.to_format(rng.standard_normal((int(L), d_model)).astype(np.float32), fmt) for L in lens]
    q = PI.to_format(rng.standard_normal((batch, H, d_h)).astype(np.float32), fmt)

    desc = R.AttnDesc(H, H_kv, d_h, G, [rank] * G, use_rope=use_rope, latent_dtype=fmt, act_dtype=fmt)
    cache = R.alloc_cache(desc, batch, max_len)
    A_kv = to_device(np.concatenate([a.T for a in Ak + Av], axis=0), fmt)
    for b in range(batch):
        R.palu_project(desc, to_device(x[b], fmt), A_kv, cache, b, 0)
    cat = lambda Bs: to_device(np.concatenate([m.reshape(-1) for m in Bs]), fmt)
    ws = torch.empty(R.decode_workspace_bytes(desc, batch, max_len), dtype=torch.uint8, device="cuda")
    tdt = torch.float16 if fmt == "f16" else torch.bfloat16
    out = torch.empty((batch, H, d_h), dtype=tdt, device="cuda")
    seq_lens = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    sm = 1.0 / math.sqrt(d_h)
    R.palu_decode_attn(desc, to_device(q, fmt), cache, cat(Bk), cat(Bv), seq_lens, None, sm, out, ws)
    torch.cuda.synchronize()
    gpu = from_device(out)

    # oracle: latents z = x A in fp64, rounded once to the latent format
    up = lambda a: oracle.upcast(a, fmt)
    zk = [[oracle.round_to(oracle.project(up(x[b]), up(Ak[j])), fmt) for b in range(batch)] for j in range(G)]
    zv = [[oracle.round_to(oracle.project(up(x[b]), up(Av[j])), fmt) for b in range(batch)] for j in range(G)]
    ref = oracle.decode_attention(up(q), zk, zv, [up(m) for m in Bk], [up(m) for m in Bv], lens, n_kv_heads=H_kv,
                                  use_rope=use_rope, sm_scale=sm)
    return gpu, ref, dict(x=x, q=q, Wk=Wk, Wv=Wv, errs=[e for _, _, e in fk + fv], fmt=fmt, sm=sm)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_factorised_rank_below_width(fmt):
    """Groups of 4 kv heads (w = 512) factorised at rank 256 (50%), RoPE: the
    MHA head-group kernel over latents that palu_project wrote."""
    gpu, ref, info = _run(H=8, H_kv=8, G=2, d_h=128, d_model=1024, rank=256, use_rope=True, batch=2,
                          lens=[300, 77], fmt=fmt, seed=11)
    assert all(0 < e < 0.5 for e in info["errs"])      # a real truncation, not a full-rank copy
    compare(gpu, ref, fmt, f"factorised r256 of w512 {fmt}")


@pytest.mark.parametrize("use_rope", [False, True])
def test_factorised_full_rank_is_standard_attention(use_rope):
    """Groups of 2 kv heads (w = 256) at full rank 256: A B = W, so the decode
    over the projected latents is standard attention over K = x W_k and
    V = x W_v (GQA, 4 query heads per kv head)."""
    import torch
    H, H_kv, G, d_h = 16, 4, 2, 128
    lens = [200, 61]
    gpu, ref, info = _run(H=H, H_kv=H_kv, G=G, d_h=d_h, d_model=512, rank=256, use_rope=use_rope, batch=2,
                          lens=lens, fmt="f16", seed=5)
    compare(gpu, ref, "f16", f"factorised full rank rope={use_rope}")
    if use_rope:
        return
    # standard attention over the unfactorised weights (fp64), no RoPE
    up = lambda a: oracle.upcast(a, "f16")
    n_g = H_kv // G
    sdpa = np.zeros_like(ref)
    for b, L in enumerate(lens):
        xb = up(info["x"][b])
        for h in range(H):
            kv = h // (H // H_kv)
            j, c = kv // n_g, kv % n_g
            K = (xb @ info["Wk"][j])[:, c * d_h:(c + 1) * d_h]
            V = (xb @ info["Wv"][j])[:, c * d_h:(c + 1) * d_h]
            qh = torch.from_numpy(up(info["q"][b, h]))[None, None, None]
            sdpa[b, h] = torch.nn.functional.scaled_dot_product_attention(
                qh, torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None], scale=info["sm"])[0, 0, 0].numpy()
    # (the factors are rounded to fp16 once, so this is a looser bar than the oracle's)
    compare(gpu, sdpa, "f16", "factorised full rank vs SDPA(x W)")
