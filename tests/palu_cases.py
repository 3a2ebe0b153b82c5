"""Shared helpers of the GPU parity tests: build device inputs for a workload
from the seeded generators, run the library through its binding, build the
matching fp64 oracle inputs, and compare.

Tolerances (the accuracy bar of the decode outputs):
  fp16 / bf16 outputs: max |gpu - ref| <= 2e-3 + half an ulp of the output
  format at |ref| (the output is stored in that format), and
  ||gpu - ref||_2 / ||ref||_2 <= 1e-2;
  fp32 outputs: max-abs <= 1e-5 and relative <= 1e-5.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

import oracle
import palu_inputs as PI

TOL = {"f32": (1e-5, 1e-5), "f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2)}
_ULP_BITS = {"f32": 23, "f16": 10, "bf16": 7}


def desc_of(wl: PI.Workload):
    import rank_decode_attention_amd as R
    r = PI.ranks(wl).tolist()
    return R.AttnDesc(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.n_groups, r, r, use_rope=wl.use_rope,
                      rope_base=wl.rope_base, latent_dtype=wl.latent, act_dtype=wl.act)


def _torch_dtype(fmt: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[fmt]


def to_device(arr: np.ndarray, fmt: str, device="cuda"):
    """Upload an array in a stored format ('bf16' = uint16 bits) as a torch tensor."""
    import torch
    if fmt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def from_device(t) -> np.ndarray:
    import torch
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype != torch.float32 else \
        t.detach().cpu().numpy().astype(np.float64)


def padded_rows(arr: np.ndarray, fmt: str, r: int) -> np.ndarray:
    """[n][r] stored-format rows -> [n][pitch] bytes with zero row padding."""
    import rank_decode_attention_amd as R
    esz = 4 if fmt == "f32" else 2
    pitch = R.row_pitch(fmt, r)
    n = arr.shape[0]
    out = np.zeros((n, pitch // esz), dtype=arr.dtype)
    out[:, :r] = arr
    return out.view(np.uint8)


class LazyLatents:
    """zk[j][b] / zv[j][b] in fp64 for the oracle, regenerated on demand."""

    def __init__(self, wl: PI.Workload, which: str, j: int, lens: np.ndarray):
        self.wl, self.which, self.j, self.lens = wl, which, j, lens

    def __getitem__(self, b):
        L = int(self.lens[b])
        if self.wl.latent == "i4":
            packed, scales = PI.latent_int4(self.wl, self.which, b, self.j, n=max(L, 1))
            return oracle.int4_latent(packed, scales, int(PI.ranks(self.wl)[self.j]))
        a = PI.latent(self.wl, self.which, b, self.j, n=max(L, 1))
        return oracle.upcast(a, self.wl.latent)


def build_decode_case(wl: PI.Workload, q_scale: float = 1.0, lens: Optional[np.ndarray] = None,
                      device="cuda") -> Dict:
    """Device inputs of one decode step of workload wl (fp16/bf16/fp32 or int4 latents)."""
    import torch
    import rank_decode_attention_amd as R
    desc = desc_of(wl)
    ranks = PI.ranks(wl)
    lens = PI.lengths(wl) if lens is None else np.asarray(lens, dtype=np.int32)
    q = PI.query(wl)
    if q_scale != 1.0:
        q = PI.to_format(oracle.upcast(q, wl.act).astype(np.float32) * np.float32(q_scale), wl.act)
    Bk = [PI.factor(wl, "Bk", j) for j in range(wl.n_groups)]
    Bv = [PI.factor(wl, "Bv", j) for j in range(wl.n_groups)]

    def rows(which, b, j):
        n = int(min(max(lens[b], 1), wl.max_len))
        if wl.latent == "i4":
            return PI.latent_int4(wl, "k" if which == 0 else "v", b, j, n=n)
        a = PI.latent(wl, "k" if which == 0 else "v", b, j, n=n)
        return padded_rows(a, wl.latent, int(ranks[j]))

    cache = R.fill_cache(desc, wl.batch, wl.max_len, rows, device=device)
    catB = lambda Bs: to_device(np.concatenate([b.reshape(-1) for b in Bs]), wl.act, device)
    ws = torch.empty(R.decode_workspace_bytes(desc, wl.batch, wl.max_len), dtype=torch.uint8, device=device)
    out = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=_torch_dtype(wl.act), device=device)
    return dict(wl=wl, desc=desc, cache=cache, q=to_device(q, wl.act, device), q_host=q, Bk=catB(Bk), Bv=catB(Bv),
                Bk_host=Bk, Bv_host=Bv, lens=lens, seq_lens=torch.from_numpy(lens).to(device), ws=ws, out=out,
                sm_scale=1.0 / math.sqrt(wl.head_dim))


def paged_from(case: Dict, page_size: int, seed: int = 0, extra_pages: int = 3, share_first: bool = False):
    """Scatter the latent rows of a contiguous decode case into pages of
    page_size tokens placed in random order in the pools (data placement
    only).  Pool bytes that no history reaches, and rows past a history,
    are 0xFF.  share_first: sequence 1's first page is sequence 0's (its
    rows must then be equal in the contiguous cache too, which this makes
    so).  Returns (PagedCache, block_table numpy)."""
    import torch
    import rank_decode_attention_amd as R
    wl, desc, lens, cache = case["wl"], case["desc"], case["lens"], case["cache"]
    ps, batch, max_len = int(page_size), wl.batch, wl.max_len
    q4 = desc.latent_dtype == "i4"
    host = {(w, sc): (cache.sv if sc else cache.zv) if w else (cache.sk if sc else cache.zk)
            for w in (0, 1) for sc in ((False, True) if q4 else (False,))}
    host = {k: t.cpu().numpy() for k, t in host.items()}
    if share_first:
        assert batch >= 2 and lens[0] >= ps and lens[1] >= ps
        for (w, sc), buf in host.items():
            ranks = desc.rank_v if w else desc.rank_k
            for j in range(desc.n_groups):
                pitch = R.scale_pitch(ranks[j]) if sc else R.row_pitch(desc.latent_dtype, ranks[j])
                o0 = R.latent_offset(desc, max_len, w, sc, 0, j, 0)
                o1 = R.latent_offset(desc, max_len, w, sc, 1, j, 0)
                buf[o1:o1 + ps * pitch] = buf[o0:o0 + ps * pitch]
        for (w, sc), buf in host.items():
            t = (cache.sv if sc else cache.zv) if w else (cache.sk if sc else cache.zk)
            t.copy_(torch.from_numpy(buf))
    npg = [(int(L) + ps - 1) // ps for L in lens]
    total = sum(npg) + extra_pages
    rng = np.random.default_rng(seed)
    perm = rng.permutation(total)
    max_pages = (max_len + ps - 1) // ps
    bt = np.full((batch, max_pages), -1, dtype=np.int32)
    i = 0
    for b in range(batch):
        for k in range(npg[b]):
            if share_first and b == 1 and k == 0:
                bt[1, 0] = bt[0, 0]
                continue
            bt[b, k] = perm[i]
            i += 1
    pools = {}
    for (w, sc), buf in host.items():
        pool = np.full(max(16, R.latent_bytes(desc, total, ps, w, sc)), 0xFF, dtype=np.uint8)
        ranks = desc.rank_v if w else desc.rank_k
        for b in range(batch):
            for j in range(desc.n_groups):
                pitch = R.scale_pitch(ranks[j]) if sc else R.row_pitch(desc.latent_dtype, ranks[j])
                for k in range(npg[b]):
                    t0, t1 = k * ps, min((k + 1) * ps, int(lens[b]))
                    src = R.latent_offset(desc, max_len, w, sc, b, j, t0)
                    dst = R.latent_offset(desc, ps, w, sc, int(bt[b, k]), j, 0)
                    pool[dst:dst + (t1 - t0) * pitch] = buf[src:src + (t1 - t0) * pitch]
        pools[(w, sc)] = torch.from_numpy(pool).cuda()
    pc = R.PagedCache(pools[(0, False)], pools[(1, False)], pools.get((0, True)), pools.get((1, True)),
                      torch.from_numpy(bt).cuda(), ps, total)
    return pc, bt


def run_decode_paged(case: Dict, pc, q_pos=None):
    import torch
    import rank_decode_attention_amd as R
    out = torch.empty_like(case["out"])
    # (the workspace is sized for the paged history bound, max_pages * page_size)
    wsb = R.decode_workspace_bytes(case["desc"], case["wl"].batch, pc.max_pages * pc.page_size)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    R.palu_decode_attn_paged(case["desc"], case["q"], pc, case["Bk"], case["Bv"], case["seq_lens"], q_pos,
                             case["sm_scale"], out, ws)
    torch.cuda.synchronize()
    return from_device(out)


def run_decode(case: Dict, q_pos=None):
    import torch
    import rank_decode_attention_amd as R
    R.palu_decode_attn(case["desc"], case["q"], case["cache"], case["Bk"], case["Bv"], case["seq_lens"], q_pos,
                       case["sm_scale"], case["out"], case["ws"])
    torch.cuda.synchronize()
    return from_device(case["out"])


def oracle_decode(case: Dict, heads: Optional[Sequence[Tuple[int, int]]] = None, q_pos=None) -> np.ndarray:
    wl = case["wl"]
    lens = case["lens"]
    zk = [LazyLatents(wl, "k", j, lens) for j in range(wl.n_groups)]
    zv = [LazyLatents(wl, "v", j, lens) for j in range(wl.n_groups)]
    Bk = [oracle.upcast(b, wl.act) for b in case["Bk_host"]]
    Bv = [oracle.upcast(b, wl.act) for b in case["Bv_host"]]
    q = oracle.upcast(case["q_host"], wl.act)
    return oracle.decode_attention(q, zk, zv, Bk, Bv, lens, q_pos, n_kv_heads=wl.n_kv_heads,
                                   use_rope=wl.use_rope, rope_base=wl.rope_base, sm_scale=case["sm_scale"],
                                   heads=heads)


def run_chunk(case: Dict, q_len: int, paged=None):
    """Chunk attention of q_len seeded queries per sequence over the case's
    cache (or a PagedCache of the same rows); returns (gpu, host queries)."""
    import torch
    import rank_decode_attention_amd as R
    wl = case["wl"]
    qh = PI.query_chunk(wl, q_len)
    q = to_device(qh, wl.act)
    out = torch.empty(qh.shape, dtype=_torch_dtype(wl.act), device="cuda")
    cache = paged if paged is not None else case["cache"]
    if paged is not None:
        wsb = R.chunk_workspace_bytes(case["desc"], wl.batch, q_len, paged.max_pages * paged.page_size, paged.max_pages)
    else:
        wsb = R.chunk_workspace_bytes(case["desc"], wl.batch, q_len, wl.max_len, 1)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    R.palu_decode_attn_chunk(case["desc"], q, cache, case["Bk"], case["Bv"], case["seq_lens"], case["sm_scale"], out, ws)
    torch.cuda.synchronize()
    return from_device(out), qh


def oracle_chunk(case: Dict, qh: np.ndarray) -> np.ndarray:
    wl, lens = case["wl"], case["lens"]
    zk = [LazyLatents(wl, "k", j, lens) for j in range(wl.n_groups)]
    zv = [LazyLatents(wl, "v", j, lens) for j in range(wl.n_groups)]
    Bk = [oracle.upcast(b, wl.act) for b in case["Bk_host"]]
    Bv = [oracle.upcast(b, wl.act) for b in case["Bv_host"]]
    return oracle.chunk_attention(oracle.upcast(qh, wl.act), zk, zv, Bk, Bv, lens, n_kv_heads=wl.n_kv_heads,
                                  use_rope=wl.use_rope, rope_base=wl.rope_base, sm_scale=case["sm_scale"])


def half_ulp(ref: np.ndarray, fmt: str) -> np.ndarray:
    mag = np.maximum(np.abs(ref), 2.0 ** -14)
    return 0.5 * 2.0 ** (np.floor(np.log2(mag)) - _ULP_BITS[fmt])


# every comparison of the session: (what, fmt, elements, max_abs, max |err| / allowance, rel, rel / rtol),
# written out by tests/conftest.py when PALU_PARITY_SUMMARY names a file
RESULTS: List[Tuple[str, str, int, float, float, float, float]] = []


def compare(gpu: np.ndarray, ref: np.ndarray, fmt: str, what: str = "") -> Dict[str, float]:
    atol, rtol = TOL[fmt]
    err = np.abs(gpu - ref)
    allow = atol + (half_ulp(ref, fmt) if fmt != "f32" else 0.0)
    rel = float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30))
    stats = dict(max_abs=float(err.max()) if err.size else 0.0, rel=rel)
    used = float((err / allow).max()) if err.size else 0.0
    RESULTS.append((what, fmt, int(err.size), stats["max_abs"], used, rel, rel / rtol))
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    bad = err > allow
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond tolerance, max_abs={stats['max_abs']:.3e}"
    assert rel <= rtol, f"{what}: relative error {rel:.3e} > {rtol}"
    return stats
