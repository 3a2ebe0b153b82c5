"""Benchmark of palu_decode_attn on one MI355X.

Workload: one decode step of a Llama-2-7B-shaped attention layer over the
low-rank latent cache (batch 16, history 4096, 32 heads x 128, 8 head-groups
of 4 heads, rank 256 per group = 50% of the group width, fp16 latents and
factors, RoPE base 10000), synthetic seeded inputs resident in HBM.

A step is one palu_decode_attn call (every decode step of the method: query
rotation, latent streaming, key rebuild, RoPE, scores, online softmax, the
latent-space value accumulation, split merge and the B_v output projection).
Before each timed step a 1 GiB buffer is read once, so that no latent bytes
are served from the 256 MB Infinity Cache or the L2s (cold-cache timing); a
read pass leaves clean lines behind, where overwriting the buffer would
leave ~256 MB of dirty lines whose write-back competes with the step.

Output (stdout, one JSON line): decode tokens/s (batch / step time), plus
`roofline` for the dominant kernel (the decode kernel the library picks,
timed with HIP events stamped by its own dispatch) and `cpu_baseline` (the
fp64 oracle on the host cores on a bounded sample of the same workload).

Other modes: `--workload NAME` (any workload of palu_inputs; prefill
workloads time palu_project and palu_quant_latent), `--page-size N` (the
latents through a paged cache), `--q-len N` (chunk attention, N new tokens
per sequence).  `--gpus` above 1 is refused: the path runs on one GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published
# HBM bytes per launch of the main kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE
# passes, calibrated against a plain copy of known size; valid only for the
# kernel sources it was measured on (their hash is stored beside the figures).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "palu_decode_mha_kernel_llama2_7b_traffic.json")
KERNEL_SOURCES = ["decode.hip", "decode_mha.hip", "decode.h", "common.h", "int4.h"]
MFMA_F16_PEAK_TFLOPS = 2516.6  # MI355X dense fp16/bf16 MFMA, AMD published
METRIC = "decode attn tokens/s and latent GB/s (% of HBM peak) at Llama-2-7B shape"


def _hip():
    import torch  # noqa: F401  (torch's HIP runtime is the one in the process)
    lib = ctypes.CDLL("libamdhip64.so.7")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


def setup(wl, page_size: int = 0):
    import torch
    import palu_inputs as PI
    import rank_decode_attention_amd as R

    ranks = PI.ranks(wl)
    desc = R.AttnDesc(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.n_groups, ranks.tolist(), use_rope=wl.use_rope,
                      rope_base=wl.rope_base, latent_dtype=wl.latent, act_dtype=wl.act)
    lens = PI.lengths(wl)
    esz = 4 if wl.latent == "f32" else 2

    def rows(which, b, j):
        if wl.latent == "i4":
            return PI.latent_int4(wl, "k" if which == 0 else "v", b, j, n=max(int(lens[b]), 1))
        a = PI.latent(wl, "k" if which == 0 else "v", b, j, n=int(lens[b]))
        pitch = R.row_pitch(wl.latent, int(ranks[j]))
        out = np.zeros((a.shape[0], pitch // esz), dtype=a.dtype)
        out[:, :a.shape[1]] = a
        return out.view(np.uint8)

    if page_size:
        # paged cache: pages in a seeded random order, histories up to max_pages * page_size
        cache = R.fill_paged_cache(desc, lens, page_size, rows, seed=wl.seed)
        ws_len = cache.max_pages * cache.page_size
    else:
        cache = R.fill_cache(desc, wl.batch, wl.max_len, rows)
        ws_len = wl.max_len
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[wl.act]

    def dev(a):
        if wl.act == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    Bk = dev(np.concatenate([PI.factor(wl, "Bk", j).reshape(-1) for j in range(wl.n_groups)]))
    Bv = dev(np.concatenate([PI.factor(wl, "Bv", j).reshape(-1) for j in range(wl.n_groups)]))
    q = dev(PI.query(wl))
    seq_lens = torch.from_numpy(lens).cuda()
    ws = torch.empty(R.decode_workspace_bytes(desc, wl.batch, ws_len), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=tdt, device="cuda")
    if wl.latent == "i4":
        # half a byte per code plus one binary16 scale per 32 elements, keys and values
        row_bytes = sum(int(r) / 2 + 2 * ((int(r) + 31) // 32) for r in ranks) * 2
        latent_bytes = int(sum(int(lens[b]) for b in range(wl.batch)) * row_bytes)
    else:
        latent_bytes = int(sum(int(lens[b]) * int(ranks.sum()) * 2 * esz for b in range(wl.batch)))
    n_lat = int(sum(int(lens[b]) for b in range(wl.batch)))
    nq = wl.n_q_heads // wl.n_groups
    # score side: the key rebuild with RoPE, the absorbed query against the
    # latent rows without; value side: P z_v of every query head
    if wl.use_rope:
        recon_flops = n_lat * sum(2 * int(r) * wl.group_width for r in ranks)
    else:
        recon_flops = n_lat * sum(2 * int(r) * nq for r in ranks)
    pv_flops = n_lat * sum(2 * int(r) * nq for r in ranks)
    return dict(desc=desc, cache=cache, paged=bool(page_size), Bk=Bk, Bv=Bv, q=q, seq_lens=seq_lens, ws=ws, out=out,
                sm_scale=1.0 / math.sqrt(wl.head_dim), latent_bytes=latent_bytes,
                flops=recon_flops + pv_flops, lens=lens)


def evict(scrub):
    """Cold caches: one read pass over a 1 GiB buffer (its result is dropped)."""
    if scrub is not None:
        import torch
        torch.amax(scrub.view(torch.int64))


def run_steps(st, steps, scrub, hip, ev_main):
    import torch
    import rank_decode_attention_amd as R
    t_call, t_main = [], []
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    mains = []
    for i in range(steps):
        evict(scrub)
        before, after = ctypes.c_void_p(), ctypes.c_void_p()
        if ev_main:
            hip.hipEventCreate(ctypes.byref(before))
            hip.hipEventCreate(ctypes.byref(after))
            R.palu_profile_events(before, after)
            mains.append((before, after))
        starts[i].record()
        call = R.palu_decode_attn_paged if st["paged"] else R.palu_decode_attn
        call(st["desc"], st["q"], st["cache"], st["Bk"], st["Bv"], st["seq_lens"], None, st["sm_scale"], st["out"],
             st["ws"])
        ends[i].record()
    R.palu_profile_events(None, None)
    torch.cuda.synchronize()
    for i in range(steps):
        t_call.append(starts[i].elapsed_time(ends[i]))
    for before, after in mains:
        ms = ctypes.c_float()
        hip.hipEventElapsedTime(ctypes.byref(ms), before, after)
        t_main.append(ms.value)
        hip.hipEventDestroy(before)
        hip.hipEventDestroy(after)
    return t_call, t_main


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "rank_decode_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch from the stored counter passes, or None when they
    were taken on other kernel sources or another workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash() or t.get("workload") != workload:
        return None
    return int(t["read_bytes_per_launch"] + t["write_bytes_per_launch"])


def copy_calibration(nbytes: int, reps: int):
    """A plain device-to-device copy of known size: its FETCH_SIZE / WRITE_SIZE
    counter readings give the scale from counter units to bytes."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4, "reps": reps}),
          flush=True)


def main_kernel_name(wl) -> str:
    """Name of the decode kernel the library runs for a workload: the fused
    MHA-group kernel where it applies (16-bit latents, head_dim 128, groups of
    4 kv heads with one query head each, RoPE, ranks multiples of 32 up to 256),
    the absorbed-query kernel without RoPE (16-bit latents, at most 8 query
    heads per group, ranks up to 320), the general split-attention kernel
    otherwise."""
    import palu_inputs as PI
    r = PI.ranks(wl)
    q4 = wl.latent == "i4"
    mha = ((wl.latent in ("f16", "bf16") or q4) and wl.head_dim == 128 and wl.kv_per_group == 4
           and wl.n_q_heads == wl.n_kv_heads and wl.use_rope
           and all((q4 or int(x) % 32 == 0) and int(x) <= 256 for x in r))
    if mha:
        # (int4 codes are expanded into the kernel's LDS tiles)
        return "palu_decode_mha_kernel (fused, MHA head-groups" + (", int4 codes)" if q4 else ")")
    nq = wl.n_q_heads // wl.n_groups
    if (not wl.use_rope and wl.latent in ("f16", "bf16", "i4") and nq <= 8
            and all(int(x) <= 320 for x in r)):
        # (int4 caches are first expanded to 16-bit rows of the rank rounded up to 32)
        return ("palu_dequant_kernel, then " if q4 else "") + "palu_decode_abs_kernel (absorbed query)"
    # (int4 caches are first expanded to 16-bit rows of the rank rounded up to 32)
    return ("palu_dequant_kernel, then " if q4 else "") + "palu_decode_kernel (split attention)"


def record_traffic(prof_dir: str, workload: str, copy_bytes: int, out_path: str = TRAFFIC_FILE):
    """Derive HBM bytes per main-kernel launch from four rocprofv3 --pmc runs
    under prof_dir (FETCH_SIZE / WRITE_SIZE of this benchmark, and of the
    copy calibration) and store them with the kernel sources' hash."""
    import csv
    import glob

    def values(sub, name_part):
        f = glob.glob(os.path.join(prof_dir, sub, "*counter_collection.csv"))[0]
        return [float(r["Counter_Value"]) for r in csv.DictReader(open(f)) if name_part in r["Kernel_Name"]]

    def med(v):
        return statistics.median(v)

    scale_r = copy_bytes / (1024 * med([v for v in values("copy_FETCH_SIZE", "copyBuffer") if v > 1024]))
    scale_w = copy_bytes / (1024 * med([v for v in values("copy_WRITE_SIZE", "copyBuffer") if v > 1024]))
    # (both decode kernels carry "palu_decode" in their names; the merge kernel does not)
    rd = med(values("FETCH_SIZE", "palu_decode")) * 1024 * scale_r
    wr = med(values("WRITE_SIZE", "palu_decode")) * 1024 * scale_w
    rec = {"workload": workload, "source_sha256": kernel_source_hash(), "kernel": "palu_decode",
           "read_bytes_per_launch": int(round(rd)), "write_bytes_per_launch": int(round(wr)),
           "fetch_scale": round(scale_r, 5), "write_scale": round(scale_w, 5),
           "how": "rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE (KiB per dispatch, median over dispatches), "
                  "each times the bytes-per-counted-byte of a plain copy of known size"}
    # (optional third pass: read requests that leave the L2 for the memory
    # side, in 32-byte units, scaled the same way; Infinity-Cache hits are
    # among them)
    if glob.glob(os.path.join(prof_dir, "DRAM_32B", "*counter_collection.csv")):
        scale_d = copy_bytes / (32 * med([v for v in values("copy_DRAM_32B", "copyBuffer") if v > 1024]))
        dr = med(values("DRAM_32B", "palu_decode")) * 32 * scale_d
        rec["l2_to_memory_read_bytes_per_launch"] = int(round(dr))
        rec["l2_to_memory_scale"] = round(scale_d, 5)
        rec["how_l2_to_memory"] = ("rocprofv3 --pmc TCC_EA0_RDREQ_DRAM_32B_sum (32-byte read requests from the L2 "
                                   "towards memory, median over dispatches), times the same calibration")
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def _blas_threads() -> int:
    """Threads of the BLAS the oracle's numpy calls run on."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(wl, n_seq: int, reps: int = 3):
    """The fp64 oracle (as it stands) on the first n_seq sequences of the workload."""
    import oracle
    import palu_inputs as PI
    cores = _blas_threads()
    n_seq = min(n_seq, wl.batch)
    lens = PI.lengths(wl)[:n_seq]

    def lat(which, b, j):
        if wl.latent == "i4":
            packed, scales = PI.latent_int4(wl, which, b, j, n=int(lens[b]))
            return oracle.int4_latent(packed, scales, int(PI.ranks(wl)[j]))
        return oracle.upcast(PI.latent(wl, which, b, j, n=int(lens[b])), wl.latent)
    zk = [[lat("k", b, j) for b in range(n_seq)] for j in range(wl.n_groups)]
    zv = [[lat("v", b, j) for b in range(n_seq)] for j in range(wl.n_groups)]
    Bk = [oracle.upcast(PI.factor(wl, "Bk", j), wl.act) for j in range(wl.n_groups)]
    Bv = [oracle.upcast(PI.factor(wl, "Bv", j), wl.act) for j in range(wl.n_groups)]
    q = oracle.upcast(PI.query(wl), wl.act)[:n_seq]
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.decode_attention(q, zk, zv, Bk, Bv, lens, n_kv_heads=wl.n_kv_heads, use_rope=wl.use_rope,
                                rope_base=wl.rope_base, sm_scale=1.0 / math.sqrt(wl.head_dim))
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    out = {"value": n_seq / t, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
           "sample": f"{n_seq} of {wl.batch} sequences (history {int(lens[0])}, all {wl.n_q_heads} heads), "
                     f"fp64 numpy, median of {reps} runs of {t:.2f} s"}
    try:
        # the same oracle on one host thread, first sequence only
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            oracle.decode_attention(q[:1], [z[:1] for z in zk], [z[:1] for z in zv], Bk, Bv, lens[:1],
                                    n_kv_heads=wl.n_kv_heads, use_rope=wl.use_rope, rope_base=wl.rope_base,
                                    sm_scale=1.0 / math.sqrt(wl.head_dim))
            t1 = time.perf_counter() - t0
        out["one_thread"] = {"value": 1 / t1, "unit": "tokens/s", "sample": f"1 sequence, one run of {t1:.2f} s"}
    except ImportError:  # pragma: no cover
        pass
    return out


def bench_prefill(wl, args, hip):
    """Prefill workloads (n_tok > 0): palu_project (z = x A for every latent
    row, int4-quantised in its epilogue when the cache is int4) over one chunk
    of n_tok tokens, and palu_quant_latent over the same number of latent rows
    on its own.  One JSON line; roofline: the projection against the dense
    MFMA peak of its dtype, the quantiser against HBM."""
    import torch
    import palu_inputs as PI
    import oracle
    import rank_decode_attention_amd as R

    ranks = PI.ranks(wl)
    desc = R.AttnDesc(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.n_groups, ranks.tolist(), use_rope=wl.use_rope,
                      rope_base=wl.rope_base, latent_dtype=wl.latent, act_dtype=wl.act)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[wl.act]

    def dev(a):
        if wl.act == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    n_tok = wl.n_tok
    x = dev(PI.prefill_x(wl))
    As = PI.prefill_A(wl)
    A_kv = dev(np.concatenate([a.T for a in As], axis=0))
    cache = R.alloc_cache(desc, 1, n_tok)
    n_lat = int(2 * ranks.sum())
    flops = 2.0 * n_tok * wl.d_model * n_lat
    scrub = None if args.no_scrub else torch.zeros(1 << 30, dtype=torch.uint8, device="cuda")

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ts = []
        for i in range(steps):
            evict(scrub)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ts.append((a, b))
        torch.cuda.synchronize()
        return statistics.mean(a.elapsed_time(b) for a, b in ts)

    ms_proj = timed(lambda: R.palu_project(desc, x, A_kv, cache, 0, 0), args.steps, args.warmup)
    # the projection kernel's own duration: dispatch-stamped events (the
    # library's timing hook) over as many calls again, after the timed ones
    mains = []
    for _ in range(args.steps):
        evict(scrub)
        before, after = ctypes.c_void_p(), ctypes.c_void_p()
        hip.hipEventCreate(ctypes.byref(before))
        hip.hipEventCreate(ctypes.byref(after))
        R.palu_profile_events(before, after)
        R.palu_project(desc, x, A_kv, cache, 0, 0)
        mains.append((before, after))
    R.palu_profile_events(None, None)
    torch.cuda.synchronize()
    kms = []
    for before, after in mains:
        ms = ctypes.c_float()
        hip.hipEventElapsedTime(ctypes.byref(ms), before, after)
        kms.append(ms.value)
        hip.hipEventDestroy(before)
        hip.hipEventDestroy(after)
    ms_kern = statistics.mean(kms)
    # the quantiser alone on n_tok x (2 G) latent rows of rank r in the activation format
    r = int(ranks[0])
    rows = [PI.latent_f32(wl, which, 0, j, n=n_tok) for which in ("k", "v") for j in range(wl.n_groups)]
    z = dev(PI.to_format(np.concatenate(rows), wl.act))
    nc = (r + 31) // 32
    codes = torch.empty((z.shape[0], 16 * nc), dtype=torch.uint8, device="cuda")
    scales = torch.empty((z.shape[0], nc), dtype=torch.int16, device="cuda")
    ms_q = timed(lambda: R.palu_quant_latent(z, r, r, codes, scales), args.steps, args.warmup)
    q_bytes = z.numel() * z.element_size() + codes.numel() + scales.numel() * 2

    line = {
        "metric": "prefill latent write tokens/s (palu_project, z = x A with the int4 epilogue)",
        "value": round(n_tok / (ms_proj * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_proj, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.act,
        "data": "synthetic (seeded N(0,1) activations, Gaussian A with std 1/sqrt(d_model))",
        "config": {"workload": f"{wl.name}: prefill chunk of {n_tok} tokens x d_model {wl.d_model}, {n_lat} latent "
                               f"columns ({wl.n_groups} groups, rank {r}, keys and values), {wl.latent} latents",
                   "global_batch": 1, "seq_len": n_tok, "parallelism": "single GPU",
                   "cache": "cold (1 GiB read pass before each step)" if scrub is not None else "warm"},
        "roofline": {"bound": "mfma", "achieved": round(flops / (ms_kern * 1e-3) / 1e12, 1),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / (ms_kern * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "palu_project_kernel", "kernel_ms": round(ms_kern, 4), "flops": flops,
                     "call_frac": round(flops / (ms_proj * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)},
        "quant_latent": {"rows": int(z.shape[0]), "rank": r, "ms": round(ms_q, 4), "bytes": int(q_bytes),
                         "bound": "hbm", "achieved_GBps": round(q_bytes / (ms_q * 1e-3) / 1e9, 1),
                         "frac": round(q_bytes / (ms_q * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    if args.cpu_seqs > 0:
        n_cpu = n_tok
        xs = oracle.upcast(PI.prefill_x(wl, n_cpu), wl.act)
        Aup = [oracle.upcast(a, wl.act) for a in As]
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            for a in Aup:
                zc = oracle.project(xs, a)
                if wl.latent == "i4":
                    oracle.quant_int4(zc.astype(np.float32))
            times.append(time.perf_counter() - t0)
        t = statistics.median(times)
        line["cpu_baseline"] = {"value": n_cpu / t, "unit": "tokens/s", "cores": _blas_threads(),
                                "kind": "oracle", "sample": f"{n_cpu} of {n_tok} tokens, every latent column, "
                                                             f"fp64 numpy, median of 3 runs of {t:.2f} s"}
    print(json.dumps(line), flush=True)


def bench_chunk(wl, args, hip):
    """Chunk attention (palu_decode_attn_chunk): q_len new tokens per
    sequence, causal within the chunk, over the workload's cache.  The
    queries run as batch * q_len decode sequences; `achieved` counts each
    sequence's latent bytes once (what the chunk has to read)."""
    import torch
    import palu_inputs as PI
    import rank_decode_attention_amd as R
    st = setup(wl, args.page_size)
    ql = args.q_len
    qh = PI.query_chunk(wl, ql)
    if wl.act == "bf16":
        q = torch.from_numpy(np.ascontiguousarray(qh).view(np.int16)).cuda().view(torch.bfloat16)
    else:
        q = torch.from_numpy(np.ascontiguousarray(qh)).cuda()
    out = torch.empty(q.shape, dtype=q.dtype, device="cuda")
    cache = st["cache"]
    if st["paged"]:
        wsb = R.chunk_workspace_bytes(st["desc"], wl.batch, ql, cache.max_pages * cache.page_size, cache.max_pages)
    else:
        wsb = R.chunk_workspace_bytes(st["desc"], wl.batch, ql, wl.max_len, 1)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    scrub = None if args.no_scrub else torch.zeros(1 << 30, dtype=torch.uint8, device="cuda")

    def call():
        R.palu_decode_attn_chunk(st["desc"], q, cache, st["Bk"], st["Bv"], st["seq_lens"], st["sm_scale"], out, ws)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    # the timed calls without the timing hook, then as many with it (the
    # decode kernel's own dispatch events)
    ts, mains = [], []
    for i in range(args.steps):
        evict(scrub)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        ts.append((a, b))
    torch.cuda.synchronize()
    for i in range(args.steps):
        evict(scrub)
        before, after = ctypes.c_void_p(), ctypes.c_void_p()
        hip.hipEventCreate(ctypes.byref(before))
        hip.hipEventCreate(ctypes.byref(after))
        R.palu_profile_events(before, after)
        call()
        mains.append((before, after))
    R.palu_profile_events(None, None)
    torch.cuda.synchronize()
    ms_step = statistics.mean(a.elapsed_time(b) for a, b in ts)
    kms = []
    for before, after in mains:
        ms = ctypes.c_float()
        hip.hipEventElapsedTime(ctypes.byref(ms), before, after)
        kms.append(ms.value)
        hip.hipEventDestroy(before)
        hip.hipEventDestroy(after)
    ms_main = statistics.mean(kms)
    achieved = st["latent_bytes"] / (ms_main * 1e-3) / 1e9
    line = {
        "metric": f"chunk attention tokens/s ({ql} new tokens per sequence, causal) at {wl.name} workload shape",
        "value": round(wl.batch * ql / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.act, "data": "synthetic (seeded latents, queries and factors)",
        "config": {"workload": f"{wl.name} with {ql}-token chunks", "global_batch": wl.batch, "seq_len": wl.max_len,
                   "q_len": ql, "parallelism": "single GPU",
                   "layout": f"paged, {args.page_size}-token pages" if args.page_size else "contiguous"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": main_kernel_name(wl),
                     "kernel_ms": round(ms_main, 4), "algorithmic_bytes": st["latent_bytes"]},
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama2_7b")
    ap.add_argument("--no-scrub", action="store_true", help="time with warm caches")
    ap.add_argument("--q-len", type=int, default=1,
                    help="new tokens per sequence: above 1, time the chunk attention (causal within the chunk)")
    ap.add_argument("--page-size", type=int, default=0,
                    help="read the latents through a paged cache with pages of this many tokens")
    ap.add_argument("--cpu-seqs", type=int, default=16,
                    help="sequences in the CPU-oracle sample (0: skip; prefill workloads: any value > 0 runs it on the whole chunk)")
    ap.add_argument("--detail", default="", help="also write a detailed JSON record to this path")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES (counter calibration) and exit")
    ap.add_argument("--record-traffic", default="", metavar="DIR",
                    help="derive the main kernel's HBM bytes from the counter runs under DIR and store them")
    ap.add_argument("--traffic-out", default=TRAFFIC_FILE, help="where --record-traffic writes")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.record_traffic, args.workload, 1 << 30, args.traffic_out)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the decode hot path measured "
              f"here runs on one GPU)", file=sys.stderr)
        sys.exit(2)

    import torch
    import palu_inputs as PI
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(1, args.steps))
        return
    wl = PI.workload(args.workload)
    hip = _hip()
    if wl.n_tok > 0:
        bench_prefill(wl, args, hip)
        return
    if args.q_len > 1:
        bench_chunk(wl, args, hip)
        return
    st = setup(wl, args.page_size)
    scrub = None if args.no_scrub else torch.zeros(1 << 30, dtype=torch.uint8, device="cuda")

    run_steps(st, args.warmup, scrub, hip, ev_main=False)
    torch.cuda.synchronize()
    # the K timed steps are the call as a caller makes it; the decode kernel's
    # own time comes from as many further calls with the timing hook set (the
    # dispatch events it attaches add a few microseconds to a call)
    t_call, _ = run_steps(st, args.steps, scrub, hip, ev_main=False)
    torch.cuda.synchronize()
    _, t_main = run_steps(st, args.steps, scrub, hip, ev_main=True)
    torch.cuda.synchronize()

    ms_step = statistics.mean(t_call)
    ms_main = statistics.mean(t_main)
    # warm caches (no scrub), for information
    n_w = max(5, args.steps // 5)
    t_call_w, _ = run_steps(st, n_w, None, hip, ev_main=False)
    _, t_main_w = run_steps(st, n_w, None, hip, ev_main=True)
    tokens_per_s = wl.batch / (ms_step * 1e-3)
    # int4 caches: the rate is taken over the whole call (where the expansion
    # runs as a kernel of its own, it is part of the step)
    ms_roof = ms_step if wl.latent == "i4" else ms_main
    achieved = st["latent_bytes"] / (ms_roof * 1e-3) / 1e9
    traffic = measured_traffic(wl.name)
    line = {
        "metric": METRIC if wl.name == "llama2_7b" else METRIC.replace("Llama-2-7B", f"{wl.name} workload"),
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.act,
        "data": "synthetic (seeded N(0,1) latents and queries, Gaussian factors with std 1/sqrt(fan_in))",
        "config": {
            "workload": f"{wl.name}: decode step, batch {wl.batch}, history {wl.max_len}, {wl.n_q_heads} heads x "
                        f"{wl.head_dim}, {wl.n_groups} head-groups of {wl.kv_per_group} kv heads, rank "
                        f"{int(PI.ranks(wl)[0])} per group, {wl.latent} latents, RoPE {wl.use_rope}",
            "global_batch": wl.batch, "seq_len": wl.max_len, "parallelism": "single GPU",
            "cache": "cold (1 GiB read pass before each step)" if scrub is not None else "warm",
            "layout": f"paged, {args.page_size}-token pages in random order" if args.page_size else "contiguous",
        },
        "ms_per_step_p10_p50_p90": [round(float(x), 4) for x in np.percentile(t_call, [10, 50, 90])],
        "warm": {"ms_per_step": round(statistics.mean(t_call_w), 4), "kernel_ms": round(statistics.mean(t_main_w), 4),
                 "cache": "warm (no scrub; latents partly served from the 256 MB Infinity Cache)"},
        "latent_GBps": round(st["latent_bytes"] / (ms_step * 1e-3) / 1e9, 1),
        "latent_frac_of_hbm_peak": round(st["latent_bytes"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": main_kernel_name(wl), "kernel_ms": round(ms_roof, 4),
            "decode_kernel_ms": round(ms_main, 4),
            "algorithmic_bytes": st["latent_bytes"],
            "mfma_frac_f16": round(st["flops"] / (ms_roof * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
        },
    }
    if args.cpu_seqs > 0:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seqs)
    if args.detail:
        with open(args.detail, "w") as f:
            json.dump({"line": line, "t_call_ms": t_call, "t_main_ms": t_main,
                       "t_call_p10_p50_p90": np.percentile(t_call, [10, 50, 90]).tolist()}, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
