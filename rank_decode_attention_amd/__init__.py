"""Python binding of libpalu (Palu decode attention over a low-rank latent KV cache).

Argument marshalling only: every step of the method runs in the HIP kernels
of ``libpalu.so`` behind the C ABI declared in ``include/palu.h``.  PyTorch
provides device memory and streams.  The names mirror the C entry points:
``palu_project``, ``palu_quant_latent``, ``palu_decode_attn`` and the layout /
workspace queries.  There is no fallback path: if the library is missing or
a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "PaluError", "AttnDesc", "LatentCache", "PagedCache", "lib_path", "load",
    "latent_bytes", "latent_offset", "row_pitch", "scale_pitch", "alloc_cache", "fill_cache",
    "fill_paged_cache", "decode_workspace_bytes", "palu_decode_attn", "palu_decode_attn_paged", "palu_project",
    "palu_project_paged", "palu_quant_latent", "palu_dequant_latent", "palu_profile_events",
    "chunk_workspace_bytes", "palu_decode_attn_chunk", "palu_decode_attn_noalloc", "NOALLOC_SCRATCH_BYTES",
    "palu_quant_latent_rotated",
]

_DIR = os.path.dirname(os.path.abspath(__file__))
_DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "i4": 3}
_ESZ = {"f32": 4, "f16": 2, "bf16": 2}


def lib_path() -> str:
    return os.path.join(_DIR, "libpalu.so")


class PaluError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status
        self.name = name
        self.detail = detail


class _Desc(ctypes.Structure):
    _fields_ = [
        ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("n_groups", ctypes.c_int32), ("rank_k", ctypes.POINTER(ctypes.c_int32)),
        ("rank_v", ctypes.POINTER(ctypes.c_int32)), ("use_rope", ctypes.c_int32), ("rope_base", ctypes.c_double),
        ("latent_dtype", ctypes.c_int), ("act_dtype", ctypes.c_int),
    ]


class _Cache(ctypes.Structure):
    _fields_ = [("zk", ctypes.c_void_p), ("zv", ctypes.c_void_p), ("sk", ctypes.c_void_p), ("sv", ctypes.c_void_p),
                ("max_len", ctypes.c_int32)]


class _PagedCache(ctypes.Structure):
    _fields_ = [("zk", ctypes.c_void_p), ("zv", ctypes.c_void_p), ("sk", ctypes.c_void_p), ("sv", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("n_pages", ctypes.c_int32)]


_LIB = None


def load():
    """Load libpalu.so (after torch, so that both use the same HIP runtime)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    import torch  # noqa: F401  (loads torch's libamdhip64 first; the library binds to it by soname)
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m rank_decode_attention_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D, C = ctypes.POINTER(_Desc), ctypes.POINTER(_Cache)
    lib.palu_status_string.argtypes = [ctypes.c_int]
    lib.palu_status_string.restype = ctypes.c_char_p
    lib.palu_last_error.argtypes = []
    lib.palu_last_error.restype = ctypes.c_char_p
    lib.palu_latent_bytes.argtypes = [D, i32, i32, i32, i32]
    lib.palu_latent_bytes.restype = sz
    lib.palu_latent_offset.argtypes = [D, i32, i32, i32, i32, i32, i32]
    lib.palu_latent_offset.restype = i64
    lib.palu_quant_latent.argtypes = [vp, ctypes.c_int, i64, i32, i64, vp, vp, vp]
    lib.palu_quant_latent.restype = ctypes.c_int
    lib.palu_quant_latent_rotated.argtypes = [vp, ctypes.c_int, i64, i32, i64, vp, vp, vp]
    lib.palu_quant_latent_rotated.restype = ctypes.c_int
    lib.palu_dequant_latent.argtypes = [vp, vp, i64, i32, ctypes.c_int, vp, vp]
    lib.palu_dequant_latent.restype = ctypes.c_int
    lib.palu_project.argtypes = [D, vp, i32, i64, vp, C, i32, i32, vp]
    lib.palu_project_paged.argtypes = [D, vp, i32, i64, vp, ctypes.POINTER(_PagedCache), i32, i32, vp]
    lib.palu_project_paged.restype = ctypes.c_int
    lib.palu_project.restype = ctypes.c_int
    lib.palu_decode_workspace_bytes.argtypes = [D, i32, i32]
    lib.palu_decode_workspace_bytes.restype = sz
    lib.palu_decode_attn.argtypes = [D, vp, C, vp, vp, vp, vp, i32, ctypes.c_float, vp, vp, sz, vp]
    lib.palu_decode_attn.restype = ctypes.c_int
    lib.palu_decode_attn_noalloc.argtypes = [D, vp, C, vp, vp, vp, vp, i32, ctypes.c_float, vp, vp]
    lib.palu_decode_attn_noalloc.restype = ctypes.c_int
    lib.palu_decode_attn_paged.argtypes = [D, vp, ctypes.POINTER(_PagedCache), vp, vp, vp, vp, i32, ctypes.c_float,
                                           vp, vp, sz, vp]
    lib.palu_decode_attn_paged.restype = ctypes.c_int
    lib.palu_decode_attn_chunk.argtypes = [D, vp, i32, C, vp, vp, vp, i32, ctypes.c_float, vp, vp, sz, vp]
    lib.palu_decode_attn_chunk.restype = ctypes.c_int
    lib.palu_decode_attn_chunk_paged.argtypes = [D, vp, i32, ctypes.POINTER(_PagedCache), vp, vp, vp, i32,
                                                 ctypes.c_float, vp, vp, sz, vp]
    lib.palu_decode_attn_chunk_paged.restype = ctypes.c_int
    lib.palu_decode_chunk_workspace_bytes.argtypes = [D, i32, i32, i32, i32]
    lib.palu_decode_chunk_workspace_bytes.restype = sz
    lib.palu_profile_events.argtypes = [vp, vp]
    lib.palu_profile_events.restype = ctypes.c_int
    _LIB = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = load()
        raise PaluError(status, lib.palu_status_string(status).decode(), lib.palu_last_error().decode())


class AttnDesc:
    """One attention layer (mirrors palu_attn_desc)."""

    def __init__(self, n_q_heads: int, n_kv_heads: int, head_dim: int, n_groups: int,
                 rank_k: Sequence[int], rank_v: Optional[Sequence[int]] = None, *, use_rope: bool = True,
                 rope_base: float = 10000.0, latent_dtype: str = "f16", act_dtype: Optional[str] = None):
        self.n_q_heads, self.n_kv_heads, self.head_dim, self.n_groups = n_q_heads, n_kv_heads, head_dim, n_groups
        self.rank_k = [int(r) for r in rank_k]
        self.rank_v = [int(r) for r in (rank_v if rank_v is not None else rank_k)]
        self.use_rope, self.rope_base = bool(use_rope), float(rope_base)
        self.latent_dtype = latent_dtype
        self.act_dtype = act_dtype or (latent_dtype if latent_dtype != "i4" else "f16")
        self._rk = (ctypes.c_int32 * max(1, len(self.rank_k)))(*self.rank_k)
        self._rv = (ctypes.c_int32 * max(1, len(self.rank_v)))(*self.rank_v)
        self._c = _Desc(n_q_heads, n_kv_heads, head_dim, n_groups, self._rk, self._rv, int(self.use_rope),
                        self.rope_base, _DTYPES[latent_dtype], _DTYPES[self.act_dtype])

    @property
    def group_width(self) -> int:
        return (self.n_kv_heads // self.n_groups) * self.head_dim

    def ref(self):
        return ctypes.byref(self._c)


class LatentCache:
    """Caller-owned latent buffers of one layer (uint8 device tensors)."""

    def __init__(self, zk, zv, sk=None, sv=None, max_len: int = 0):
        self.zk, self.zv, self.sk, self.sv, self.max_len = zk, zv, sk, sv, int(max_len)

    def c(self) -> _Cache:
        ptr = lambda t: None if t is None else t.data_ptr()
        return _Cache(ptr(self.zk), ptr(self.zv), ptr(self.sk), ptr(self.sv), self.max_len)


class PagedCache:
    """Caller-owned paged latent pools of one layer (uint8 device tensors) and
    the block table (int32 device tensor [batch][max_pages])."""

    def __init__(self, zk, zv, sk, sv, block_table, page_size: int, n_pages: int):
        self.zk, self.zv, self.sk, self.sv, self.block_table = zk, zv, sk, sv, block_table
        self.page_size, self.n_pages = int(page_size), int(n_pages)
        self.max_pages = int(block_table.shape[1])

    def c(self) -> _PagedCache:
        ptr = lambda t: None if t is None else t.data_ptr()
        return _PagedCache(ptr(self.zk), ptr(self.zv), ptr(self.sk), ptr(self.sv), ptr(self.block_table),
                           self.page_size, self.max_pages, self.n_pages)


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ------------------------------------------------------------------ layout
def row_pitch(dtype: str, r: int) -> int:
    """Bytes per latent row (the layout of include/palu.h)."""
    if dtype == "f32":
        return 4 * (-(-r // 4) * 4)
    if dtype in ("f16", "bf16"):
        return 2 * (-(-r // 8) * 8)
    return 16 * (-(-r // 32))


def scale_pitch(r: int) -> int:
    return 2 * (-(-r // 32))


def latent_bytes(desc: AttnDesc, batch: int, max_len: int, which: int, scales: bool = False) -> int:
    return int(load().palu_latent_bytes(desc.ref(), batch, max_len, which, int(scales)))


def latent_offset(desc: AttnDesc, max_len: int, which: int, scales: bool, b: int, j: int, t: int) -> int:
    off = int(load().palu_latent_offset(desc.ref(), max_len, which, int(scales), b, j, t))
    if off < 0:
        raise ValueError("invalid latent coordinates")
    return off


def alloc_cache(desc: AttnDesc, batch: int, max_len: int, device="cuda") -> LatentCache:
    import torch
    nb = lambda which, sc: max(16, latent_bytes(desc, batch, max_len, which, sc))
    zk = torch.zeros(nb(0, False), dtype=torch.uint8, device=device)
    zv = torch.zeros(nb(1, False), dtype=torch.uint8, device=device)
    sk = sv = None
    if desc.latent_dtype == "i4":
        sk = torch.zeros(nb(0, True), dtype=torch.uint8, device=device)
        sv = torch.zeros(nb(1, True), dtype=torch.uint8, device=device)
    return LatentCache(zk, zv, sk, sv, max_len)


def fill_cache(desc: AttnDesc, batch: int, max_len: int, rows, device="cuda") -> LatentCache:
    """Build a cache from host rows: ``rows(which, b, j)`` returns a numpy array
    [n <= max_len][pitch_bytes] (uint8) or (codes, scales) byte arrays for I4.
    Pure data placement into the documented layout."""
    import torch
    bufs = {}
    for which in (0, 1):
        for sc in ((False, True) if desc.latent_dtype == "i4" else (False,)):
            bufs[(which, sc)] = np.zeros(max(16, latent_bytes(desc, batch, max_len, which, sc)), dtype=np.uint8)
    for which in (0, 1):
        ranks = desc.rank_k if which == 0 else desc.rank_v
        for b in range(batch):
            for j in range(desc.n_groups):
                data = rows(which, b, j)
                parts = data if isinstance(data, tuple) else (data,)
                for sc, arr in zip((False, True), parts):
                    pitch = scale_pitch(ranks[j]) if sc else row_pitch(desc.latent_dtype, ranks[j])
                    arr = np.ascontiguousarray(arr).view(np.uint8).reshape(arr.shape[0], -1)
                    assert arr.shape[1] == pitch and arr.shape[0] <= max_len, (arr.shape, pitch)
                    off = latent_offset(desc, max_len, which, sc, b, j, 0)
                    bufs[(which, sc)][off:off + arr.size] = arr.reshape(-1)
    t = {k: torch.from_numpy(v).to(device) for k, v in bufs.items()}
    return LatentCache(t[(0, False)], t[(1, False)], t.get((0, True)), t.get((1, True)), max_len)


def fill_paged_cache(desc: AttnDesc, lens, page_size: int, rows, seed: int = 0, extra_pages: int = 0,
                     device="cuda") -> PagedCache:
    """Build a paged cache from host rows: ``rows(which, b, j)`` returns the
    first lens[b] rows of (sequence b, group j) as in fill_cache.  Pages are
    placed in a seeded random order in the pools (extra_pages unused pages,
    pool bytes no history reaches are zero).  Pure data placement."""
    import torch
    ps, batch = int(page_size), len(lens)
    npg = [(int(L) + ps - 1) // ps for L in lens]
    total = sum(npg) + int(extra_pages)
    max_pages = max(1, max(npg) if npg else 1)
    order = np.random.default_rng(seed).permutation(max(total, 1))
    table = np.full((batch, max_pages), -1, dtype=np.int32)
    i = 0
    for b in range(batch):
        for k in range(npg[b]):
            table[b, k] = order[i]
            i += 1
    pools = {}
    for which in (0, 1):
        ranks = desc.rank_k if which == 0 else desc.rank_v
        for sc in ((False, True) if desc.latent_dtype == "i4" else (False,)):
            pools[(which, sc)] = np.zeros(max(16, latent_bytes(desc, max(total, 1), ps, which, sc)), dtype=np.uint8)
        for b in range(batch):
            for j in range(desc.n_groups):
                data = rows(which, b, j)
                parts = data if isinstance(data, tuple) else (data,)
                for sc, arr in zip((False, True), parts):
                    pitch = scale_pitch(ranks[j]) if sc else row_pitch(desc.latent_dtype, ranks[j])
                    arr = np.ascontiguousarray(arr).view(np.uint8).reshape(arr.shape[0], -1)
                    assert arr.shape[1] == pitch, (arr.shape, pitch)
                    for k in range(npg[b]):
                        t0, t1 = k * ps, min((k + 1) * ps, int(lens[b]))
                        off = latent_offset(desc, ps, which, sc, int(table[b, k]), j, 0)
                        pools[(which, sc)][off:off + (t1 - t0) * pitch] = arr[t0:t1].reshape(-1)
    t = {k: torch.from_numpy(v).to(device) for k, v in pools.items()}
    return PagedCache(t[(0, False)], t[(1, False)], t.get((0, True)), t.get((1, True)),
                      torch.from_numpy(table).to(device), ps, max(total, 1))


# ------------------------------------------------------------------ entry points
def decode_workspace_bytes(desc: AttnDesc, batch: int, max_len: int) -> int:
    n = int(load().palu_decode_workspace_bytes(desc.ref(), batch, max_len))
    if n == 0:
        lib = load()
        raise PaluError(-1, "palu_decode_workspace_bytes", lib.palu_last_error().decode())
    return n


def palu_profile_events(before_main, after_main):
    """Set (or clear with None, None) HIP events that palu_decode_attn records
    around its main kernel, and palu_project around its projection kernel, on
    the calling thread (palu_profile_events)."""
    _check(load().palu_profile_events(before_main, after_main))


def palu_decode_attn(desc: AttnDesc, q, cache: LatentCache, B_k, B_v, seq_lens, q_pos, sm_scale: float, out,
                     workspace, stream=None):
    """One decode step (palu_decode_attn).  Tensors are device tensors in the
    layouts of include/palu.h; q_pos may be None."""
    c = cache.c()
    _check(load().palu_decode_attn(desc.ref(), q.data_ptr(), ctypes.byref(c), B_k.data_ptr(), B_v.data_ptr(),
                                   seq_lens.data_ptr(), None if q_pos is None else q_pos.data_ptr(),
                                   int(q.shape[0]), float(sm_scale), out.data_ptr(), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))


def palu_decode_attn_noalloc(desc: AttnDesc, q, cache: LatentCache, B_k, B_v, seq_lens, q_pos, sm_scale: float, out,
                             stream=None):
    """One decode step without a workspace argument (palu_decode_attn_noalloc):
    the library's static device scratch of NOALLOC_SCRATCH_BYTES is used."""
    c = cache.c()
    _check(load().palu_decode_attn_noalloc(desc.ref(), q.data_ptr(), ctypes.byref(c), B_k.data_ptr(), B_v.data_ptr(),
                                           seq_lens.data_ptr(), None if q_pos is None else q_pos.data_ptr(),
                                           int(q.shape[0]), float(sm_scale), out.data_ptr(), _stream(stream)))


# bytes of that scratch (PALU_NOALLOC_SCRATCH_BYTES in include/palu.h)
NOALLOC_SCRATCH_BYTES = 16 << 20


def palu_decode_attn_paged(desc: AttnDesc, q, cache: PagedCache, B_k, B_v, seq_lens, q_pos, sm_scale: float, out,
                           workspace, stream=None):
    """One decode step over a paged latent cache (palu_decode_attn_paged)."""
    c = cache.c()
    _check(load().palu_decode_attn_paged(desc.ref(), q.data_ptr(), ctypes.byref(c), B_k.data_ptr(), B_v.data_ptr(),
                                         seq_lens.data_ptr(), None if q_pos is None else q_pos.data_ptr(),
                                         int(q.shape[0]), float(sm_scale), out.data_ptr(), workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(), _stream(stream)))


def chunk_workspace_bytes(desc: AttnDesc, batch: int, q_len: int, max_len: int, max_pages: int = 1) -> int:
    n = int(load().palu_decode_chunk_workspace_bytes(desc.ref(), batch, q_len, max_len, max_pages))
    if n == 0:
        raise PaluError(-1, "palu_decode_chunk_workspace_bytes", load().palu_last_error().decode())
    return n


def palu_decode_attn_chunk(desc: AttnDesc, q, cache, B_k, B_v, seq_lens, sm_scale: float, out, workspace,
                           stream=None):
    """Causal attention of a chunk of q_len tokens per sequence
    (palu_decode_attn_chunk / _paged): q and out are [batch][q_len][H][d_h];
    cache is a LatentCache or a PagedCache."""
    paged = isinstance(cache, PagedCache)
    c = cache.c()
    fn = load().palu_decode_attn_chunk_paged if paged else load().palu_decode_attn_chunk
    _check(fn(desc.ref(), q.data_ptr(), int(q.shape[1]), ctypes.byref(c), B_k.data_ptr(), B_v.data_ptr(),
              seq_lens.data_ptr(), int(q.shape[0]), float(sm_scale), out.data_ptr(), workspace.data_ptr(),
              workspace.numel() * workspace.element_size(), _stream(stream)))


def palu_project(desc: AttnDesc, x, A_kv, cache: LatentCache, seq: int, pos0: int, stream=None):
    """Prefill latent write (palu_project): x [n_tok][d_model], A_kv [n_lat][d_model]."""
    c = cache.c()
    _check(load().palu_project(desc.ref(), x.data_ptr(), int(x.shape[1]), int(x.shape[0]), A_kv.data_ptr(),
                               ctypes.byref(c), int(seq), int(pos0), _stream(stream)))


def palu_project_paged(desc: AttnDesc, x, A_kv, cache: PagedCache, seq: int, pos0: int, stream=None):
    """Prefill latent write into a paged cache (palu_project_paged)."""
    c = cache.c()
    _check(load().palu_project_paged(desc.ref(), x.data_ptr(), int(x.shape[1]), int(x.shape[0]), A_kv.data_ptr(),
                                     ctypes.byref(c), int(seq), int(pos0), _stream(stream)))


def palu_dequant_latent(codes, scales, n_rows: int, r: int, out, stream=None):
    """int4 rows -> 16-bit rows (palu_dequant_latent); out is a float16 or
    bfloat16 device tensor of n_rows x 32*ceil(r/32) elements."""
    import torch
    dt = {torch.float16: 1, torch.bfloat16: 2}[out.dtype]
    _check(load().palu_dequant_latent(codes.data_ptr(), scales.data_ptr(), int(n_rows), int(r), dt, out.data_ptr(),
                                      _stream(stream)))


def palu_quant_latent_rotated(z, r: int, row_stride: int, codes, scales, stream=None):
    """Low-rank-aware int4 quantisation (palu_quant_latent_rotated): every full
    32-element chunk is rotated by the order-32 Hadamard matrix first."""
    import torch
    dt = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}[z.dtype]
    _check(load().palu_quant_latent_rotated(z.data_ptr(), dt, int(z.shape[0]), int(r), int(row_stride),
                                            codes.data_ptr(), scales.data_ptr(), _stream(stream)))


def palu_quant_latent(z, r: int, row_stride: int, codes, scales, stream=None):
    """int4 quantisation of latent rows (palu_quant_latent); z is a 2-D device
    tensor of float32 / float16 / bfloat16."""
    import torch
    dt = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}[z.dtype]
    n_rows = z.shape[0]
    _check(load().palu_quant_latent(z.data_ptr(), dt, int(n_rows), int(r), int(row_stride), codes.data_ptr(),
                                    scales.data_ptr(), _stream(stream)))
