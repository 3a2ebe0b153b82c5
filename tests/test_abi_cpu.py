"""CPU-side checks of the C-ABI library: it loads, exports every entry point
declared in include/palu.h, and rejects bad arguments on the host before any
HIP call.  No kernel is launched here."""
import ctypes
import os
import re

import pytest

import rank_decode_attention_amd as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INVALID, UNSUP, WS, HIP = 1, 2, 3, 4


def _declared():
    with open(os.path.join(ROOT, "include", "palu.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(palu_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    if not os.path.exists(R.lib_path()):
        pytest.skip("libpalu.so not built")
    lib = R.load()
    names = _declared()
    assert {"palu_decode_attn", "palu_project", "palu_quant_latent"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(R.lib_path()):
        pytest.skip("libpalu.so not built")
    return R.load()


def _desc(**kw):
    base = dict(n_q_heads=32, n_kv_heads=32, head_dim=128, n_groups=8, rank_k=[256] * 8, latent_dtype="f16")
    base.update(kw)
    return R.AttnDesc(**base)


def test_status_strings(lib):
    assert lib.palu_status_string(0) == b"PALU_OK"
    assert lib.palu_status_string(3) == b"PALU_ERR_WORKSPACE_TOO_SMALL"


def test_layout_host_logic(lib):
    d = _desc()
    # f16 rank 256: 512-byte rows, 8 groups per sequence block
    assert R.latent_bytes(d, 2, 100, 0) == 2 * 8 * 100 * 512
    assert R.latent_offset(d, 100, 0, False, 1, 3, 7) == 1 * 8 * 100 * 512 + 3 * 100 * 512 + 7 * 512
    # ragged ranks and rank not a multiple of 8: rows pad to 16 bytes
    d2 = _desc(n_groups=2, n_kv_heads=32, rank_k=[154, 40], latent_dtype="bf16")
    assert R.row_pitch("bf16", 154) == 320 and R.row_pitch("bf16", 40) == 80
    assert R.latent_offset(d2, 10, 1, False, 0, 1, 2) == 10 * 320 + 2 * 80
    # int4: 16 bytes per 32 elements, scales 2 bytes per 32 elements
    d3 = _desc(rank_k=[154] * 8, latent_dtype="i4", act_dtype="f16")
    assert R.latent_bytes(d3, 1, 4, 1) == 8 * 4 * 80
    assert R.latent_bytes(d3, 1, 4, 1, scales=True) == 8 * 4 * 10
    assert R.latent_offset(d3, 4, 0, True, 0, 2, 3) == 2 * 4 * 10 + 3 * 10
    # scales of a float layout and out-of-range coordinates are errors
    assert lib.palu_latent_bytes(d.ref(), 1, 4, 0, 1) == 0
    assert lib.palu_latent_offset(d.ref(), 4, 0, 0, 0, 8, 0) == -1
    assert lib.palu_latent_offset(d.ref(), 4, 0, 0, 0, 0, 4) == -1


def _call_decode(lib, d, batch=1, sm_scale=0.1, null=None, max_len=64, ws_bytes=1 << 20):
    cache = R._Cache(16, 16, None, None, max_len)
    ptr = {k: ctypes.c_void_p(256) for k in ("q", "Bk", "Bv", "lens", "out", "ws")}
    if null:
        ptr[null] = None
    return lib.palu_decode_attn(d.ref() if d is not None else None, ptr["q"], ctypes.byref(cache), ptr["Bk"],
                                ptr["Bv"], ptr["lens"], None, batch, sm_scale, ptr["out"], ptr["ws"], ws_bytes,
                                None)


def test_decode_argument_errors(lib):
    assert _call_decode(lib, None) == INVALID
    assert _call_decode(lib, _desc(n_q_heads=30)) == INVALID           # H % H_kv
    assert _call_decode(lib, _desc(n_groups=3, rank_k=[256] * 3)) == INVALID  # H_kv % G
    assert _call_decode(lib, _desc(head_dim=127)) == INVALID
    assert _call_decode(lib, _desc(rank_k=[256] * 7 + [0])) == INVALID
    assert _call_decode(lib, _desc(n_groups=32, rank_k=[64] * 32)) == UNSUP  # more groups than supported
    assert _call_decode(lib, _desc(), batch=-1) == INVALID
    assert _call_decode(lib, _desc(), max_len=0) == INVALID
    assert _call_decode(lib, _desc(), batch=5000) == UNSUP
    assert _call_decode(lib, _desc(latent_dtype="i4", act_dtype="f32")) == UNSUP
    assert _call_decode(lib, _desc(latent_dtype="f16", act_dtype="bf16")) == UNSUP
    assert _call_decode(lib, _desc(head_dim=96)) == UNSUP                # no kernel for this head_dim
    assert _call_decode(lib, _desc(rank_k=[512] * 8)) == UNSUP          # rank above every compiled cap
    assert b"no decode kernel" in lib.palu_last_error()


def test_decode_paged_argument_errors(lib):
    d = _desc()
    p = ctypes.c_void_p(256)

    def call(page_size=64, max_pages=4, n_pages=8, table=p, batch=1):
        cache = R._PagedCache(16, 16, None, None, table, page_size, max_pages, n_pages)
        return lib.palu_decode_attn_paged(d.ref(), p, ctypes.byref(cache), p, p, p, None, batch, 0.1, p, p, 1 << 20,
                                          None)
    assert call(page_size=48) == INVALID        # not a power of two
    assert call(page_size=16) == INVALID        # below one tile
    assert call(max_pages=0) == INVALID
    assert call(n_pages=0) == INVALID
    assert call(table=None) == INVALID
    assert b"block_table" in lib.palu_last_error()
    assert lib.palu_decode_attn_paged(d.ref(), p, None, p, p, p, None, 1, 0.1, p, p, 1 << 20, None) == INVALID


def test_chunk_argument_errors(lib):
    d = _desc()
    p = ctypes.c_void_p(256)
    cache = R._Cache(16, 16, None, None, 64)
    call = lambda q_len, batch=1: lib.palu_decode_attn_chunk(d.ref(), p, q_len, ctypes.byref(cache), p, p, p, batch,
                                                             0.1, p, p, 1 << 30, None)
    assert call(0) == INVALID
    assert call(-2) == INVALID
    assert call(64, batch=64) == UNSUP                 # more than 2048 virtual sequences
    assert lib.palu_decode_chunk_workspace_bytes(d.ref(), 1, 0, 64, 1) == 0


def test_quant_argument_errors(lib):
    p = ctypes.c_void_p(256)
    assert lib.palu_quant_latent(None, 0, 4, 32, 32, p, p, None) == INVALID
    assert lib.palu_quant_latent(p, 0, -1, 32, 32, p, p, None) == INVALID
    assert lib.palu_quant_latent(p, 0, 4, 0, 32, p, p, None) == INVALID
    assert lib.palu_quant_latent(p, 0, 4, 40, 32, p, p, None) == INVALID   # stride < r
    assert lib.palu_quant_latent(p, 3, 4, 32, 32, p, p, None) == UNSUP     # int4 input
    assert lib.palu_quant_latent(p, 0, 4, 32, 32, ctypes.c_void_p(8), p, None) == INVALID  # misaligned codes
    assert lib.palu_quant_latent(p, 0, 0, 32, 32, p, p, None) == 0        # nothing to do
    # rows more than 64 MiB apart (the kernel addresses 34 rows with 32-bit offsets)
    assert lib.palu_quant_latent(p, 0, 4, 32, (1 << 24) + 1, p, p, None) == UNSUP     # fp32: 4 B per element
    assert lib.palu_quant_latent(p, 1, 4, 32, (1 << 25) + 1, p, p, None) == UNSUP     # fp16: 2 B per element
    assert lib.palu_quant_latent_rotated(p, 2, 4, 32, (1 << 25) + 1, p, p, None) == UNSUP


def test_dequant_argument_errors(lib):
    p = ctypes.c_void_p(256)
    assert lib.palu_dequant_latent(None, p, 4, 32, 1, p, None) == INVALID
    assert lib.palu_dequant_latent(p, p, -1, 32, 1, p, None) == INVALID
    assert lib.palu_dequant_latent(p, p, 4, 0, 1, p, None) == INVALID
    assert lib.palu_dequant_latent(p, p, 4, 32, 0, p, None) == UNSUP        # fp32 output
    assert lib.palu_dequant_latent(p, p, 4, 32, 3, p, None) == UNSUP        # int4 output
    assert lib.palu_dequant_latent(ctypes.c_void_p(258), p, 4, 32, 1, p, None) == INVALID  # codes misaligned
    assert lib.palu_dequant_latent(p, ctypes.c_void_p(257), 4, 32, 1, p, None) == INVALID  # scales misaligned
    assert lib.palu_dequant_latent(p, p, 4, 32, 1, ctypes.c_void_p(264), None) == INVALID  # out misaligned
    assert lib.palu_dequant_latent(p, p, 1 << 23, 1024, 1, p, None) == UNSUP  # too many rows for one call
    assert lib.palu_dequant_latent(p, p, 0, 32, 1, p, None) == 0            # nothing to do


def test_project_argument_errors(lib):
    d = _desc()
    p = ctypes.c_void_p(256)
    cache = R._Cache(256, 256, None, None, 64)
    assert lib.palu_project(d.ref(), None, 4096, 8, p, ctypes.byref(cache), 0, 0, None) == INVALID
    assert lib.palu_project(d.ref(), p, 4096, 8, p, ctypes.byref(cache), 0, 60, None) == INVALID  # past max_len
    assert lib.palu_project(d.ref(), p, 4000, 8, p, ctypes.byref(cache), 0, 0, None) == UNSUP    # d_model % 64
    d4 = _desc(latent_dtype="i4", act_dtype="f16")
    assert lib.palu_project(d4.ref(), p, 4096, 8, p, ctypes.byref(cache), 0, 0, None) == INVALID  # no scales
    assert lib.palu_project(d.ref(), p, 4096, 0, p, ctypes.byref(cache), 0, 0, None) == 0         # nothing to do
    # latent rows are cut into column tiles of 160 channels, at most 256 per call:
    # 32 rows of rank 1280 fit (8 tiles each), rank 1300 (9 each) does not
    wide = _desc(n_groups=16, rank_k=[1300] * 16)
    assert lib.palu_project(wide.ref(), p, 4096, 8, p, ctypes.byref(cache), 0, 0, None) == UNSUP
