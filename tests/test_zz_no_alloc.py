"""GPU: palu_decode_attn_noalloc (the workspace comes from the library's
static device scratch) against palu_decode_attn with a caller workspace,
through the C ABI: identical outputs on two calls in a row, the second with a
smaller input, on the MHA kernel (RoPE), the absorbed-query path (no RoPE)
and an int4 cache; a call whose workspace exceeds the scratch is refused."""
import ctypes

import numpy as np
import pytest

import palu_inputs as PI
from palu_cases import build_decode_case, compare, from_device, oracle_decode, run_decode

pytestmark = pytest.mark.gpu


def _noalloc(case):
    import torch
    import rank_decode_attention_amd as R
    out = torch.full_like(case["out"], float("nan"))
    R.palu_decode_attn_noalloc(case["desc"], case["q"], case["cache"], case["Bk"], case["Bv"], case["seq_lens"], None,
                               case["sm_scale"], out)
    torch.cuda.synchronize()
    return from_device(out)


SEQUENCES = [
    # (first call, second call with a smaller input)
    (PI.scaled("llama2_7b", batch=4, max_len=700, fixed_lengths=(700, 1, 333, 64), name="noalloc_7b_a"),
     PI.scaled("llama2_7b", batch=2, max_len=100, fixed_lengths=(100, 37), name="noalloc_7b_b")),
    (PI.scaled("gqa_norope", batch=3, max_len=300, fixed_lengths=(300, 0, 129), name="noalloc_norope_a"),
     PI.scaled("gqa_norope", batch=1, max_len=40, fixed_lengths=(40,), name="noalloc_norope_b")),
    (PI.scaled("int4", batch=3, max_len=400, fixed_lengths=(400, 5, 260), name="noalloc_int4_a"),
     PI.scaled("int4", batch=2, max_len=64, fixed_lengths=(64, 33), name="noalloc_int4_b")),
]


@pytest.mark.parametrize("first,second", SEQUENCES, ids=[a.name for a, _ in SEQUENCES])
def test_noalloc_matches_workspace_call(first, second):
    import rank_decode_attention_amd as R
    for wl in (first, second):
        case = build_decode_case(wl)
        assert R.decode_workspace_bytes(case["desc"], wl.batch, wl.max_len) <= R.NOALLOC_SCRATCH_BYTES
        want = run_decode(case)
        got = _noalloc(case)
        assert np.array_equal(got, want), f"{wl.name}: no-alloc call differs from the workspace call"
        compare(got, oracle_decode(case), wl.act, f"{wl.name} no-alloc")


def test_noalloc_refuses_oversized_workspace():
    """An int4 cache without RoPE is expanded into the workspace: at batch 8 and
    4096 tokens that is far above the scratch, so the call is refused before
    anything is read (the pointers are never touched)."""
    import rank_decode_attention_amd as R
    desc = R.AttnDesc(32, 32, 128, 8, [154] * 8, use_rope=False, latent_dtype="i4", act_dtype="f16")
    assert R.decode_workspace_bytes(desc, 8, 4096) > R.NOALLOC_SCRATCH_BYTES
    lib = R.load()
    cache = R._Cache(8, 8, 8, 8, 4096)
    p = ctypes.c_void_p(256)
    st = lib.palu_decode_attn_noalloc(desc.ref(), p, ctypes.byref(cache), p, p, p, None, 8, 0.1, p, None)
    assert st == 2 and b"no-alloc" in lib.palu_last_error()
