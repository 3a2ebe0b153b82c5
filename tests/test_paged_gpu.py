"""GPU: palu_decode_attn_paged.  The latent rows of a contiguous decode case
are scattered into pages placed in random order (unused pool bytes and rows
past a history are 0xFF), and the paged call must give exactly the
contiguous call's output (same kernels and arithmetic, other addresses), and
so meet the oracle bar as well."""
import numpy as np
import pytest

import palu_inputs as PI
from palu_cases import (build_decode_case, compare, oracle_decode, paged_from, run_decode,
                        run_decode_paged)

pytestmark = pytest.mark.gpu

CASES = [
    # (name, workload, page size)
    ("7b_ps32", PI.scaled("llama2_7b", batch=3, max_len=300, fixed_lengths=(300, 1, 77)), 32),
    ("7b_ps256_empty", PI.scaled("llama2_7b", batch=3, max_len=600, fixed_lengths=(600, 257, 0)), 256),
    ("long_bf16_ps64", PI.scaled("long_b4", batch=3, max_len=700), 64),
    ("gqa_rope_ps64", PI.scaled("gqa_rope", batch=3, max_len=200, fixed_lengths=(200, 33, 129)), 64),
    ("gqa_norope_ps128", PI.scaled("gqa_norope", batch=2, max_len=300, fixed_lengths=(300, 129)), 128),
    ("int4_ps64", PI.scaled("int4", batch=3, max_len=300, fixed_lengths=(300, 1, 77)), 64),
    ("tiny_f32_ps32", PI.workload("tiny"), 32),
]


@pytest.mark.parametrize("name,wl,ps", CASES, ids=[c[0] for c in CASES])
def test_paged_equals_contiguous(name, wl, ps):
    case = build_decode_case(wl)
    ref = run_decode(case)
    pc, _ = paged_from(case, ps, seed=len(name))
    got = run_decode_paged(case, pc)
    assert np.all(np.isfinite(got)), name
    assert np.array_equal(got, ref), f"{name}: paged and contiguous outputs differ"
    compare(got, oracle_decode(case), wl.act, name)


def test_paged_shared_prefix_page():
    """Two sequences whose first page is one shared page."""
    wl = PI.scaled("llama2_7b", batch=2, max_len=256, fixed_lengths=(256, 200))
    case = build_decode_case(wl)
    pc, bt = paged_from(case, 64, seed=3, share_first=True)
    assert bt[0, 0] == bt[1, 0]
    ref = run_decode(case)          # contiguous cache with the same (copied) prefix rows
    got = run_decode_paged(case, pc)
    assert np.array_equal(got, ref)


def test_paged_full_size_7b():
    """The benchmark shape through pages of 64 tokens: equal to the contiguous call."""
    wl = PI.workload("llama2_7b")
    case = build_decode_case(wl)
    ref = run_decode(case)
    pc, _ = paged_from(case, 64, seed=11, extra_pages=0)
    got = run_decode_paged(case, pc)
    assert np.array_equal(got, ref)
    heads = [(0, 0), (9, 17), (15, 31)]
    o = oracle_decode(case, heads=heads)
    bs, hs = [b for b, _ in heads], [h for _, h in heads]
    compare(got[bs, hs], o[bs, hs], wl.act, "7b paged")


def test_paged_int4_unsupported_shape():
    """int4 pools are read by the MHA head-group kernel only."""
    import rank_decode_attention_amd as R
    wl = PI.scaled("int4", use_rope=False, batch=2, max_len=128, fixed_lengths=(128, 64))
    case = build_decode_case(wl)
    pc, _ = paged_from(case, 64)
    with pytest.raises(R.PaluError, match="paged int4"):
        run_decode_paged(case, pc)
