"""GPU: palu_decode_attn_paged.  The latent rows of a contiguous decode case
are scattered into pages placed in random order (unused pool bytes and rows
past a history are 0xFF), and with the same history bound the paged call
must give exactly the contiguous call's output (same kernels, same split of
the history, other addresses), and so meet the oracle bar as well."""
import numpy as np
import pytest

import palu_inputs as PI
from palu_cases import (build_decode_case, compare, oracle_decode, paged_from, run_decode,
                        run_decode_paged)

pytestmark = pytest.mark.gpu

CASES = [
    # (name, workload, page size); history bounds are multiples of the page
    # size, so that both calls plan the same split of the history
    ("7b_ps32", PI.scaled("llama2_7b", batch=3, max_len=320, fixed_lengths=(300, 1, 77)), 32),
    ("7b_ps256_empty", PI.scaled("llama2_7b", batch=3, max_len=768, fixed_lengths=(600, 257, 0)), 256),
    ("long_bf16_ps64", PI.scaled("long_b4", batch=3, max_len=704), 64),
    ("gqa_rope_ps64", PI.scaled("gqa_rope", batch=3, max_len=256, fixed_lengths=(200, 33, 129)), 64),
    ("gqa_norope_ps128", PI.scaled("gqa_norope", batch=2, max_len=384, fixed_lengths=(300, 129)), 128),
    ("int4_ps64", PI.scaled("int4", batch=3, max_len=320, fixed_lengths=(300, 1, 77)), 64),
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


@pytest.mark.parametrize("fmt", ["bf16", "i4"])
def test_project_paged_equals_contiguous(fmt):
    """palu_project_paged writes, row for row, the bytes palu_project writes
    into a contiguous cache; pool bytes of other pages stay untouched."""
    import torch
    import rank_decode_attention_amd as R
    from palu_cases import desc_of, to_device
    wl = PI.scaled("int4_prefill", latent=fmt, d_model=512, batch=2, max_len=400, n_tok=300)
    desc = desc_of(wl)
    n_tok, seq, pos0, ps = 300, 1, 50, 64
    x = to_device(PI.prefill_x(wl, n_tok), wl.act)
    A_kv = to_device(np.ascontiguousarray(np.concatenate([a.T for a in PI.prefill_A(wl)], axis=0)), wl.act)
    ref = R.alloc_cache(desc, wl.batch, wl.max_len)
    R.palu_project(desc, x, A_kv, ref, seq, pos0)
    # pages of sequence 1 in a shuffled pool of 16 pages; block table rows for 2 sequences
    max_pages = (wl.max_len + ps - 1) // ps
    n_pages = 16
    table = np.full((wl.batch, max_pages), -1, dtype=np.int32)
    table[1, :] = np.random.default_rng(5).permutation(n_pages)[:max_pages]
    q4 = fmt == "i4"
    pool = lambda w, sc: torch.full((max(16, R.latent_bytes(desc, n_pages, ps, w, sc)),), 0, dtype=torch.uint8,
                                    device="cuda")
    pc = R.PagedCache(pool(0, False), pool(1, False), pool(0, True) if q4 else None, pool(1, True) if q4 else None,
                      torch.from_numpy(table).cuda(), ps, n_pages)
    R.palu_project_paged(desc, x, A_kv, pc, seq, pos0)
    torch.cuda.synchronize()
    for which in (0, 1):
        ranks = desc.rank_k if which == 0 else desc.rank_v
        for sc in ((False, True) if q4 else (False,)):
            got_pool = (pc.sv if sc else pc.zv) if which else (pc.sk if sc else pc.zk)
            got_pool = got_pool.cpu().numpy()
            ref_buf = ((ref.sv if sc else ref.zv) if which else (ref.sk if sc else ref.zk)).cpu().numpy()
            touched = np.zeros(got_pool.size, dtype=bool)
            for j in range(desc.n_groups):
                pitch = R.scale_pitch(ranks[j]) if sc else R.row_pitch(desc.latent_dtype, ranks[j])
                for t in range(pos0, pos0 + n_tok):
                    o_ref = R.latent_offset(desc, wl.max_len, which, sc, seq, j, t)
                    o_pg = R.latent_offset(desc, ps, which, sc, int(table[seq, t // ps]), j, t % ps)
                    assert np.array_equal(got_pool[o_pg:o_pg + pitch], ref_buf[o_ref:o_ref + pitch]), (which, sc, j, t)
                    touched[o_pg:o_pg + pitch] = True
            assert np.all(got_pool[~touched] == 0), "bytes outside the written rows changed"
