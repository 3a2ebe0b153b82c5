"""GPU: palu_decode_attn_chunk (several new tokens per sequence, causal
within the chunk) against the oracle's chunk attention, through the C ABI;
q_len = 1 is exactly the decode call."""
import numpy as np
import pytest

import palu_inputs as PI
from palu_cases import (build_decode_case, compare, oracle_chunk, paged_from, run_chunk, run_decode)

pytestmark = pytest.mark.gpu

CASES = [
    # (name, workload, q_len); a history shorter than the chunk leaves its first queries empty
    ("7b_q4", PI.scaled("llama2_7b", batch=3, max_len=300, fixed_lengths=(300, 2, 77)), 4),
    ("7b_q7_bf16_long", PI.scaled("long_b4", batch=2, max_len=500, fixed_lengths=(500, 260)), 7),
    ("gqa_rope_q3", PI.scaled("gqa_rope", batch=2, max_len=200, fixed_lengths=(200, 33)), 3),
    ("gqa_norope_q5", PI.scaled("gqa_norope", batch=2, max_len=200, fixed_lengths=(129, 64)), 5),
    ("tiny_f32_q2", PI.workload("tiny"), 2),
    ("int4_q4", PI.scaled("int4", batch=2, max_len=300, fixed_lengths=(300, 96)), 4),
]


@pytest.mark.parametrize("name,wl,q_len", CASES, ids=[c[0] for c in CASES])
def test_chunk_parity(name, wl, q_len):
    case = build_decode_case(wl)
    gpu, qh = run_chunk(case, q_len)
    ref = oracle_chunk(case, qh)
    stats = compare(gpu, ref, wl.act, name)
    for b, L in enumerate(case["lens"]):
        for i in range(q_len):
            if L - q_len + i < 0:
                assert np.all(gpu[b, i] == 0), f"{name}: query {i} of sequence {b} sees nothing"
    print(name, stats)


def test_chunk_paged_parity():
    wl = PI.scaled("llama2_7b", batch=2, max_len=256, fixed_lengths=(256, 70))
    case = build_decode_case(wl)
    pc, _ = paged_from(case, 64, seed=2)
    gpu, qh = run_chunk(case, 5, paged=pc)
    compare(gpu, oracle_chunk(case, qh), wl.act, "chunk paged")
    gpu_c, _ = run_chunk(case, 5)
    assert np.array_equal(gpu, gpu_c)    # same history bound: same split, same bits


def test_chunk_of_one_is_the_decode_step():
    import torch
    wl = PI.scaled("llama2_7b", batch=3, max_len=200, fixed_lengths=(200, 1, 77))
    case = build_decode_case(wl)
    gpu, qh = run_chunk(case, 1)
    # the decode call with the chunk's queries
    case["q"] = torch.from_numpy(np.ascontiguousarray(qh[:, 0])).cuda()
    ref = run_decode(case)
    assert np.array_equal(gpu[:, 0], ref)
