"""GPU parity of palu_decode_attn against the fp64 oracle, through the C ABI.

Small cases (the oracle computes every output): several 32-token tiles with
ragged tails, empty and single-token histories, explicit query positions,
peaked attention.  Full-size cases (the shapes the benchmark times, same
launch configuration): sampled (sequence, head) outputs, each computed by the
oracle on its own.
"""
import math

import numpy as np
import pytest

import palu_inputs as PI
from palu_cases import build_decode_case, compare, oracle_decode, run_decode

pytestmark = pytest.mark.gpu


def _small(base, **over):
    return PI.scaled(base, **over)


SMALL = [
    ("tiny", PI.workload("tiny"), None),
    ("tiny_norope", PI.scaled("tiny", use_rope=False, name="tiny_norope"), None),
    ("tiny_ragged", PI.scaled("tiny", batch=3, max_len=200, fixed_lengths=(200, 37, 1)), None),
    ("7b_small", _small("llama2_7b", batch=3, max_len=320, fixed_lengths=(300, 1, 77)), None),
    ("7b_small_norope", _small("llama2_7b", batch=2, max_len=256, fixed_lengths=(256, 45), use_rope=False), None),
    ("long_small", _small("long_b4", batch=3, max_len=600, ragged=True), None),
    ("gqa_rope_small", _small("gqa_rope", batch=3, max_len=200, fixed_lengths=(200, 33, 129)), None),
    ("gqa_norope_small", _small("gqa_norope", batch=3, max_len=200, fixed_lengths=(200, 33, 129)), None),
    ("7b_f16_gqa_shape", PI.scaled("gqa_rope", latent="f16", act="f16", batch=2, max_len=96,
                                   fixed_lengths=(96, 50)), None),
    # int4 latents: expanded to 16-bit rows (rank rounded up to 32), then the
    # MHA-group kernel (rank 154 -> 160, 100 -> 128) or the split kernel
    ("int4_small", _small("int4", batch=3, max_len=300, fixed_lengths=(300, 1, 77)), None),
    ("int4_bf16_r100", _small("int4", act="bf16", rank=100, batch=2, max_len=200, fixed_lengths=(200, 65)), None),
    ("int4_empty_seq", _small("int4", batch=3, max_len=100, fixed_lengths=(0, 100, 33)), None),
    ("int4_norope", _small("int4", use_rope=False, batch=2, max_len=160, fixed_lengths=(160, 3)), None),
    ("int4_gqa", _small("gqa_rope", latent="i4", batch=3, max_len=200, fixed_lengths=(200, 33, 129)), None),
    # MHA-group kernel with fewer than 8 key chunks, and per-group ranks
    ("7b_r160", _small("llama2_7b", rank=160, batch=2, max_len=300, fixed_lengths=(300, 77)), None),
    ("long_r128_bf16", _small("long_b4", rank=128, batch=2, max_len=400), None),
    ("7b_mixed_ranks", _small("llama2_7b", rank=None, rank_choices=(96, 160, 256), batch=2, max_len=200,
                              fixed_lengths=(200, 45)), None),
    ("int4_mixed_ranks", _small("int4", rank=None, rank_choices=(70, 154, 200), batch=2, max_len=260,
                                fixed_lengths=(260, 31)), None),
    # absorbed-query kernel (no RoPE, 16-bit): histories of at most 16 tokens
    # leave the second token half of every tile masked (its stream never sees
    # a token), an empty sequence, tile boundaries, odd ranks (chunk counts
    # rounded up to even), and capacity 256 with ranks below it
    ("gqa_norope_short", _small("gqa_norope", batch=6, max_len=70, fixed_lengths=(1, 16, 0, 17, 33, 70)), None),
    ("gqa_norope_odd_ranks", _small("gqa_norope", rank=None, rank_choices=(90, 150, 200, 300), batch=3,
                                    max_len=150, fixed_lengths=(150, 9, 64)), None),
    ("7b_norope_short", _small("llama2_7b", use_rope=False, rank=None, rank_choices=(64, 96, 256), batch=4,
                               max_len=100, fixed_lengths=(16, 100, 1, 48)), None),
]


@pytest.mark.parametrize("name,wl,_", SMALL, ids=[s[0] for s in SMALL])
def test_small_full_compare(name, wl, _):
    case = build_decode_case(wl)
    gpu = run_decode(case)
    ref = oracle_decode(case)
    stats = compare(gpu, ref, wl.act, name)
    print(name, stats)


@pytest.mark.parametrize("q_scale", [8.0])
def test_peaked_attention(q_scale):
    wl = _small("llama2_7b", batch=2, max_len=160, fixed_lengths=(160, 99), name="7b_peaked")
    case = build_decode_case(wl, q_scale=q_scale)
    compare(run_decode(case), oracle_decode(case), wl.act, "peaked")
    wl = _small("gqa_rope", batch=2, max_len=160, fixed_lengths=(160, 99), name="gqa_peaked")
    case = build_decode_case(wl, q_scale=q_scale)
    compare(run_decode(case), oracle_decode(case), wl.act, "gqa peaked")


def test_empty_sequences_and_explicit_positions():
    import torch
    wl = _small("llama2_7b", batch=4, max_len=128, fixed_lengths=(0, 128, 0, 5), name="7b_empty")
    case = build_decode_case(wl)
    gpu = run_decode(case)
    assert np.all(gpu[0] == 0) and np.all(gpu[2] == 0)
    compare(gpu, oracle_decode(case), wl.act, "empty")
    qpos = np.array([0, 1000, 3, 70000], dtype=np.int32)
    gpu2 = run_decode(case, q_pos=torch.from_numpy(qpos).cuda())
    compare(gpu2, oracle_decode(case, q_pos=qpos), wl.act, "q_pos")


def test_batch_zero_is_noop():
    import torch
    import rank_decode_attention_amd as R
    wl = _small("llama2_7b", batch=1, max_len=64, name="7b_b1")
    case = build_decode_case(wl)
    q0 = case["q"][:0]
    out0 = case["out"][:0]
    R.palu_decode_attn(case["desc"], q0, case["cache"], case["Bk"], case["Bv"], case["seq_lens"], None,
                       case["sm_scale"], out0, case["ws"])
    torch.cuda.synchronize()


def test_int4_workspace_and_errors():
    """int4 latents on shapes the MHA kernel covers are expanded inside it (no
    extra workspace); elsewhere (here: no RoPE) the 16-bit expansion (rank
    rounded up to 32, keys and values) is added to the workspace.  Missing
    scales are an argument error."""
    import rank_decode_attention_amd as R
    batch, max_len = 3, 100
    wl = _small("int4", batch=batch, max_len=max_len)
    dense = batch * max_len * 8 * 2 * 160
    for rope, extra in ((True, 0), (False, 2 * ((dense + 255) // 256 * 256))):
        f = R.AttnDesc(32, 32, 128, 8, [154] * 8, use_rope=rope, latent_dtype="f16", act_dtype="f16")
        i = R.AttnDesc(32, 32, 128, 8, [154] * 8, use_rope=rope, latent_dtype="i4", act_dtype="f16")
        assert R.decode_workspace_bytes(i, batch, max_len) == R.decode_workspace_bytes(f, batch, max_len) + extra
    case = build_decode_case(wl)
    c = case["cache"]
    no_scales = R.LatentCache(c.zk, c.zv, None, None, c.max_len)
    with pytest.raises(R.PaluError, match="scales"):
        R.palu_decode_attn(case["desc"], case["q"], no_scales, case["Bk"], case["Bv"], case["seq_lens"], None,
                           case["sm_scale"], case["out"], case["ws"])


def test_deterministic():
    wl = _small("long_b4", batch=2, max_len=2000, ragged=True, name="long_det")
    case = build_decode_case(wl)
    a = run_decode(case)
    b = run_decode(case)
    assert np.array_equal(a, b)


FULL = [
    ("llama2_7b", [(0, 0), (0, 31), (7, 13), (15, 22)]),
    ("long_b1", [(0, 0), (0, 17)]),
    ("long_b4", [(0, 3), (3, 28)]),
    ("gqa_rope", [(0, 0), (5, 9), (31, 31)]),
    ("gqa_norope", [(0, 1), (17, 20), (31, 30)]),
    ("int4", [(0, 0), (3, 17), (7, 31)]),
]


@pytest.mark.parametrize("name,heads", FULL, ids=[f[0] for f in FULL])
def test_full_size_sampled(name, heads):
    wl = PI.workload(name)
    case = build_decode_case(wl)
    gpu = run_decode(case)
    ref = oracle_decode(case, heads=heads)
    bs = [b for b, _ in heads]
    hs = [h for _, h in heads]
    stats = compare(gpu[bs, hs], ref[bs, hs], wl.act, name)
    assert np.all(np.isfinite(gpu))
    print(name, stats)


def test_maximum_batch_and_groups():
    """The largest batch the library takes (2048 sequences, short ragged
    histories) and the largest group count (16 groups of 2 kv heads)."""
    wl = PI.scaled("tiny", name="tiny_b2048", batch=2048, max_len=64, ragged=True)
    case = build_decode_case(wl)
    gpu = run_decode(case)
    seqs = [0, 1, 1023, 2046, 2047]
    heads = [(b, h) for b in seqs for h in (0, 7)]
    ref = oracle_decode(case, heads=heads)
    bs, hs = [b for b, _ in heads], [h for _, h in heads]
    compare(gpu[bs, hs], ref[bs, hs], wl.act, "batch 2048")
    wl = PI.scaled("gqa_rope", name="gqa_g16", n_q_heads=128, n_kv_heads=32, n_groups=16, batch=2, max_len=100,
                   fixed_lengths=(100, 37), rank_choices=(64, 128))
    case = build_decode_case(wl)
    compare(run_decode(case), oracle_decode(case), wl.act, "16 groups")
