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
    # int4 latents (the oracle attends over the exact code * scale): the MHA
    # head-group kernel reads the codes itself (rank 154 -> 5 chunks, 100 ->
    # 4); other shapes attend over exact hi/lo 16-bit rows of twice the rank
    # rounded up to 32 (no RoPE: the absorbed-query kernel; GQA: the split
    # kernel, ranks up to 160)
    ("int4_small", _small("int4", batch=3, max_len=300, fixed_lengths=(300, 1, 77)), None),
    ("int4_bf16_r100", _small("int4", act="bf16", rank=100, batch=2, max_len=200, fixed_lengths=(200, 65)), None),
    ("int4_empty_seq", _small("int4", batch=3, max_len=100, fixed_lengths=(0, 100, 33)), None),
    ("int4_norope", _small("int4", use_rope=False, batch=2, max_len=160, fixed_lengths=(160, 3)), None),
    ("int4_norope_bf16", _small("int4", act="bf16", use_rope=False, batch=2, max_len=130, fixed_lengths=(130, 64)),
     None),
    ("int4_gqa", _small("gqa_rope", latent="i4", rank_choices=(64, 128, 160), batch=3, max_len=200,
                        fixed_lengths=(200, 33, 129)), None),
    # MHA-group kernel with fewer than 8 key chunks, and per-group ranks
    ("7b_r160", _small("llama2_7b", rank=160, batch=2, max_len=300, fixed_lengths=(300, 77)), None),
    ("long_r128_bf16", _small("long_b4", rank=128, batch=2, max_len=400), None),
    ("7b_mixed_ranks", _small("llama2_7b", rank=None, rank_choices=(96, 160, 256), batch=2, max_len=200,
                              fixed_lengths=(200, 45)), None),
    ("int4_mixed_ranks", _small("int4", rank=None, rank_choices=(70, 154, 200), batch=2, max_len=260,
                                fixed_lengths=(260, 31)), None),
    # ranks of one and two 32-rank chunks (the MHA kernel's B_k staging waits
    # differ there), one-tile blocks and blocks of several tiles
    ("7b_low_ranks", _small("llama2_7b", rank=None, rank_choices=(32, 64), batch=3, max_len=300,
                            fixed_lengths=(300, 1, 77)), None),
    ("7b_low_ranks_long", _small("llama2_7b", rank=None, rank_choices=(32, 64), batch=2, max_len=2048,
                                 fixed_lengths=(2048, 1100)), None),
    # absorbed-query kernel (no RoPE, 16-bit): histories of at most 16 tokens
    # leave the second token half of every tile masked (its stream never sees
    # a token), an empty sequence, tile boundaries, odd ranks (chunk counts
    # rounded up to even), and capacity 256 with ranks below it
    ("gqa_norope_short", _small("gqa_norope", batch=6, max_len=70, fixed_lengths=(1, 16, 0, 17, 33, 70)), None),
    ("gqa_norope_odd_ranks", _small("gqa_norope", rank=None, rank_choices=(90, 150, 200, 300), batch=3,
                                    max_len=150, fixed_lengths=(150, 9, 64)), None),
    ("7b_norope_short", _small("llama2_7b", use_rope=False, rank=None, rank_choices=(64, 96, 256), batch=4,
                               max_len=100, fixed_lengths=(16, 100, 1, 48)), None),
    # one or two sequences split over every block of their group: the merge
    # shares an output item between several threads (each merging every
    # nsub-th record, several rounds here) and combines their partials
    ("7b_batch1_all_blocks", _small("llama2_7b", batch=1, max_len=2085, fixed_lengths=(2085,)), None),
    ("7b_batch2_all_blocks", _small("llama2_7b", batch=2, max_len=1500, fixed_lengths=(1500, 701)), None),
]


@pytest.mark.parametrize("name,wl,_", SMALL, ids=[s[0] for s in SMALL])
def test_small_full_compare(name, wl, _):
    case = build_decode_case(wl)
    gpu = run_decode(case)
    ref = oracle_decode(case)
    stats = compare(gpu, ref, wl.act, name)
    print(name, stats)


@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("q_scale", [1.0, 8.0])
def test_int4_exact_latents(act, q_scale):
    """int4 decode against the oracle's exact code * scale, flat and peaked
    attention, fp16 and bf16 activations (rounding the latent to bf16 first
    would miss the bar under peaked attention by an order of magnitude)."""
    wl = _small("int4", act=act, batch=3, max_len=260, fixed_lengths=(260, 97, 32), name=f"int4_{act}")
    case = build_decode_case(wl, q_scale=q_scale)
    stats = compare(run_decode(case), oracle_decode(case), wl.act, f"int4 {act} q x{q_scale:g}")
    print(f"int4 {act} q x{q_scale:g}", stats)


def test_int4_unsupported_rank():
    """Shapes attended over hi/lo rows need twice the rank (rounded up to 32)
    within a kernel's capacity (GQA: 320): rank 192 is refused."""
    import rank_decode_attention_amd as R
    wl = _small("gqa_rope", latent="i4", rank=192, batch=1, max_len=64)
    with pytest.raises(R.PaluError, match="hi/lo"):
        build_decode_case(wl)


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
    """int4 latents on shapes the MHA kernel covers are read by it directly (no
    extra workspace); elsewhere (here: no RoPE) the workspace adds the exact
    hi/lo expansion (rank 160 -> 320, keys and values) and the factors with
    duplicated rows.  Missing scales are an argument error."""
    import rank_decode_attention_amd as R
    batch, max_len = 3, 100
    wl = _small("int4", batch=batch, max_len=max_len)
    r256 = lambda x: (x + 255) // 256 * 256
    dense = batch * max_len * 8 * 2 * 320
    dup = 8 * 320 * 512 * 2
    for rope, extra in ((True, 0), (False, 2 * r256(dense) + 2 * r256(dup))):
        f = R.AttnDesc(32, 32, 128, 8, [154] * 8, use_rope=rope, latent_dtype="f16", act_dtype="f16")
        f2 = R.AttnDesc(32, 32, 128, 8, [320] * 8, use_rope=rope, latent_dtype="f16", act_dtype="f16")
        i = R.AttnDesc(32, 32, 128, 8, [154] * 8, use_rope=rope, latent_dtype="i4", act_dtype="f16")
        base = R.decode_workspace_bytes(f if rope else f2, batch, max_len)
        assert R.decode_workspace_bytes(i, batch, max_len) == base + extra
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


def _one_head_per_group(wl):
    """One query head of every (sequence, head-group): head b mod (H/G) of
    group g, so that the sampled heads vary inside the groups too."""
    per = wl.n_q_heads // wl.n_groups
    return [(b, g * per + (b + g) % per) for b in range(wl.batch) for g in range(wl.n_groups)]


FULL = [("llama2_7b", 1.0), ("llama2_7b", 8.0), ("long_b1", 1.0), ("long_b4", 1.0), ("gqa_rope", 1.0),
        ("gqa_rope", 8.0), ("gqa_norope", 1.0), ("int4", 1.0), ("int4", 8.0)]


@pytest.mark.parametrize("name,q_scale", FULL, ids=[f"{n}_q{s:g}" for n, s in FULL])
def test_full_size_sampled(name, q_scale):
    """The workloads at full size, in the benchmark's launch configuration:
    one query head of every (sequence, group) against the oracle (which
    rebuilds that group's keys and values in fp64), flat and peaked (q x 8)
    attention."""
    wl = PI.workload(name)
    case = build_decode_case(wl, q_scale=q_scale)
    gpu = run_decode(case)
    heads = _one_head_per_group(wl)
    ref = oracle_decode(case, heads=heads)
    bs = [b for b, _ in heads]
    hs = [h for _, h in heads]
    stats = compare(gpu[bs, hs], ref[bs, hs], wl.act, f"{name} full q x{q_scale:g}")
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


@pytest.mark.parametrize("rope", [True, False], ids=["mha_fused", "expanded"])
def test_int4_padding_and_rows_past_history_are_ignored(rope):
    """int4 codes past the rank (the padding nibbles of a row's last 32-rank
    chunk) and rows past each history (codes and scales) may hold anything:
    the decode output is bit-identical to that of the clean cache (the fused
    kernel carries the codes unmasked into the MFMAs, where the keys' meet
    zero rows of B_k and the values' land in ranks the merge never reads), and
    it still matches the oracle."""
    import rank_decode_attention_amd as R
    wl = _small("int4", use_rope=rope, batch=3, max_len=200, fixed_lengths=(200, 77, 33), name=f"int4_dirty_{rope}")
    case = build_decode_case(wl)
    clean = run_decode(case)
    ranks = PI.ranks(wl)
    rng = np.random.default_rng(123)

    def rows(which, b, j):
        L = int(case["lens"][b])
        codes, scales = PI.latent_int4(wl, "k" if which == 0 else "v", b, j, n=max(L, 1))
        r, nc = int(ranks[j]), scales.shape[1]
        codes = np.concatenate([codes, rng.integers(0, 256, size=(wl.max_len - codes.shape[0], codes.shape[1]),
                                                    dtype=np.uint8)])
        scales = np.concatenate([scales, rng.uniform(-1e4, 1e4, size=(wl.max_len - scales.shape[0], nc))
                                 .astype(np.float16)])
        nib = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(codes.shape[0], -1)
        nib[:, r:] = rng.integers(1, 16, size=(codes.shape[0], nib.shape[1] - r), dtype=np.uint8)
        return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8), scales

    dirty = dict(case)
    dirty["cache"] = R.fill_cache(case["desc"], wl.batch, wl.max_len, rows)
    gpu = run_decode(dirty)
    assert np.array_equal(gpu, clean)
    compare(gpu, oracle_decode(case), wl.act, f"int4 dirty padding rope={rope}")
