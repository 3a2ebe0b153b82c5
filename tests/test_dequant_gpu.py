"""GPU: palu_dequant_latent (int4 rows -> 16-bit rows) is bit-exact against
the oracle's 16-bit rows of int4 latents (code * scale, exact, rounded once to
fp16 / bf16; zero past the rank), through the C ABI."""
import numpy as np
import pytest

import oracle
import palu_inputs as PI

pytestmark = pytest.mark.gpu


def _bits(x64: np.ndarray, fmt: str) -> np.ndarray:
    """uint16 bit patterns of values already representable in fmt."""
    if fmt == "f16":
        return x64.astype(np.float16).view(np.uint16)
    return (x64.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _expand(packed, scales, r, fmt):
    import torch
    import rank_decode_attention_amd as R
    n, nc = scales.shape
    out = torch.full((n, 32 * nc), float("nan"), dtype=torch.float16 if fmt == "f16" else torch.bfloat16,
                     device="cuda")
    R.palu_dequant_latent(torch.from_numpy(np.ascontiguousarray(packed)).cuda(),
                          torch.from_numpy(np.ascontiguousarray(scales).view(np.int16)).cuda(), n, r, out)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("fmt,r,n", [("f16", 154, 1000), ("bf16", 154, 777), ("f16", 320, 300), ("bf16", 32, 64),
                                     ("f16", 100, 513), ("bf16", 1, 17)])
def test_dequant_bit_exact(fmt, r, n):
    wl = PI.scaled("int4", rank=r, act=fmt)
    packed, scales = PI.latent_int4(wl, "k", 0, 0, n=n)
    got = _expand(packed, scales, r, fmt)
    want = oracle.int4_rows16(packed, scales, r, fmt)
    assert np.array_equal(got[:, :r], _bits(want, fmt))
    assert np.all(got[:, r:] == 0)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_dequant_every_code_and_odd_scales(fmt):
    """All 16 nibble values (including -8, which the quantiser never writes),
    zero, subnormal, tiny and large binary16 scales, and non-zero pad nibbles
    (which must not leak into the elements past the rank)."""
    rng = np.random.default_rng(11)
    r, n = 50, 256                     # two chunks, the second with 18 elements
    nib = rng.integers(0, 16, size=(n, 64), dtype=np.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    s = rng.uniform(0.01, 3.0, size=(n, 2)).astype(np.float16)
    s[0] = 0.0
    s[1] = np.float16(2.0 ** -20)      # subnormal
    s[2] = np.float16(6.1e-5)          # smallest normal
    s[3] = np.float16(4096.0)          # large
    s[4] = np.float16(-0.75)           # negative (never written by the quantiser; still code * scale)
    got = _expand(packed, s, r, fmt)
    want = oracle.int4_rows16(packed, s, r, fmt)
    assert np.array_equal(got[:, :r], _bits(want, fmt))
    assert np.all(got[:, r:] == 0)
