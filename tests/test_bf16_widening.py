"""The reading of a bf16 probability entry used by topk_topp_sample_bf16 and
by its parity tests: an entry means its exact fp32 widening, the 16 bits
moved into the upper half of an fp32 word.  Pinned against torch's own
bf16 -> fp32 conversion over all 65,536 bit patterns, and the widened order
against the bf16 values' own order (the sampler ranks widened bits)."""

import numpy as np
import torch

from tests.test_gpu_bf16 import to_bf16_bits


def _all_patterns():
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def test_widening_equals_torch_conversion():
    b16 = _all_patterns()
    wide = (b16.astype(np.uint32) << 16).view(np.float32)
    ref = torch.from_numpy(b16.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(wide), nan)
    assert np.array_equal(wide[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_widened_bits_keep_the_order_of_non_negative_values():
    # Non-negative, non-NaN bf16 values order like their widened fp32 bits
    # read as integers, which is how the sampler compares keys.
    b16 = _all_patterns()
    vals = torch.from_numpy(b16.view(np.int16)).view(torch.bfloat16).float().numpy()
    keep = (b16 < 0x8000) & ~np.isnan(vals)
    bits = (b16[keep].astype(np.uint32) << 16)
    order_bits = np.argsort(bits, kind="stable")
    order_vals = np.argsort(vals[keep], kind="stable")
    assert np.array_equal(order_bits, order_vals)


def test_rounding_helper_rounds_to_nearest_even():
    # The parity tests round fp32 rows to bf16 with torch; its result must be
    # the nearest bf16 value, ties to an even mantissa, for finite inputs.
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.random(20000).astype(np.float32),
        (rng.random(2000) * 1e-30).astype(np.float32),
        # exact halfway cases between two bf16 values
        ((np.arange(1, 2001, dtype=np.uint32) << 16) | 0x8000).view(np.float32),
    ])
    b16, wide = to_bf16_bits(x[None, :])
    bits = x.view(np.uint32)
    lo = bits & 0xFFFF0000
    rem = bits & 0xFFFF
    up = (rem > 0x8000) | ((rem == 0x8000) & ((bits >> 16) & 1).astype(bool))
    want = lo + np.where(up, 0x10000, 0).astype(np.uint32)
    assert np.array_equal(wide[0].view(np.uint32), want)
