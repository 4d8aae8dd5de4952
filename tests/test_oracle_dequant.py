"""Exhaustive pin of the oracle's Q8G64 -> bf16 dequantisation.

The row format (page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache
Offloading", section "Separate historical capacity from the current working
set") is an int8 latent with one fp16 scale per group of 64 values.  The value
is q * scale, rounded to the nearest bf16 with ties to even.  |q| <= 2^7 and an
fp16 significand has 11 bits, so the product itself is exact and the rounding
to bf16 is the only one.

Two independent references, over every int8 q and every finite fp16 scale:
  * exact integer arithmetic: product = (|q| * significand) * 2^exp, rounded
    to 8 significant bits by integer shifts (round half to even);
  * torch's float32 multiply and its float32 -> bfloat16 conversion.
"""
import numpy as np
import torch

import oracle


def _finite_scales():
    bits = np.arange(65536, dtype=np.int64)
    return bits[((bits >> 10) & 31) != 31]


def exact_bf16_of_product(q, h):
    """bf16 bits of RNE(q * fp16(h)), by integer arithmetic only.
    q, h: int64 arrays of equal shape, h finite fp16 bit patterns."""
    q = np.asarray(q, np.int64)
    h = np.asarray(h, np.int64)
    e = (h >> 10) & 31
    m = h & 1023
    sig = np.where(e == 0, m, m + 1024)          # integer significand
    exp2 = np.where(e == 0, -24, e - 25)         # value = sig * 2^exp2
    sign = ((q < 0).astype(np.int64) ^ (h >> 15)) & 1
    n = np.abs(q) * sig                          # exact |product| / 2^exp2
    # bit length of n (n < 2^18, exact in float64)
    _, bl = np.frexp(n.astype(np.float64))
    bl = bl.astype(np.int64)
    sh = np.maximum(bl - 8, 0)
    r = n >> sh
    rem = n & ((np.int64(1) << sh) - 1)
    half = np.where(sh > 0, np.int64(1) << np.maximum(sh - 1, 0), 0)
    up = (sh > 0) & ((rem > half) | ((rem == half) & ((r & 1) == 1)))
    r = r + up
    carry = r == 256
    r = np.where(carry, 128, r)
    sh = sh + carry
    # normalise small n (< 128) up to an 8-bit significand
    lz = np.where(n > 0, 8 - np.minimum(bl, 8), 0)
    r = r << lz
    sh = sh - lz
    E = exp2 + sh + 7 + 127
    bits = (sign << 15) | (E << 7) | (r - 128)
    bits = np.where(n == 0, sign << 15, bits)
    return bits.astype(np.uint16)


def test_integer_reference_on_hand_values():
    # the reference itself, on values worked out by hand
    q = np.array([1, -1, 127, -128, 3, 127, 0, -127])
    h = np.array([0x3C00, 0x3C00, 0x3C00, 0x3C00, 0x3555, 0x7BFF, 0xBC00, 0x2E66])
    expect = [0x3F80, 0xBF80, 0x42FE, 0xC300, 0x3F80, 0x4AFE, 0x8000, 0xC14B]
    np.testing.assert_array_equal(exact_bf16_of_product(q, h), np.array(expect, np.uint16))


def test_oracle_dequant_is_exact_for_every_int8_and_every_finite_fp16():
    table = oracle.dequant_table()               # [256, 65536]
    scales = _finite_scales()
    assert scales.size == 63488
    for qi in range(256):
        q = qi - 128
        got = table[qi, scales]
        want = exact_bf16_of_product(np.full(scales.size, q), scales)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (q, hex(int(scales[bad[0]])), hex(got[bad[0]]), hex(want[bad[0]]))


def test_oracle_dequant_matches_torch_float32_product_to_bfloat16():
    table = oracle.dequant_table()
    scales = _finite_scales()
    s32 = torch.from_numpy(scales.astype(np.uint16).view(np.float16)).to(torch.float32)
    for qi in range(0, 256, 5):
        q = float(qi - 128)
        ref = (s32 * q).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(table[qi, scales], ref, err_msg=f"q={qi - 128}")


def test_non_finite_scales():
    table = oracle.dequant_table()
    inf, ninf, nan = 0x7C00, 0xFC00, 0x7E00
    assert table[128 + 3, inf] == 0x7F80 and table[128 - 3, inf] == 0xFF80
    assert table[128 + 3, ninf] == 0xFF80
    assert table[128 + 0, inf] == 0x7FC0          # 0 * Inf = NaN (canonical)
    assert table[128 + 1, nan] == 0x7FC0
    # NaN scales of either sign, times q of either sign, give the one canonical NaN
    neg_nan = 0xFE00
    assert table[128 + 1, neg_nan] == 0x7FC0
    assert table[128 - 1, nan] == 0x7FC0 and table[128 - 1, neg_nan] == 0x7FC0
    assert table[128 + 0, neg_nan] == 0x7FC0
