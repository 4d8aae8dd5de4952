"""Pins of the 656-B Q8G64 row format and of the oracle's row layout.

The page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading"
describes a row as 512 B latent + 16 B scales + 128 B RoPE (section "Separate
historical capacity from the current working set") and prints payload sizes
derived from it; tests/golden/capacity.tsv holds those printed figures.
"""
import os
import re

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
UNIT = {"MiB": 2 ** 20, "GiB": 2 ** 30, "TiB": 2 ** 40}


def _golden():
    rows = []
    with open(os.path.join(HERE, "golden", "capacity.tsv")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            r, l, rep, cp, unit, printed, *_ = line.rstrip("\n").split("\t")
            rows.append((int(r), int(l), int(rep), int(cp), unit, printed))
    return rows


def test_row_is_656_bytes_and_reproduces_every_printed_payload():
    assert 512 + 8 * 2 + 64 * 2 == 656 == oracle.ROW_BYTES
    golden = _golden()
    assert len(golden) == 8
    for r, l, rep, cp, unit, printed in golden:
        value = r * l * rep * cp * oracle.ROW_BYTES / UNIT[unit]
        digits = len(printed.split(".")[1]) if "." in printed else 0
        assert f"{value:.{digits}f}" == printed, (r, l, rep, cp, unit, printed, value)


def test_exact_byte_counts_of_selection_and_cache():
    assert 2048 * 656 == 1_343_488 == int(1.28125 * 2 ** 20)
    assert 32768 * 656 == 21_495_808 == int(20.5 * 2 ** 20)
    # one gathered row in bf16: 512 dequantised + 64 RoPE values
    assert oracle.OUT_ELEMS * 2 == 1152


def test_header_constants_match_the_format():
    text = open(os.path.join(ROOT, "include", "hc.h")).read()
    consts = dict(re.findall(r"#define\s+(HC_\w+)\s+(\d+)", text))
    assert int(consts["HC_ROW_BYTES"]) == 656
    assert int(consts["HC_LATENT_BYTES"]) == 512
    assert int(consts["HC_SCALE_OFFSET"]) == 512
    assert int(consts["HC_ROPE_OFFSET"]) == 528
    assert int(consts["HC_OUT_ELEMS"]) == 576


def _one_hot_row(j, q, g, scale_bits):
    row = np.zeros(656, np.uint8)
    row[j] = np.uint8(q & 0xFF)
    row[512 + 2 * g] = scale_bits & 0xFF
    row[513 + 2 * g] = scale_bits >> 8
    return row


def test_scale_group_g_covers_latent_bytes_64g_to_64g_plus_64():
    one = 0x3C00  # fp16 1.0
    for j in (0, 1, 63, 64, 127, 128, 300, 447, 448, 511):
        for g in range(8):
            out = oracle.dequant_row(_one_hot_row(j, 3, g, one))
            # bf16 3.0 = 0x4040 where the scale applies, +0 (scale 0) elsewhere
            expect = np.zeros(576, np.uint16)
            if j // 64 == g:
                expect[j] = 0x4040
            np.testing.assert_array_equal(out, expect, err_msg=f"j={j} g={g}")


def test_rope_is_copied_bit_for_bit_little_endian():
    rng = np.random.default_rng(7)
    row = rng.integers(0, 256, 656, dtype=np.uint8)
    row[512:528] = 0  # zero scales
    out = oracle.dequant_row(row)
    rope = row[528:656].view("<u2")
    np.testing.assert_array_equal(out[512:], rope)
    # latent with zero scale: +0 for q >= 0, -0 for q < 0 (sign of the product)
    q = row[:512].view(np.int8)
    np.testing.assert_array_equal(out[:512], np.where(q < 0, 0x8000, 0).astype(np.uint16))


def test_dequant_worked_values():
    # value(scale) * q for hand-computed cases; bf16 bits written out by hand.
    cases = [
        (1, 0x3C00, 0x3F80),      # 1 * 1.0 = 1.0
        (-1, 0x3C00, 0xBF80),     # -1.0
        (127, 0x3C00, 0x42FE),    # 127.0 = 1.984375 * 2^6
        (-128, 0x3C00, 0xC300),   # -128.0
        (2, 0x3800, 0x3F80),      # 2 * 0.5
        (3, 0x3555, 0x3F80),      # 3 * 0.333251953125 = 0.999755859375 -> 1.0
        (1, 0x0001, 0x3380),      # smallest fp16 subnormal 2^-24
        (127, 0x7BFF, 0x4AFE),    # 127 * 65504 = 8319008 -> 254 * 2^15 = 8323072 (RNE)
        (0, 0xBC00, 0x8000),      # 0 * -1.0 = -0
        (-5, 0x8000, 0x0000),     # -5 * -0 = +0
    ]
    for q, s, expect in cases:
        assert oracle.dequant_elem(q, s) == expect, (q, hex(s))
    # -127 * 0.0999755859375 = -12.6968994140625; bf16 neighbours -12.6875
    # (0xC14B) and -12.75 (0xC14C); the nearer is -12.6875.
    assert oracle.dequant_elem(-127, 0x2E66) == 0xC14B
