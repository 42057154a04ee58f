"""Pins for the oracle's q6_K decode (CPU only).

The decode is checked against what the pages fix, not against itself:
  * hand-built blocks whose codes follow from the byte map of a block
    ("r41 — q6_K B-expand widened to uint4 group loads (LANDED)", sec. 2; "r38 — q6_K BT-style
    raw-byte mma kernel (LANDED)", sec. 2.1);
  * the worked example of element 70 (r38 sec. 2.1), stored under tests/golden/;
  * the two other statements of the same index map that the pages print: the dense load-time
    expander that walks a block in (half, 64-byte run) order ("r53 — q6_K bundle: W_exp
    pre-expansion plane + cp.async B staging (LANDED)", sec. 3.2) and the 16-element group closed form of the wide-load expand (r41 sec. 3.2),
    re-expressed here in vectorised numpy;
  * the f16 d conversion against numpy's own binary16 decoder, including subnormals.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def blank_block():
    return np.zeros(210, np.uint8)


def codes(oracle_mod, blk):
    return np.array([oracle_mod.code(blk, e) for e in range(256)])


def test_all_zero_block_is_minus_32(oracle_mod):
    wc, sc, d = oracle_mod.decode(blank_block(), 1, 256)
    assert (wc == -32).all() and (sc == 0).all() and d[0, 0] == 0.0


def test_all_ones_block_is_plus_31(oracle_mod):
    blk = blank_block()
    blk[0:192] = 0xFF
    wc, _, _ = oracle_mod.decode(blk, 1, 256)
    assert (wc == 31).all()


def test_single_ql_high_nibble_hits_element_70_only(oracle_mod):
    blk = blank_block()
    blk[6] = 0xF0  # high nibble of ql[6]
    c = codes(oracle_mod, blk)
    assert c[70] == 15
    assert (np.delete(c, 70) == 0).all()
    blk[6] = 0x0F  # low nibble of ql[6] -> element 6
    c = codes(oracle_mod, blk)
    assert c[6] == 15 and (np.delete(c, 6) == 0).all()


def test_second_half_ql(oracle_mod):
    blk = blank_block()
    blk[64 + 9] = 0x5A  # ql[73]: low nibble 0xA -> element 128+9, high 0x5 -> element 128+64+9
    c = codes(oracle_mod, blk)
    assert c[137] == 0xA and c[201] == 0x5
    assert (np.delete(c, [137, 201]) == 0).all()


@pytest.mark.parametrize("j", [0, 6, 31, 32, 45, 63])
def test_single_qh_byte_fields(oracle_mod, j):
    # fields 0,1,2,3 of one qh byte serve the same offset in the four 32-element chunks of a half
    blk = blank_block()
    blk[128 + j] = 0b11100100  # fields (from bit 0): 0, 1, 2, 3
    c = codes(oracle_mod, blk)
    base = 128 * (j // 32) + (j % 32)
    want = np.zeros(256, int)
    for f in range(4):
        want[base + 32 * f] = f << 4
    np.testing.assert_array_equal(c, want)


def test_scales_and_d(oracle_mod):
    blk = blank_block()
    blk[192:208] = (np.arange(16) - 8).astype(np.int8).view(np.uint8)
    for bits, val in [(0x3800, 0.5), (0xBC00, -1.0), (0x0001, 2.0**-24), (0x03FF, 1023 * 2.0**-24),
                      (0x7BFF, 65504.0), (0x0000, 0.0)]:
        blk[208] = bits & 0xFF
        blk[209] = bits >> 8
        _, sc, d = oracle_mod.decode(blk, 1, 256)
        np.testing.assert_array_equal(sc[0], np.arange(16) - 8)
        assert d[0, 0] == val
        w = oracle_mod.dequant(blk, 1, 256)
        # every q is 0 -> value -32; element e uses scale sc[e // 16]
        np.testing.assert_array_equal(w[0], val * np.repeat(np.arange(16) - 8, 16) * -32.0)


def test_known_values_block(oracle_mod):
    # ql bytes 0x21: low nibble 1 (elements in the first 64 of each half), high nibble 2 (last 64)
    # qh bytes 0b00011011: fields 3,2,1,0 for the four 32-element chunks of each half
    blk = blank_block()
    blk[0:128] = 0x21
    blk[128:192] = 0b00011011
    blk[192:208] = 3
    blk[208], blk[209] = 0x00, 0x38  # d = 0.5
    w = oracle_mod.dequant(blk, 1, 256)[0]
    for e in range(256):
        n = e % 128
        lo = 1 if n < 64 else 2
        hi = 3 - (n // 32)
        assert w[e] == 0.5 * 3 * ((lo | (hi << 4)) - 32)


def test_worked_example_element_70(oracle_mod):
    with open(os.path.join(GOLDEN, "worked_example_elem70.json")) as f:
        g = json.load(f)
    e = g["element"]
    assert e // 256 == g["super_block"] and e // 16 == g["sub_block"]
    assert e // 32 == g["chunk"] and e % 32 == g["offset_in_chunk"] and e % 128 == g["offset_in_half"]
    # the element's scale is sub-block 4's
    blk = blank_block()
    blk[192 + g["sub_block"]] = 5
    blk[208], blk[209] = 0x00, 0x3C  # d = 1
    w = oracle_mod.dequant(blk, 1, 256)[0]
    assert w[e] == 5 * -32.0 and (w[np.arange(256) // 16 != g["sub_block"]] == 0).all()
    # ql index = offset in the half (mod 64) -> only bytes 6 can move it; qh index = offset in chunk
    for byte in range(192):
        blk2 = blank_block()
        blk2[byte] = 0xFF
        moved = codes(oracle_mod, blk2)[e] != 0
        assert moved == (byte == g["offset_in_half"] % 64 or byte == 128 + g["offset_in_chunk"])


def _dense_expander(block):
    """Second statement of the map (r53 sec. 3.2): per half and per byte r of a 64-byte ql run,
    one ql byte and one qh byte feed element (half*128 + r) from the low nibble and qh phase
    2*(r//32), and element (half*128 + r + 64) from the high nibble and phase 2*(r//32) + 4."""
    out = np.zeros(256, int)
    for half in range(2):
        r = np.arange(64)
        ql = block[64 * half + r].astype(int)
        qh = block[128 + 32 * half + (r % 32)].astype(int)
        phase = 2 * (r // 32)
        out[128 * half + r] = (ql & 15) | (((qh >> phase) & 3) << 4)
        out[128 * half + r + 64] = (ql >> 4) | (((qh >> (phase + 4)) & 3) << 4)
    return out


def _group_form(block):
    """Third statement ("r41 — q6_K B-expand widened to uint4 group loads (LANDED)", sec. 3.2):
    the expand works on 16-element groups, and every group reads exactly one 16-byte run of ql
    bytes (runs start at 0, 16, ..., 112) and one 16-byte run of qh bytes (runs start at 128,
    144, 160, 176).  Restated per group: group gi (elements 16*gi .. 16*gi+15) lies in half
    hf = gi // 8 of the block at position pos = gi % 8 of that half; it reads the ql run at
    64*hf + 16*(pos % 4), taking the high nibble for pos >= 4, and the qh run at
    128 + 32*hf + 16*(pos % 2), taking 2-bit field pos // 2 of each byte."""
    out = np.zeros(256, int)
    for gi in range(16):
        hf, pos = divmod(gi, 8)
        ql_run = block[64 * hf + 16 * (pos % 4):][:16].astype(int)
        qh_run = block[128 + 32 * hf + 16 * (pos % 2):][:16].astype(int)
        low = (ql_run >> (4 * (pos // 4))) & 15
        high = (qh_run >> (2 * (pos // 2))) & 3
        out[16 * gi:16 * gi + 16] = low | (high << 4)
    return out


def test_three_statements_of_the_map_agree(oracle_mod):
    rng = np.random.default_rng(7)
    for _ in range(200):
        blk = rng.integers(0, 256, 210, dtype=np.uint8)
        c = codes(oracle_mod, blk)
        np.testing.assert_array_equal(c, _dense_expander(blk))
        np.testing.assert_array_equal(c, _group_form(blk))


def test_decode_multi_row_multi_block_layout(oracle_mod):
    # decode of row r, block b must equal the single-block decode of bytes (r*nsb + b)*210
    rng = np.random.default_rng(3)
    m, k = 3, 768
    raw = rng.integers(0, 256, m * (k // 256) * 210, dtype=np.uint8)
    wc, sc, d = oracle_mod.decode(raw, m, k)
    for r in range(m):
        for b in range(k // 256):
            blk = raw[(r * 3 + b) * 210:(r * 3 + b + 1) * 210]
            np.testing.assert_array_equal(wc[r, b * 256:(b + 1) * 256], codes(oracle_mod, blk) - 32)
            np.testing.assert_array_equal(sc[r, b * 16:(b + 1) * 16], blk[192:208].view(np.int8))
            np.testing.assert_equal(d[r, b], float(blk[208:210].view("<f2")[0]))


def test_f16_conversion_all_finite(oracle_mod):
    # every one of the 65536 binary16 bit patterns: finite values exactly as numpy converts them
    # (subnormals included), infinities as infinities, NaNs as NaNs
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle_mod.f16_to_f64(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert fin.sum() == 0x10000 - 2 * 1024
    np.testing.assert_array_equal(got[fin], ref[fin])
    np.testing.assert_array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])
    assert np.isnan(got[np.isnan(ref)]).all()
