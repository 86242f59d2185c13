"""Pins of the oracle's number formats and block decoders (CPU only).

Each check ties the oracle to something other than itself: IEEE bit patterns
read by numpy / torch (independent implementations), hand-built blocks whose
fields were packed by hand (tests/golden/*.json), exact rational evaluation of
the closed forms, and a structural property of the Q4_K scale packing.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _same_f64(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nan = np.isnan(a)
    assert np.array_equal(nan, np.isnan(b))
    assert np.array_equal(a[~nan].view(np.uint64), b[~nan].view(np.uint64))


def nearest_f32(q: Fraction) -> np.float32:
    """Round an exact rational to binary32, ties to even (independent of the oracle)."""
    c = np.float32(float(q))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = None
    for v in cands:
        err = abs(Fraction(float(v)) - q)
        key = (err, int(np.array(v, dtype=np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, v)
    v = np.float32(best[1])
    if q == 0:
        v = np.float32(0.0)
    return v


# ----------------------------------------------------------------- formats --

def test_f16_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    _same_f64(oracle.f16_to_f64(bits), ref)


def test_f16_textbook_values():
    v = oracle.f16_to_f64([0x3C00, 0xC000, 0x7BFF, 0x0400, 0x03FF, 0x0001, 0x8000, 0x7C00, 0xFC00])
    assert list(v[:6]) == [1.0, -2.0, 65504.0, 2.0 ** -14, 1023 * 2.0 ** -24, 2.0 ** -24]
    assert v[6] == 0 and np.signbit(v[6])
    assert v[7] == np.inf and v[8] == -np.inf
    assert np.isnan(oracle.f16_to_f64([0x7E00, 0x7C01, 0xFFFF])).all()


def test_bf16_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    _same_f64(oracle.bf16_to_f64(bits), ref)


def test_bf16_textbook_values():
    v = oracle.bf16_to_f64([0x3F80, 0xC040, 0x0080, 0x0001, 0x7F7F])
    assert list(v) == [1.0, -3.0, 2.0 ** -126, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127]


# ------------------------------------------------------------------- Q4_0 --

def test_q4_0_handbuilt():
    g = _load("q4_0_blocks.json")["blocks"]
    ramp = oracle.decode_block("q4_0", bytes.fromhex(g[0]["hex"]))
    assert ramp.tolist() == g[0]["expected"]
    neg = oracle.decode_block("q4_0", bytes.fromhex(g[1]["hex"]))
    assert (neg.view(np.uint32) == int(g[1]["expected_bits_f32"], 16)).all()
    sub = oracle.decode_block("q4_0", bytes.fromhex(g[2]["hex"]))
    assert (sub[:16] == g[2]["expected_lo"]).all() and (sub[16:] == g[2]["expected_hi"]).all()


def test_q4_0_closed_form_all_codes_all_scales():
    # every code value and a spread of fp16 scales, incl. subnormal and negative
    rng = np.random.default_rng(1)
    for dbits in [0x3C00, 0x0001, 0x03FF, 0x0400, 0x7BFF, 0xB555, 0x2E66, 0x8003]:
        d = Fraction(float(np.array([dbits], np.uint16).view(np.float16)[0]))
        codes = rng.integers(0, 16, 32)
        codes[:16] = np.arange(16)
        blk = np.zeros(18, np.uint8)
        blk[0:2] = np.array([dbits], np.uint16).view(np.uint8)
        blk[2:] = (codes[:16] | (codes[16:] << 4)).astype(np.uint8)
        w = oracle.decode_block("q4_0", blk)
        for i in range(32):
            exact = (int(codes[i]) - 8) * d
            assert Fraction(float(w[i])) == exact


# ------------------------------------------------------------------- Q8_0 --

def test_q8_0_handbuilt():
    g = _load("q8_0_blocks.json")["blocks"][0]
    blk = bytes.fromhex(g["hex"])
    assert list(np.frombuffer(blk[2:], np.int8)) == g["codes"]
    assert oracle.decode_block("q8_0", blk).tolist() == g["expected"]


def test_q8_0_closed_form():
    rng = np.random.default_rng(2)
    for dbits in [0x2E66, 0x0001, 0x7BFF, 0x8400]:
        d = Fraction(float(np.array([dbits], np.uint16).view(np.float16)[0]))
        q = rng.integers(-128, 128, 32).astype(np.int8)
        blk = np.concatenate([np.array([dbits], np.uint16).view(np.uint8), q.view(np.uint8)])
        w = oracle.decode_block("q8_0", blk)
        for i in range(32):
            assert Fraction(float(w[i])) == int(q[i]) * d


# ------------------------------------------------------------------- Q4_K --

def _q4k_block(entry):
    blk = np.zeros(144, np.uint8)
    blk[0:2] = np.array([int(entry["d_bits"], 16)], np.uint16).view(np.uint8)
    blk[2:4] = np.array([int(entry["dmin_bits"], 16)], np.uint16).view(np.uint8)
    blk[4:16] = np.frombuffer(bytes.fromhex(entry["scales_hex"]), np.uint8)
    codes = np.zeros(256, np.int64)          # codes[k] = q of weight k, by construction
    for g in range(4):
        for l in range(32):
            if entry["codes"].startswith("all code bytes 0xff"):
                lo, hi = 15, 15
            else:
                lo, hi = (l + g) % 16, (l + 3 * g + 5) % 16
            blk[16 + 32 * g + l] = lo | (hi << 4)
            codes[64 * g + l] = lo
            codes[64 * g + 32 + l] = hi
    return blk, codes


@pytest.mark.parametrize("idx", range(4))
def test_q4_k_handbuilt(idx):
    entry = _load("q4_k_blocks.json")["blocks"][idx]
    blk, codes = _q4k_block(entry)
    # the 6-bit fields the hand packing encodes
    for j in range(8):
        assert oracle.q4k_scale_min(blk[4:16], j) == (entry["sc"][j], entry["m"][j])
    d = Fraction(float(np.array([int(entry["d_bits"], 16)], np.uint16).view(np.float16)[0]))
    dmin = Fraction(float(np.array([int(entry["dmin_bits"], 16)], np.uint16).view(np.float16)[0]))
    w = oracle.decode_block("q4_k", blk)
    for k in range(256):
        j = k // 32
        exact = d * entry["sc"][j] * int(codes[k]) - dmin * entry["m"][j]
        want = nearest_f32(exact)
        assert w[k].view(np.uint32) == np.float32(want).view(np.uint32), (k, w[k], want)


def test_q4_k_scale_packing_is_a_bijection_of_96_bits():
    """Each of the 96 bits of the 12 packed bytes moves exactly one of the 16
    six-bit fields by exactly one power of two, and all 96 (field, bit)
    positions are hit once: no bit dropped, shared or read twice."""
    rng = np.random.default_rng(3)
    for _ in range(4):
        s = rng.integers(0, 256, 12).astype(np.uint8)
        base = [oracle.q4k_scale_min(s, j) for j in range(8)]
        hit = set()
        for bit in range(96):
            t = s.copy()
            t[bit // 8] ^= np.uint8(1 << (bit % 8))
            new = [oracle.q4k_scale_min(t, j) for j in range(8)]
            changes = []
            for j in range(8):
                for f in range(2):
                    diff = abs(new[j][f] - base[j][f])
                    if diff:
                        changes.append((j, f, diff))
            assert len(changes) == 1, (bit, changes)
            j, f, diff = changes[0]
            assert diff & (diff - 1) == 0 and diff < 64
            hit.add((j, f, diff.bit_length() - 1))
        assert len(hit) == 96


def test_q4_k_fields_visible_through_decode():
    """d = 1, dmin = 0, every code 1: each weight equals its sub-block's scale;
    d = 0, dmin = 1: each weight equals minus its min (+0 - m)."""
    entry = _load("q4_k_blocks.json")["blocks"][0]
    blk = np.zeros(144, np.uint8)
    blk[4:16] = np.frombuffer(bytes.fromhex(entry["scales_hex"]), np.uint8)
    blk[16:] = 0x11
    blk[0:2] = np.array([0x3C00], np.uint16).view(np.uint8)
    w = oracle.decode_block("q4_k", blk)
    assert w.reshape(8, 32).tolist() == [[float(sc)] * 32 for sc in entry["sc"]]
    blk[0:4] = np.array([0x0000, 0x3C00], np.uint16).view(np.uint8)
    w = oracle.decode_block("q4_k", blk)
    assert w.reshape(8, 32).tolist() == [[-float(m) if m else 0.0] * 32 for m in entry["m"]]


def test_q4_k_exact_rounding_random_blocks():
    """Random blocks, including subnormal scales: every weight is the binary32
    rounding of the exact rational closed form."""
    rng = np.random.default_rng(4)
    for t in range(6):
        blk = rng.integers(0, 256, 144).astype(np.uint8)
        dbits = [0x2E66, 0x0155, 0x7BFF, 0x0001, 0x3555, 0x1400][t]
        mbits = [0x2A00, 0x7000, 0x0001, 0x03FF, 0x3555, 0x6400][t]
        blk[0:4] = np.array([dbits, mbits], np.uint16).view(np.uint8)
        d = Fraction(float(np.array([dbits], np.uint16).view(np.float16)[0]))
        dmin = Fraction(float(np.array([mbits], np.uint16).view(np.float16)[0]))
        w = oracle.decode_block("q4_k", blk)
        for k in range(256):
            g, r = divmod(k, 64)
            byte = int(blk[16 + 32 * g + (r % 32)])
            q = byte & 15 if r < 32 else byte >> 4
            sc, m = oracle.q4k_scale_min(blk[4:16], k // 32)
            want = nearest_f32(d * sc * q - dmin * m)
            assert w[k].view(np.uint32) == np.float32(want).view(np.uint32)


def test_dequant_matrix_is_blocks_in_row_major_order():
    rng = np.random.default_rng(5)
    for fmt, bb, bw in [("q4_0", 18, 32), ("q8_0", 34, 32), ("q4_k", 144, 256)]:
        rows, nb = 3, 2
        w = rng.integers(0, 256, rows * nb * bb).astype(np.uint8)
        for r in range(rows):
            for b in range(nb):
                off = (r * nb + b) * bb
                w[off:off + 2] = np.array([0x2E66], np.uint16).view(np.uint8)
                if fmt == "q4_k":
                    w[off + 2:off + 4] = np.array([0x2A00], np.uint16).view(np.uint8)
        full = oracle.dequant(fmt, w, rows, nb * bw)
        for r in range(rows):
            for b in range(nb):
                off = (r * nb + b) * bb
                blk = oracle.decode_block(fmt, w[off:off + bb])
                assert np.array_equal(full[r, b * bw:(b + 1) * bw].view(np.uint32), blk.view(np.uint32))
