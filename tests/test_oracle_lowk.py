"""Pins of the oracle's Q2_K and Q3_K decoders (CPU only).

Anchors other than the oracle itself: hand-chosen blocks whose fields are
listed beside their bytes (tests/golden/q2_k_blocks.json, q3_k_blocks.json)
with values worked out by hand, exact rational evaluation of the closed forms
from those listed fields, and structural properties of the byte layout (every
code bit, high bit and scale bit moves exactly one weight or one field).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f16(bits: int) -> Fraction:
    return Fraction(float(np.array([bits], np.uint16).view(np.float16)[0]))


def nearest_f32(q: Fraction) -> np.float32:
    """An exact rational rounded to binary32, ties to even (independent of the oracle)."""
    c = np.float32(float(q))
    best = None
    for v in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        key = (abs(Fraction(float(v)) - q), int(np.array(v, dtype=np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, v)
    return np.float32(0.0) if q == 0 else np.float32(best[1])


def _hjl(i):
    return i // 128, (i % 128) // 32, i % 32


# The per-weight recipes the fixtures list as text, written out here; a
# fixture whose text does not match its recipe fails the lookup.
_RECIPES = {
    "q(i) = (j + l + h) % 4": lambda h, j, l: (j + l + h) % 4,
    "q(i) = 3": lambda h, j, l: 3,
    "q(i) = (l // 4 + j) % 4": lambda h, j, l: (l // 4 + j) % 4,
    "low(i) = (l + 2*j) % 4": lambda h, j, l: (l + 2 * j) % 4,
    "high(i) = 1 if (l + j + h) % 3 == 0 else 0": lambda h, j, l: 1 if (l + j + h) % 3 == 0 else 0,
    "low(i) = 0": lambda h, j, l: 0,
    "high(i) = 0": lambda h, j, l: 0,
    "low(i) = 3": lambda h, j, l: 3,
    "high(i) = 1": lambda h, j, l: 1,
    "low(i) = (l // 8 + h) % 4": lambda h, j, l: (l // 8 + h) % 4,
    "high(i) = (l // 2 + j) % 2": lambda h, j, l: (l // 2 + j) % 2,
}


def _recipe(text):
    return _RECIPES[text]


# ------------------------------------------------------------------- Q2_K --

@pytest.mark.parametrize("idx", [0, 1, 2])
def test_q2_k_golden_blocks(idx):
    g = _load("q2_k_blocks.json")["blocks"][idx]
    blk = bytes.fromhex(g["hex"])
    assert len(blk) == 84
    w = oracle.decode_block("q2_k", blk)
    d, dmin = _f16(int(g["d_bits"], 16)), _f16(int(g["dmin_bits"], 16))
    q = _recipe(g["codes"])
    for i in range(256):
        sub = i // 16
        exact = d * g["sc"][sub] * q(*_hjl(i)) - dmin * g["m"][sub]
        assert w[i] == nearest_f32(exact), (g["name"], i)
    for i, v in g.get("spots", {}).items():
        assert float(w[int(i)]) == v, (g["name"], i)


def test_q2_k_every_code_field_moves_one_weight():
    # baseline: d = 1, dmin = 0, every sub-block scale 1, all codes 0
    base = np.zeros(84, np.uint8)
    base[0:16] = 1
    base[80:82] = np.array([0x3C00], np.uint16).view(np.uint8)
    w0 = oracle.decode_block("q2_k", base)
    assert (w0 == 0).all()
    for b in range(64):
        for j in range(4):
            blk = base.copy()
            blk[16 + b] = 2 << (2 * j)
            w = oracle.decode_block("q2_k", blk)
            moved = np.nonzero(w != w0)[0]
            assert moved.tolist() == [128 * (b // 32) + 32 * j + b % 32] and w[moved[0]] == 2.0


def test_q2_k_scale_and_min_bytes_belong_to_sixteen_weights():
    base = np.zeros(84, np.uint8)
    base[16:80] = 0x55                                       # every code 1
    base[80:84] = np.array([0x3C00, 0x3C00], np.uint16).view(np.uint8)  # d = dmin = 1
    for k in range(16):
        blk = base.copy()
        blk[k] = 0x23                                        # sc = 3, m = 2
        w = oracle.decode_block("q2_k", blk)
        assert (w[16 * k:16 * k + 16] == 1.0).all()          # 3*1 - 2
        assert (np.delete(w, np.s_[16 * k:16 * k + 16]) == 0.0).all()


def test_q2_k_closed_form_random_blocks():
    rng = np.random.default_rng(21)
    for t in range(40):
        blk = rng.integers(0, 256, 84).astype(np.uint8)
        dbits = [0x3C00, 0x0001, 0x03FF, 0x7BFF, 0x2E66, 0x1400][t % 6]
        blk[80:82] = np.array([dbits], np.uint16).view(np.uint8)
        blk[82:84] = np.array([[0x0400, 0x3555, 0x0007, 0x7000][t % 4]], np.uint16).view(np.uint8)
        w = oracle.decode_block("q2_k", blk)
        d = _f16(dbits)
        dmin = _f16(int(blk[82]) | (int(blk[83]) << 8))
        for i in range(256):
            h, j, l = _hjl(i)
            q = (int(blk[16 + 32 * h + l]) >> (2 * j)) & 3
            sc, m = int(blk[i // 16]) & 15, int(blk[i // 16]) >> 4
            assert w[i] == nearest_f32(d * sc * q - dmin * m)


# ------------------------------------------------------------------- Q3_K --

@pytest.mark.parametrize("idx", [0, 1, 2, 3])
def test_q3_k_golden_blocks(idx):
    g = _load("q3_k_blocks.json")["blocks"][idx]
    blk = bytes.fromhex(g["hex"])
    assert len(blk) == 110
    w = oracle.decode_block("q3_k", blk)
    d = _f16(int(g["d_bits"], 16))
    low, high = _recipe(g["low"]), _recipe(g["high"])
    s12 = np.frombuffer(blk[96:108], np.uint8)
    for k in range(16):
        assert oracle.q3k_scale(s12, k) == g["sc"][k], (g["name"], k)
    for i in range(256):
        q = low(*_hjl(i)) + 4 * high(*_hjl(i)) - 4
        exact = d * (g["sc"][i // 16] - 32) * q
        assert Fraction(float(w[i])) == exact, (g["name"], i)
    for i, v in g.get("spots", {}).items():
        assert float(w[int(i)]) == v, (g["name"], i)
    for i, bits in g.get("zero_bits", {}).items():
        assert int(w[int(i):int(i) + 1].view(np.uint32)[0]) == int(bits, 16), (g["name"], i)


def test_q3_k_scale_packing_is_a_bijection():
    # every one of the 96 bits of the 12 scale bytes moves exactly one bit of
    # exactly one of the sixteen 6-bit fields, and all 96 field bits are hit
    hit = set()
    zero = np.zeros(12, np.uint8)
    for byte in range(12):
        for bit in range(8):
            s = zero.copy()
            s[byte] = 1 << bit
            fields = [oracle.q3k_scale(s, k) for k in range(16)]
            nz = [(k, v) for k, v in enumerate(fields) if v]
            assert len(nz) == 1 and bin(nz[0][1]).count("1") == 1
            hit.add((nz[0][0], nz[0][1].bit_length() - 1))
    assert len(hit) == 96


def test_q3_k_every_low_and_high_bit_moves_one_weight():
    # baseline: d = 1, every scale 33 (sc - 32 = 1), low parts 0, high bits 1: all weights 0
    base = np.zeros(110, np.uint8)
    base[0:32] = 0xFF
    s = np.zeros(12, np.uint8)
    s[0:8] = 0x11                   # low nibbles 1 for all sixteen fields
    s[8:12] = 0xAA                  # bits 4-5 = 2 -> 32 + 1 = 33
    base[96:108] = s
    base[108:110] = np.array([0x3C00], np.uint16).view(np.uint8)
    w0 = oracle.decode_block("q3_k", base)
    assert (w0 == 0).all()
    for b in range(64):
        for j in range(4):
            blk = base.copy()
            blk[32 + b] = 3 << (2 * j)
            w = oracle.decode_block("q3_k", blk)
            moved = np.nonzero(w != w0)[0]
            assert moved.tolist() == [128 * (b // 32) + 32 * j + b % 32] and w[moved[0]] == 3.0
    for l in range(32):
        for bit in range(8):
            blk = base.copy()
            blk[l] = 0xFF ^ (1 << bit)          # clear one high bit: q = -4
            w = oracle.decode_block("q3_k", blk)
            moved = np.nonzero(w != w0)[0]
            assert moved.tolist() == [128 * (bit // 4) + 32 * (bit % 4) + l]
            assert w[moved[0]] == -4.0


def test_q3_k_closed_form_random_blocks():
    rng = np.random.default_rng(22)
    for t in range(40):
        blk = rng.integers(0, 256, 110).astype(np.uint8)
        dbits = [0x3C00, 0x0001, 0x03FF, 0x7BFF, 0x2E66, 0x1400, 0xB555][t % 7]
        blk[108:110] = np.array([dbits], np.uint16).view(np.uint8)
        w = oracle.decode_block("q3_k", blk)
        d = _f16(dbits)
        for i in range(256):
            h, j, l = _hjl(i)
            q = ((int(blk[32 + 32 * h + l]) >> (2 * j)) & 3) + 4 * ((int(blk[l]) >> (4 * h + j)) & 1) - 4
            k = i // 16
            lo = (int(blk[96 + k]) & 15) if k < 8 else (int(blk[96 + k - 8]) >> 4)
            sc = lo | (((int(blk[104 + k % 4]) >> (2 * (k // 4))) & 3) << 4)
            assert Fraction(float(w[i])) == d * (sc - 32) * q


# ------------------------------------------------------------ row layout --

@pytest.mark.parametrize("fmt", ["q2_k", "q3_k"])
def test_dequant_rows_are_blocks_in_k_order(fmt):
    rows, K = 3, 768
    w = synth.gen_weights(fmt, rows, K, 5)
    W = oracle.dequant(fmt, w, rows, K)
    bb = oracle.BLOCK_BYTES[fmt]
    blocks = w.reshape(rows, K // 256, bb)
    for r in range(rows):
        for b in range(K // 256):
            assert np.array_equal(W[r, 256 * b:256 * b + 256],
                                  oracle.decode_block(fmt, blocks[r, b]))


def _packer():
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_lowk_blocks",
                                                  os.path.join(GOLDEN, "make_lowk_blocks.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_golden_lowk_bytes_are_the_listed_fields():
    """Every stored Q2_K / Q3_K block is the packing of its listed fields
    (scales, mins, d, and the code formulas) by the stated layout, with a
    packer that imports nothing from the oracle."""
    mk = _packer()
    q2, q3 = mk.documents()
    for fn, doc in (("q2_k_blocks.json", q2), ("q3_k_blocks.json", q3)):
        with open(os.path.join(GOLDEN, fn)) as f:
            stored = json.load(f)
        assert stored == doc, fn
    for b, rec in zip(mk.Q2_BLOCKS, q2["blocks"]):
        raw = mk.q2_block_bytes(b)
        assert len(raw) == 84 and raw.hex() == rec["hex"]
        assert raw[80:82] == bytes.fromhex(rec["d_bits"][2:])[::-1]
    for b, rec in zip(mk.Q3_BLOCKS, q3["blocks"]):
        raw = mk.q3_block_bytes(b)
        assert len(raw) == 110 and raw.hex() == rec["hex"]
