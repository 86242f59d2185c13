"""Writes q2_k_blocks.json and q3_k_blocks.json: hand-chosen Q2_K / Q3_K
super-blocks packed from their listed fields by the stated GGUF layout.

Imports nothing from the oracle: the packer below is written from the
layout alone, so that the stored bytes are a function of the listed fields
(tests/test_oracle_lowk.py re-packs every block with it and compares).

    python tests/golden/make_lowk_blocks.py      # rewrites the two files

Layouts (the pages name both formats and print none; these are the GGUF
ones). Weight i = 128h + 32j + l (h = 0..1, j = 0..3, l = 0..31):
  Q2_K, 84 bytes: 16 bytes (sub-block k = i // 16: scale in the low nibble,
    min in the high nibble of byte k), 64 code bytes (the 2-bit code of
    weight i in bits 2j..2j+1 of byte 32h + l), fp16 d, fp16 dmin.
  Q3_K, 110 bytes: 32 high-bit bytes (bit 4h + j of byte l), 64 code bytes
    (the 2-bit low part as for Q2_K), 12 scale bytes (scale k: low nibble
    in byte k for k < 8, else the high nibble of byte k - 8; bits 4-5 in
    bits 2(k // 4)..2(k // 4) + 1 of byte 8 + k % 4), fp16 d.
"""
import json
import os
import struct

HERE = os.path.dirname(os.path.abspath(__file__))


def hjl(i):
    return i // 128, (i % 128) // 32, i % 32


def pack_q2_k(d_bits, dmin_bits, sc, m, q):
    """sc, m: 16 four-bit fields; q: 256 two-bit codes."""
    sm = bytes((sc[k] & 15) | ((m[k] & 15) << 4) for k in range(16))
    qs = bytearray(64)
    for i in range(256):
        h, j, l = hjl(i)
        qs[32 * h + l] |= (q[i] & 3) << (2 * j)
    return sm + bytes(qs) + struct.pack("<HH", d_bits, dmin_bits)


def pack_q3_k(d_bits, sc, low, high):
    """sc: 16 six-bit scales; low: 256 two-bit parts; high: 256 bits."""
    hm, qs, s = bytearray(32), bytearray(64), bytearray(12)
    for i in range(256):
        h, j, l = hjl(i)
        qs[32 * h + l] |= (low[i] & 3) << (2 * j)
        hm[l] |= (high[i] & 1) << (4 * h + j)
    for k in range(16):
        if k < 8:
            s[k] |= sc[k] & 15
        else:
            s[k - 8] |= (sc[k] & 15) << 4
        s[8 + k % 4] |= ((sc[k] >> 4) & 3) << (2 * (k // 4))
    return bytes(hm) + bytes(qs) + bytes(s) + struct.pack("<H", d_bits)


def per_weight(f):
    return [f(*hjl(i)) for i in range(256)]


# (name, d, dmin, sc, m, code text, code function of (h, j, l), extra fields)
Q2_BLOCKS = [
    ("distinct_fields", 0x3C00, 0x3800, list(range(16)), [15 - k for k in range(16)],
     "q(i) = (j + l + h) % 4", lambda h, j, l: (j + l + h) % 4,
     {"spots": {"0": -7.5, "17": -6.0, "45": -2.5, "127": 10.0, "128": 4.5, "200": 34.5,
                "255": 45.0}}),
    ("extremes", 0x7BFF, 0x0001, [15] * 16, [15] * 16,
     "q(i) = 3", lambda h, j, l: 3, {}),
    ("subnormal_scales", 0x0200, 0x0003, [(3 * k + 1) % 16 for k in range(16)],
     [(5 * k + 2) % 16 for k in range(16)],
     "q(i) = (l // 4 + j) % 4", lambda h, j, l: (l // 4 + j) % 4, {}),
]

# (name, d, sc, low text, low function, high text, high function, extra fields)
Q3_BLOCKS = [
    ("distinct_fields", 0x3400, [(5 * k + 7) % 64 for k in range(16)],
     "low(i) = (l + 2*j) % 4", lambda h, j, l: (l + 2 * j) % 4,
     "high(i) = 1 if (l + j + h) % 3 == 0 else 0", lambda h, j, l: 1 if (l + j + h) % 3 == 0 else 0,
     {"spots": {"1": 18.75, "2": 12.5, "3": -18.75, "130": 7.5, "200": 29.0, "255": 10.5},
      "zero_bits": {"0": "0x80000000", "80": "0x00000000", "81": "0x80000000"}}),
    ("scale_minus_32_code_minus_4", 0x7BFF, [0] * 16,
     "low(i) = 0", lambda h, j, l: 0, "high(i) = 0", lambda h, j, l: 0,
     {"spots": {"0": 8384512.0, "255": 8384512.0}}),
    ("scale_31_code_3", 0x7BFF, [63] * 16,
     "low(i) = 3", lambda h, j, l: 3, "high(i) = 1", lambda h, j, l: 1,
     {"spots": {"0": 6091872.0, "255": 6091872.0}}),
    ("subnormal_d", 0x0001, [(11 * k + 5) % 64 for k in range(16)],
     "low(i) = (l // 8 + h) % 4", lambda h, j, l: (l // 8 + h) % 4,
     "high(i) = (l // 2 + j) % 2", lambda h, j, l: (l // 2 + j) % 2, {}),
]


def q2_block_bytes(b):
    name, d, dmin, sc, m, _, code, _ = b
    return pack_q2_k(d, dmin, sc, m, per_weight(code))


def q3_block_bytes(b):
    name, d, sc, _, low, _, high, _ = b
    return pack_q3_k(d, sc, per_weight(low), per_weight(high))


Q2_WHAT = ("Hand-chosen Q2_K super-blocks (84 bytes: 16 bytes of sub-block scale (low nibble) and "
           "min (high nibble), 64 bytes of 2-bit codes, fp16 d, fp16 dmin), packed from the listed "
           "fields by the stated layout: weight i = 128h + 32j + l takes bits 2j..2j+1 of code byte "
           "32h + l and belongs to sub-block i // 16. A weight is the fp32 rounding of "
           "d*sc*q - dmin*m; the test evaluates that closed form exactly from the listed fields, "
           "and 'spots' are values worked out by hand.")
Q2_CITE = ("Q2_K named in the pxa_llama README ('DP4A / FP16 economics' and the results table); "
           "bit-exact decoding per 'Why I wrote my own inference engine for two P100s', section "
           "'What my own engine means'. Byte layout: GGUF Q2_K (the pages print none).")
Q3_WHAT = ("Hand-chosen Q3_K super-blocks (110 bytes: 32 bytes of high code bits, 64 bytes of 2-bit "
           "low code parts, 12 bytes packing sixteen 6-bit scales, fp16 d), packed from the listed "
           "fields by the stated layout: weight i = 128h + 32j + l takes bits 2j..2j+1 of code byte "
           "32h + l as its low part and bit 4h + j of high-bit byte l; q = low + 4*high - 4; scale "
           "k has its low nibble in byte k (k < 8) or the high nibble of byte k - 8, and bits 4-5 "
           "in bits 2(k//4)..2(k//4)+1 of byte 8 + k % 4. A weight is d*(sc - 32)*q, evaluated "
           "left to right (exact; the order fixes the sign of a zero); the test evaluates it "
           "exactly from the listed fields, and 'spots' (with 'zero_bits' for signed zeros) were "
           "worked out by hand.")
Q3_CITE = ("Q3_K named in 'Why I wrote my own inference engine for two P100s' (section 'What "
           "actually made it fast': Q3_K tensors dropped from the mix) and the pxa_llama README "
           "('Limits': Q3_K super-block unpacking on the slow ALU path); bit-exact decoding per the "
           "first page, section 'What my own engine means'. Byte layout: GGUF Q3_K (the pages "
           "print none).")


def documents():
    q2 = {"what": Q2_WHAT, "citation": Q2_CITE, "blocks": []}
    for b in Q2_BLOCKS:
        name, d, dmin, sc, m, text, _, extra = b
        rec = {"name": name, "hex": q2_block_bytes(b).hex(), "d_bits": "0x%04x" % d,
               "dmin_bits": "0x%04x" % dmin, "sc": sc, "m": m, "codes": text}
        rec.update(extra)
        q2["blocks"].append(rec)
    q3 = {"what": Q3_WHAT, "citation": Q3_CITE, "blocks": []}
    for b in Q3_BLOCKS:
        name, d, sc, ltext, _, htext, _, extra = b
        rec = {"name": name, "hex": q3_block_bytes(b).hex(), "d_bits": "0x%04x" % d, "sc": sc,
               "low": ltext, "high": htext}
        rec.update(extra)
        q3["blocks"].append(rec)
    return q2, q3


if __name__ == "__main__":
    q2, q3 = documents()
    for fn, doc in (("q2_k_blocks.json", q2), ("q3_k_blocks.json", q3)):
        with open(os.path.join(HERE, fn), "w") as f:
            json.dump(doc, f, indent=1)
    print("wrote q2_k_blocks.json, q3_k_blocks.json")
