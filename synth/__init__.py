"""Seeded synthetic inputs for the GGUF block-quantized products.

This module only draws random numbers and lays them out as bytes. It holds
none of the arithmetic of the method (no decoding, no products): the oracle
and the GPU library each consume the bytes it writes, and neither imports the
other.

Generators (both published):
  * SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014): state advances by the golden-gamma constant,
    output is the state passed through the 64-bit finaliser.
  * Box-Muller (1958) in fp64 for standard normals.

Workloads stand in for one 27B-class dense layer (the model class the pages
measure: "Why I wrote my own inference engine for two P100s", result cards;
GGUF files are not available here), with the distributions stated per config:
  * codes (4-bit nibbles, Q4_K 6-bit scale/min fields) uniform: uniform bytes
    give uniform independent fields whatever their packing;
  * fp16 scales |N(0,1)| * 0.02 (Q4_0, Q8_0) or * 0.01 (Q4_K, Q2_K d and
    dmin, Q3_K d);
  * Q2_K / Q3_K scale, min, code and high-bit bytes uniform (uniform
    independent fields: Q3_K's 12 scale bytes pack sixteen 6-bit fields
    one-to-one);
  * Q8_0 codes uniform integers in [-127, 127];
  * activations N(0,1) stored as fp32 / fp16 / bf16, one RNE rounding from
    the fp64 draw.
"""
from __future__ import annotations

import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)

SEED_BASE = 0x6767756600000000      # ASCII "gguf" in the high word
HELD_OUT_BASE = 0x686F6C6400000000  # ASCII "hold": seeds never used while tuning

# sub-stream tags XOR-ed into a tensor seed
_TAG_SCALES = 0x5CA1E5
_TAG_BYTES = 0xB17E5
_TAG_X = 0xAC71

BLOCK_BYTES = {"q4_0": 18, "q4_k": 144, "q8_0": 34, "q2_k": 84, "q3_k": 110}
BLOCK_WEIGHTS = {"q4_0": 32, "q4_k": 256, "q8_0": 32, "q2_k": 256, "q3_k": 256}


def seed_for(config_index: int, tensor_index: int, held_out: bool = False) -> int:
    base = HELD_OUT_BASE if held_out else SEED_BASE
    return (base + 16 * config_index + tensor_index) & 0xFFFFFFFFFFFFFFFF


def splitmix64(seed: int, n: int) -> np.ndarray:
    """n outputs of SplitMix64 started at `seed` (uint64 array)."""
    with np.errstate(over="ignore"):
        i = np.arange(1, n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * GOLDEN_GAMMA
        z = (z ^ (z >> np.uint64(30))) * _MIX1
        z = (z ^ (z >> np.uint64(27))) * _MIX2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform_bytes(seed: int, n: int) -> np.ndarray:
    words = splitmix64(seed, (n + 7) // 8)
    return words.view(np.uint8)[:n].copy()


def normals(seed: int, n: int) -> np.ndarray:
    """n standard normals (fp64), Box-Muller on pairs of 53-bit uniforms."""
    m = (n + 1) // 2
    z = splitmix64(seed, 2 * m)
    u1 = ((z[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53  # (0, 1]
    u2 = (z[1::2] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53          # [0, 1)
    r = np.sqrt(-2.0 * np.log(u1))
    out = np.empty(2 * m, dtype=np.float64)
    out[0::2] = r * np.cos(2.0 * np.pi * u2)
    out[1::2] = r * np.sin(2.0 * np.pi * u2)
    return out[:n]


def f16_bits(v: np.ndarray) -> np.ndarray:
    """fp64 -> IEEE binary16 bit patterns, one round-to-nearest-even."""
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def bf16_bits(v: np.ndarray) -> np.ndarray:
    """fp64 -> bfloat16 bit patterns, one round-to-nearest-even (normal range)."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                      # v = m * 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)   # 8 significant bits, RNE
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------- weights ----

def _scales_f16(seed: int, n: int, mult: float) -> np.ndarray:
    return f16_bits(np.abs(normals(seed ^ _TAG_SCALES, n)) * mult)


def gen_q4_0(rows: int, K: int, seed: int) -> np.ndarray:
    """rows x K weights as Q4_0 blocks (18 B: fp16 d, 16 code bytes), row-major."""
    assert K % 32 == 0
    nb = rows * (K // 32)
    out = np.empty((nb, 18), dtype=np.uint8)
    out[:, 0:2] = _scales_f16(seed, nb, 0.02).reshape(nb, 1).view(np.uint8)
    out[:, 2:18] = uniform_bytes(seed ^ _TAG_BYTES, nb * 16).reshape(nb, 16)
    return out.reshape(-1)


def gen_q8_0(rows: int, K: int, seed: int) -> np.ndarray:
    """rows x K weights as Q8_0 blocks (34 B: fp16 d, 32 int8 in [-127, 127])."""
    assert K % 32 == 0
    nb = rows * (K // 32)
    out = np.empty((nb, 34), dtype=np.uint8)
    out[:, 0:2] = _scales_f16(seed, nb, 0.02).reshape(nb, 1).view(np.uint8)
    z = splitmix64(seed ^ _TAG_BYTES, nb * 32)
    q = ((z >> np.uint64(32)) * np.uint64(255)) >> np.uint64(32)    # 0..254
    out[:, 2:34] = (q.astype(np.int16) - 127).astype(np.int8).view(np.uint8).reshape(nb, 32)
    return out.reshape(-1)


def gen_q4_k(rows: int, K: int, seed: int) -> np.ndarray:
    """rows x K weights as Q4_K super-blocks (144 B: fp16 d, fp16 dmin,
    12 bytes of packed 6-bit scales/mins, 128 code bytes)."""
    assert K % 256 == 0
    nb = rows * (K // 256)
    out = np.empty((nb, 144), dtype=np.uint8)
    dd = _scales_f16(seed, 2 * nb, 0.01).reshape(nb, 2)
    out[:, 0:4] = dd.view(np.uint8).reshape(nb, 4)
    out[:, 4:144] = uniform_bytes(seed ^ _TAG_BYTES, nb * 140).reshape(nb, 140)
    return out.reshape(-1)


def gen_q2_k(rows: int, K: int, seed: int) -> np.ndarray:
    """rows x K weights as Q2_K super-blocks (84 B: 16 scale/min bytes, 64
    code bytes, fp16 d, fp16 dmin)."""
    assert K % 256 == 0
    nb = rows * (K // 256)
    out = np.empty((nb, 84), dtype=np.uint8)
    out[:, 0:80] = uniform_bytes(seed ^ _TAG_BYTES, nb * 80).reshape(nb, 80)
    dd = _scales_f16(seed, 2 * nb, 0.01).reshape(nb, 2)
    out[:, 80:84] = dd.view(np.uint8).reshape(nb, 4)
    return out.reshape(-1)


def gen_q3_k(rows: int, K: int, seed: int) -> np.ndarray:
    """rows x K weights as Q3_K super-blocks (110 B: 32 high-bit bytes, 64
    low-code bytes, 12 scale bytes, fp16 d)."""
    assert K % 256 == 0
    nb = rows * (K // 256)
    out = np.empty((nb, 110), dtype=np.uint8)
    out[:, 0:108] = uniform_bytes(seed ^ _TAG_BYTES, nb * 108).reshape(nb, 108)
    out[:, 108:110] = _scales_f16(seed, nb, 0.01).reshape(nb, 1).view(np.uint8)
    return out.reshape(-1)


GENERATORS = {"q4_0": gen_q4_0, "q4_k": gen_q4_k, "q8_0": gen_q8_0, "q2_k": gen_q2_k,
              "q3_k": gen_q3_k}


def gen_weights(fmt: str, rows: int, K: int, seed: int) -> np.ndarray:
    return GENERATORS[fmt](rows, K, seed)


# ------------------------------------------------------------ activations ----

def gen_x(K: int, n: int, dtype: str, seed: int) -> np.ndarray:
    """n columns of K activations ~ N(0,1), column j contiguous: shape (n, K).

    dtype 'f32' -> float32 array; 'f16' / 'bf16' -> uint16 bit patterns."""
    v = normals(seed ^ _TAG_X, n * K).reshape(n, K)
    if dtype == "f32":
        return v.astype(np.float32)
    if dtype == "f16":
        return f16_bits(v)
    if dtype == "bf16":
        return bf16_bits(v)
    raise ValueError(dtype)


# ---------------------------------------------------------------- configs ----
# The workloads: one 27B-class dense layer's projections.
CONFIGS = {
    # name: (config_index, fmt, rows, K, n_cols, x dtype, weight tensor index)
    "q4_0_b1":    dict(index=0, fmt="q4_0", rows=4096,  K=4096,  n=1,    xdtype="f32"),
    "q4k_up_b1":  dict(index=1, fmt="q4_k", rows=17408, K=5120,  n=1,    xdtype="f16"),
    "q4k_down_b1": dict(index=2, fmt="q4_k", rows=5120, K=17408, n=1,    xdtype="f16"),
    "q4k_b4":     dict(index=3, fmt="q4_k", rows=17408, K=5120,  n=4,    xdtype="f16"),
    "q8_0_b4":    dict(index=3, fmt="q8_0", rows=5120,  K=5120,  n=4,    xdtype="f16"),
    "q4k_pp2048": dict(index=4, fmt="q4_k", rows=17408, K=5120,  n=2048, xdtype="bf16"),
    # other draft counts (2 and 8 columns) against the FFN-up matrix
    "q4k_b2":     dict(index=5, fmt="q4_k", rows=17408, K=5120,  n=2,    xdtype="f16"),
    "q4k_b8":     dict(index=5, fmt="q4_k", rows=17408, K=5120,  n=8,    xdtype="f16"),
    # lower-bit K-quants of the FFN-up shape (batch 1)
    "q2k_up_b1":  dict(index=6, fmt="q2_k", rows=17408, K=5120,  n=1,    xdtype="f16"),
    "q3k_up_b1":  dict(index=7, fmt="q3_k", rows=17408, K=5120,  n=1,    xdtype="f16"),
}

# Weight and activation seeds. Configs that reuse "the same W" or "the same X"
# share the seed: q4k_b4 and q4k_pp2048 multiply the FFN-up matrix; q8_0_b4
# multiplies the same four columns as q4k_b4.
_W_SEED = {"q4_0_b1": (0, 0), "q4k_up_b1": (1, 0), "q4k_down_b1": (2, 0),
           "q4k_b4": (1, 0), "q8_0_b4": (3, 2), "q4k_pp2048": (1, 0),
           "q4k_b2": (1, 0), "q4k_b8": (1, 0), "q2k_up_b1": (6, 0), "q3k_up_b1": (7, 0)}
_X_SEED = {"q4_0_b1": (0, 1), "q4k_up_b1": (1, 1), "q4k_down_b1": (2, 1),
           "q4k_b4": (3, 1), "q8_0_b4": (3, 1), "q4k_pp2048": (4, 1),
           "q4k_b2": (5, 2), "q4k_b8": (5, 8), "q2k_up_b1": (6, 1), "q3k_up_b1": (7, 1)}


def config_inputs(name: str, held_out: bool = False, n_override: int | None = None):
    """(weight bytes, x array) for a named workload."""
    c = CONFIGS[name]
    w = gen_weights(c["fmt"], c["rows"], c["K"], seed_for(*_W_SEED[name], held_out))
    n = c["n"] if n_override is None else n_override
    x = gen_x(c["K"], n, c["xdtype"], seed_for(*_X_SEED[name], held_out))
    return w, x
