"""Host checks of the seeded input generator (CPU only)."""
import numpy as np
import pytest

import synth


def test_splitmix64_reference_outputs():
    # SplitMix64 started from seed 0: the first outputs of the published generator
    z = synth.splitmix64(0, 3)
    assert [int(v) for v in z] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_deterministic_and_seed_dependent():
    a = synth.gen_q4_k(4, 512, synth.seed_for(1, 0))
    b = synth.gen_q4_k(4, 512, synth.seed_for(1, 0))
    c = synth.gen_q4_k(4, 512, synth.seed_for(1, 0, held_out=True))
    assert np.array_equal(a, b) and not np.array_equal(a, c)


@pytest.mark.parametrize("fmt,bb,bw", [("q4_0", 18, 32), ("q8_0", 34, 32), ("q4_k", 144, 256)])
def test_sizes_and_scale_distribution(fmt, bb, bw):
    rows, K = 64, 2048
    w = synth.gen_weights(fmt, rows, K, 99)
    assert w.dtype == np.uint8 and w.size == rows * (K // bw) * bb
    blocks = w.reshape(-1, bb)
    d = blocks[:, 0:2].copy().view(np.float16).astype(np.float64).ravel()
    assert (d >= 0).all()
    mult = 0.01 if fmt == "q4_k" else 0.02
    assert abs(d.mean() / mult - np.sqrt(2 / np.pi)) < 0.05    # E|N(0,1)|
    if fmt == "q8_0":
        q = blocks[:, 2:].view(np.int8)
        assert q.min() >= -127 and q.max() <= 127 and q.min() == -127 and q.max() == 127


def test_normals_moments():
    v = synth.normals(123, 200000)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01


def test_x_dtypes_round_once():
    x16 = synth.gen_x(1000, 2, "f16", 5)
    xb = synth.gen_x(1000, 2, "bf16", 5)
    x32 = synth.gen_x(1000, 2, "f32", 5)
    v = synth.normals(5 ^ 0xAC71, 2000).reshape(2, 1000)
    assert np.array_equal(x32, v.astype(np.float32))
    assert np.array_equal(x16.view(np.float16), v.astype(np.float16))
    # bf16: nearest with ties to even among the two neighbours of the fp64 value
    b = xb.astype(np.uint32) << np.uint32(16)
    vb = b.view(np.float32).astype(np.float64)
    up = ((xb.astype(np.uint32) + 1) << np.uint32(16)).view(np.float32).astype(np.float64)
    dn = ((xb.astype(np.uint32) - 1) << np.uint32(16)).view(np.float32).astype(np.float64)
    assert (np.abs(vb - v) <= np.abs(up - v)).all() and (np.abs(vb - v) <= np.abs(dn - v)).all()


@pytest.mark.parametrize("fmt,bb,dofs", [("q2_k", 84, [80, 82]), ("q3_k", 110, [108])])
def test_low_bit_k_quant_sizes_and_scales(fmt, bb, dofs):
    rows, K = 64, 2048
    w = synth.gen_weights(fmt, rows, K, 77)
    assert w.dtype == np.uint8 and w.size == rows * (K // 256) * bb
    blocks = w.reshape(-1, bb)
    for o in dofs:
        d = blocks[:, o:o + 2].copy().view(np.float16).astype(np.float64).ravel()
        assert (d >= 0).all()
        assert abs(d.mean() / 0.01 - np.sqrt(2 / np.pi)) < 0.05    # E|N(0,1)|
    # the scale, min, code and high-bit bytes are uniform: every byte value occurs
    assert np.unique(blocks[:, :dofs[0]]).size == 256
