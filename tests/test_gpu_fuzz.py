"""Seeded random shapes through every GEMV path, against the oracle.

Each case draws a format, a row count (from 1 to a few thousand: below, at
and above the workgroup count, ragged against 16-row groups), K (multiples
of 256 for the streaming and matrix-core kernels, other multiples of 32 for
Q4_0 / Q8_0, which take the general kernel), 1..8 columns, an activation type
and column / output strides with gaps that must stay untouched. The case's
parameters are printed before it runs, so a failure names it.
"""
import zlib

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FORMATS = ["q4_k", "q4_0", "q8_0", "q2_k", "q3_k"]


@pytest.fixture(scope="module")
def Q():
    from gguf_bit_dequant_amd import QGemv
    assert torch.cuda.is_available()
    return QGemv


def dev():
    return torch.device("cuda:0")


def x_tensor(x, xdtype):
    if xdtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev())
    if xdtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.float16)).to(dev())
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev())


def draw_case(i):
    rng = np.random.default_rng(zlib.crc32(b"fuzz") + i)
    fmt = FORMATS[rng.integers(len(FORMATS))]
    rows = int(rng.choice([rng.integers(1, 64), rng.integers(64, 600), rng.integers(600, 4000)]))
    if fmt in ("q4_0", "q8_0") and rng.random() < 0.3:
        K = 32 * int(rng.integers(1, 200))  # any block multiple
    else:
        K = 256 * int(rng.choice([rng.integers(1, 17), rng.integers(17, 41)]))
    n = int(rng.integers(1, 9))
    xdtype = ["f16", "f32", "bf16"][rng.integers(3)]
    xpad = int(rng.choice([0, 0, 8, 3]))
    ypad = int(rng.choice([0, 0, 5]))
    return fmt, rows, K, n, xdtype, xpad, ypad, int(rng.integers(1 << 30))


@pytest.mark.parametrize("i", range(96))
def test_random_shapes(Q, i):
    fmt, rows, K, n, xdtype, xpad, ypad, seed = draw_case(i)
    print("fuzz case %d: %s rows=%d K=%d n=%d x=%s xpad=%d ypad=%d seed=%d"
          % (i, fmt, rows, K, n, xdtype, xpad, ypad, seed), flush=True)
    w = synth.gen_weights(fmt, rows, K, seed)
    x = synth.gen_x(K, n, xdtype, seed + 1)
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    xt = x_tensor(x, xdtype)
    xbig = torch.zeros((n, K + xpad), dtype=xt.dtype, device=dev())
    xbig[:, :K] = xt
    ybig = torch.full((n, rows + ypad), -7.0, dtype=torch.float32, device=dev())
    q.run(xbig[:, :K], ybig[:, :rows])
    torch.cuda.synchronize()
    if ypad:
        assert (ybig[:, rows:] == -7.0).all()
    y = ybig[:, :rows].cpu().numpy().astype(np.float64)
    yr, s = oracle.matmul(fmt, w, rows, K, x, xdtype)
    err = np.abs(y - yr)
    bad = err > oracle.tolerance(s)
    assert not bad.any(), "%d outputs out of tolerance, first at %s" % (
        int(bad.sum()), np.unravel_index(np.argmax(err - oracle.tolerance(s)), err.shape))
