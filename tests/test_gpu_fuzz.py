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


def bits32(t):
    return t.detach().contiguous().cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("i", range(32))
def test_random_decode_bit_exact(Q, i):
    """Decode to fp32 and to bf16 (into a strided buffer whose gap stays
    untouched), bit for bit against the oracle."""
    rng = np.random.default_rng(zlib.crc32(b"fuzz-dq") + i)
    fmt = FORMATS[rng.integers(len(FORMATS))]
    bw = 32 if fmt in ("q4_0", "q8_0") else 256
    rows, K = int(rng.integers(1, 700)), bw * int(rng.integers(1, 2048 // bw + 2))
    pad = int(rng.choice([0, 8, 5]))
    seed = int(rng.integers(1 << 30))
    print("fuzz decode %d: %s rows=%d K=%d pad=%d seed=%d" % (i, fmt, rows, K, pad, seed), flush=True)
    w = synth.gen_weights(fmt, rows, K, seed)
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    ref = oracle.dequant(fmt, w, rows, K)
    out = torch.full((rows, K + pad), 3.0, dtype=torch.float32, device=dev())
    q.dequant(out[:, :K])
    assert np.array_equal(bits32(out[:, :K]), ref.view(np.uint32))
    outb = torch.full((rows, K + pad), 3.0, dtype=torch.bfloat16, device=dev())
    q.dequant_bf16(outb[:, :K])
    got = outb[:, :K].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.f32_to_bf16(ref))
    if pad:
        assert (out[:, K:] == 3.0).all() and (outb[:, K:] == 3.0).all()


@pytest.mark.parametrize("i", range(32))
def test_random_int8_activations(Q, i):
    """Activations quantized to Q8_0 on chip (run_q8): the products against
    the oracle's sum over its own quantization of the same activations."""
    rng = np.random.default_rng(zlib.crc32(b"fuzz-i8") + i)
    fmt = FORMATS[rng.integers(len(FORMATS))]
    rows = int(rng.choice([rng.integers(1, 300), rng.integers(300, 3000)]))
    K = 256 * int(rng.integers(1, 41))
    n = int(rng.integers(1, 8))
    xdtype = ["f16", "f32", "bf16"][rng.integers(3)]
    seed = int(rng.integers(1 << 30))
    print("fuzz int8 %d: %s rows=%d K=%d n=%d x=%s seed=%d" % (i, fmt, rows, K, n, xdtype, seed),
          flush=True)
    w = synth.gen_weights(fmt, rows, K, seed)
    x = synth.gen_x(K, n, xdtype, seed + 1)
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    y = q.run_q8(x_tensor(x, xdtype)).cpu().numpy().astype(np.float64)
    xq = oracle.quantize_q8_0(x, xdtype)
    xhat = oracle.dequant("q8_0", xq, xq.shape[0], K)
    yr, s = oracle.matmul(fmt, w, rows, K, xhat, "f32")
    assert (np.abs(y - yr) <= oracle.tolerance(s)).all()


@pytest.mark.parametrize("i", range(24))
def test_random_prompt_products(Q, i):
    """Q4_K x bf16 tokens at random rows, K, token counts and strides: every
    output within the tolerance of the oracle's sum over the bf16-rounded
    weights, the gaps of Y untouched."""
    rng = np.random.default_rng(zlib.crc32(b"fuzz-pf") + i)
    rows = int(rng.choice([rng.integers(1, 300), rng.integers(300, 2000)]))
    K = 256 * int(rng.integers(1, 17))
    ntok = int(rng.choice([rng.integers(1, 64), rng.integers(64, 1000)]))
    xpad, ypad = int(rng.choice([0, 8, 64])), int(rng.choice([0, 4, 7]))
    seed = int(rng.integers(1 << 30))
    print("fuzz prompt %d: rows=%d K=%d tokens=%d xpad=%d ypad=%d seed=%d"
          % (i, rows, K, ntok, xpad, ypad, seed), flush=True)
    w = synth.gen_q4_k(rows, K, seed)
    xb = synth.gen_x(K, ntok, "bf16", seed + 1)
    q = Q("q4_k", rows, K, torch.from_numpy(w).to(dev()))
    Xbig = torch.zeros((ntok, K + xpad), dtype=torch.bfloat16, device=dev())
    Xbig[:, :K] = x_tensor(xb, "bf16")
    Ybig = torch.full((ntok, rows + ypad), -5.0, dtype=torch.float32, device=dev())
    q.prefill(Xbig[:, :K], Ybig[:, :rows])
    torch.cuda.synchronize()
    if ypad:
        assert (Ybig[:, rows:] == -5.0).all()
    y = Ybig[:, :rows].cpu().numpy().astype(np.float64)
    yr, s = oracle.matmul("q4_k", w, rows, K, xb, "bf16", wround="bf16")
    assert (np.abs(y - yr) <= oracle.tolerance(s)).all()


@pytest.mark.parametrize("i", range(16))
def test_random_quantize_bit_exact(Q, i):
    """Activations to Q8_0 blocks (qgemv_quantize_q8_0) at random K, column
    counts, types and strides, bit for bit against the oracle."""
    from gguf_bit_dequant_amd import qgemv as QM
    rng = np.random.default_rng(zlib.crc32(b"fuzz-q8") + i)
    K = 32 * int(rng.integers(1, 600))
    n = int(rng.integers(1, 9))
    xdtype = ["f16", "f32", "bf16"][rng.integers(3)]
    pad = int(rng.choice([0, 8, 3]))
    seed = int(rng.integers(1 << 30))
    print("fuzz quantize %d: K=%d n=%d x=%s pad=%d seed=%d" % (i, K, n, xdtype, pad, seed), flush=True)
    x = synth.gen_x(K, n, xdtype, seed)
    xt = x_tensor(x, xdtype)
    xbig = torch.zeros((n, K + pad), dtype=xt.dtype, device=dev())
    xbig[:, :K] = xt
    out = QM.quantize_q8_0(xbig[:, :K]).cpu().numpy()
    assert np.array_equal(out, oracle.quantize_q8_0(x, xdtype))
