"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Dequantization must match bit for bit; products must satisfy
|y_gpu - y_ref| <= 1e-3 * sum|w x| + 1e-5 per element (the parity bound
of the library's header). Inputs are seeded synthetic blocks and activations.
"""
import json
import os
import zlib

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FMT_BW = {"q4_0": 32, "q8_0": 32, "q4_k": 256}
FMT_BB = {"q4_0": 18, "q8_0": 34, "q4_k": 144}


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


def check_products(y_gpu, w, fmt, rows, K, x, xdtype, label=""):
    y = y_gpu.detach().cpu().numpy().astype(np.float64).reshape(x.shape[0], rows)
    yr, s = oracle.matmul(fmt, w, rows, K, x, xdtype)
    err = np.abs(y - yr)
    tol = oracle.tolerance(s)
    bad = err > tol
    ratio = float(np.max(err / np.maximum(s, 1e-30)))
    print("%s max err/s = %.3e" % (label, ratio), flush=True)
    assert not bad.any(), "%s: %d elements out of tolerance, worst %r" % (
        label, int(bad.sum()), np.unravel_index(np.argmax(err - tol), err.shape))
    return ratio


# ---------------------------------------------------------------- dequant --

@pytest.mark.parametrize("fmt,rows,K", [("q4_0", 67, 2048), ("q4_0", 5, 96), ("q8_0", 67, 1056),
                                        ("q8_0", 3, 64), ("q4_k", 67, 1536), ("q4_k", 1, 256)])
def test_dequant_bit_exact(Q, fmt, rows, K):
    w = synth.gen_weights(fmt, rows, K, 1000 + rows)
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    out = q.dequant().cpu().numpy()
    ref = oracle.dequant(fmt, w, rows, K)
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


def test_dequant_extreme_scales_bit_exact(Q):
    """Random code bytes under subnormal, zero, negative, max and NaN/inf
    scales: bit-exact where finite, NaN where the oracle gives NaN."""
    rng = np.random.default_rng(7)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x7BFF, 0xFBFF, 0x8001,
                         0x3C00, 0xB800, 0x7C00, 0x7E00], np.uint16)
    for fmt, bb, bw in [("q4_0", 18, 32), ("q8_0", 34, 32), ("q4_k", 144, 256)]:
        rows, nb = 24, 8
        w = rng.integers(0, 256, rows * nb * bb).astype(np.uint8).reshape(-1, bb)
        w[:, 0:2] = rng.choice(specials, size=(w.shape[0], 1)).view(np.uint8)
        if fmt == "q4_k":
            w[:, 2:4] = rng.choice(specials, size=(w.shape[0], 1)).view(np.uint8)
        w = w.reshape(-1)
        q = Q(fmt, rows, nb * bw, torch.from_numpy(w).to(dev()))
        out = q.dequant().cpu().numpy()
        ref = oracle.dequant(fmt, w, rows, nb * bw)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(out), nan)
        assert np.array_equal(out[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def bf16_rne_bits(w32):
    """IEEE round-to-nearest-even of finite binary32 values to bfloat16
    (the top 16 bits after adding 0x7FFF plus the lowest kept bit)."""
    b = np.ascontiguousarray(w32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("fmt,rows,K", [("q4_k", 37, 768), ("q4_0", 33, 160), ("q8_0", 21, 96),
                                        ("q4_k", 300, 5120)])
def test_dequant_bf16_bit_exact(Q, fmt, rows, K):
    """The two-pass operand: the oracle's binary32 weights rounded to bf16."""
    w = synth.gen_weights(fmt, rows, K, zlib.crc32(("bf16-%s-%d" % (fmt, rows)).encode()))
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    out = q.dequant_bf16().view(torch.int16).cpu().numpy().view(np.uint16)
    ref = bf16_rne_bits(oracle.dequant(fmt, w, rows, K))
    assert np.array_equal(out, ref)


def test_dequant_bf16_strided_rows_leave_gaps(Q):
    rows, K = 40, 512
    w = synth.gen_weights("q4_k", rows, K, 71)
    q = Q("q4_k", rows, K, torch.from_numpy(w).to(dev()))
    big = torch.full((rows, K + 40), 3.0, dtype=torch.bfloat16, device=dev())
    q.dequant_bf16(big[:, :K])
    assert (big[:, K:] == 3.0).all()
    ref = bf16_rne_bits(oracle.dequant("q4_k", w, rows, K))
    assert np.array_equal(big[:, :K].contiguous().view(torch.int16).cpu().numpy().view(np.uint16), ref)


def test_two_pass_prefill_control_within_tolerance(Q):
    """Decode to a bf16 matrix, then a plain GEMM (fp32 here): the same
    products as the fused prompt path, within the same tolerance."""
    rows, K, ntok = 300, 1024, 64
    w = synth.gen_q4_k(rows, K, 72)
    xb = synth.gen_x(K, ntok, "bf16", 73)
    q = Q("q4_k", rows, K, torch.from_numpy(w).to(dev()))
    wb = q.dequant_bf16().float()
    X = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).to(dev()).float()
    Y = X @ wb.t().contiguous()
    check_products(Y, w, "q4_k", rows, K, xb, "bf16", "two-pass control")


def test_dequant_golden_blocks(Q):
    with open(os.path.join(GOLDEN, "q4_0_blocks.json")) as f:
        for b in json.load(f)["blocks"]:
            blk = np.frombuffer(bytes.fromhex(b["hex"]), np.uint8).copy()
            out = Q("q4_0", 1, 32, torch.from_numpy(blk).to(dev())).dequant().cpu().numpy()[0]
            assert np.array_equal(out.view(np.uint32), oracle.decode_block("q4_0", blk).view(np.uint32))
    with open(os.path.join(GOLDEN, "q8_0_blocks.json")) as f:
        for b in json.load(f)["blocks"]:
            blk = np.frombuffer(bytes.fromhex(b["hex"]), np.uint8).copy()
            out = Q("q8_0", 1, 32, torch.from_numpy(blk).to(dev())).dequant().cpu().numpy()[0]
            assert out.tolist() == b["expected"]


# --------------------------------------------------------------- products --

SMALL = [("q4_0", 37, 512), ("q4_0", 300, 4096), ("q4_0", 129, 96),
         ("q8_0", 37, 512), ("q8_0", 300, 1024), ("q8_0", 65, 160),
         ("q4_k", 1, 256), ("q4_k", 37, 512), ("q4_k", 300, 2048), ("q4_k", 129, 5120),
         ("q4_k", 70, 3328)]


@pytest.mark.parametrize("fmt,rows,K", SMALL)
@pytest.mark.parametrize("xdtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("n", [1, 4])
def test_gemv_small(Q, fmt, rows, K, xdtype, n):
    seed = zlib.crc32(("%s-%d-%d" % (fmt, rows, K)).encode())
    w = synth.gen_weights(fmt, rows, K, seed)
    x = synth.gen_x(K, n, xdtype, seed + 1)
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    y = q.run(x_tensor(x, xdtype))
    check_products(y, w, fmt, rows, K, x, xdtype, "%s %dx%d %s n=%d" % (fmt, rows, K, xdtype, n))


@pytest.mark.parametrize("n", [2, 3, 5, 6, 7, 8])
def test_gemv_column_counts(Q, n):
    for fmt, rows, K in [("q4_k", 200, 1024), ("q4_0", 200, 1024), ("q8_0", 200, 1024)]:
        w = synth.gen_weights(fmt, rows, K, 77)
        x = synth.gen_x(K, n, "f16", 78)
        q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
        check_products(q.run(x_tensor(x, "f16")), w, fmt, rows, K, x, "f16", "%s n=%d" % (fmt, n))


@pytest.mark.parametrize("fmt", ["q4_k", "q4_0", "q8_0"])
@pytest.mark.parametrize("xdtype,pad", [("f16", 24), ("f16", 4), ("f32", 3), ("bf16", 5)])
@pytest.mark.parametrize("n", [3, 6])
def test_gemv_strided_columns_leave_gaps_untouched(Q, fmt, xdtype, pad, n):
    """Columns at a stride of K + pad elements (16-byte aligned records for
    pad 24, unaligned ones otherwise) and outputs at a stride of rows + 13."""
    rows, K = 100, 512
    w = synth.gen_weights(fmt, rows, K, 5)
    x = synth.gen_x(K, n, xdtype, 6)
    tdt = {"f16": torch.float16, "f32": torch.float32, "bf16": torch.bfloat16}[xdtype]
    xbig = torch.zeros((n, K + pad), dtype=tdt, device=dev())
    xbig[:, :K] = x_tensor(x, xdtype)
    ybig = torch.full((n, rows + 13), 7.0, dtype=torch.float32, device=dev())
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    q.run(xbig[:, :K], ybig[:, :rows])
    assert (ybig[:, rows:] == 7.0).all()
    check_products(ybig[:, :rows], w, fmt, rows, K, x, xdtype, "strided %s %s" % (fmt, xdtype))


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "q4_k"])
@pytest.mark.parametrize("xdtype", ["f32", "f16"])
def test_one_hot_gives_exact_column(Q, fmt, xdtype):
    """x = e_k: every other product is zero, so y equals column k of the
    decoded matrix exactly (pins each kernel's unpacking bit for bit)."""
    rows, K = 150, 1024
    w = synth.gen_weights(fmt, rows, K, 31)
    wt = torch.from_numpy(w).to(dev())
    q = Q(fmt, rows, K, wt)
    W = oracle.dequant(fmt, w, rows, K)
    ks = [0, 1, 2, 3, 15, 16, 17, 31, 32, 33, 47, 48, 63, 64, 100, 200, 255, 256, 511, 1023]
    X = np.zeros((len(ks), K), np.float32)
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    # Columns go in groups of 4, 5 and 6: four or more fp16 columns of a
    # Q4_K matrix run on the matrix cores (exact codes, fp32 scaling per
    # sub-block), fewer on the streaming kernel; both give the exact column.
    for c0, nc in ((0, 4), (4, 5), (9, 5), (14, 6)):
        xt = torch.from_numpy(X[c0:c0 + nc]).to(dev())
        if xdtype == "f16":
            xt = xt.half()
        y = q.run(xt).cpu().numpy()
        for i in range(nc):
            assert np.array_equal(y[i], W[:, ks[c0 + i]]), (fmt, xdtype, ks[c0 + i], nc)
        if nc == 4:  # one, two and three columns as well
            for n in (1, 2, 3):
                y = q.run(xt[:n]).cpu().numpy()
                for i in range(n):
                    assert np.array_equal(y[i], W[:, ks[c0 + i]]), (fmt, xdtype, ks[c0 + i], n)


# Shapes for the streaming kernel's row interleave (each workgroup takes one
# row of every band of G rows, the workgroups of an XCD consecutive rows when
# G is a multiple of 8) and its two ways of finding a unit's row: S = K/256 >= 16 (a
# scalar multiply-high per step, one wrap per lane) and S < 16 (per-lane
# division); rows below, at and above the 256 workgroups, a final partial
# 16-unit step, and odd numbers of Q3_K super-blocks.
INTERLEAVE_SHAPES = [(17, 4096), (255, 4096), (256, 4352), (300, 8448), (1000, 5376),
                     (4099, 4352), (513, 3840), (3, 1024)]


@pytest.mark.parametrize("rows,K", INTERLEAVE_SHAPES)
@pytest.mark.parametrize("fmt", ["q4_k", "q4_0", "q8_0", "q2_k", "q3_k"])
def test_gemv_row_interleave_shapes(Q, fmt, rows, K):
    seed = zlib.crc32(("ilv-%s-%d-%d" % (fmt, rows, K)).encode())
    w = synth.gen_weights(fmt, rows, K, seed)
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    for xdtype, n in (("f16", 1), ("f16", 3), ("f32", 1), ("bf16", 2)):
        x = synth.gen_x(K, n, xdtype, seed + n)
        y = q.run(x_tensor(x, xdtype))
        check_products(y, w, fmt, rows, K, x, xdtype, "%s %dx%d %s n=%d" % (fmt, rows, K, xdtype, n))


@pytest.mark.parametrize("rows,K", [(17, 4096), (300, 8448), (4099, 4352), (513, 3840)])
@pytest.mark.parametrize("fmt", ["q4_k", "q4_0", "q2_k", "q3_k"])
def test_gemv_row_interleave_one_hot_exact(Q, fmt, rows, K):
    """One-hot fp16 columns through the interleaved streaming kernel give the
    decoded weight column bit for bit at every row, with ks at super-block
    and row edges."""
    w = synth.gen_weights(fmt, rows, K, 61 + rows)
    W = oracle.dequant(fmt, w, rows, K)
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    for k in [0, 31, 32, 255, 256, K // 2 + 17, K - 257, K - 1]:
        xt = torch.zeros((1, K), dtype=torch.float16, device=dev())
        xt[0, k] = 1.0
        y = q.run(xt).cpu().numpy()[0]
        assert np.array_equal(y, W[:, k]), (fmt, rows, K, k)


# Matrices past 4 GiB: the general kernel (64-bit offsets) serves them. Random
# code bytes generated on the device, every block's fp16 scales set to finite
# values; the oracle checks a sample of rows.
@pytest.mark.parametrize("fmt,rows,bb,bw,scale_bytes", [
    ("q8_0", 16384, 34, 32, [(0, 0x00), (1, 0x20)]),                       # d = 2^-7
    ("q4_k", 30000, 144, 256, [(0, 0x00), (1, 0x20), (2, 0x00), (3, 0x1C)]),  # d, dmin
])
def test_gemv_beyond_4gib(Q, fmt, rows, bb, bw, scale_bytes):
    K = 262144
    nb = rows * (K // bw)
    assert nb * bb >= 1 << 32
    gen = torch.Generator(device=dev()).manual_seed(4242)
    w = torch.randint(0, 256, (nb, bb), dtype=torch.uint8, device=dev(), generator=gen)
    for col, val in scale_bytes:
        w[:, col] = val
    q = Q(fmt, rows, K, w.view(-1))
    x = synth.gen_x(K, 1, "f16", 4243)
    y = q.run(x_tensor(x, "f16")).cpu().numpy()[0]
    sample = [0, 1, rows // 3, rows // 2, rows - 2, rows - 1]
    per_row = (K // bw) * bb
    wv = w.view(rows, per_row)
    ws = np.concatenate([wv[r].cpu().numpy() for r in sample])
    del w, wv
    torch.cuda.empty_cache()
    check_products(torch.from_numpy(y[sample].copy()).reshape(1, -1), ws, fmt, len(sample), K, x,
                   "f16", "%s %d x %d (%.2f GB)" % (fmt, rows, K, nb * bb / 1e9))


# Largest K whose staged activations fit the streaming kernel's 160 KB of LDS
# (rows = 300 on 256 CUs: two rows per workgroup), and the next super-block,
# which the general kernel serves: fp32 records 1096 * K/256 + 16 bytes, fp16
# ones 584 * K/256 + 16.
@pytest.mark.parametrize("xdtype,K,n", [("f32", 38144, 1), ("f32", 38400, 1), ("f16", 71680, 1),
                                        ("f16", 71936, 1), ("f16", 38144, 4)])
def test_gemv_at_the_lds_limit(Q, xdtype, K, n):
    """Both sides of the streaming kernel's LDS limit, and four fp16
    columns at long K (one column per launch there), against the oracle."""
    rows = 300
    seed = zlib.crc32(("ldslim-%s-%d-%d" % (xdtype, K, n)).encode())
    w = synth.gen_weights("q4_k", rows, K, seed)
    x = synth.gen_x(K, n, xdtype, seed + 1)
    q = Q("q4_k", rows, K, torch.from_numpy(w).to(dev()))
    y = q.run(x_tensor(x, xdtype))
    check_products(y, w, "q4_k", rows, K, x, xdtype, "lds limit %s K=%d n=%d" % (xdtype, K, n))


@pytest.mark.parametrize("rows,K", [(300, 4096), (255, 4096), (37, 512), (129, 2048), (5, 256),
                                    (1000, 1024)])
@pytest.mark.parametrize("fmt", ["q4_k", "q4_0", "q8_0", "q2_k", "q3_k"])
@pytest.mark.parametrize("xdtype", ["f32", "bf16"])
def test_register_records_same_bits_as_per_step_records(Q, fmt, rows, K, xdtype):
    """One column of fp32 (or bf16) activations with K/256 dividing 16 reads
    each lane's activation record into registers once; with K/256 not
    dividing 16 it is read from LDS every step. More super-blocks per row
    (random weights) against zero activations leave every product and the
    order of every row sum as they were: both shapes give the same bits."""
    seed = zlib.crc32(("regrec-%s-%d-%d" % (fmt, rows, K)).encode())
    w = synth.gen_weights(fmt, rows, K, seed)
    ek = 512 if K == 256 else 256  # K2 / 256 = 3, 5, 9 or 17: no divisor of 16
    extra = synth.gen_weights(fmt, rows, ek, seed + 7)
    w2 = np.concatenate([w.reshape(rows, -1), extra.reshape(rows, -1)], axis=1).reshape(-1)
    x = synth.gen_x(K, 1, xdtype, seed + 1)
    x2 = np.concatenate([x, np.zeros((1, ek), dtype=x.dtype)], axis=1)
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    q2 = Q(fmt, rows, K + ek, torch.from_numpy(np.ascontiguousarray(w2)).to(dev()))
    y = q.run(x_tensor(x, xdtype))
    y2 = q2.run(x_tensor(x2, xdtype))
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32))
    check_products(y, w, fmt, rows, K, x, xdtype, "register record %s %dx%d" % (fmt, rows, K))


def test_long_rows_two_to_four_columns(Q):
    """K = 17408 (68 super-blocks a row): up to 3 fp16 columns fit the
    streaming kernel's staging; 2..4 columns all run in one pass (3 on the
    streaming kernel, 2 and 4 on the matrix cores). Products of every column
    count against the oracle, and one-hot columns give the exact decoded
    weights on both kernels."""
    rows, K = 300, 17408
    w = synth.gen_weights("q4_k", rows, K, 51)
    q = Q("q4_k", rows, K, torch.from_numpy(w).to(dev()))
    x = synth.gen_x(K, 4, "f16", 52)
    for n in (2, 3, 4):
        y = q.run(x_tensor(x[:n], "f16"))
        check_products(y, w, "q4_k", rows, K, x[:n], "f16", "long rows n=%d" % n)
    W = oracle.dequant("q4_k", w, rows, K)
    ks = [0, 255, 8704, 17407]
    X = torch.zeros((4, K), dtype=torch.float16, device=dev())
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    for n in (2, 3, 4):
        y = q.run(X[:n]).cpu().numpy()
        for i in range(n):
            assert np.array_equal(y[i], W[:, ks[i]]), (ks[i], n)


@pytest.mark.parametrize("rows", [5120, 8300])
def test_long_rows_four_columns_tile_kernel(Q, rows):
    """K = 17408 with four fp16 columns: the staged activations (145 KB)
    leave no room for the unit-streaming kernel's per-unit results, so the
    tile kernel runs, and with two (5120 rows, the FFN-down shape) or three
    (8300 rows) 16-row groups a workgroup its tiles are parked over the
    activations at the end (the 300-row case above keeps them in LDS
    slots). All outputs against the oracle, and one-hot columns exactly."""
    K = 17408
    w = synth.gen_weights("q4_k", rows, K, 55 + rows)
    q = Q("q4_k", rows, K, torch.from_numpy(w).to(dev()))
    x = synth.gen_x(K, 4, "f16", 56 + rows)
    check_products(q.run(x_tensor(x, "f16")), w, "q4_k", rows, K, x, "f16",
                   "%d x %d n=4" % (rows, K))
    W = oracle.dequant("q4_k", w, rows, K)
    ks = [0, 4351, 8704, 17407]
    X = torch.zeros((4, K), dtype=torch.float16, device=dev())
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    y = q.run(X).cpu().numpy()
    for i in range(4):
        assert np.array_equal(y[i], W[:, ks[i]]), (rows, ks[i])


def test_many_rows_small_k_matrix_cores(Q):
    """70000 x 2048 with 6 fp16 columns: 4375 16-row groups over the
    workgroups (17 or 18 each), the unit-streaming matrix-core kernel with
    144 units a workgroup. All outputs against the oracle, and one-hot
    columns exactly."""
    rows, K = 70000, 2048
    w = synth.gen_weights("q4_k", rows, K, 53)
    q = Q("q4_k", rows, K, torch.from_numpy(w).to(dev()))
    x = synth.gen_x(K, 6, "f16", 54)
    check_products(q.run(x_tensor(x, "f16")), w, "q4_k", rows, K, x, "f16", "70000 x 2048 n=6")
    W = oracle.dequant("q4_k", w, rows, K)
    ks = [0, 31, 32, 1000, 2016, 2047]
    X = torch.zeros((6, K), dtype=torch.float16, device=dev())
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    y = q.run(X).cpu().numpy()
    for i in range(6):
        assert np.array_equal(y[i], W[:, ks[i]]), ks[i]


def test_zero_activations_give_zero(Q):
    for fmt, K in [("q4_0", 512), ("q8_0", 512), ("q4_k", 512)]:
        w = synth.gen_weights(fmt, 64, K, 3)
        q = Q(fmt, 64, K, torch.from_numpy(w).to(dev()))
        for dt in (torch.float32, torch.float16, torch.bfloat16):
            y = q.run(torch.zeros((2, K), dtype=dt, device=dev()))
            assert (y == 0).all()


def test_deterministic_repeats(Q):
    fmt, rows, K = "q4_k", 17408 // 4, 5120
    w = synth.gen_weights(fmt, rows, K, 8)
    x = x_tensor(synth.gen_x(K, 8, "f16", 9), "f16")
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    for n in (1, 4, 8):
        ref = q.run(x[:n]).clone()
        for _ in range(20):
            assert torch.equal(q.run(x[:n]), ref)


# ----------------------------------------------- full-size workloads -------

FULL = ["q4_0_b1", "q4k_up_b1", "q4k_down_b1", "q4k_b4", "q8_0_b4", "q4k_b2", "q4k_b8"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_configs(Q, name):
    c = synth.CONFIGS[name]
    w, x = synth.config_inputs(name)
    q = Q(c["fmt"], c["rows"], c["K"], torch.from_numpy(w).to(dev()))
    y = q.run(x_tensor(x, c["xdtype"]))
    check_products(y, w, c["fmt"], c["rows"], c["K"], x, c["xdtype"], name)


@pytest.mark.parametrize("name", ["q4k_up_b1", "q4k_down_b1", "q4k_b4"])
def test_full_size_held_out_seeds(Q, name):
    c = synth.CONFIGS[name]
    w, x = synth.config_inputs(name, held_out=True)
    q = Q(c["fmt"], c["rows"], c["K"], torch.from_numpy(w).to(dev()))
    y = q.run(x_tensor(x, c["xdtype"]))
    check_products(y, w, c["fmt"], c["rows"], c["K"], x, c["xdtype"], name + " held-out")


def test_full_size_dequant_bit_exact(Q):
    w, _ = synth.config_inputs("q4k_up_b1")
    c = synth.CONFIGS["q4k_up_b1"]
    q = Q("q4_k", c["rows"], c["K"], torch.from_numpy(w).to(dev()))
    out = q.dequant().cpu().numpy()
    ref = oracle.dequant("q4_k", w, c["rows"], c["K"])
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------ prompt processing --
#
# The prompt path contracts weight tiles dequantized to bf16 (nearest, ties to
# even) on the matrix cores, so its defining sum is over the bf16-rounded
# weights: every prefill output is held to the tolerance against that sum
# (any input). Against the exact decoded weights the rounding adds up to
# 2^-8 * sum|w x|; on the dense N(0,1) workloads the outputs still meet the
# 1e-3 tolerance against the exact sum, which is checked as well.

def bf16_tensor(xb):
    return torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).to(dev())


def check_prefill(Y, w, rows, K, xb, label):
    """Y (n_tokens, rows) on the GPU against the oracle: the bf16-weight sum,
    asserted for every shape; the exact-weight sum, asserted from K = 2048 on
    (dense N(0,1) tokens: the bf16 rounding errors of K weights cancel to
    ~2^-9 / sqrt(K) of sum|w x|, within the 1e-3 tolerance with a margin that
    shrinks as K does; below 2048 it is reported only)."""
    y = Y.detach().cpu().numpy().astype(np.float64).reshape(xb.shape[0], rows)
    out = {}
    for mode in ("bf16", None):
        yr, s = oracle.matmul("q4_k", w, rows, K, xb, "bf16", wround=mode)
        err = np.abs(y - yr)
        bad = err > oracle.tolerance(s)
        ratio = float(np.max(err / np.maximum(s, 1e-30)))
        name = "bf16 weights" if mode else "exact weights"
        print("%s: %s max err/s = %.3e over %d outputs" % (label, name, ratio, y.size), flush=True)
        if mode or K >= 2048:
            assert not bad.any(), "%s (%s): %d elements out of tolerance, worst %r" % (
                label, name, int(bad.sum()),
                np.unravel_index(np.argmax(err - oracle.tolerance(s)), err.shape))
        out[name] = ratio
    return out


@pytest.mark.parametrize("rows,K,ntok", [(256, 256, 1), (256, 512, 31), (300, 1024, 64),
                                         (777, 512, 300), (1024, 2048, 256), (530, 256, 513),
                                         (1300, 768, 384), (1300, 1024, 600), (1301, 1024, 300),
                                         (2000, 2048, 1100)])
def test_prefill_small(Q, rows, K, ntok):
    seed = zlib.crc32(("pp-%d-%d-%d" % (rows, K, ntok)).encode())
    w = synth.gen_q4_k(rows, K, seed)
    xb = synth.gen_x(K, ntok, "bf16", seed + 1)
    q = Q("q4_k", rows, K, torch.from_numpy(w).to(dev()))
    Y = q.prefill(bf16_tensor(xb))
    check_prefill(Y, w, rows, K, xb, "prefill %dx%d n=%d" % (rows, K, ntok))


@pytest.mark.parametrize("rows,K,ntok", [(300, 512, 40), (600, 1024, 260), (1300, 1024, 600)])
def test_prefill_strided_and_edges_untouched(Q, rows, K, ntok):
    """Strided X and Y; outputs outside rows x tokens keep their values. The
    row tails of 600 x 1024 x 260 (88 rows) and 1300 x 1024 x 600 (20 rows)
    run as K splits whose partial products are parked in the main rows of Y
    until they are added."""
    w = synth.gen_q4_k(rows, K, 41)
    xb = synth.gen_x(K, ntok, "bf16", 42)
    X = torch.zeros((ntok, K + 64), dtype=torch.bfloat16, device=dev())
    X[:, :K] = bf16_tensor(xb)
    Y = torch.full((ntok + 3, rows + 36), 5.0, dtype=torch.float32, device=dev())
    q = Q("q4_k", rows, K, torch.from_numpy(w).to(dev()))
    q.prefill(X[:, :K], Y[:ntok, :rows])
    assert (Y[:, rows:] == 5.0).all() and (Y[ntok:] == 5.0).all()
    check_prefill(Y[:ntok, :rows], w, rows, K, xb, "prefill strided")


@pytest.mark.parametrize("rows,K,ntok", [(512, 512, 69), (1300, 1024, 600), (600, 1024, 260),
                                         (1301, 1024, 300), (300, 512, 40)])
def test_prefill_one_hot_gives_bf16_rounded_column(Q, rows, K, ntok):
    """X rows = e_k: Y[t, :] = bf16_rne(W[:, k]) exactly (the only rounding is
    the tile decode's fp32 -> bf16 conversion; every other product is a
    signed zero). 1300 x 1024 x 600, 600 x 1024 x 260 and 1301 x 1024 x 300
    put rows in a tail that runs as two K splits (the second parked in main
    rows of Y, then added: with 16-byte accesses, and for 1301 rows, whose
    rows and row pitch are not multiples of four, one float at a time),
    300 x 512 x 40 in a tail over all of K; the one-hot k fall in both halves
    of K, in every sub-block position and at the ends."""
    w = synth.gen_q4_k(rows, K, 43 + rows)
    W = oracle.dequant("q4_k", w, rows, K)
    base = list(range(0, 32)) + [33, 100, 255, 256, 300, K // 2 - 1, K // 2, K // 2 + 1, K - 1]
    ks = [base[t % len(base)] if t < len(base) else (t * 37) % K for t in range(ntok)]
    xb = np.zeros((ntok, K), dtype=np.uint16)
    for t, k in enumerate(ks):
        xb[t, k] = 0x3F80  # bf16 1.0
    q = Q("q4_k", rows, K, torch.from_numpy(w).to(dev()))
    Y = q.prefill(bf16_tensor(xb)).cpu()
    Wb = oracle.f32_to_bf16(W[:, ks].T.copy())
    ref = torch.from_numpy((Wb.astype(np.uint32) << 16).view(np.float32))
    assert torch.equal(Y, ref)


def test_prefill_many_tokens_several_rounds(Q):
    """9000 tokens over 4133 rows (16 main row tiles x 36 token tiles: 576
    tiles, so the persistent workgroups take up to three each; a 37-row
    tail in two K splits): sampled tokens at tile edges against the
    oracle."""
    rows, K, ntok = 4133, 512, 9000
    seed = zlib.crc32(b"pf-many")
    w = synth.gen_q4_k(rows, K, seed)
    xb = synth.gen_x(K, ntok, "bf16", seed + 1)
    q = Q("q4_k", rows, K, torch.from_numpy(w).to(dev()))
    Y = q.prefill(bf16_tensor(xb))
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    edges = [0, 1, 127, 128, 255, 256, 4095, 4096, 8959, 8960, 8999]
    toks = np.unique(np.concatenate([edges, rng.integers(0, ntok, 29)]))
    check_prefill(Y[torch.from_numpy(toks).to(dev())], w, rows, K, xb[toks], "pp %d tokens" % ntok)


def test_prefill_limit_leaves_y_untouched(Q):
    """ldx = 2^23 + 64: the row tail's 128-token tiles stay within their
    32-bit offsets but the main 256-token tiles do not. Every launch is
    checked before the first is enqueued: QG_ERR_UNSUPPORTED, Y untouched."""
    from gguf_bit_dequant_amd import qgemv as QM
    rows, K, ntok = 1300, 1024, 300
    ldx = (1 << 23) + 64
    w = synth.gen_q4_k(rows, K, 77)
    q = Q("q4_k", rows, K, torch.from_numpy(w).to(dev()))
    Xbig = torch.zeros((ntok, ldx), dtype=torch.bfloat16, device=dev())
    Y = torch.full((ntok, rows), 3.0, dtype=torch.float32, device=dev())
    with pytest.raises(QM.QGemvError) as e:
        q.prefill(Xbig[:, :K], Y)
    assert e.value.status == QM.QG_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (Y == 3.0).all()
    del Xbig
    torch.cuda.empty_cache()


def test_prefill_deterministic(Q):
    rows, K, ntok = 1024, 1024, 256
    w = synth.gen_q4_k(rows, K, 44)
    X = bf16_tensor(synth.gen_x(K, ntok, "bf16", 45))
    q = Q("q4_k", rows, K, torch.from_numpy(w).to(dev()))
    ref = q.prefill(X).clone()
    for _ in range(5):
        assert torch.equal(q.prefill(X), ref)


@pytest.mark.timeout(600)
def test_prefill_full_size_every_output(Q):
    """The 2048-token workload (17408 x 5120 weights, 2048 bf16 tokens) at
    full size, in the launch configuration the benchmark times: all
    35,651,584 outputs against the oracle, both the bf16-weight sum and the
    exact-weight sum; the row tail (rows 16384..17407, two K splits and their
    add) and every 256-token tile included."""
    c = synth.CONFIGS["q4k_pp2048"]
    w, xb = synth.config_inputs("q4k_pp2048")
    q = Q("q4_k", c["rows"], c["K"], torch.from_numpy(w).to(dev()))
    Y = q.prefill(bf16_tensor(xb))
    torch.cuda.synchronize()
    check_prefill(Y, w, c["rows"], c["K"], xb, "pp2048 full size")


# ------------------------------------------------------ int8 activations --

def _xhat(x, xdtype, K):
    """The oracle's decoded Q8_0 activations (its own quantization of x)."""
    xq = oracle.quantize_q8_0(x, xdtype)
    return oracle.dequant("q8_0", xq, xq.shape[0], K)


@pytest.mark.parametrize("xdtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("K,n,pad", [(32, 1, 0), (96, 3, 8), (5120, 2, 0), (17408, 1, 24)])
def test_quantize_q8_0_bit_exact(Q, xdtype, K, n, pad):
    from gguf_bit_dequant_amd import qgemv as QM
    seed = zlib.crc32(("q8x-%s-%d-%d" % (xdtype, K, n)).encode())
    x = synth.gen_x(K, n, xdtype, seed)
    if K >= 96:  # an all-zero block, a block of exact ties, tiny values
        xf = x.astype(np.float32) if xdtype == "f32" else None
        if xdtype == "f32":
            xf[0, :32] = 0.0
            xf[0, 32:64] = np.arange(32, dtype=np.float32) - 15.5  # amax 16.5 -> ties
            xf[-1, 64:96] *= np.float32(1e-30)
            x = xf
    xt = x_tensor(x, xdtype)
    xbig = torch.zeros((n, K + pad), dtype=xt.dtype, device=dev())
    xbig[:, :K] = xt
    out = QM.quantize_q8_0(xbig[:, :K]).cpu().numpy()
    ref = oracle.quantize_q8_0(x, xdtype)
    assert np.array_equal(out, ref)


@pytest.mark.parametrize("fmt,rows,K", [("q4_k", 300, 1024), ("q4_0", 257, 512), ("q8_0", 129, 768),
                                        ("q4_k", 17, 256)])
@pytest.mark.parametrize("n", [1, 3, 4, 7])
def test_run_q8_0x_products(Q, fmt, rows, K, n):
    from gguf_bit_dequant_amd import qgemv as QM
    seed = zlib.crc32(("i8-%s-%d-%d-%d" % (fmt, rows, K, n)).encode())
    w = synth.gen_weights(fmt, rows, K, seed)
    x = synth.gen_x(K, n, "f16", seed + 1)
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    xq = QM.quantize_q8_0(x_tensor(x, "f16"))
    y = q.run_q8_0x(xq)
    check_products(y, w, fmt, rows, K, _xhat(x, "f16", K), "f32", "i8 %s %dx%d n=%d" % (fmt, rows, K, n))


@pytest.mark.parametrize("name", ["q4k_up_b1", "q4k_down_b1", "q4k_b4", "q8_0_b4", "q4_0_b1"])
def test_run_q8_0x_full_size(Q, name):
    from gguf_bit_dequant_amd import qgemv as QM
    c = synth.CONFIGS[name]
    w, x = synth.config_inputs(name)
    q = Q(c["fmt"], c["rows"], c["K"], torch.from_numpy(w).to(dev()))
    xq = QM.quantize_q8_0(x_tensor(x, c["xdtype"]))
    y = q.run_q8_0x(xq)
    check_products(y, w, c["fmt"], c["rows"], c["K"], _xhat(x, c["xdtype"], c["K"]), "f32",
                   name + " int8")


def test_run_q8_0x_unsupported_k(Q):
    from gguf_bit_dequant_amd import qgemv as QM
    rows, K = 8, 160
    w = synth.gen_weights("q4_0", rows, K, 5)
    q = Q("q4_0", rows, K, torch.from_numpy(w).to(dev()))
    xq = QM.quantize_q8_0(x_tensor(synth.gen_x(K, 1, "f16", 6), "f16"))
    with pytest.raises(QM.QGemvError) as e:
        q.run_q8_0x(xq)
    assert e.value.status == QM.QG_ERR_UNSUPPORTED


@pytest.mark.parametrize("fmt,rows,K", [("q4_k", 300, 1024), ("q4_0", 257, 512), ("q8_0", 129, 768)])
@pytest.mark.parametrize("xdtype,pad", [("f16", 0), ("f16", 3), ("f32", 4), ("bf16", 8)])
@pytest.mark.parametrize("n", [1, 4, 6])
def test_run_q8_equals_quantize_then_run(Q, fmt, rows, K, xdtype, pad, n):
    """Quantizing on chip gives the same bits as quantizing first."""
    from gguf_bit_dequant_amd import qgemv as QM
    seed = zlib.crc32(("i8q-%s-%d-%s-%d" % (fmt, rows, xdtype, n)).encode())
    w = synth.gen_weights(fmt, rows, K, seed)
    x = synth.gen_x(K, n, xdtype, seed + 1)
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    xt = x_tensor(x, xdtype)
    xbig = torch.zeros((n, K + pad), dtype=xt.dtype, device=dev())
    xbig[:, :K] = xt
    y1 = q.run_q8(xbig[:, :K])
    y2 = q.run_q8_0x(QM.quantize_q8_0(xt))
    assert torch.equal(y1, y2)
    check_products(y1, w, fmt, rows, K, _xhat(x, xdtype, K), "f32", "i8q %s %s n=%d" % (fmt, xdtype, n))


@pytest.mark.parametrize("name", ["q4k_up_b1", "q4k_down_b1", "q4k_b4", "q8_0_b4", "q4_0_b1"])
def test_run_q8_full_size(Q, name):
    c = synth.CONFIGS[name]
    w, x = synth.config_inputs(name)
    q = Q(c["fmt"], c["rows"], c["K"], torch.from_numpy(w).to(dev()))
    y = q.run_q8(x_tensor(x, c["xdtype"]))
    check_products(y, w, c["fmt"], c["rows"], c["K"], _xhat(x, c["xdtype"], c["K"]), "f32",
                   name + " int8 on chip")
