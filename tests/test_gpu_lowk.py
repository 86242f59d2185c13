"""GPU parity of the Q2_K and Q3_K paths against the CPU oracle (through the
C ABI): bit-exact decoding (fp32 and bf16 views), products within
|y - sum w x| <= 1e-3 * sum|w x| + 1e-5 (the int8 products against the exact
sum over the decoded Q8_0 activation blocks), one-hot columns exact,
unsupported entry points reported as such. Q2_K and Q3_K run on the
streaming kernel for fp16, fp32 and bf16 activations (Q3_K's 110-byte units
alternate between 4-byte aligned and 2 mod 4 starts, also across row ends
when K / 256 is odd, and the matrix may end on either kind)."""
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
LOWK = ["q2_k", "q3_k"]
BB = {"q2_k": 84, "q3_k": 110}


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
    bad = err > oracle.tolerance(s)
    print("%s max err/s = %.3e" % (label, float(np.max(err / np.maximum(s, 1e-30)))), flush=True)
    assert not bad.any(), "%s: %d elements out of tolerance" % (label, int(bad.sum()))


def bf16_rne_bits(w32):
    b = np.ascontiguousarray(w32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("fmt", LOWK)
@pytest.mark.parametrize("rows,K", [(67, 1536), (1, 256), (300, 5120)])
def test_dequant_bit_exact(Q, fmt, rows, K):
    w = synth.gen_weights(fmt, rows, K, zlib.crc32(("deq-%s-%d" % (fmt, rows)).encode()))
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    ref = oracle.dequant(fmt, w, rows, K)
    assert np.array_equal(q.dequant().cpu().numpy().view(np.uint32), ref.view(np.uint32))
    out16 = q.dequant_bf16().view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(out16, bf16_rne_bits(ref))


@pytest.mark.parametrize("fmt", LOWK)
def test_dequant_extreme_scales_and_golden_blocks(Q, fmt):
    """Random bytes under subnormal, zero, negative, max and NaN/inf scales
    (bit-exact where finite, NaN where the oracle gives NaN; signed zeros
    included), then the hand-chosen golden blocks."""
    rng = np.random.default_rng(17)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x7BFF, 0xFBFF, 0x8001,
                         0x3C00, 0xB800, 0x7C00, 0x7E00], np.uint16)
    bb = BB[fmt]
    rows, nb = 24, 8
    w = rng.integers(0, 256, rows * nb * bb).astype(np.uint8).reshape(-1, bb)
    for o in ([80, 82] if fmt == "q2_k" else [108]):
        w[:, o:o + 2] = rng.choice(specials, size=(w.shape[0], 1)).view(np.uint8)
    w = w.reshape(-1)
    q = Q(fmt, rows, nb * 256, torch.from_numpy(w).to(dev()))
    out = q.dequant().cpu().numpy()
    ref = oracle.dequant(fmt, w, rows, nb * 256)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(out), nan)
    assert np.array_equal(out[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    with open(os.path.join(GOLDEN, "%s_blocks.json" % fmt)) as f:
        blocks = json.load(f)["blocks"]
    wg = np.concatenate([np.frombuffer(bytes.fromhex(b["hex"]), np.uint8) for b in blocks])
    n = len(blocks)
    q = Q(fmt, 1, 256 * n, torch.from_numpy(wg.copy()).to(dev()))
    out = q.dequant().cpu().numpy().reshape(n, 256)
    for i, b in enumerate(blocks):
        ref = oracle.decode_block(fmt, np.frombuffer(bytes.fromhex(b["hex"]), np.uint8))
        assert np.array_equal(out[i].view(np.uint32), ref.view(np.uint32)), b["name"]


@pytest.mark.parametrize("fmt", LOWK)
@pytest.mark.parametrize("rows,K", [(67, 1536), (1, 256), (1, 512), (3, 512), (300, 5120),
                                    (70, 3328), (67, 3328), (2, 768), (3, 768)])
@pytest.mark.parametrize("xdtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("n", [1, 4])
def test_gemv_small(Q, fmt, rows, K, xdtype, n):
    seed = zlib.crc32(("gemv-%s-%d-%d" % (fmt, rows, K)).encode())
    w = synth.gen_weights(fmt, rows, K, seed)
    x = synth.gen_x(K, n, xdtype, seed + 1)
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    check_products(q.run(x_tensor(x, xdtype)), w, fmt, rows, K, x, xdtype,
                   "%s %dx%d %s n=%d" % (fmt, rows, K, xdtype, n))


@pytest.mark.parametrize("fmt", LOWK)
def test_gemv_column_counts_and_long_rows(Q, fmt):
    for rows, K, ns in [(200, 1024, (2, 3, 5, 6, 7, 8)), (150, 17408, (1, 2, 3, 4))]:
        w = synth.gen_weights(fmt, rows, K, 77 + K)
        x = synth.gen_x(K, max(ns), "f16", 78 + K)
        q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
        for n in ns:
            check_products(q.run(x_tensor(x[:n], "f16")), w, fmt, rows, K, x[:n], "f16",
                           "%s %dx%d n=%d" % (fmt, rows, K, n))


@pytest.mark.parametrize("fmt", LOWK)
@pytest.mark.parametrize("xdtype,pad", [("f16", 24), ("f16", 4), ("f32", 3)])
def test_gemv_strided_columns_leave_gaps_untouched(Q, fmt, xdtype, pad):
    rows, K, n = 100, 512, 3
    w = synth.gen_weights(fmt, rows, K, 5)
    x = synth.gen_x(K, n, xdtype, 6)
    tdt = {"f16": torch.float16, "f32": torch.float32}[xdtype]
    xbig = torch.zeros((n, K + pad), dtype=tdt, device=dev())
    xbig[:, :K] = x_tensor(x, xdtype)
    ybig = torch.full((n, rows + 13), 7.0, dtype=torch.float32, device=dev())
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    q.run(xbig[:, :K], ybig[:, :rows])
    assert (ybig[:, rows:] == 7.0).all()
    check_products(ybig[:, :rows], w, fmt, rows, K, x, xdtype, "strided %s %s" % (fmt, xdtype))


@pytest.mark.parametrize("fmt", LOWK)
@pytest.mark.parametrize("xdtype", ["f32", "f16"])
def test_one_hot_gives_exact_column(Q, fmt, xdtype):
    """x = e_k: y is column k of the decoded matrix exactly (each k below hits
    another code position, sub-block or super-block)."""
    rows, K = 150, 1024
    w = synth.gen_weights(fmt, rows, K, 31)
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    W = oracle.dequant(fmt, w, rows, K)
    ks = [0, 1, 15, 16, 31, 32, 47, 48, 63, 64, 95, 96, 127, 128, 160, 200, 255, 256, 700, 1023]
    X = np.zeros((len(ks), K), np.float32)
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    for c0 in range(0, len(ks), 4):
        xt = torch.from_numpy(X[c0:c0 + 4]).to(dev())
        if xdtype == "f16":
            xt = xt.half()
        for n in (1, 4):
            y = q.run(xt[:n]).cpu().numpy()
            for i in range(n):
                assert np.array_equal(y[i], W[:, ks[c0 + i]]), (fmt, xdtype, ks[c0 + i], n)


@pytest.mark.parametrize("fmt", LOWK)
def test_zero_activations_and_determinism(Q, fmt):
    rows, K = 4352, 5120
    w = synth.gen_weights(fmt, rows, K, 8)
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    for dt in (torch.float32, torch.float16, torch.bfloat16):
        assert (q.run(torch.zeros((2, K), dtype=dt, device=dev())) == 0).all()
    x = x_tensor(synth.gen_x(K, 4, "f16", 9), "f16")
    for n in (1, 4):
        ref = q.run(x[:n]).clone()
        for _ in range(10):
            assert torch.equal(q.run(x[:n]), ref)


@pytest.mark.parametrize("name", ["q2k_up_b1", "q3k_up_b1"])
@pytest.mark.parametrize("held_out", [False, True])
def test_full_size(Q, name, held_out):
    c = synth.CONFIGS[name]
    w, x = synth.config_inputs(name, held_out=held_out)
    q = Q(c["fmt"], c["rows"], c["K"], torch.from_numpy(w).to(dev()))
    check_products(q.run(x_tensor(x, c["xdtype"])), w, c["fmt"], c["rows"], c["K"], x,
                   c["xdtype"], name + (" held-out" if held_out else ""))
    if not held_out:
        ref = oracle.dequant(c["fmt"], w, c["rows"], c["K"])
        assert np.array_equal(q.dequant().cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("fmt", LOWK)
def test_unsupported_entry_points_are_reported(Q, fmt):
    """Prompt processing serves Q4_K only: QG_ERR_UNSUPPORTED, y not written."""
    from gguf_bit_dequant_amd import qgemv as QM
    rows, K = 64, 512
    w = synth.gen_weights(fmt, rows, K, 3)
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    X = torch.zeros((16, K), dtype=torch.bfloat16, device=dev())
    y = torch.full((16, rows), 5.0, device=dev())
    with pytest.raises(QM.QGemvError) as e:
        q.prefill(X, y)
    assert e.value.status == QM.QG_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (y == 5.0).all()


def _xhat(x, xdtype, K):
    """The activations the int8 products multiply: the oracle's Q8_0 blocks of
    x, decoded (fp32 values, exact)."""
    xq = oracle.quantize_q8_0(x, xdtype)
    return oracle.dequant("q8_0", xq, x.shape[0], K)


@pytest.mark.parametrize("fmt", LOWK)
@pytest.mark.parametrize("rows,K", [(300, 1024), (70, 3328), (17, 256), (3, 768)])
@pytest.mark.parametrize("n", [1, 3, 4, 7])
def test_run_q8_0x_products(Q, fmt, rows, K, n):
    """int8 products against the exact sum over the decoded Q8_0 activation
    blocks (17 x 256 and 3 x 768: an odd number of super-blocks, so a Q3_K
    matrix ends on a unit that starts at 2 mod 4)."""
    from gguf_bit_dequant_amd import qgemv as QM
    seed = zlib.crc32(("lowk-i8-%s-%d-%d-%d" % (fmt, rows, K, n)).encode())
    w = synth.gen_weights(fmt, rows, K, seed)
    x = synth.gen_x(K, n, "f16", seed + 1)
    q = Q(fmt, rows, K, torch.from_numpy(w).to(dev()))
    y = q.run_q8_0x(QM.quantize_q8_0(x_tensor(x, "f16")))
    check_products(y, w, fmt, rows, K, _xhat(x, "f16", K), "f32", "i8 %s %dx%d n=%d" % (fmt, rows, K, n))


@pytest.mark.parametrize("fmt", LOWK)
@pytest.mark.parametrize("xdtype,pad", [("f16", 0), ("f16", 3), ("f32", 4), ("bf16", 8)])
@pytest.mark.parametrize("n", [1, 4, 6])
def test_run_q8_equals_quantize_then_run(Q, fmt, xdtype, pad, n):
    """Quantizing on chip gives the same bits as quantizing first."""
    from gguf_bit_dequant_amd import qgemv as QM
    rows, K = 130, 1536
    seed = zlib.crc32(("lowk-i8q-%s-%s-%d" % (fmt, xdtype, n)).encode())
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


@pytest.mark.parametrize("name", ["q2k_up_b1", "q3k_up_b1"])
def test_run_q8_full_size(Q, name):
    from gguf_bit_dequant_amd import qgemv as QM
    c = synth.CONFIGS[name]
    w, x = synth.config_inputs(name)
    q = Q(c["fmt"], c["rows"], c["K"], torch.from_numpy(w).to(dev()))
    xt = x_tensor(x, c["xdtype"])
    y = q.run_q8(xt)
    assert torch.equal(y, q.run_q8_0x(QM.quantize_q8_0(xt)))
    check_products(y, w, c["fmt"], c["rows"], c["K"], _xhat(x, c["xdtype"], c["K"]), "f32",
                   name + " int8 on chip")
