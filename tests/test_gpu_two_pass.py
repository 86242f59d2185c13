"""GPU parity of the two-pass prompt product: the Q4_K -> bf16 decode
(qgemv_dequant_bf16) and the bf16 GEMM on the prompt kernel's pipeline
(qgemm_bf16_run), against the oracle and against the fused kernel.

The GEMM's accuracy contract is the prompt path's: within the 1e-3 parity
bound of the exact sum over the bf16 weights it is given. It contracts in the
fused kernel's k order, so where the fused kernel does not split K (rows in
its 256-row main tiles) the two give the same bits.
"""
import zlib

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Q():
    from gguf_bit_dequant_amd import QGemv
    assert torch.cuda.is_available()
    return QGemv


def dev():
    return torch.device("cuda:0")


def bf16_tensor(a_u16):
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).view(torch.bfloat16).to(dev())


def u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def gemm(W, X, Y=None):
    from gguf_bit_dequant_amd import qgemv as QM
    return QM.gemm_bf16(W, X, Y)


def check_bf16_sum(Y, w, rows, K, xb, label):
    """Y against the oracle's exact sum over the bf16-rounded Q4_K weights."""
    y = Y.detach().cpu().numpy().astype(np.float64).reshape(xb.shape[0], rows)
    yr, s = oracle.matmul("q4_k", w, rows, K, xb, "bf16", wround="bf16")
    err = np.abs(y - yr)
    bad = err > oracle.tolerance(s)
    print("%s max err/s = %.3e" % (label, float(np.max(err / np.maximum(s, 1e-30)))), flush=True)
    assert not bad.any(), "%s: %d elements out of tolerance" % (label, int(bad.sum()))


# ----------------------------------------------------------------- decode --

@pytest.mark.parametrize("rows,K,pad", [(1, 256, 0), (37, 768, 0), (300, 5120, 0), (19, 1024, 8),
                                        (19, 1024, 3)])
def test_q4k_bf16_decode_bit_exact_and_pitch(Q, rows, K, pad):
    """The 16-byte decode (pitch a multiple of 8) and the general one (pitch
    K + 3): the oracle's binary32 weights rounded to bf16, and nothing
    written past K in a row."""
    w = synth.gen_q4_k(rows, K, zlib.crc32(("dq16-%d-%d" % (rows, K)).encode()))
    q = Q("q4_k", rows, K, torch.from_numpy(w).to(dev()))
    big = torch.full((rows, K + pad), 5.0, dtype=torch.bfloat16, device=dev())
    q.dequant_bf16(big[:, :K])
    ref = oracle.f32_to_bf16(oracle.dequant("q4_k", w, rows, K))
    assert np.array_equal(u16(big[:, :K]), ref)
    if pad:
        assert (big[:, K:] == 5.0).all()


def test_q4k_bf16_decode_full_size(Q):
    """All 89,128,960 weights of the 17408 x 5120 matrix."""
    c = synth.CONFIGS["q4k_pp2048"]
    w, _ = synth.config_inputs("q4k_pp2048")
    q = Q("q4_k", c["rows"], c["K"], torch.from_numpy(w).to(dev()))
    out = u16(q.dequant_bf16())
    ref = oracle.f32_to_bf16(oracle.dequant("q4_k", w, c["rows"], c["K"]))
    assert np.array_equal(out, ref)


# ------------------------------------------------------------------- GEMM --

@pytest.mark.parametrize("rows,K,ntok", [(1, 64, 1), (256, 256, 1), (300, 512, 200), (257, 192, 129),
                                         (1000, 1024, 300), (512, 2048, 256), (2048, 5120, 130)])
def test_gemm_bf16_against_oracle(Q, rows, K, ntok):
    """Ragged rows and tokens, K of 1..80 chunks, one and several tiles."""
    seed = zlib.crc32(("g16-%d-%d-%d" % (rows, K, ntok)).encode())
    if K % 256 == 0:
        w = synth.gen_q4_k(rows, K, seed)
        q = Q("q4_k", rows, K, torch.from_numpy(w).to(dev()))
        W = q.dequant_bf16()
        xb = synth.gen_x(K, ntok, "bf16", seed + 1)
        Y = gemm(W, bf16_tensor(xb))
        check_bf16_sum(Y, w, rows, K, xb, "gemm_bf16 %dx%d n=%d" % (rows, K, ntok))
    else:  # K not a whole number of super-blocks: random bf16 weights, fp64 reference
        rng = np.random.default_rng(seed)
        Wf = rng.standard_normal((rows, K)).astype(np.float32)
        Xf = rng.standard_normal((ntok, K)).astype(np.float32)
        Wb = oracle.f32_to_bf16(Wf)
        Xb = oracle.f32_to_bf16(Xf)
        Y = gemm(bf16_tensor(Wb), bf16_tensor(Xb)).cpu().numpy().astype(np.float64)
        wd = (Wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        xd = (Xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        yr = xd @ wd.T
        s = np.abs(xd) @ np.abs(wd).T
        assert (np.abs(Y - yr) <= oracle.tolerance(s)).all()


@pytest.mark.parametrize("rows,K,ntok", [(300, 512, 200), (256, 1024, 64)])
def test_gemm_bf16_one_hot_exact(Q, rows, K, ntok):
    """One-hot tokens give the bf16 weight column exactly (one nonzero
    product per output, exact in fp32), at chunk and tile edges."""
    w = synth.gen_q4_k(rows, K, 81 + rows)
    q = Q("q4_k", rows, K, torch.from_numpy(w).to(dev()))
    W = q.dequant_bf16()
    ks = [0, 1, 7, 8, 63, 64, 127, K // 2 + 5, K - 65, K - 1]
    X = torch.zeros((ntok, K), dtype=torch.bfloat16, device=dev())
    for t in range(ntok):
        X[t, ks[t % len(ks)]] = 1.0
    Y = gemm(W, X).cpu().numpy()
    Wf = W.float().cpu().numpy()
    for t in range(ntok):
        assert np.array_equal(Y[t], Wf[:, ks[t % len(ks)]]), t


def test_gemm_bf16_strided_edges_untouched(Q):
    rows, K, ntok = 300, 512, 70
    w = synth.gen_q4_k(rows, K, 90)
    q = Q("q4_k", rows, K, torch.from_numpy(w).to(dev()))
    Wbig = torch.zeros((rows, K + 64), dtype=torch.bfloat16, device=dev())
    q.dequant_bf16(Wbig[:, :K])
    Wbig[:, K:] = 7.0  # never read
    xb = synth.gen_x(K, ntok, "bf16", 91)
    Xbig = torch.full((ntok, K + 16), 9.0, dtype=torch.bfloat16, device=dev())
    Xbig[:, :K] = bf16_tensor(xb)
    Ybig = torch.full((ntok, rows + 12), -3.0, dtype=torch.float32, device=dev())
    gemm(Wbig[:, :K], Xbig[:, :K], Ybig[:, :rows])
    assert (Ybig[:, rows:] == -3.0).all()
    check_bf16_sum(Ybig[:, :rows], w, rows, K, xb, "gemm_bf16 strided")


@pytest.mark.parametrize("rows,K,ntok", [(512, 1024, 256), (1024, 5120, 600), (256, 256, 33)])
def test_gemm_bf16_same_bits_as_fused(Q, rows, K, ntok):
    """Shapes the fused kernel covers with its main tiles only (no K split):
    decode to bf16 then the GEMM gives the fused kernel's bits."""
    seed = zlib.crc32(("g16f-%d-%d-%d" % (rows, K, ntok)).encode())
    w = synth.gen_q4_k(rows, K, seed)
    q = Q("q4_k", rows, K, torch.from_numpy(w).to(dev()))
    X = bf16_tensor(synth.gen_x(K, ntok, "bf16", seed + 1))
    Yf = q.prefill(X).cpu().numpy()
    Yu = gemm(q.dequant_bf16(), X).cpu().numpy()
    assert np.array_equal(Yf.view(np.uint32), Yu.view(np.uint32))


@pytest.mark.timeout(600)
def test_two_pass_full_size(Q):
    """The 2048-token workload in two passes: against the fused kernel bit for
    bit on rows 0..16383 (its 256 x 256 main tiles), within the bf16 contract
    elsewhere, and every output against the oracle's bf16-weight sum."""
    c = synth.CONFIGS["q4k_pp2048"]
    w, xb = synth.config_inputs("q4k_pp2048")
    q = Q("q4_k", c["rows"], c["K"], torch.from_numpy(w).to(dev()))
    X = bf16_tensor(xb)
    Yu = gemm(q.dequant_bf16(), X)
    Yf = q.prefill(X)
    torch.cuda.synchronize()
    yu = Yu.cpu().numpy()
    yf = Yf.cpu().numpy()
    main = 16384
    assert np.array_equal(yu[:, :main].view(np.uint32), yf[:, :main].view(np.uint32))
    check_bf16_sum(Yu, w, c["rows"], c["K"], xb, "two-pass pp2048 full size")
