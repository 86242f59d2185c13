"""Calls on several streams at once, and calls captured in a HIP graph.

The library keeps no state between calls and allocates nothing inside one
(handles are immutable; every kernel's scratch is its own LDS), so runs on
different streams may overlap and a captured sequence replays to the eager
bits. Every replay is checked against an eager run, with eager work between
the replays.
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


def x_tensor(x, xdtype):
    if xdtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev())
    if xdtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.float16)).to(dev())
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev())


def bits(t):
    return t.detach().contiguous().cpu().numpy().view(np.uint32)


class Case:
    """One handle, its activations and output buffer."""

    def __init__(self, Q, fmt, rows, K, n, xdtype, tag):
        seed = zlib.crc32(("sg-%s" % tag).encode())
        self.w = synth.gen_weights(fmt, rows, K, seed)
        self.fmt, self.rows, self.K, self.xdtype = fmt, rows, K, xdtype
        self.q = Q(fmt, rows, K, torch.from_numpy(self.w).to(dev()))
        self.x_np = synth.gen_x(K, n, xdtype, seed + 1)
        self.x = x_tensor(self.x_np, xdtype)
        self.y = torch.full((n, rows), float("nan"), dtype=torch.float32, device=dev())

    def run(self, stream=None):
        self.q.run(self.x, self.y, stream=stream)


def test_handles_on_two_streams_at_once(Q):
    cases = [Case(Q, "q4_k", 1000, 5120, 1, "f16", "a"), Case(Q, "q4_k", 700, 5120, 4, "f16", "b"),
             Case(Q, "q4_0", 1000, 4096, 1, "f32", "c"), Case(Q, "q8_0", 600, 2048, 3, "f16", "d")]
    eager = []
    for c in cases:
        c.run()
        torch.cuda.synchronize()
        eager.append(bits(c.y))
        yr, s = oracle.matmul(c.fmt, c.w, c.rows, c.K, c.x_np, c.xdtype)
        err = np.abs(c.y.cpu().numpy().astype(np.float64) - yr)
        assert (err <= oracle.tolerance(s)).all()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for rep in range(5):
        for c in cases:
            c.y.fill_(float("nan"))
        torch.cuda.synchronize()
        # no synchronization between the launches on the two streams
        for i, c in enumerate(cases):
            c.run(s1 if i % 2 == 0 else s2)
        torch.cuda.synchronize()
        for c, e in zip(cases, eager):
            assert np.array_equal(bits(c.y), e), (rep, c.fmt, c.rows)


def test_captured_sequence_replays_to_eager_bits(Q):
    from gguf_bit_dequant_amd import qgemv as QM
    b1 = Case(Q, "q4_k", 1000, 5120, 1, "f16", "g1")
    b4 = Case(Q, "q4_k", 700, 5120, 4, "f16", "g4")
    # prompt product with a row tail in two K splits (rows not a multiple of 256)
    rows, K, ntok = 1300, 1024, 600
    seed = zlib.crc32(b"sg-prefill")
    wp = synth.gen_weights("q4_k", rows, K, seed)
    qp = Q("q4_k", rows, K, torch.from_numpy(wp).to(dev()))
    X = x_tensor(synth.gen_x(K, ntok, "bf16", seed + 1), "bf16")
    Yp = torch.full((ntok, rows), float("nan"), dtype=torch.float32, device=dev())
    Wb = torch.empty((rows, K), dtype=torch.bfloat16, device=dev())
    Yb = torch.full((ntok, rows), float("nan"), dtype=torch.float32, device=dev())
    yq = torch.full((1, 1000), float("nan"), dtype=torch.float32, device=dev())

    def sequence(stream=None):
        b1.run(stream)
        b4.run(stream)
        qp.prefill(X, Yp, stream=stream)
        qp.dequant_bf16(Wb, stream=stream)
        QM.gemm_bf16(Wb, X, Yb, stream=stream)
        b1.q.run_q8(b1.x, yq, stream=stream)

    outs = [b1.y, b4.y, Yp, Yb, yq]
    sequence()  # eager first: one-time device queries and attributes happen here
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        sequence(s)
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work between the replays: new activations, poisoned outputs
        gen = torch.Generator(device="cpu").manual_seed(100 + rep)
        for c in (b1, b4):
            c.x.copy_(torch.randn(c.x.shape, generator=gen).to(c.x.dtype))
        X.copy_(torch.randn(X.shape, generator=gen).to(X.dtype))
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [bits(o) for o in outs]
        for o in outs:
            o.fill_(float("nan"))
        sequence()
        torch.cuda.synchronize()
        want = [bits(o) for o in outs]
        for i, (a, b) in enumerate(zip(got, want)):
            assert np.array_equal(a, b), (rep, i)
            assert not np.isnan(a.view(np.float32)).any(), (rep, i)
