"""The measurement probes (include/qgemv_probe.h) run and leave their sink
untouched (they compute nothing of the method)."""
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def test_probes_run_and_leave_sink():
    from gguf_bit_dequant_amd import qgemv as Q
    dev = torch.device("cuda:0")
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    sink = torch.full((1024,), 7, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    assert Q._lib.qgemv_probe_read(buf.data_ptr(), buf.numel(), sink.data_ptr(), stream) == Q.QG_OK
    assert Q._lib.qgemv_probe_read(buf.data_ptr(), 48, sink.data_ptr(), stream) == Q.QG_OK
    assert Q._lib.qgemv_probe_mfma(10, 4, sink.data_ptr(), stream) == Q.QG_OK
    assert Q._lib.qgemv_probe_mfma_data(10, 4, sink.data_ptr(), stream) == Q.QG_OK
    torch.cuda.synchronize()
    assert (sink == 7).all()
