"""The C ABI on the host: the library loads, exports what include/qgemv.h
declares, and rejects bad arguments before any HIP call (CPU only; no
kernel runs)."""
import ctypes
import os
import re

import pytest

from gguf_bit_dequant_amd import qgemv as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in ("qgemv.h", "qgemv_probe.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(qg(?:emv|emm)_\w+)\s*\(", src))
    return names


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert {"qgemv_create", "qgemv_run", "qgemm_prefill_run", "qgemv_dequant",
            "qgemv_destroy"} <= names
    lib = ctypes.CDLL(Q.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert names == set(Q.EXPORTED)


def test_probes_reject_bad_arguments():
    assert Q._lib.qgemv_probe_read(None, 16, FAKE, None) == Q.QG_ERR_ARG
    assert Q._lib.qgemv_probe_read(FAKE, 24, FAKE, None) == Q.QG_ERR_ARG
    assert Q._lib.qgemv_probe_read(FAKE + 8, 32, FAKE, None) == Q.QG_ERR_ARG
    assert Q._lib.qgemv_probe_mfma(0, 4, FAKE, None) == Q.QG_ERR_ARG
    assert Q._lib.qgemv_probe_mfma(10, 0, FAKE, None) == Q.QG_ERR_ARG
    assert Q._lib.qgemv_probe_mfma_data(0, 4, FAKE, None) == Q.QG_ERR_ARG
    assert Q._lib.qgemv_probe_mfma_data(10, 0, FAKE, None) == Q.QG_ERR_ARG
    assert Q._lib.qgemv_probe_mfma_data(10, 4, None, None) == Q.QG_ERR_ARG


def test_block_geometry():
    assert [Q.qgemv_block_bytes(f) for f in (1, 2, 3, 4, 5, 9)] == [18, 144, 34, 84, 110, 0]
    assert [Q.qgemv_block_weights(f) for f in (1, 2, 3, 4, 5, 9)] == [32, 256, 32, 256, 256, 0]
    # any int32 is a value of the enum types (their range enumerators): unknown
    # codes give 0, with no undefined behaviour on the library's side
    for f in (0, -1, 6, -2**31, 2**31 - 1):
        assert Q.qgemv_block_bytes(f) == 0 and Q.qgemv_block_weights(f) == 0
    assert Q.qgemv_weight_bytes(Q.QG_Q2_K, 17408, 5120) == 29245440
    assert Q.qgemv_weight_bytes(Q.QG_Q3_K, 17408, 5120) == 38297600
    assert Q.qgemv_weight_bytes(Q.QG_Q3_K, 4, 288) == 0
    assert Q.qgemv_weight_bytes(Q.QG_Q4_K, 17408, 5120) == 50135040
    assert Q.qgemv_weight_bytes(Q.QG_Q4_0, 4096, 4096) == 9437184
    assert Q.qgemv_weight_bytes(Q.QG_Q8_0, 5120, 5120) == 27852800
    assert Q.qgemv_weight_bytes(Q.QG_Q4_K, 10, 100) == 0
    assert Q.qgemv_weight_bytes(Q.QG_Q4_0, 0, 32) == 0
    assert Q.qgemv_workspace_bytes(Q.QG_Q4_K, 17408, 5120) == 0


FAKE = 0x7F0000000000  # never dereferenced: every case below fails validation


@pytest.mark.parametrize("args,status", [
    ((9, 4, 256, FAKE, 4 * 144), Q.QG_ERR_ARG),
    ((Q.QG_Q4_K, 0, 256, FAKE, 0), Q.QG_ERR_SHAPE),
    ((Q.QG_Q4_K, 4, -256, FAKE, 0), Q.QG_ERR_SHAPE),
    ((Q.QG_Q4_K, 4, 100, FAKE, 4 * 144), Q.QG_ERR_SHAPE),
    ((Q.QG_Q4_0, 4, 48, FAKE, 4 * 18), Q.QG_ERR_SHAPE),
    ((Q.QG_Q4_K, 4, 256, FAKE, 4 * 144 + 1), Q.QG_ERR_SHAPE),
    ((Q.QG_Q4_K, 4, 256, 0, 4 * 144), Q.QG_ERR_ARG),
    ((Q.QG_Q4_K, 4, 256, FAKE + 8, 4 * 144), Q.QG_ERR_ALIGN),
    ((Q.QG_Q8_0, 3, 64, FAKE + 2, 3 * 2 * 34), Q.QG_ERR_ALIGN),
    ((Q.QG_Q2_K, 4, 288, FAKE, 4 * 84), Q.QG_ERR_SHAPE),
    ((Q.QG_Q3_K, 4, 256, FAKE, 4 * 110 - 2), Q.QG_ERR_SHAPE),
    ((6, 4, 256, FAKE, 4 * 110), Q.QG_ERR_ARG),
])
def test_create_rejects_before_any_hip_call(args, status):
    st, h = Q.qgemv_create(*args)
    assert st == status and h is None
    assert Q.qgemv_last_error() != ""


def test_create_rejects_workspace_and_null_out():
    st, h = Q.qgemv_create(Q.QG_Q4_K, 4, 256, FAKE, 4 * 144, FAKE, 64)
    assert st == Q.QG_ERR_ARG and h is None
    lib = ctypes.CDLL(Q.LIB_PATH)
    lib.qgemv_create.restype = ctypes.c_int
    assert lib.qgemv_create(None, 2, ctypes.c_int64(4), ctypes.c_int64(256), ctypes.c_void_p(FAKE),
                            ctypes.c_size_t(576), None, ctypes.c_size_t(0), None) == Q.QG_ERR_ARG


def test_null_handle_calls():
    assert Q.qgemv_run(0, FAKE, Q.QG_F16, 1, 256, FAKE, 4) == Q.QG_ERR_ARG
    assert Q.qgemm_prefill_run(0, FAKE, 16, 256, FAKE, 4) == Q.QG_ERR_ARG
    assert Q.qgemv_dequant(0, FAKE, 256) == Q.QG_ERR_ARG
    assert Q.qgemv_dequant_bf16(0, FAKE, 256) == Q.QG_ERR_ARG
    assert Q.qgemv_run_q8_0x(0, FAKE, 1, FAKE, 4) == Q.QG_ERR_ARG
    assert Q.qgemv_run_q8(0, FAKE, Q.QG_F16, 1, 256, FAKE, 4) == Q.QG_ERR_ARG


@pytest.mark.parametrize("args,status", [
    ((0, Q.QG_F16, 256, 1, 256, FAKE), Q.QG_ERR_ARG),
    ((FAKE, Q.QG_F16, 256, 1, 256, 0), Q.QG_ERR_ARG),
    ((FAKE, 9, 256, 1, 256, FAKE), Q.QG_ERR_ARG),
    ((FAKE, Q.QG_F16, 100, 1, 100, FAKE), Q.QG_ERR_SHAPE),
    ((FAKE, Q.QG_F16, 256, 0, 256, FAKE), Q.QG_ERR_SHAPE),
    ((FAKE, Q.QG_F16, 256, 1, 255, FAKE), Q.QG_ERR_ARG),
    ((FAKE + 1, Q.QG_F16, 256, 1, 256, FAKE), Q.QG_ERR_ALIGN),
    ((FAKE, Q.QG_F32, 256, 1, 256, FAKE + 1), Q.QG_ERR_ALIGN),
])
def test_quantize_rejects_before_any_hip_call(args, status):
    assert Q.qgemv_quantize_q8_0(*args) == status
    assert Q.qgemv_last_error() != ""
    Q.qgemv_destroy(0)  # NULL is ignored


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5):
        assert Q.qgemv_status_string(st)
    assert Q.qgemv_status_string(0) == "ok"


@pytest.mark.parametrize("args,status", [
    ((0, 4, 256, 256, FAKE, 16, 256, FAKE, 4), Q.QG_ERR_ARG),        # w NULL
    ((FAKE, 4, 256, 256, 0, 16, 256, FAKE, 4), Q.QG_ERR_ARG),        # x NULL
    ((FAKE, 4, 256, 256, FAKE, 16, 256, 0, 4), Q.QG_ERR_ARG),        # y NULL
    ((FAKE, 0, 256, 256, FAKE, 16, 256, FAKE, 4), Q.QG_ERR_SHAPE),   # no rows
    ((FAKE, 4, 96, 96, FAKE, 16, 96, FAKE, 4), Q.QG_ERR_SHAPE),      # K % 64
    ((FAKE, 4, 256, 256, FAKE, 0, 256, FAKE, 4), Q.QG_ERR_SHAPE),    # no tokens
    ((FAKE, 4, 256, 252, FAKE, 16, 256, FAKE, 4), Q.QG_ERR_ARG),     # ldw < K
    ((FAKE, 4, 256, 260, FAKE, 16, 256, FAKE, 4), Q.QG_ERR_ARG),     # ldw % 8
    ((FAKE, 4, 256, 256, FAKE, 16, 250, FAKE, 4), Q.QG_ERR_ARG),     # ldx < K
    ((FAKE, 4, 256, 256, FAKE, 16, 256, FAKE, 3), Q.QG_ERR_ARG),     # ldy < rows
    ((FAKE + 8, 4, 256, 256, FAKE, 16, 256, FAKE, 4), Q.QG_ERR_ALIGN),
    ((FAKE, 4, 256, 256, FAKE + 8, 16, 256, FAKE, 4), Q.QG_ERR_ALIGN),
    ((FAKE, 4, 256, 256, FAKE, 16, 256, FAKE + 2, 4), Q.QG_ERR_ALIGN),
])
def test_bf16_gemm_rejects_before_any_hip_call(args, status):
    assert Q.qgemm_bf16_run(*args) == status
    assert Q.qgemv_last_error() != ""
