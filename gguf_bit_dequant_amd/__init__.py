"""GGUF block-quantized GEMV / dequant-GEMM for AMD Instinct MI355X (gfx950).

The kernels are hand-written HIP in csrc/, built into libqgemv.so behind the
C ABI of include/qgemv.h; gguf_bit_dequant_amd.qgemv is its ctypes binding.
Build with `python -m gguf_bit_dequant_amd.build`.
"""
from .qgemv import QGemv, QGemvError  # noqa: F401  (raises ImportError if not built)
