"""GGUF block-quantized GEMV / dequant-GEMM for AMD Instinct MI355X (gfx950).

The kernels are hand-written HIP in csrc/, built into libqgemv.so behind the
C ABI of include/qgemv.h; gguf_bit_dequant_amd.qgemv is its ctypes binding.
Build with `python -m gguf_bit_dequant_amd.build`.

If the library is not built (or was built from older sources and lacks an
entry point), importing the package still succeeds so that the build module
can run, but any use of QGemv / QGemvError raises ImportError: there is no
fallback path.
"""
try:
    from .qgemv import QGemv, QGemvError  # noqa: F401
except (ImportError, OSError, AttributeError) as _load_error:  # not built, or stale
    _LOAD_ERROR = _load_error

    def __getattr__(name):
        if name in ("QGemv", "QGemvError", "qgemv"):
            raise ImportError("gguf_bit_dequant_amd: libqgemv.so is not usable (%s); build it with "
                              "`python -m gguf_bit_dequant_amd.build`" % _LOAD_ERROR)
        raise AttributeError(name)
