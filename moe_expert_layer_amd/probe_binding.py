"""ctypes binding of the measurement probes in include/moe_probes.h (libmoe_probes.so).

The probes are not part of the layer; the tests and the bench use them to measure the
matrix instructions' accumulation precision, the achievable matrix-core and HBM rates, and the
per-CU rate of the GEMMs' operand stream.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(PKG, "libmoe_probes.so")

FORMS = {"scaled_32x32x64": 0, "scaled_16x16x128": 1, "fp8_32x32x16": 2, "bf16_32x32x16": 3, "fp32_fma": 4,
         "scaled_32x32x64_split": 5}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError(f"probe library not built: {PROBE_LIB_PATH} (run __graft_entry__.build())")
        L = ctypes.CDLL(PROBE_LIB_PATH)
        P, I32 = ctypes.c_void_p, ctypes.c_int
        L.moe_probe_mfma_gemm.restype = I32
        L.moe_probe_mfma_gemm.argtypes = [I32, I32, I32, I32, P, P, P, P]
        L.moe_probe_mfma_loop.restype = I32
        L.moe_probe_mfma_loop.argtypes = [I32, I32, I32, P, P]
        L.moe_probe_hbm_read.restype = I32
        L.moe_probe_hbm_read.argtypes = [P, ctypes.c_size_t, I32, P, P]
        L.moe_probe_dma_stream.restype = I32
        L.moe_probe_dma_stream.argtypes = [P, ctypes.c_size_t, I32, I32, I32, I32, I32, P, P]
        L.moe_probe_cvt_bf16.restype = I32
        L.moe_probe_cvt_bf16.argtypes = [I32, I32, P, P, P, P]
        _lib = L
    return _lib


def _stream(stream):
    import torch
    return (torch.cuda.current_stream() if stream is None else stream).cuda_stream


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def mfma_gemm(form: str, a, b, c, b_fp4: bool = False, stream=None):
    """a: uint8 [n, 32, K] E4M3; b: uint8 [n, 32, K] E4M3 or [n, 32, K/2] E2M1 pairs; c: float32 [n, 32, 32]."""
    n, _, K = a.shape
    _check(lib().moe_probe_mfma_gemm(FORMS[form], n, K, int(b_fp4), a.data_ptr(), b.data_ptr(), c.data_ptr(),
                                     _stream(stream)), "moe_probe_mfma_gemm")


def mfma_loop(blocks: int, iters: int, sink, b_fp4: bool = False, stream=None):
    _check(lib().moe_probe_mfma_loop(blocks, iters, int(b_fp4), sink.data_ptr(), _stream(stream)),
           "moe_probe_mfma_loop")


def hbm_read(src, blocks: int, sink, stream=None):
    _check(lib().moe_probe_hbm_read(src.data_ptr(), src.numel() * src.element_size(), blocks, sink.data_ptr(),
                                    _stream(stream)), "moe_probe_hbm_read")


def dma_stream(src, K: int, blocks: int, panels: int, passes: int, depth: int, sink, stream=None):
    """Operand-stream probe: blocks x passes x 512 x K bytes into LDS (see include/moe_probes.h)."""
    _check(lib().moe_probe_dma_stream(src.data_ptr(), src.numel() * src.element_size(), K, blocks, panels, passes,
                                      depth, sink.data_ptr(), _stream(stream)), "moe_probe_dma_stream")


def cvt_bf16(fmt: int, codes, scale_bytes, out, stream=None):
    """fmt 0 E4M3, 1 E5M2, 2 E2M1 pairs; out uint16/int16 [n] (n = values)."""
    _check(lib().moe_probe_cvt_bf16(fmt, out.numel(), codes.data_ptr(), scale_bytes.data_ptr(), out.data_ptr(),
                                    _stream(stream)), "moe_probe_cvt_bf16")
