"""Hardware micro-benchmarks on the current GPU (libdualkv_microbench.so).

mfma_tflops(): sustained dense bf16 MFMA rate (32x32x16, register operands,
independent chains, every CU): the ceiling the attention kernels are also
compared with.
copy(): a plain device copy of known size, whose HBM byte counters scale the
counters taken on the attention kernels.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdualkv_microbench.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            from . import build as _build
            _build.build()
        _lib = ctypes.CDLL(_LIB)
        for name in ("dkv_mb_mfma", "dkv_mb_mfma8"):
            fn = getattr(_lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        _lib.dkv_mb_copy.restype = ctypes.c_int
        _lib.dkv_mb_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p]
    return _lib


def _time(fn, blocks, iters, reps=3):
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    assert fn(blocks, max(1, iters // 8), out.data_ptr(), s.cuda_stream) == 0
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        assert fn(blocks, iters, out.data_ptr(), s.cuda_stream) == 0
        e1.record(s)
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    return best


def cu_count() -> int:
    return torch.cuda.get_device_properties(0).multi_processor_count


def clock_hz() -> float:
    """Peak shader clock (Hz) as the runtime reports it."""
    props = torch.cuda.get_device_properties(0)
    khz = getattr(props, "clock_rate", 0) or 2_400_000
    return khz * 1e3


def copy(nbytes: int, reps: int = 3) -> dict:
    """Run the plain copy kernel `reps` times over nbytes (multiple of 16);
    returns the bytes each launch reads and writes and the best GB/s."""
    lib = _load()
    n16 = nbytes // 16
    src = torch.ones(n16 * 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    s = torch.cuda.current_stream()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        assert lib.dkv_mb_copy(src.data_ptr(), dst.data_ptr(), n16, s.cuda_stream) == 0
        e1.record(s)
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    assert torch.equal(src, dst)
    return {"bytes_read": n16 * 16, "bytes_written": n16 * 16, "launches": reps,
            "gbs": 2 * n16 * 16 / best / 1e9}


def mfma_tflops(iters: int = 4096) -> float:
    """Best of: 8 waves/CU x 4 chains, and 4 waves/CU x 8 chains."""
    lib = _load()
    blocks = cu_count() * 2  # 8 waves per CU
    a = blocks * 4 * iters * 4 * 32768 / _time(lib.dkv_mb_mfma, blocks, iters) / 1e12
    blocks = cu_count()      # 4 waves per CU
    b = blocks * 4 * iters * 8 * 32768 / _time(lib.dkv_mb_mfma8, blocks, iters) / 1e12
    return max(a, b)


if __name__ == "__main__":
    print({"cus": cu_count(), "clock_hz": clock_hz(), "mfma_bf16_tflops": mfma_tflops()})
