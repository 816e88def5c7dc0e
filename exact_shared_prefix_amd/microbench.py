"""Hardware micro-benchmarks on the current GPU (libdualkv_microbench.so).

mfma_tflops(): sustained dense bf16 MFMA rate (32x32x16, register operands,
four independent chains per wave, 8 waves per CU on every CU).
lds_bytes_per_clk(): LDS read bandwidth per CU for 16-byte reads and for
8-byte transpose reads, from the measured time and the GPU's clock.
atomic_lanes_per_s(): sustained fp32 atomic-add rate (lanes per second).
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
        for name in ("dkv_mb_mfma", "dkv_mb_mfma8", "dkv_mb_lds_b128", "dkv_mb_lds_b64",
                     "dkv_mb_lds_tr", "dkv_mb_lds_b128_deep"):
            fn = getattr(_lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        _lib.dkv_mb_atomic.restype = ctypes.c_int
        _lib.dkv_mb_atomic.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        _lib.dkv_mb_valu.restype = ctypes.c_int
        _lib.dkv_mb_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        _lib.dkv_mb_mix.restype = ctypes.c_int
        _lib.dkv_mb_mix.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p]
        _lib.dkv_mb_mfma_chain.restype = ctypes.c_int
        _lib.dkv_mb_mfma_chain.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p]
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


def atomic_lanes_per_s(rows: int = 139264 * 32, blocks: int = 2048, iters: int = 50) -> float:
    """Sustained fp32 atomic-add lanes per second into a [rows][128] fp32 buffer."""
    lib = _load()
    buf = torch.zeros(rows * 128, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    assert lib.dkv_mb_atomic(blocks, 2, buf.data_ptr(), rows, s.cuda_stream) == 0
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    assert lib.dkv_mb_atomic(blocks, iters, buf.data_ptr(), rows, s.cuda_stream) == 0
    e1.record(s)
    torch.cuda.synchronize()
    return blocks * 256 * iters * 16 / (e0.elapsed_time(e1) * 1e-3)


def mfma_tflops(iters: int = 4096) -> float:
    """Best of: 8 waves/CU x 4 chains, and 4 waves/CU x 8 chains."""
    lib = _load()
    blocks = cu_count() * 2  # 8 waves per CU
    a = blocks * 4 * iters * 4 * 32768 / _time(lib.dkv_mb_mfma, blocks, iters) / 1e12
    blocks = cu_count()      # 4 waves per CU
    b = blocks * 4 * iters * 8 * 32768 / _time(lib.dkv_mb_mfma8, blocks, iters) / 1e12
    return max(a, b)


def lds_bytes_per_clk(iters: int = 4096) -> dict:
    lib = _load()
    blocks = cu_count() * 2
    res = {}
    for name, fn, width in (("b128", lib.dkv_mb_lds_b128, 16), ("b64", lib.dkv_mb_lds_b64, 8),
                            ("tr_b64", lib.dkv_mb_lds_tr, 8)):
        sec = _time(fn, blocks, iters)
        total = blocks * 256 * iters * 8 * width
        res[name] = total / sec / cu_count() / clock_hz()
    for wg_per_cu in (2, 4):
        blocks = cu_count() * wg_per_cu
        sec = _time(lib.dkv_mb_lds_b128_deep, blocks, iters)
        total = blocks * 256 * iters * 8 * 16
        res[f"b128_deep_{4 * wg_per_cu}waves"] = total / sec / cu_count() / clock_hz()
    return res


def valu_cycles_per_instruction(iters: int = 8192) -> dict:
    """SIMD cycles per wave64 instruction for exp2, fma and cvt_pk_bf16, at
    4 and 8 waves per CU, from the measured time and the reported clock."""
    lib = _load()
    res = {}
    for wg in (1, 2):
        blocks = cu_count() * wg
        for op, name in ((0, "exp2"), (1, "fma"), (2, "cvt_pk_bf16")):
            sec = _time(lambda b, it, o, s: lib.dkv_mb_valu(op, b, it, o, s), blocks, iters)
            insts_per_simd = blocks * 4 * iters * 8 / (cu_count() * 4)
            res[f"{name}_{4 * wg}waves"] = sec * clock_hz() / insts_per_simd
    return res


def mfma_chain_cycles(iters: int = 2048) -> dict:
    """SIMD cycles per 32x32x16 MFMA (reported clock) with 1, 2, 4, 8
    dependent accumulator chains per wave, at 1 and 2 waves per SIMD."""
    lib = _load()
    res = {}
    for wg in (1, 2):
        blocks = cu_count() * wg
        for ch in (1, 2, 4, 8):
            sec = _time(lambda b, it, o, s: lib.dkv_mb_mfma_chain(ch, b, it, o, s), blocks, iters)
            res[f"{ch}chains_{wg}waves"] = sec * clock_hz() / (iters * 8 * wg)
    return res


def mfma_exp_overlap(iters: int = 4096) -> dict:
    """Time per round (4 MFMAs and/or nexp exp2 per wave), in SIMD cycles per
    wave, for MFMA alone, exp alone and both, at 4 and 8 waves per CU."""
    lib = _load()
    res = {}
    for wg in (1, 2):
        blocks = cu_count() * wg
        for nexp in (16, 32, 64):
            for mf, tag in ((1, "mfma"), (0, "exp"), (1, "both")):
                ne = 0 if tag == "mfma" else nexp
                sec = _time(lambda b, it, o, s: lib.dkv_mb_mix(b, it, mf, ne, o, s), blocks, iters)
                res[f"{4 * wg}w_nexp{nexp}_{tag}"] = sec * clock_hz() / (iters * wg)
    return res


if __name__ == "__main__":
    print({"cus": cu_count(), "clock_hz": clock_hz(), "mfma_bf16_tflops": mfma_tflops(),
           "lds_bytes_per_clk_per_cu": lds_bytes_per_clk(),
           "fp32_atomic_lanes_per_s": atomic_lanes_per_s()})
