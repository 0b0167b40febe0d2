"""Measured hardware peaks on one MI355X: ctypes binding of libmla_peaks.so
(C ABI in ``include/mla_peaks.h``) and the measurements bench.py reports.

* ``hbm_read``: streaming read of a buffer larger than the last-level cache;
* ``page_stream``: 36,864-byte pages through a random page list into LDS by
  LDS-DMA, the decode kernel's staging, at 1-4 pages in flight per wave;
* ``latency``: dependent loads over a random 4 KB-strided cycle;
* ``mfma_bf16``: v_mfma_f32_16x16x32_bf16 throughput and the shader clock.

Times are HIP events on the stream the kernels run on.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_peaks.so")
PAGE_BYTES = 36864


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python long_context_mla_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, L = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.mla_peak_stream_read.argtypes = [P, L, P, I, P]
    lib.mla_peak_stream_pages.argtypes = [P, I, P, I, I, I, P, P]
    lib.mla_peak_latency.argtypes = [P, L, I, P, P, P]
    lib.mla_peak_mfma.argtypes = [I, I, I, P, P, P]
    for f in ("mla_peak_stream_read", "mla_peak_stream_pages", "mla_peak_latency", "mla_peak_mfma"):
        getattr(lib, f).restype = I
    return lib


LIB = _load()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ok(name, rc):
    if rc != 0:
        raise RuntimeError(f"{name} failed with status {rc}")


def _timed(fn, reps):
    """Mean milliseconds per call over `reps` back-to-back calls (after one warm call)."""
    fn()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def hbm_read(nbytes=2 << 30, grids=(256, 512, 1024, 2048, 4096), reps=10):
    """GB/s of a streaming read of `nbytes` (default 2 GiB, eight times the
    256 MB last-level cache) for each grid size; returns (best GB/s, table)."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(3)
    table = {}
    for g in grids:
        sink = torch.empty(g * 256, dtype=torch.int32, device="cuda")
        ms = _timed(lambda: _ok("mla_peak_stream_read", LIB.mla_peak_stream_read(
            ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), g, _stream())), reps)
        table[g] = nbytes / (ms * 1e-3) / 1e9
    del buf
    return max(table.values()), table


def page_stream(nbytes=2 << 30, wgs=256, depths=(1, 2, 3, 4), reps=10, seed=0):
    """GB/s moving random pages HBM -> LDS by LDS-DMA with `wgs` workgroups
    (one per compute unit) and `depth` pages of 36,864 bytes in flight per
    workgroup; returns {depth: GB/s}."""
    n_pages = nbytes // PAGE_BYTES
    buf = torch.empty(n_pages * PAGE_BYTES, dtype=torch.uint8, device="cuda").fill_(5)
    g = torch.Generator().manual_seed(seed)
    ids = torch.randperm(n_pages, generator=g).to(torch.int32).cuda()
    ppw = (n_pages + wgs - 1) // wgs
    out = {}
    for d in depths:
        sink = torch.empty(((n_pages + ppw - 1) // ppw) * 256, dtype=torch.int32, device="cuda")
        ms = _timed(lambda: _ok("mla_peak_stream_pages", LIB.mla_peak_stream_pages(
            ctypes.c_void_p(buf.data_ptr()), n_pages, ctypes.c_void_p(ids.data_ptr()), n_pages, ppw, d,
            ctypes.c_void_p(sink.data_ptr()), _stream())), reps)
        out[d] = n_pages * PAGE_BYTES / (ms * 1e-3) / 1e9
    del buf
    return out


def latency(nbytes=1 << 30, stride_bytes=4096, steps=20000, seed=0):
    """Nanoseconds per dependent load over a random cycle of 4 KB-strided slots
    spanning `nbytes`."""
    stride = stride_bytes // 4
    n = nbytes // 4
    slots = n // stride
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(slots, generator=g).to(torch.int64)
    chain = torch.zeros(n, dtype=torch.int32)
    chain[perm * stride] = (torch.roll(perm, -1) * stride).to(torch.int32)
    chain = chain.cuda()
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    ticks = torch.zeros(1, dtype=torch.int64, device="cuda")
    for _ in range(2):
        _ok("mla_peak_latency", LIB.mla_peak_latency(ctypes.c_void_p(chain.data_ptr()), n, steps,
                                                     ctypes.c_void_p(out.data_ptr()),
                                                     ctypes.c_void_p(ticks.data_ptr()), _stream()))
        torch.cuda.synchronize()
    return float(ticks.item()) * 10.0 / steps  # 100 MHz ticks -> ns


def mfma_bf16(waves_per_simd=2, grid=1024, iters=20000, reps=3):
    """TFLOP/s of independent v_mfma_f32_16x16x32_bf16 chains and the shader
    clock (GHz) the loop ran at."""
    sink = torch.empty(grid * 256 * waves_per_simd, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2 * grid, dtype=torch.int64, device="cuda")
    ms = _timed(lambda: _ok("mla_peak_mfma", LIB.mla_peak_mfma(
        grid, waves_per_simd, iters, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(clocks.data_ptr()),
        _stream())), reps)
    flops = grid * 4 * waves_per_simd * iters * 8 * 16 * 16 * 32 * 2
    c = clocks.view(grid, 2).double()
    ghz = float((c[:, 0] / c[:, 1]).median()) * 0.1  # shader ticks per 10 ns tick
    return flops / (ms * 1e-3) / 1e12, ghz
