"""Helpers for the GPU parity tests: build the HIP-side state and the oracle-side
state of a synthetic workload from the same seeded inputs.

The HIP side quantises with its own kv_append_fp8 kernel; the oracle side with
oracle.mla.  Nothing computed on the GPU ever feeds the oracle.
"""

from __future__ import annotations

import math
import sys
import time

import numpy as np
import torch

import synth
from oracle import mla as omla

TOL_MAX_ABS = 2e-2
TOL_MEAN_ABS = 2e-3
TOL_LSE = 1e-3


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_tensor_to_f64(t: torch.Tensor) -> np.ndarray:
    u = t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class GpuState:
    """Device buffers of a workload: q, cache, scales, page map, lengths, new rows."""

    def __init__(self, w: synth.Workload, device=None, chunk_pages=4096):
        import long_context_mla_amd as mla

        self.w = w
        d = device or dev()
        self.device = d
        self.q = to_bf16_tensor(w.q_bits(), d)
        self.block_table = torch.from_numpy(w.block_table).to(d)
        self.seq_lens = torch.from_numpy(w.seq_lens).to(d)
        self.scale_mode = w.scale_mode
        self.new_rows = to_bf16_tensor(w.new_row_bits(), d) if w.n_new else None
        if w.cache_dtype == "bf16":
            self.cache = torch.empty((w.num_pages, 64, 576), dtype=torch.bfloat16, device=d)
            for c0 in range(0, w.num_pages, chunk_pages):
                c1 = min(c0 + chunk_pages, w.num_pages)
                self.cache[c0:c1] = to_bf16_tensor(w.page_bits(np.arange(c0, c1)), d)
            self.kv_scale = None
            return
        self.cache = torch.zeros((w.num_pages, 64, 576), dtype=torch.uint8, device=d)
        if w.scale_mode == "token":
            self.kv_scale = torch.zeros((w.num_pages, 64), dtype=torch.float32, device=d)
        else:
            self.kv_scale = torch.tensor([float(w.tensor_scale())], dtype=torch.float32, device=d)
        # quantise the pool with the product's append over an identity page map
        for c0 in range(0, w.num_pages, chunk_pages):
            c1 = min(c0 + chunk_pages, w.num_pages)
            n = c1 - c0
            rows = to_bf16_tensor(w.page_bits(np.arange(c0, c1)).reshape(1, n * 64, 576), d)
            bt = torch.arange(c0, c1, dtype=torch.int32, device=d).view(1, n)
            sl = torch.tensor([n * 64], dtype=torch.int32, device=d)
            mla.kv_append_fp8(rows, self.cache, self.kv_scale, w.scale_mode, bt, sl)
        torch.cuda.synchronize()

    def step(self, pages_per_split=None, max_splits=None, num_cus=0):
        """append (FP8) + decode + combine; returns (out fp64 [B,n_q,H,512], lse fp64)."""
        import long_context_mla_amd as mla

        w = self.w
        st = mla.DecodeStep(w.B, w.n_q, w.H, w.max_blocks, int(w.seq_lens.max()), w.total_tokens(),
                            self.device, num_cus=num_cus, pages_per_split=pages_per_split,
                            max_splits=max_splits, seq_lens_host=w.seq_lens, cache_dtype=w.cache_dtype)
        out, lse = st(self.q, self.cache, self.kv_scale, self.scale_mode, self.block_table,
                      self.seq_lens, w.softmax_scale, new_rows=self.new_rows)
        torch.cuda.synchronize()
        self.last_step = st
        return bf16_tensor_to_f64(out), lse.detach().cpu().double().numpy()

    def decode_only(self, pages_per_split, max_splits):
        import long_context_mla_amd as mla

        w = self.w
        st = mla.DecodeStep(w.B, w.n_q, w.H, w.max_blocks, int(w.seq_lens.max()), w.total_tokens(),
                            self.device, pages_per_split=pages_per_split, max_splits=max_splits, cache_dtype=w.cache_dtype)
        st.decode(self.q, self.cache, self.kv_scale, self.scale_mode, self.block_table, self.seq_lens,
                  w.softmax_scale)
        st.combine(self.seq_lens)
        torch.cuda.synchronize()
        return bf16_tensor_to_f64(st.out), st.lse.detach().cpu().double().numpy()


def oracle_state(w: synth.Workload, requests=None):
    """Oracle cache (codes or bf16 bits, scales) holding at least the pages of
    ``requests`` (all requests by default), after the step's append."""
    reqs = range(w.B) if requests is None else requests
    if requests is None:
        pages = np.arange(w.num_pages)
    else:
        pages = np.unique(np.concatenate([w.pages_of(b) for b in reqs]))
    ts = w.tensor_scale() if w.scale_mode == "tensor" else None
    if w.cache_dtype == "bf16":
        cache = np.zeros((w.num_pages, 64, 576), np.uint16)
        cache[pages] = w.page_bits(pages)
        return cache, None, None
    cache = np.zeros((w.num_pages, 64, 576), np.uint8)
    scales = np.zeros((w.num_pages, 64), np.float32)
    for c0 in range(0, pages.size, 2048):
        sel = pages[c0:c0 + 2048]
        codes, sc = omla.fill_pages_ref(w.page_bits(sel), w.scale_mode, ts)
        cache[sel] = codes
        scales[sel] = sc
    if w.n_new:
        omla.append_ref(w.new_row_bits(), cache, scales, w.block_table, w.seq_lens, w.scale_mode, ts)
    return cache, scales, ts


def oracle_pool(w: synth.Workload):
    """The oracle's quantised pool, every page, before the step's append:
    (codes [num_pages, 64, 576], per-token scales [num_pages, 64], tensor scale)."""
    ts = w.tensor_scale() if w.scale_mode == "tensor" else None
    cache = np.zeros((w.num_pages, 64, 576), np.uint8)
    scales = np.zeros((w.num_pages, 64), np.float32)
    for c0 in range(0, w.num_pages, 2048):
        sel = np.arange(c0, min(c0 + 2048, w.num_pages))
        codes, sc = omla.fill_pages_ref(w.page_bits(sel), w.scale_mode, ts)
        cache[sel] = codes
        scales[sel] = sc
    return cache, scales, ts


def assert_cache_equals(g: "GpuState", cache: np.ndarray, scales: np.ndarray, tag=""):
    """The GPU cache (and per-token scales) byte for byte as the oracle's."""
    got = g.cache.cpu().numpy()
    bad = np.nonzero((got != cache).any(axis=2))
    assert bad[0].size == 0, f"{tag}: cache rows differ at (page, slot) {list(zip(*bad))[:8]}"
    if g.scale_mode == "token":
        gs = g.kv_scale.cpu().numpy()
        assert np.array_equal(gs.view(np.uint32), scales.view(np.uint32)), f"{tag}: scales differ"
    log(f"{tag}: cache and scales equal the oracle's")


def oracle_decode(w: synth.Workload, requests=None):
    cache, scales, ts = oracle_state(w, requests)
    return omla.decode_ref(w.q_bits(), cache, scales, w.block_table, w.seq_lens, n_q=w.n_q, H=w.H,
                           cache_dtype=w.cache_dtype, scale_mode=w.scale_mode,
                           softmax_scale=w.softmax_scale, tensor_scale=ts, requests=requests)


def compare(out, lse, ref_out, ref_lse, requests=None, tag=""):
    """Assert the parity bar on the selected requests; returns the error summary."""
    sel = slice(None) if requests is None else list(requests)
    o, r = out[sel], ref_out[sel]
    l, rl = lse[sel], ref_lse[sel]
    err = np.abs(o - r)
    fin = np.isfinite(rl)
    lse_err = np.abs(l[fin] - rl[fin]) if fin.any() else np.zeros(1)
    summ = dict(max_abs=float(err.max()), mean_abs=float(err.mean()), lse_max=float(lse_err.max()),
                max_ref=float(np.abs(r).max()),
                rel_rms=float(math.sqrt((err ** 2).mean() / max((r ** 2).mean(), 1e-300))))
    log(f"{tag} parity {summ}")
    assert np.all(np.isfinite(o)), f"{tag}: non-finite output"
    assert np.array_equal(np.isinf(l) & (l < 0), np.isinf(rl) & (rl < 0)), f"{tag}: -inf lse mismatch"
    assert summ["max_abs"] <= TOL_MAX_ABS, f"{tag}: max-abs {summ['max_abs']}"
    assert summ["mean_abs"] <= TOL_MEAN_ABS, f"{tag}: mean-abs {summ['mean_abs']}"
    assert summ["lse_max"] <= TOL_LSE, f"{tag}: lse {summ['lse_max']}"
    return summ
