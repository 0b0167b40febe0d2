"""mla_decode_paged_append_noalloc against mla_decode_paged_append +
mla_decode_combine on the same inputs, through the C-ABI: two calls in a row,
the second on a smaller batch, each compared bit for bit (same kernels, same
split plan), cache and scales included."""

import numpy as np
import pytest
import torch

import synth
from _gpu import GpuState, dev, log

pytestmark = pytest.mark.gpu


def _pair(w):
    """Two GPU states of one workload (the pool quantised by the product's
    append), the first for the two-call path, the second for the no-alloc call."""
    a = GpuState(w)
    b = GpuState(w)
    assert torch.equal(a.cache, b.cache) and torch.equal(a.kv_scale, b.kv_scale)
    return a, b


def _run_both(w, pps, ms):
    import long_context_mla_amd as mla

    a, b = _pair(w)
    d = dev()
    B, n_q, H = w.B, w.n_q, w.H
    new_a = a.new_rows if a.new_rows is not None else torch.empty((B, 0, 576), dtype=torch.bfloat16, device=d)
    new_b = b.new_rows if b.new_rows is not None else torch.empty((B, 0, 576), dtype=torch.bfloat16, device=d)
    out_a = torch.empty((B, n_q, H, 512), dtype=torch.bfloat16, device=d)
    lse_a = torch.empty((B, n_q, H), dtype=torch.float32, device=d)
    if ms > 1:
        o_part = torch.empty((B, ms, n_q, H, 512), dtype=torch.bfloat16, device=d)
        l_part = torch.empty((B, ms, n_q, H), dtype=torch.float32, device=d)
        mla.mla_decode_paged_append(new_a, a.q, a.cache, a.kv_scale, w.scale_mode, a.block_table, a.seq_lens,
                                    w.softmax_scale, pps, ms, o_partial=o_part, lse_partial=l_part)
        mla.mla_decode_combine(o_part, l_part, a.seq_lens, w.max_blocks, pps, out_a, lse_a)
    else:
        mla.mla_decode_paged_append(new_a, a.q, a.cache, a.kv_scale, w.scale_mode, a.block_table, a.seq_lens,
                                    w.softmax_scale, pps, ms, out=out_a, lse=lse_a)
    # outputs pre-filled with a pattern the call must overwrite everywhere
    out_b = torch.full((B, n_q, H, 512), 7.0, dtype=torch.bfloat16, device=d)
    lse_b = torch.full((B, n_q, H), 7.0, dtype=torch.float32, device=d)
    mla.mla_decode_paged_append_noalloc(new_b, b.q, b.cache, b.kv_scale, w.scale_mode, b.block_table,
                                        b.seq_lens, w.softmax_scale, pps, ms, out_b, lse_b)
    torch.cuda.synchronize()
    assert torch.equal(a.cache, b.cache), f"{w.name}: cache bytes differ"
    assert torch.equal(a.kv_scale, b.kv_scale), f"{w.name}: scales differ"
    ua = out_a.view(torch.int16).cpu().numpy()
    ub = out_b.view(torch.int16).cpu().numpy()
    la = lse_a.cpu().numpy()
    lb = lse_b.cpu().numpy()
    n_diff = int((ua != ub).sum())
    log(f"{w.name} B={B} n_q={n_q} H={H} pps={pps} splits={ms} rows={B * ms * n_q * H}: "
        f"out bits differing {n_diff}, lse equal {np.array_equal(la, lb)}")
    assert n_diff == 0, f"{w.name}: {n_diff} output values differ"
    assert np.array_equal(la.view(np.int32), lb.view(np.int32)), f"{w.name}: lse differs"
    assert np.isfinite(la).any()


def test_noalloc_matches_two_call_path_twice_second_smaller():
    import long_context_mla_amd as mla

    # the 100k-token single-request step in the launch configuration the
    # throughput measurement uses (the planner's split, 224 x 64 partial rows)
    w1 = synth.make("fp8_single_100k")
    pps1, ms1 = mla.mla_decode_plan_lens(w1.seq_lens, w1.n_q, w1.H)
    assert w1.B * ms1 * w1.n_q * w1.H <= mla.NOALLOC_MAX_PARTIAL_ROWS
    _run_both(w1, pps1, ms1)
    # then a smaller batch: 3 requests, 2 causal queries, 16 heads, ragged
    # lengths with a partial last page and per-token scales
    w2 = synth.custom("noalloc_small", B=3, n_q=2, H=16, context_lens=(5000, 130, 62), scale_mode="token",
                      seed=11)
    pps2, ms2 = mla.mla_decode_plan_lens(w2.seq_lens, w2.n_q, w2.H)
    assert w2.B * ms2 * w2.n_q * w2.H < w1.B * ms1 * w1.n_q * w1.H
    _run_both(w2, pps2, ms2)
    # one split: the decode writes out / lse itself, the scratch is not used
    _run_both(w2, 10_000, 1)


def test_noalloc_rejects_partials_beyond_the_scratch():
    import long_context_mla_amd as mla

    w = synth.custom("noalloc_limit", B=1, n_q=1, H=64, context_lens=(200,), scale_mode="tensor", seed=3)
    s = GpuState(w)
    d = dev()
    out = torch.empty((1, 1, 64, 512), dtype=torch.bfloat16, device=d)
    lse = torch.empty((1, 1, 64), dtype=torch.float32, device=d)
    ms = mla.NOALLOC_MAX_PARTIAL_ROWS // 64 + 1
    with pytest.raises(mla.MlaError) as e:
        mla.mla_decode_paged_append_noalloc(s.new_rows, s.q, s.cache, s.kv_scale, "tensor", s.block_table,
                                            s.seq_lens, w.softmax_scale, 1, ms, out, lse)
    assert e.value.status == 5
