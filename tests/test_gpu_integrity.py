"""GPU parity of the KV page-tag check (kv_check_pages) with the oracle, bit for
bit, on allocator histories with planted faults; and the check in front of a
decode step: a flagged request reads and writes no page and gets zero rows,
the others still match the attention oracle.  All calls go through the C ABI."""

import json
import os

import numpy as np
import pytest
import torch

import synth
from oracle import integrity as oi
from oracle import mla as omla
from synth import integrity as si

from _gpu import GpuState, assert_cache_equals, bf16_tensor_to_f64, compare, log, oracle_decode, oracle_pool

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_tag_check_small.json")


def _dev(a, dtype=np.int32):
    return torch.from_numpy(np.ascontiguousarray(a).view(dtype)).to("cuda:0")


def _gpu_check(tags, bt, et, lens, ep=None, in_place=False):
    import long_context_mla_amd as mla

    B = bt.shape[0]
    t_lens = _dev(lens)
    status = torch.full((B,), -7, dtype=torch.int32, device="cuda:0")
    checked = t_lens if in_place else torch.full((B,), -7, dtype=torch.int32, device="cuda:0")
    mla.kv_check_pages(_dev(tags), _dev(bt), _dev(et), t_lens, status, checked,
                       None if ep is None else _dev(ep))
    torch.cuda.synchronize()
    return status.cpu().numpy(), checked.cpu().numpy()


def _assert_same(case, tag):
    for ep in (case.expected_pages, None):
        for in_place in (False, True):
            want_s, want_l = oi.check_pages_ref(case.page_tags, case.block_table, case.expected_tags,
                                                case.seq_lens, ep)
            got_s, got_l = _gpu_check(case.page_tags, case.block_table, case.expected_tags, case.seq_lens,
                                      ep, in_place)
            log(f"{tag} record={'pages' if ep is not None else 'map'} in_place={in_place} "
                f"flagged={int((want_s != 0).sum())}/{want_s.size}")
            assert np.array_equal(got_s, want_s), (tag, np.nonzero(got_s != want_s))
            assert np.array_equal(got_l, want_l), (tag, np.nonzero(got_l != want_l))


def test_hand_worked_case():
    with open(GOLDEN) as f:
        g = json.load(f)
    case = si.TagCase(np.asarray(g["page_tags"], np.uint32), np.asarray(g["block_table"], np.int32),
                      np.asarray(g["expected_pages"], np.int32), np.asarray(g["expected_tags"], np.uint32),
                      np.asarray(g["seq_lens"], np.int32))
    got_s, got_l = _gpu_check(case.page_tags, case.block_table, case.expected_tags, case.seq_lens,
                              case.expected_pages)
    assert got_s.tolist() == g["status"] and got_l.tolist() == g["checked_lens"]
    _assert_same(case, "golden")


KINDS = ["stale", "wrong", "oob", "neg", "len", "neglen", "tail"]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_batch_with_planted_faults(seed):
    rng = np.random.default_rng(1000 + seed)
    B, mb = 64, 300
    lens = [int(x) for x in rng.integers(0, mb * 64 + 1, size=B)]
    lens[:6] = [0, 1, 64, 65, mb * 64, mb * 64 - 1]
    faults = []
    for _ in range(16):
        b = int(rng.integers(0, B))
        n = (lens[b] + 63) // 64
        kind = KINDS[int(rng.integers(0, len(KINDS)))]
        if kind in ("stale", "wrong", "oob", "neg") and n == 0:
            continue
        if kind == "tail" and n >= mb:
            continue
        j = int(rng.integers(0, n)) if kind != "tail" else int(rng.integers(n, mb))
        faults.append((kind, b, j))
    need = sum((x + 63) // 64 for x in lens)
    c = si.make_case(seed, lens, mb, num_pages=need + 700, faults=faults, churn=100)
    _assert_same(c, f"batch seed={seed} faults={len(faults)}")


def test_long_requests_take_several_passes():
    """Requests of more than 4096 pages: faults in the first and the second
    pass of the workgroup, at the last page and exactly at page 4096."""
    mb = 5000
    lens = [mb * 64 - 3, 4097 * 64, 4096 * 64 + 1, 4096 * 64, mb * 64]
    faults = [("stale", 0, 4999), ("wrong", 1, 4096), ("oob", 2, 4096), ("tail", 3, 4096)]
    c = si.make_case(11, lens, mb, num_pages=sum((x + 63) // 64 for x in lens) + 100, faults=faults)
    _assert_same(c, "long")


def test_empty_batch_launches_nothing():
    import long_context_mla_amd as mla

    e = torch.empty((0,), dtype=torch.int32, device="cuda:0")
    mla.kv_check_pages(torch.zeros(4, dtype=torch.int32, device="cuda:0"),
                       torch.empty((0, 3), dtype=torch.int32, device="cuda:0"),
                       torch.empty((0, 3), dtype=torch.int32, device="cuda:0"), e, e.clone(), e.clone())
    torch.cuda.synchronize()


def _e2e_workload():
    w = synth.custom("check_e2e", B=4, n_q=1, H=64, context_lens=(300, 200, 1000, 65), cache_dtype="fp8",
                     scale_mode="token", seed=5)
    rng = np.random.default_rng(9)
    tags = rng.integers(0, 2**32, size=w.num_pages, dtype=np.uint64).astype(np.uint32)
    bt = w.block_table
    et = np.where(bt >= 0, tags[np.clip(bt, 0, w.num_pages - 1)], 0).astype(np.uint32)
    victim = 1
    last = (int(w.seq_lens[victim]) - 1) // 64  # the page the victim's new row goes to
    page = int(bt[victim, last])
    tags[page] ^= np.uint32(1)  # the page was handed out again
    return w, tags, et, victim, page


def _e2e_step(w, g, tags, et, fuse_append, check_mode, stream=None):
    import long_context_mla_amd as mla

    npg = int(-(-w.seq_lens.max() // 64))
    st = mla.DecodeStep(w.B, w.n_q, w.H, w.max_blocks, int(w.seq_lens.max()), w.total_tokens(), g.device,
                        pages_per_split=2, max_splits=-(-npg // 2), fuse_append=fuse_append,
                        check_mode=check_mode, cache_dtype=w.cache_dtype)
    check = (_dev(tags), _dev(et), None)
    return st, check


MODES = [("fused", True, "front"), ("fused_overlapped", True, "stream"), ("fused_in_launch", True, "launch"),
         ("separate", False, "front")]


@pytest.mark.parametrize("mode", MODES, ids=[m[0] for m in MODES])
def test_flagged_request_is_aborted_within_the_step(mode):
    name, fuse_append, check_mode = mode
    w, tags, et, victim, page = _e2e_workload()
    want_s, want_l = oi.check_pages_ref(tags, w.block_table, et, w.seq_lens)
    log(f"e2e {name} L={w.seq_lens.tolist()} status={want_s.tolist()}")
    assert want_s.tolist() == [0, oi.STALE_TAG, 0, 0]

    g = GpuState(w)
    before = g.cache[page].clone()
    st, check = _e2e_step(w, g, tags, et, fuse_append, check_mode)
    out, lse = st(g.q, g.cache, g.kv_scale, g.scale_mode, g.block_table, g.seq_lens, w.softmax_scale,
                  new_rows=g.new_rows, page_check=check)
    torch.cuda.synchronize()
    assert st.status.cpu().numpy().tolist() == want_s.tolist()
    if check_mode != "launch":  # the in-launch check writes the status only
        assert st.checked_lens.cpu().numpy().tolist() == want_l.tolist()
    o = bf16_tensor_to_f64(out)
    l = lse.detach().cpu().double().numpy()
    assert not o[victim].any() and np.all(np.isneginf(l[victim]))
    assert torch.equal(g.cache[page], before), "an aborted request wrote into the cache"
    # the cache after the step: in front of the decode, the check zeroes a flagged
    # request's length, so none of its rows is stored; inside the launch each row
    # is stored iff its own page passes
    cache, scales, ts = oracle_pool(w)
    if check_mode == "launch":
        oi.append_checked_ref(w.new_row_bits(), cache, scales, w.block_table, w.seq_lens, w.scale_mode, ts,
                              tags, et)
    else:
        omla.append_ref(w.new_row_bits(), cache, scales, w.block_table, want_l, w.scale_mode, ts)
    assert_cache_equals(g, cache, scales, f"e2e {name}")
    keep = [0, 2, 3]
    ref_o, ref_l = oracle_decode(w, requests=keep)
    compare(o, l, ref_o, ref_l, requests=keep, tag=f"e2e {name}")


def test_overlapped_check_matches_the_sequential_one():
    """The check beside the decode (side stream) and inside the decode launch
    against the check in front of it: same outputs, same cache bytes and scales
    after the step, bit for bit (the flagged request's stale page is the one
    its new row goes to, so no mode stores it); and a HIP graph of each step
    gives the same on every replay."""
    w, tags, et, victim, page = _e2e_workload()
    res = {}
    for name, mode in (("sequential", "front"), ("overlapped", "stream"), ("in_launch", "launch")):
        g = GpuState(w)
        st, check = _e2e_step(w, g, tags, et, True, mode)
        out, lse = st(g.q, g.cache, g.kv_scale, g.scale_mode, g.block_table, g.seq_lens, w.softmax_scale,
                      new_rows=g.new_rows, page_check=check)
        torch.cuda.synchronize()
        res[name] = (out.clone(), lse.clone(), g.cache.clone(), g.kv_scale.clone())
        if mode != "front":
            eager = res[name]
            graph = torch.cuda.CUDAGraph()
            cap = torch.cuda.Stream()
            cap.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cap):
                with torch.cuda.graph(graph, stream=cap):
                    st(g.q, g.cache, g.kv_scale, g.scale_mode, g.block_table, g.seq_lens, w.softmax_scale,
                       new_rows=g.new_rows, page_check=check, stream=cap)
            torch.cuda.current_stream().wait_stream(cap)
            for rep in range(3):
                st.out.zero_()
                st.lse.zero_()
                st.status.fill_(-1)
                torch.cuda.synchronize()
                graph.replay()
                torch.cuda.synchronize()
                log(f"graph replay {rep}")
                assert torch.equal(st.out, eager[0]) and torch.equal(st.lse, eager[1])
                assert torch.equal(g.cache, eager[2]) and torch.equal(g.kv_scale, eager[3])
                assert st.status.cpu().numpy().tolist() == [0, oi.STALE_TAG, 0, 0]
    a = res["sequential"]
    for other in ("overlapped", "in_launch"):
        b = res[other]
        for k, nm in enumerate(("out", "lse", "cache", "kv_scale")):
            assert torch.equal(a[k], b[k]), (other, nm)


@pytest.mark.parametrize("name", ["fp8_single_100k", "fp8_prefix_shared_b32", "fp8_pool_b64", "bf16_pool_b32",
                                  "fp8_spec4_b16"])
def test_full_size_page_maps(name):
    """The check on the page maps of the named workloads at their full sizes (the
    shapes the benchmark times), with faults planted at random pages."""
    w = synth.make(name)
    rng = np.random.default_rng(2024)
    bt = w.block_table.copy()
    tags = rng.integers(0, 2**32, size=w.num_pages, dtype=np.uint64).astype(np.uint32)
    et = np.where(bt >= 0, tags[np.clip(bt, 0, w.num_pages - 1)], 0).astype(np.uint32)
    ep = bt.copy()
    lens = w.seq_lens.copy()
    npg = (lens.astype(np.int64) + 63) // 64
    picks = rng.choice(w.B, size=min(w.B, 4), replace=False)
    for k, b in enumerate(picks):
        j = int(rng.integers(0, npg[b]))
        if k == 0:
            tags[bt[b, j]] ^= np.uint32(1 << 31)  # handed out again (shared pages flag every sharer)
        elif k == 1:
            bt[b, j] = (bt[b, j] + 1) % w.num_pages
        elif k == 2:
            bt[b, j] = w.num_pages
        else:
            lens[b] = w.max_blocks * 64 + 1
    c = si.TagCase(tags, bt, ep, et, lens)
    _assert_same(c, f"{name} B={w.B} pages={int(npg.sum())}")


def test_in_launch_check_with_an_earlier_stale_page():
    """The check inside the decode launch when a flagged request's stale page is
    not the one its new row goes to: the row is stored into its own last page
    (which passes), the stale page is left alone, and the request's rows still
    come out 0 / -inf while the others match the oracle."""
    w, tags, et, victim, last_page = _e2e_workload()
    tags[last_page] ^= np.uint32(1)  # undo: the last page passes again
    first_page = int(w.block_table[victim, 0])
    tags[first_page] ^= np.uint32(1 << 7)  # the first page was handed out again
    want_s, _ = oi.check_pages_ref(tags, w.block_table, et, w.seq_lens)
    assert want_s.tolist() == [0, oi.STALE_TAG, 0, 0]
    g = GpuState(w)
    before = g.cache[first_page].clone()
    st, check = _e2e_step(w, g, tags, et, True, "launch")
    out, lse = st(g.q, g.cache, g.kv_scale, g.scale_mode, g.block_table, g.seq_lens, w.softmax_scale,
                  new_rows=g.new_rows, page_check=check)
    torch.cuda.synchronize()
    assert st.status.cpu().numpy().tolist() == want_s.tolist()
    o = bf16_tensor_to_f64(out)
    l = lse.detach().cpu().double().numpy()
    assert not o[victim].any() and np.all(np.isneginf(l[victim]))
    assert torch.equal(g.cache[first_page], before)
    # the victim's new row went to its own last page, which passes: the cache
    # and scales are byte for byte the oracle's store rule for the in-launch check
    cache, scales, ts = oracle_pool(w)
    kept = oi.append_checked_ref(w.new_row_bits(), cache, scales, w.block_table, w.seq_lens, w.scale_mode, ts,
                                 tags, et)
    assert kept[victim].all()
    assert_cache_equals(g, cache, scales, "in-launch, earlier stale page")
    keep = [0, 2, 3]
    ref_o, ref_l = oracle_decode(w, requests=keep)
    compare(o, l, ref_o, ref_l, requests=keep, tag="in-launch, earlier stale page")


def test_in_launch_status_matches_oracle():
    """The check role of the decode launch (512 threads, so a 140k-token request
    takes two passes) on one planted fault of each kind: status bit for bit as
    the oracle's, flagged rows 0 / -inf, clean requests as the attention oracle."""
    import long_context_mla_amd as mla

    w = synth.custom("check_status", B=7, n_q=1, H=16, context_lens=(140000, 300, 5000, 64, 1, 2100, 777),
                     cache_dtype="fp8", scale_mode="token", seed=21)
    rng = np.random.default_rng(5)
    tags = rng.integers(0, 2**32, size=w.num_pages, dtype=np.uint64).astype(np.uint32)
    bt_h = w.block_table.copy()
    et = np.where(bt_h >= 0, tags[np.clip(bt_h, 0, w.num_pages - 1)], 0).astype(np.uint32)
    ep = bt_h.copy()
    lens = w.seq_lens.copy()
    tags[bt_h[0, 2100]] ^= np.uint32(3)           # second pass of the 512-thread check
    bt_h[1, 2] = (bt_h[1, 2] + 1) % w.num_pages   # another page in the map
    bt_h[2, 40] = w.num_pages + 3                 # outside the pool
    lens[3] = w.max_blocks * 64 + 5               # length past the map
    last5 = (int(lens[5]) - 1) // 64
    tags[bt_h[5, last5]] ^= np.uint32(1 << 30)    # the page the new row goes to
    want_s, _ = oi.check_pages_ref(tags, bt_h, et, lens, ep)
    log(f"in-launch status want={want_s.tolist()}")
    assert want_s.tolist()[:6] == [oi.STALE_TAG, oi.WRONG_PAGE | oi.STALE_TAG, oi.OUT_OF_RANGE | oi.WRONG_PAGE,
                                   oi.BAD_LEN, 0, oi.STALE_TAG] and want_s[6] == 0

    g = GpuState(w)
    stale5 = int(bt_h[5, last5])
    before = g.cache[stale5].clone()
    g.block_table = _dev(bt_h)
    g.seq_lens = _dev(lens)
    npg = int(-(-w.seq_lens.max() // 64))
    st = mla.DecodeStep(w.B, w.n_q, w.H, w.max_blocks, int(w.seq_lens.max()), w.total_tokens(), g.device,
                        pages_per_split=16, max_splits=-(-npg // 16), check_mode="launch", cache_dtype=w.cache_dtype)
    out, lse = st(g.q, g.cache, g.kv_scale, g.scale_mode, g.block_table, g.seq_lens, w.softmax_scale,
                  new_rows=g.new_rows, page_check=(_dev(tags), _dev(et), _dev(ep)))
    torch.cuda.synchronize()
    assert st.status.cpu().numpy().tolist() == want_s.tolist()
    o = bf16_tensor_to_f64(out)
    l = lse.detach().cpu().double().numpy()
    for b in range(w.B):
        if want_s[b]:
            assert not o[b].any() and np.all(np.isneginf(l[b])), b
    assert torch.equal(g.cache[stale5], before), "a row was stored into a page that failed the check"
    cache, scales, ts = oracle_pool(w)
    oi.append_checked_ref(w.new_row_bits(), cache, scales, bt_h, lens, w.scale_mode, ts, tags, et, ep)
    assert_cache_equals(g, cache, scales, "in-launch status")
    keep = [4, 6]
    ref_o, ref_l = oracle_decode(w, requests=keep)
    compare(o, l, ref_o, ref_l, requests=keep, tag="in-launch status")


PATHS = [("fused", True, None), ("separate", False, None), ("in_launch", True, "launch")]


@pytest.mark.parametrize("path", PATHS, ids=[p[0] for p in PATHS])
def test_rows_without_a_slot_are_not_stored(path):
    """New rows with no slot of their own: a request whose page map is full and
    whose length is the map's capacity + 2 (of its three rows, only the first
    has a slot), and a request whose page-map entry at the append position is
    -1 (a clamp would name page 0).  The cache and scales after the step equal
    the oracle's byte for byte: the plain append (fused into the decode launch,
    or a launch of its own) stores exactly the rows with a slot; the in-launch
    check stores nothing for the request flagged for its length or its page."""
    import long_context_mla_amd as mla

    name, fuse_append, check_mode = path
    w = synth.custom("no_slot", B=3, n_q=1, H=16, context_lens=(300, 100, 200), append=3, cache_dtype="fp8",
                     scale_mode="token", seed=18)
    cap = w.max_blocks * 64
    bt = w.block_table.copy()
    lens = w.seq_lens.copy()
    assert (bt[0] >= 0).all(), "request 0 must have a full page map"
    lens[0] = cap + 2
    assert (int(lens[1]) - 3) // 64 == (int(lens[1]) - 1) // 64 == 1
    # page 0 is no row's own target here (the seed is chosen so), so any write to it is a clamped -1
    assert 0 not in (bt[0, -1], bt[1, 1], bt[2, (int(lens[2]) - 1) // 64])
    bt[1, 1] = -1
    g = GpuState(w)
    g.block_table = _dev(bt)
    g.seq_lens = _dev(lens)
    page0 = g.cache[0].clone()
    scale0 = g.kv_scale[0].clone()
    npg = -(-cap // 64) + 1
    st = mla.DecodeStep(w.B, w.n_q, w.H, w.max_blocks, int(lens.max()), int(lens.sum()), g.device,
                        pages_per_split=2, max_splits=-(-npg // 2), fuse_append=fuse_append,
                        check_mode=check_mode or "front", cache_dtype="fp8")
    page_check = None
    tags = et = None
    if check_mode:
        tags = np.arange(1, w.num_pages + 1, dtype=np.uint32)
        et = np.where(bt >= 0, tags[np.clip(bt, 0, w.num_pages - 1)], 0).astype(np.uint32)
        page_check = (_dev(tags), _dev(et), None)
    out, lse = st(g.q, g.cache, g.kv_scale, g.scale_mode, g.block_table, g.seq_lens, w.softmax_scale,
                  new_rows=g.new_rows, page_check=page_check)
    torch.cuda.synchronize()
    log(f"no-slot {name}: cap={cap} lens={lens.tolist()} splits={st.max_splits}")
    assert torch.equal(g.cache[0], page0) and torch.equal(g.kv_scale[0], scale0), "page 0 was written"
    cache, scales, ts = oracle_pool(w)
    if check_mode:
        kept = oi.append_checked_ref(w.new_row_bits(), cache, scales, bt, lens, "token", ts, tags, et)
        assert not kept[0].any() and not kept[1].any() and kept[2].all()
        want_s, _ = oi.check_pages_ref(tags, bt, et, lens)
        assert st.status.cpu().numpy().tolist() == want_s.tolist() == [oi.BAD_LEN, oi.OUT_OF_RANGE, 0]
    else:
        omla.append_ref(w.new_row_bits(), cache, scales, bt, lens, "token", ts)
        # the first row of request 0 went to the last slot of its last page
        assert np.array_equal(cache[bt[0, -1], 63], g.cache[bt[0, -1], 63].cpu().numpy())
    assert_cache_equals(g, cache, scales, f"no-slot {name}")
    ref_o, ref_l = oracle_decode(w, requests=[2])
    compare(bf16_tensor_to_f64(out), lse.detach().cpu().double().numpy(), ref_o, ref_l, requests=[2],
            tag=f"no-slot {name}")


@pytest.mark.parametrize("check_mode", ["front", "launch"])
def test_flagged_request_in_a_wide_batch(check_mode):
    """A batch of 1,024 query rows over at most 64 splits (the combine then
    merges a row per wave): the flagged request's rows come out 0 / -inf, the
    cache is as the oracle's check-and-append leaves it, the others match the
    attention oracle."""
    lens = (63, 64, 65, 700, 1500, 2999, 1, 128, 5, 900, 2000, 1280, 333, 3999, 17, 0)
    w = synth.custom("wide_check", B=16, n_q=1, H=64, context_lens=lens, cache_dtype="fp8", scale_mode="token",
                     seed=41)
    rng = np.random.default_rng(43)
    tags = rng.integers(0, 2**32, size=w.num_pages, dtype=np.uint64).astype(np.uint32)
    bt = w.block_table
    et = np.where(bt >= 0, tags[np.clip(bt, 0, w.num_pages - 1)], 0).astype(np.uint32)
    victim = 4
    tags[int(bt[victim, 3])] ^= np.uint32(1)  # an earlier page of the victim was handed out again
    want_s, want_l = oi.check_pages_ref(tags, bt, et, w.seq_lens)
    assert [i for i, s in enumerate(want_s) if s] == [victim]
    import long_context_mla_amd as mla

    for pps in (1, 2):
        npg = int(-(-w.seq_lens.max() // 64))
        ms = -(-npg // pps)
        assert ms <= 64 and w.B * w.n_q * w.H >= 1024
        log(f"wide check {check_mode} pps={pps} splits={ms} rows={w.B * w.n_q * w.H}")
        g = GpuState(w)
        st = mla.DecodeStep(w.B, w.n_q, w.H, w.max_blocks, int(w.seq_lens.max()), w.total_tokens(), g.device,
                            pages_per_split=pps, max_splits=ms, fuse_append=True, check_mode=check_mode,
                            cache_dtype=w.cache_dtype)
        out, lse = st(g.q, g.cache, g.kv_scale, g.scale_mode, g.block_table, g.seq_lens, w.softmax_scale,
                      new_rows=g.new_rows, page_check=(_dev(tags), _dev(et), None))
        torch.cuda.synchronize()
        assert st.status.cpu().numpy().tolist() == want_s.tolist()
        o = bf16_tensor_to_f64(out)
        l = lse.detach().cpu().double().numpy()
        assert not o[victim].any() and np.all(np.isneginf(l[victim]))
        cache, scales, ts = oracle_pool(w)
        if check_mode == "launch":
            oi.append_checked_ref(w.new_row_bits(), cache, scales, bt, w.seq_lens, w.scale_mode, ts, tags, et)
        else:
            omla.append_ref(w.new_row_bits(), cache, scales, bt, want_l, w.scale_mode, ts)
        assert_cache_equals(g, cache, scales, f"wide check {check_mode} pps={pps}")
        keep = [b for b in range(w.B) if b != victim]
        ref_o, ref_l = oracle_decode(w, requests=keep)
        compare(o, l, ref_o, ref_l, requests=keep, tag=f"wide check {check_mode} pps={pps}")
