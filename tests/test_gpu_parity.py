"""GPU parity of the HIP path against the CPU oracle on small workloads that
span several 64-token tiles, ragged tails, many split plans, every cache and
scale mode, several query counts and head counts, plus the invariants the
method has (one visible token, weights summing to one, page permutation,
determinism, FP8 = BF16 on the e4m3 grid).  All calls go through the C ABI."""

import numpy as np
import pytest
import torch

import synth
from oracle import mla as omla

from _gpu import GpuState, compare, log, oracle_decode, oracle_state, bf16_tensor_to_f64

pytestmark = pytest.mark.gpu

CASES = [
    dict(name="fp8tok_b3", B=3, n_q=1, H=64, context_lens=(999, 63, 333), cache_dtype="fp8", scale_mode="token"),
    dict(name="fp8ten_b1", B=1, n_q=1, H=64, context_lens=(5000,), cache_dtype="fp8", scale_mode="tensor"),
    dict(name="bf16_h16", B=2, n_q=1, H=16, context_lens=(1000, 777), cache_dtype="bf16"),
    dict(name="fp8_nq2_h16", B=2, n_q=2, H=16, context_lens=(190, 1), cache_dtype="fp8", scale_mode="token"),
    dict(name="fp8_nq3_h64", B=2, n_q=3, H=64, context_lens=(127, 700), cache_dtype="fp8", scale_mode="token"),
    dict(name="fp8_nq4_h64", B=2, n_q=4, H=64, context_lens=(1500, 60), cache_dtype="fp8", scale_mode="token"),
    dict(name="fp8_h40_odd", B=2, n_q=1, H=40, context_lens=(129, 640), cache_dtype="fp8", scale_mode="tensor"),
    dict(name="bf16_nq4_h16", B=1, n_q=4, H=16, context_lens=(300,), cache_dtype="bf16"),
    dict(name="fp8_rows64", B=18, n_q=1, H=64, context_lens=tuple(range(40, 40 + 18 * 71, 71)),
         cache_dtype="fp8", scale_mode="token"),
    dict(name="bf16_rows64", B=16, n_q=1, H=64, context_lens=tuple(range(64, 64 + 16 * 65, 65)),
         cache_dtype="bf16"),
    dict(name="fp8_edges", B=4, n_q=1, H=64, context_lens=(62, 64, 0, 127), cache_dtype="fp8",
         scale_mode="token"),
    dict(name="fp8_empty_req", B=2, n_q=1, H=64, context_lens=(0, 100), cache_dtype="fp8",
         scale_mode="token", append=0),
    # H up to 128 and n_q up to 8 (up to 16 row groups of 64 query rows), full and
    # ragged last pages
    dict(name="fp8_h128", B=2, n_q=1, H=128, context_lens=(2000, 63), cache_dtype="fp8", scale_mode="token"),
    dict(name="fp8_nq5_h64", B=2, n_q=5, H=64, context_lens=(1019, 3), cache_dtype="fp8", scale_mode="token"),
    dict(name="fp8_nq8_h128", B=1, n_q=8, H=128, context_lens=(632,), cache_dtype="fp8", scale_mode="tensor"),
    dict(name="fp8_nq8_h16", B=3, n_q=8, H=16, context_lens=(56, 0, 300), cache_dtype="fp8", scale_mode="token"),
    dict(name="bf16_h128", B=2, n_q=1, H=128, context_lens=(640, 77), cache_dtype="bf16"),
    dict(name="bf16_nq5_h64", B=1, n_q=5, H=64, context_lens=(333,), cache_dtype="bf16"),
    dict(name="bf16_nq8_h128", B=1, n_q=8, H=128, context_lens=(256,), cache_dtype="bf16"),
    # extend / prefill chunks: many new tokens, causal among themselves
    dict(name="bf16_extend_nq64", B=2, n_q=64, H=16, context_lens=(300, 1000), cache_dtype="bf16"),
    dict(name="fp8_extend_nq130", B=1, n_q=130, H=16, context_lens=(700,), cache_dtype="fp8",
         scale_mode="token"),
    # the largest chunk the header allows: 2048 new tokens (32 and 64 row groups), whose
    # append on the FP8 cache takes its own launch
    dict(name="fp8_extend_nq2048", B=1, n_q=2048, H=1, context_lens=(150,), cache_dtype="fp8",
         scale_mode="token"),
    dict(name="bf16_extend_nq2048_h2", B=1, n_q=2048, H=2, context_lens=(2200,), cache_dtype="bf16"),
]


def _make(c, seed=0, **kw):
    c = dict(c)
    name = c.pop("name")
    return synth.custom(name, seed=seed, **c, **kw)


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_step_matches_oracle(case):
    w = _make(case)
    log(f"case {case['name']} B={w.B} n_q={w.n_q} H={w.H} L={w.seq_lens.tolist()}")
    g = GpuState(w)
    ref_o, ref_l = oracle_decode(w)
    out, lse = g.step()
    compare(out, lse, ref_o, ref_l, tag=f"{case['name']} planned")
    # explicit split plans: one split, every page its own split, and a short
    # max_splits whose last split takes the rest
    max_pages = int(-(-w.seq_lens.max() // 64))
    for pps, ms in [(max(max_pages, 1), 1), (1, max(max_pages, 1)), (3, -(-max_pages // 3)), (2, 2)]:
        o, l = g.decode_only(pps, ms)
        compare(o, l, ref_o, ref_l, tag=f"{case['name']} pps={pps} splits={ms}")


def test_every_split_plan_tiny():
    w = synth.custom("tiny_all_plans", B=2, n_q=2, H=16, context_lens=(128, 200), cache_dtype="fp8",
                     scale_mode="token", seed=3)
    g = GpuState(w)
    ref_o, ref_l = oracle_decode(w)
    g.step()  # appends the new rows
    npg = int(-(-w.seq_lens.max() // 64))
    for pps in range(1, npg + 1):
        for ms in sorted({1, 2, -(-npg // pps)}):
            o, l = g.decode_only(pps, ms)
            compare(o, l, ref_o, ref_l, tag=f"pps={pps} ms={ms}")


def test_named_tiny_bf16_full():
    w = synth.make("tiny_bf16")
    g = GpuState(w)
    ref_o, ref_l = oracle_decode(w)
    out, lse = g.step()
    compare(out, lse, ref_o, ref_l, tag="tiny_bf16")


def test_append_matches_oracle_bit_exact():
    import long_context_mla_amd as mla

    for mode in ("token", "tensor"):
        w = synth.custom(f"append_{mode}", B=5, n_q=3, H=16, context_lens=(0, 61, 64, 1000, 5),
                         cache_dtype="fp8", scale_mode=mode, seed=21, sigma_kv=3.0)
        g = GpuState(w)
        g.step()
        cache, scales, _ = oracle_state(w)
        got = g.cache.cpu().numpy()
        assert np.array_equal(got, cache), f"{mode}: codes differ at {np.argwhere(got != cache)[:5]}"
        if mode == "token":
            assert np.array_equal(g.kv_scale.cpu().numpy(), scales)
    # saturation and an all-zero row, per-tensor scale too small for the data
    d = torch.device("cuda:0")
    x = np.zeros((2, 1, 576), np.float32)
    x[0, 0, :] = np.linspace(-900, 900, 576)
    bits = synth.bf16_bits(x)
    cache = torch.zeros((1, 64, 576), dtype=torch.uint8, device=d)
    bt = torch.zeros((2, 1), dtype=torch.int32, device=d)
    sl = torch.tensor([1, 2], dtype=torch.int32, device=d)
    new = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(d)
    for mode, scale in (("tensor", torch.tensor([1.0], device=d)), ("token", torch.zeros((1, 64), device=d))):
        cache.zero_()
        mla.kv_append_fp8(new, cache, scale, mode, bt, sl)
        torch.cuda.synchronize()
        ref_c = np.zeros((1, 64, 576), np.uint8)
        ref_s = np.zeros((1, 64), np.float32)
        omla.append_ref(bits, ref_c, ref_s, np.zeros((2, 1), np.int32), np.array([1, 2], np.int32), mode,
                        np.float32(1.0))
        assert np.array_equal(cache.cpu().numpy(), ref_c), mode
        if mode == "token":
            assert np.array_equal(scale.cpu().numpy(), ref_s)


@pytest.mark.parametrize("mode", ["token", "tensor"])
def test_fused_append_equals_separate(mode):
    """mla_decode_paged_append leaves the cache exactly as kv_append_fp8 does and
    decodes bit-identically to kv_append_fp8 + mla_decode_paged: new rows that
    straddle a page boundary (so land in two splits when each page is a split),
    fill a page's end, or sit in a request's first page."""
    import long_context_mla_amd as mla

    w = synth.custom(f"fused_{mode}", B=3, n_q=4, H=64, context_lens=(62, 700, 1), cache_dtype="fp8",
                     scale_mode=mode, seed=31)
    log(f"fused append {mode}: L={w.seq_lens.tolist()}")
    ref_o, ref_l = oracle_decode(w)
    max_pages = int(-(-w.seq_lens.max() // 64))
    for pps, ms in [(None, None), (1, max_pages), (max_pages, 1), (3, -(-max_pages // 3))]:
        outs = []
        for fuse in (False, True):
            g = GpuState(w)
            st = mla.DecodeStep(w.B, w.n_q, w.H, w.max_blocks, int(w.seq_lens.max()), w.total_tokens(),
                                g.device, pages_per_split=pps, max_splits=ms, fuse_append=fuse, cache_dtype=w.cache_dtype)
            o, l = st(g.q, g.cache, g.kv_scale, g.scale_mode, g.block_table, g.seq_lens, w.softmax_scale,
                      new_rows=g.new_rows)
            torch.cuda.synchronize()
            outs.append((bf16_tensor_to_f64(o), l.cpu().double().numpy(), g.cache.cpu().numpy(),
                         g.kv_scale.cpu().numpy()))
        (oa, la, ca, sa), (ob, lb, cb, sb) = outs
        tag = f"{mode} pps={pps} splits={ms}"
        assert np.array_equal(ca, cb), f"{tag}: cache differs at {np.argwhere(ca != cb)[:5]}"
        assert np.array_equal(sa, sb), f"{tag}: scales differ"
        assert np.array_equal(oa, ob) and np.array_equal(la, lb), f"{tag}: outputs differ"
        compare(ob, lb, ref_o, ref_l, tag=f"fused {tag}")


@pytest.mark.parametrize("mode", ["token", "tensor"])
def test_long_append_paths_agree(mode):
    """An append of 40 rows per request (an extend chunk): mla_decode_paged_append
    storing the rows (they then go through their own append launch), the same
    call with store_rows=0 (the rows encoded inside the decode launch) followed
    by kv_append_fp8, and kv_append_fp8 + mla_decode_paged give the same cache,
    scales, outputs and LSEs, bit for bit, and pass the oracle's bar; the new
    rows straddle page boundaries and fill a request's first page."""
    import long_context_mla_amd as mla

    w = synth.custom(f"long_append_{mode}", B=3, n_q=40, H=16, context_lens=(30, 700, 0), cache_dtype="fp8",
                     scale_mode=mode, append=40, seed=37)
    log(f"long append {mode}: L={w.seq_lens.tolist()}")
    ref_o, ref_l = oracle_decode(w)
    max_pages = int(-(-w.seq_lens.max() // 64))
    for pps, ms in [(max_pages, 1), (1, max_pages)]:
        outs = []
        for path in ("separate", "stored", "unstored"):
            g = GpuState(w)
            o = torch.empty((w.B, w.n_q, w.H, 512), dtype=torch.bfloat16, device=g.device)
            l = torch.empty((w.B, w.n_q, w.H), dtype=torch.float32, device=g.device)
            kw = dict(out=o, lse=l)
            if ms > 1:
                kw = dict(o_partial=torch.empty((w.B, ms, w.n_q, w.H, 512), dtype=torch.bfloat16, device=g.device),
                          lse_partial=torch.empty((w.B, ms, w.n_q, w.H), dtype=torch.float32, device=g.device))
            if path == "separate":
                mla.kv_append_fp8(g.new_rows, g.cache, g.kv_scale, mode, g.block_table, g.seq_lens)
                mla.mla_decode_paged(g.q, g.cache, g.kv_scale, mode, g.block_table, g.seq_lens, w.softmax_scale,
                                     pps, ms, **kw)
            else:
                mla.mla_decode_paged_append(g.new_rows, g.q, g.cache, g.kv_scale, mode, g.block_table, g.seq_lens,
                                            w.softmax_scale, pps, ms, store_rows=(path == "stored"), **kw)
                if path == "unstored":
                    mla.kv_append_fp8(g.new_rows, g.cache, g.kv_scale, mode, g.block_table, g.seq_lens)
            if ms > 1:
                mla.mla_decode_combine(kw["o_partial"], kw["lse_partial"], g.seq_lens, w.max_blocks, pps, o, l)
            torch.cuda.synchronize()
            outs.append((bf16_tensor_to_f64(o), l.cpu().double().numpy(), g.cache.cpu().numpy(),
                         g.kv_scale.cpu().numpy()))
        oa, la, ca, sa = outs[0]
        for path, (ob, lb, cb, sb) in zip(("stored", "unstored"), outs[1:]):
            tag = f"{mode} {path} pps={pps} splits={ms}"
            assert np.array_equal(ca, cb), f"{tag}: cache differs at {np.argwhere(ca != cb)[:5]}"
            assert np.array_equal(sa, sb), f"{tag}: scales differ"
            assert np.array_equal(oa, ob) and np.array_equal(la, lb), f"{tag}: outputs differ"
        compare(oa, la, ref_o, ref_l, tag=f"long append {mode} pps={pps} splits={ms}")


def test_one_visible_token_returns_its_value():
    """L = 1: the only weight is 1, so out is the (dequantised) row itself."""
    for dtype, mode in (("fp8", "tensor"), ("fp8", "token"), ("bf16", "none")):
        w = synth.custom("one", B=2, n_q=1, H=64, context_lens=(0, 0), cache_dtype=dtype,
                         scale_mode=mode, append=1, seed=5)
        if dtype == "bf16":
            w = synth.custom("one", B=2, n_q=1, H=64, context_lens=(1, 1), cache_dtype=dtype, seed=5)
        g = GpuState(w)
        out, lse = g.step()
        cache, scales, ts = oracle_state(w)
        for b in range(w.B):
            K = omla.request_rows(cache, scales, w.block_table, b, 1, w.cache_dtype, w.scale_mode, ts)
            want = np.broadcast_to(K[0, :512], (64, 512))
            if w.scale_mode == "token":
                # the row's scale rides on its weight 2^0 = 1 as a bf16 (relative
                # error <= 2^-8), then the output is rounded to bf16 (<= 2^-8)
                assert np.all(np.abs(out[b, 0] - want) <= np.abs(want) * 2.0 ** -7 * (1 + 2.0 ** -8))
            else:
                assert np.max(np.abs(out[b, 0] - want)) <= np.max(np.abs(want)) * 2.0 ** -8
            if w.scale_mode != "token":
                # bf16(v * s) with s = 1 or exactly representable products: exact
                assert np.array_equal(out[b, 0], np.asarray(
                    bf16_tensor_to_f64(torch.tensor(want, dtype=torch.float32).to(torch.bfloat16))))
        ref_o, ref_l = oracle_decode(w)
        compare(out, lse, ref_o, ref_l, tag=f"one-token {dtype}/{mode}")


def test_constant_column_gives_exactly_one():
    """Value column 0 equal to 1 on every token: out[..., 0] is the sum of the
    softmax weights, 1 exactly after bf16 rounding."""
    for dtype in ("fp8", "bf16"):
        w = synth.custom("ones", B=2, n_q=2, H=64, context_lens=(3000, 70), cache_dtype=dtype,
                         scale_mode="tensor" if dtype == "fp8" else "none", seed=6)
        g = GpuState(w)
        col = g.cache.view(torch.uint8 if dtype == "fp8" else torch.int16)
        if dtype == "fp8":
            g.kv_scale.fill_(1.0)
            col[:, :, 0] = 0x38  # 1.0
            g.new_rows = None  # keep the cache as written
        else:
            col[:, :, 0] = 0x3F80  # 1.0 in bf16
        o, l = g.decode_only(*_plan(w))
        assert np.all(o[..., 0] == 1.0), np.unique(o[..., 0])


def _plan(w):
    import long_context_mla_amd as mla

    return mla.mla_decode_plan(w.B, w.n_q, w.H, int(w.seq_lens.max()), w.total_tokens(), cache_dtype=w.cache_dtype)


def test_page_permutation_and_determinism_bitwise():
    a = synth.custom("perm", B=2, n_q=1, H=64, context_lens=(1111, 400), cache_dtype="fp8",
                     scale_mode="token", seed=7, permute=False)
    b = synth.custom("perm", B=2, n_q=1, H=64, context_lens=(1111, 400), cache_dtype="fp8",
                     scale_mode="token", seed=7, permute=True)
    # same logical rows: rebuild b's pool so that its physical pages hold a's rows
    ga = GpuState(a)
    gb = GpuState(b)
    for req in range(a.B):
        pa, pb = a.pages_of(req), b.pages_of(req)
        gb.cache[torch.from_numpy(pb.astype(np.int64)).cuda()] = ga.cache[torch.from_numpy(pa.astype(np.int64)).cuda()]
        gb.kv_scale[torch.from_numpy(pb.astype(np.int64)).cuda()] = ga.kv_scale[torch.from_numpy(pa.astype(np.int64)).cuda()]
    ga.new_rows = gb.new_rows = None
    plan = _plan(a)
    oa, la = ga.decode_only(*plan)
    ob, lb = gb.decode_only(*plan)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)
    for _ in range(3):
        o2, l2 = ga.decode_only(*plan)
        assert np.array_equal(oa, o2) and np.array_equal(la, l2)


def test_fp8_equals_bf16_on_the_e4m3_grid():
    """Cache values exactly representable in e4m3 with scale 1: the FP8 path and
    the BF16 path see identical numbers.  The two kernels feed the tokens to the
    matrix core in different orders (pages against half-page units, other k
    orders), so fp32 rounding may differ; a wrong decode of any code would
    not stay inside these bounds (the codes span the whole e4m3 range, so the
    softmax is peaked and each output row is dominated by a few decoded rows)."""
    w8 = synth.custom("grid", B=2, n_q=2, H=64, context_lens=(900, 130), cache_dtype="fp8",
                      scale_mode="tensor", seed=8, append=0)
    g8 = GpuState(w8)
    g8.kv_scale.fill_(1.0)
    codes = torch.randint(0, 256, g8.cache.shape, generator=torch.Generator().manual_seed(1),
                          dtype=torch.int32).to(torch.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38  # no NaN codes
    g8.cache.copy_(codes.cuda())
    bf = codes.view(torch.float8_e4m3fn).to(torch.bfloat16)  # exact
    wb = synth.custom("grid", B=2, n_q=2, H=64, context_lens=(900, 130), cache_dtype="bf16", seed=8)
    gb = GpuState(wb)
    gb.cache.copy_(bf.cuda())
    gb.block_table.copy_(g8.block_table)
    gb.q.copy_(g8.q)
    plan = _plan(w8)
    o8, l8 = g8.decode_only(*plan)
    ob, lb = gb.decode_only(*plan)
    scale = max(1.0, float(np.abs(ob).max()))
    err = float(np.abs(o8 - ob).max())
    lerr = float(np.abs(l8 - lb).max())
    log(f"fp8 vs bf16 on the e4m3 grid: max |out| diff {err:.3e} (max |out| {scale:.3e}), lse diff {lerr:.3e}")
    assert err <= 2.0 ** -7 * scale
    assert lerr <= 1e-5 * max(1.0, float(np.abs(lb).max()))


def test_needles_peaked_softmax():
    """Keys planted along the query: one token dominates a head, |out| ~ O(1)."""
    needles = [(0, 777, 3, 0.3), (0, 1500, 17, 0.25), (1, 10, 0, 0.35), (1, 2999, 63, 0.2)]
    w = synth.custom("needle", B=2, n_q=1, H=64, context_lens=(2000, 3000), cache_dtype="fp8",
                     scale_mode="token", seed=9, needles=needles)
    g = GpuState(w)
    ref_o, ref_l = oracle_decode(w)
    out, lse = g.step()
    summ = compare(out, lse, ref_o, ref_l, tag="needles")
    assert summ["max_ref"] > 0.3


def test_combine_matches_oracle_merge():
    """The merge kernel alone on seeded synthetic partials (some splits empty)."""
    import long_context_mla_amd as mla

    rng = np.random.default_rng(10)
    B, n_q, H, max_splits, pps, max_blocks = 3, 2, 16, 6, 2, 12
    seq = np.array([700, 64, 1], np.int32)  # 11, 1 and 1 pages -> 6, 1, 1 splits
    o_bits = synth.bf16_bits(rng.standard_normal((B, max_splits, n_q, H, 512)).astype(np.float32))
    o = (o_bits.astype(np.uint32) << 16).view(np.float32)  # the bf16 partials, exactly
    ls = rng.uniform(-20, 20, (B, max_splits, n_q, H)).astype(np.float32)
    ls[0, 2, 0, :5] = -np.inf
    ls[1, 0, 1, 3] = -np.inf  # a row with no visible token at all
    d = torch.device("cuda:0")
    out = torch.empty((B, n_q, H, 512), dtype=torch.bfloat16, device=d)
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device=d)
    o_dev = torch.from_numpy(o_bits.view(np.int16)).view(torch.bfloat16).to(d)
    mla.mla_decode_combine(o_dev, torch.from_numpy(ls).to(d),
                           torch.from_numpy(seq).to(d), max_blocks, pps, out, lse)
    torch.cuda.synchronize()
    got_o, got_l = bf16_tensor_to_f64(out), lse.cpu().double().numpy()
    for b in range(B):
        npg = -(-int(seq[b]) // 64)
        nb = min(max_splits, -(-npg // pps))
        ro, rl = omla.merge_ref(o[b, :nb], ls[b, :nb])
        assert np.max(np.abs(got_o[b] - ro)) <= 2.0 ** -8 * max(1.0, np.abs(ro).max())
        fin = np.isfinite(rl)
        assert np.array_equal(fin, np.isfinite(got_l[b]))
        assert np.max(np.abs(got_l[b][fin] - rl[fin])) <= 1e-5 * 40


@pytest.mark.parametrize("scale_mode", ["token", "tensor"])
def test_long_split_repeatable(scale_mode):
    """One request of 188 pages decoded as one split and as two (both cross the
    64-page boundaries of the page-id reads): three runs of each plan are
    bitwise identical and match the oracle.  A page read before its copy has
    landed shows up here as run-to-run differences."""
    w = synth.custom(f"long_split_{scale_mode}", B=1, n_q=1, H=64, context_lens=(12000,),
                     cache_dtype="fp8", scale_mode=scale_mode, seed=5)
    g = GpuState(w)
    ref_o, ref_l = oracle_decode(w)
    g.step()  # appends the new row
    npg = int(-(-w.seq_lens.max() // 64))
    for pps, ms in [(npg, 1), (100, 2)]:
        runs = [g.decode_only(pps, ms) for _ in range(3)]
        for o, l in runs[1:]:
            assert np.array_equal(o, runs[0][0]) and np.array_equal(l, runs[0][1]), f"pps={pps}"
        compare(runs[0][0], runs[0][1], ref_o, ref_l, tag=f"long split pps={pps} splits={ms}")


@pytest.mark.parametrize("cache_dtype", ["fp8", "bf16"])
def test_restart_on_late_large_scores(cache_dtype):
    """A key planted along its head's query (logit about 60 log2-units per unit of
    gain) in a page after the split's first one pushes a weight past 2^64 of the
    first-page reference: the split restarts with a raised reference.  Two heads
    with needles in different late pages restart a split twice; on FP8 one
    needle sits in the row appended by the same launch."""
    needles = [(0, 700, 3, 1.5), (0, 2100, 17, 1.5), (1, 1234, 40, 1.4)]
    kw = dict(scale_mode="token", append=1) if cache_dtype == "fp8" else {}
    lens = (3000, 1900)
    if cache_dtype == "fp8":
        needles.append((1, 1900, 9, 1.5))  # the appended row (positions are counted from 0)
    w = synth.custom(f"restart_{cache_dtype}", B=2, n_q=1, H=64, context_lens=lens,
                     cache_dtype=cache_dtype, seed=12, needles=tuple(needles), **kw)
    log(f"restart {cache_dtype}: L={w.seq_lens.tolist()}")
    g = GpuState(w)
    ref_o, ref_l = oracle_decode(w)
    out, lse = g.step()
    summ = compare(out, lse, ref_o, ref_l, tag=f"restart {cache_dtype} planned")
    assert summ["max_ref"] > 1.0  # the needles dominate their heads
    npg = int(-(-w.seq_lens.max() // 64))
    for pps, ms in [(npg, 1), (20, -(-npg // 20)), (1, npg)]:
        o, l = g.decode_only(pps, ms)
        compare(o, l, ref_o, ref_l, tag=f"restart {cache_dtype} pps={pps} splits={ms}")


@pytest.mark.parametrize("cache_dtype", ["fp8", "bf16"])
def test_five_score_jumps_in_one_split(cache_dtype):
    """Five keys along one head's query, in five later pages of one split, the
    first about 77 log2-units above the first page's maximum and each next one 80
    above the one before (so each would push a weight past 2^64 of the reference
    in force when it is met).  The FP8 kernel switches
    to a scan at the first and reruns once with the split's true maxima; the BF16
    kernel restarts four times and takes the fifth jump with weights near 2^80,
    still finite.  Both match the oracle.  q is N(0, 6) so that the jumps need
    only small keys (the winning value row stays near N(0, 1))."""
    lens = (2000,)
    per_gain = 0.072168784 * 36.0 * 576 / np.log(2.0)  # log2-units of score per unit of gain
    gains = [(20.0 + 80.0 * k) / per_gain for k in range(1, 6)]  # 100, 180, ..., 420 log2-units
    needles = tuple((0, t, 5, g) for t, g in zip((100, 500, 900, 1300, 1700), gains))
    kw = dict(scale_mode="token", append=1) if cache_dtype == "fp8" else {}
    w = synth.custom(f"jumps5_{cache_dtype}", B=1, n_q=1, H=64, context_lens=lens, cache_dtype=cache_dtype,
                     seed=13, sigma_q=6.0, needles=needles, **kw)
    g = GpuState(w)
    ref_o, ref_l = oracle_decode(w)
    out, lse = g.step()
    summ = compare(out, lse, ref_o, ref_l, tag=f"five jumps {cache_dtype} planned")
    assert summ["max_ref"] > 1.0  # the last needle owns head 5
    npg = int(-(-w.seq_lens.max() // 64))
    for pps, ms in [(npg, 1), (16, 2)]:
        o, l = g.decode_only(pps, ms)
        compare(o, l, ref_o, ref_l, tag=f"five jumps {cache_dtype} pps={pps} splits={ms}")


def _random_case(rng, i):
    """A seeded random configuration: batch, query tokens, heads, lengths (page
    boundaries, empty requests and sub-page tails included), cache kind, scale
    mode, appended rows and split plan."""
    dtype = ["fp8", "fp8", "bf16"][i % 3]
    B = int(rng.integers(1, 7))
    n_q = int(rng.choice([1, 1, 2, 3, 4, 7, 16]))
    H = int(rng.choice([1, 8, 16, 40, 64, 128]))
    edge = [0, 1, 63, 64, 65, 127, 128, 129]
    lens = tuple(int(rng.choice(edge)) if rng.random() < 0.35 else int(rng.integers(0, 3000)) for _ in range(B))
    kw = dict(scale_mode=str(rng.choice(["tensor", "token"]))) if dtype == "fp8" else {}
    if dtype == "fp8":
        kw["append"] = int(rng.choice([0, n_q, n_q, 3]))
    w = synth.custom(f"rand{i}", B=B, n_q=n_q, H=H, context_lens=lens, cache_dtype=dtype, seed=100 + i,
                     extra_blocks=int(rng.integers(0, 3)), **kw)
    max_pages = max(int(-(-int(w.seq_lens.max()) // 64)), 1)
    pps = int(rng.integers(1, max_pages + 1))
    return w, pps, -(-max_pages // pps)


@pytest.mark.parametrize("i", range(12))
def test_random_configurations(i):
    """Seeded random shapes against the oracle, with the planner's split plan
    and with a random one (the append stored in the first step)."""
    rng = np.random.default_rng(2024 + i)
    w, pps, ms = _random_case(rng, i)
    log(f"random {i}: {w.cache_dtype} {w.scale_mode} B={w.B} n_q={w.n_q} H={w.H} n_new={w.n_new} "
        f"L={w.seq_lens.tolist()} plan={pps}x{ms}")
    g = GpuState(w)
    ref_o, ref_l = oracle_decode(w)
    out, lse = g.step()
    compare(out, lse, ref_o, ref_l, tag=f"random {i} planned")
    o, l = g.decode_only(pps, ms)
    compare(o, l, ref_o, ref_l, tag=f"random {i} pps={pps} splits={ms}")
