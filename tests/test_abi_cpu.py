"""The C-ABI library on the CPU: it loads, exports every function the header
declares, rejects bad arguments with status codes before any HIP call, and its
split planner covers every page.  No kernel runs here."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    import long_context_mla_amd._lib as L

    return L.LIB


def test_header_declares_the_boundary():
    names = _declared()
    for fn in ("kv_append_fp8", "mla_decode_paged", "mla_decode_combine"):
        assert fn in names


def test_library_exports_every_declared_symbol(lib):
    for fn in _declared():
        assert hasattr(lib, fn), fn
    # and through the dynamic symbol table, with C linkage
    syms = os.popen(f"nm -D --defined-only {lib._name}").read()
    for fn in _declared():
        assert re.search(rf"\bT {fn}$", syms, flags=re.M), fn


def _decode(lib, **kw):
    a = dict(q=1, cache=1, dt=1, scale=1, sm=1, bt=1, sl=1, B=1, n_q=1, H=64, mb=10, np_=10,
             ss=0.07, pps=1, ms=1, op=None, lp=None, out=1, lse=1)
    a.update(kw)
    P = lambda v: None if v is None else ctypes.c_void_p(v)  # noqa: E731
    return lib.mla_decode_paged(P(a["q"]), P(a["cache"]), a["dt"], P(a["scale"]), a["sm"], P(a["bt"]),
                                P(a["sl"]), a["B"], a["n_q"], a["H"], a["mb"], a["np_"], a["ss"],
                                a["pps"], a["ms"], P(a["op"]), P(a["lp"]), P(a["out"]), P(a["lse"]), None)


def test_decode_argument_validation(lib):
    # every case fails on the host before a pointer is touched (they are dummies)
    assert _decode(lib, q=None) == 1
    assert _decode(lib, scale=None) == 1
    assert _decode(lib, out=None) == 1
    assert _decode(lib, ms=4, op=None, lp=None) == 1
    assert _decode(lib, H=0) == 2
    assert _decode(lib, H=129) == 2
    assert _decode(lib, n_q=2049) == 2
    assert _decode(lib, n_q=0) == 2
    assert _decode(lib, pps=0) == 2
    assert _decode(lib, ms=0) == 2
    assert _decode(lib, mb=0) == 2
    assert _decode(lib, np_=0) == 2
    assert _decode(lib, B=-1) == 2
    assert _decode(lib, ss=float("nan")) == 2
    assert _decode(lib, dt=7) == 3
    assert _decode(lib, sm=5) == 3
    assert _decode(lib, dt=0, sm=1) == 3  # bf16 cache takes no scale
    assert _decode(lib, pps=2**16, ms=2**15, op=1, lp=1) == 2  # split starts would pass 2^31
    assert _decode(lib, pps=2**16 - 1, ms=2**15, op=1, lp=1, B=0) == 0  # just inside, nothing to do
    assert _decode(lib, B=0) == 0  # empty batch: nothing to do


def test_binding_checks_the_scale_shape():
    # the binding rejects a scale array of the wrong shape before calling the library
    import torch

    import long_context_mla_amd as mla

    q = torch.zeros((1, 1, 64, 576), dtype=torch.bfloat16)
    cache = torch.zeros((4, 64, 576), dtype=torch.uint8)
    bt = torch.zeros((1, 4), dtype=torch.int32)
    sl = torch.ones(1, dtype=torch.int32)
    out = torch.empty((1, 1, 64, 512), dtype=torch.bfloat16)
    lse = torch.empty((1, 1, 64), dtype=torch.float32)
    for mode, scale in (("token", torch.ones((3, 64))), ("token", torch.ones(256)), ("tensor", torch.ones(2))):
        with pytest.raises(ValueError, match="kv_scale"):
            mla.mla_decode_paged(q, cache, scale, mode, bt, sl, 0.07, 4, 1, out=out, lse=lse)
    assert mla.mla_decode_paged_append_noalloc is not None
    with pytest.raises(ValueError, match="kv_scale"):
        mla.mla_decode_paged_append_noalloc(torch.zeros((1, 1, 576), dtype=torch.bfloat16), q, cache,
                                            torch.ones((4, 63)), "token", bt, sl, 0.07, 4, 1, out, lse)


def test_binding_checks_alignment():
    # q, the cache, the new rows, the partials and the output move in 16-byte pieces
    import torch

    import long_context_mla_amd as mla

    q = torch.zeros(64 * 576 + 8, dtype=torch.bfloat16)[1:1 + 64 * 576].view(1, 1, 64, 576)
    cache = torch.zeros((4, 64, 576), dtype=torch.uint8)
    bt = torch.zeros((1, 4), dtype=torch.int32)
    sl = torch.ones(1, dtype=torch.int32)
    out = torch.empty((1, 1, 64, 512), dtype=torch.bfloat16)
    lse = torch.empty((1, 1, 64), dtype=torch.float32)
    with pytest.raises(ValueError, match="16-byte aligned"):
        mla.mla_decode_paged(q, cache, torch.ones(1), "tensor", bt, sl, 0.07, 4, 1, out=out, lse=lse)


def test_item_order_is_a_balanced_bijection():
    """The decode item order (written out as the model above) covers every
    workgroup once, keeps eight consecutive items on one XCD, and spreads the
    requests of the 64-request pool over the XCDs within a few per cent."""
    import numpy as np

    lens = _lens("lognormal64")
    pages = [-(-int(L) // 64) for L in lens]
    for B, S, n in [(64, 40, 1), (32, 43, 1), (16, 4, 4), (1, 224, 1), (1, 1, 1024), (3, 5, 2)]:
        grid = (B * S + 7) // 8 * 8 * n
        full = grid // 64 * 64 if (B > 1 or n > 1) else 0
        items = [(i // 64) * 64 + ((i % 8 - i // 64) % 8) * 8 + (i // 8) % 8 if i < full else i
                 for i in range(grid)]
        assert sorted(items) == list(range(grid))
        for i in range(full):
            assert items[i] // 8 == items[i - i % 64 + (i % 8)] // 8  # same XCD, same chunk
    B, S, pps = 64, 40, 30
    load = np.zeros(8)
    for i in range(B * S):
        v = (i // 64) * 64 + ((i % 8 - i // 64) % 8) * 8 + (i // 8) % 8
        s, b = divmod(v, B)
        load[i % 8] += max(0, min(pages[b], (s + 1) * pps) - s * pps)
    assert load.max() / load.mean() < 1.1


def test_combine_rejects_split_overflow(lib):
    P = ctypes.c_void_p
    assert lib.mla_decode_combine(P(1), P(1), P(1), 1, 1, 1, 1, 2**16, 2**15, P(1), P(1), None, None) == 2


def test_append_and_combine_validation(lib):
    P = ctypes.c_void_p
    assert lib.kv_append_fp8(P(1), P(1), P(1), 0, P(1), P(1), 1, 1, 1, 1, None) == 3
    assert lib.kv_append_fp8(None, P(1), P(1), 2, P(1), P(1), 1, 1, 1, 1, None) == 1
    assert lib.kv_append_fp8(P(1), P(1), P(1), 2, P(1), P(1), -1, 1, 1, 1, None) == 2
    assert lib.kv_append_fp8(None, None, None, 2, None, None, 0, 4, 1, 1, None) == 0
    assert lib.mla_decode_combine(None, P(1), P(1), 1, 1, 1, 1, 1, 2, P(1), P(1), None, None) == 1
    assert lib.mla_decode_combine(P(1), P(1), P(1), 1, 1, 1, 1, 0, 2, P(1), P(1), None, None) == 2
    assert lib.mla_decode_combine(P(1), P(1), P(1), 1, 2049, 1, 1, 1, 2, P(1), P(1), None, None) == 2
    assert lib.mla_status_string(3) == b"unsupported configuration"


def test_page_check_validation(lib):
    P = ctypes.c_void_p
    ok = dict(tags=1, np_=10, bt=1, ep=None, et=1, sl=1, B=2, mb=4, st=1, cl=1)

    def call(**kw):
        a = dict(ok, **kw)
        Q = lambda v: None if v is None else P(v)  # noqa: E731
        return lib.kv_check_pages(Q(a["tags"]), a["np_"], Q(a["bt"]), Q(a["ep"]), Q(a["et"]), Q(a["sl"]),
                                  a["B"], a["mb"], Q(a["st"]), Q(a["cl"]), None)

    assert call(tags=None) == 1
    assert call(et=None) == 1
    assert call(st=None) == 1
    assert call(cl=None) == 1
    assert call(B=-1) == 2
    assert call(np_=0) == 2
    assert call(mb=0) == 2
    assert call(mb=2**25) == 2  # 64 * max_blocks must fit an int32
    assert call(B=0, tags=None, bt=None, et=None, sl=None, st=None, cl=None) == 0


def test_checked_decode_validation(lib):
    P = ctypes.c_void_p

    def call(ms=4, tags=1, et=1, st=1, sm=2, B=1):
        Q = lambda v: None if v is None else P(v)  # noqa: E731
        return lib.mla_decode_paged_append_checked(P(1), 1, P(1), P(1), P(1), sm, P(1), P(1), B, 1, 64, 10, 10,
                                                   0.07, 1, ms, P(1), P(1), Q(tags), None, Q(et), Q(st), None)

    assert call(ms=1) == 3  # the flagged rows are masked by the combine: splits required
    assert call(sm=0) == 3
    assert call(tags=None) == 1
    assert call(et=None) == 1
    assert call(st=None) == 1
    assert call(B=0, tags=None, et=None, st=None) == 0


def test_noalloc_decode_validation(lib):
    # the allocation-free call checks its arguments, the scratch limit included,
    # before any HIP call (the pointers are dummies)
    P = ctypes.c_void_p

    def call(ms=4, sm=2, B=1, n_q=1, H=64, n_new=1, kv_new=1, out=1, lse=1):
        Q = lambda v: None if v is None else P(v)  # noqa: E731
        return lib.mla_decode_paged_append_noalloc(Q(kv_new), n_new, P(1), P(1), P(1), sm, P(1), P(1), B, n_q, H,
                                                   10, 10, 0.07, 1, ms, Q(out), Q(lse), 1, None)

    rows = 32768
    assert call(ms=rows // 64 + 1) == 5          # 64 rows x 513 splits > 32768 partial rows
    assert call(ms=rows // 256 + 1, n_q=4) == 5  # 4 queries x 64 heads x 129 splits
    assert call(ms=rows // 32 + 1, H=16, n_q=2) == 5
    assert call(out=None) == 1
    assert call(lse=None, ms=1) == 1
    assert call(kv_new=None) == 1
    assert call(n_new=-1) == 2
    assert call(sm=0) == 3
    assert call(H=129) == 2
    assert call(B=0, kv_new=None, out=None, lse=None) == 0
    assert lib.mla_status_string(5).startswith(b"split partials exceed")


# query rows per decode workgroup: 64 on an FP8 cache, 32 on a BF16 cache
ROWS = {"fp8": 64, "bf16": 64}


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
@pytest.mark.parametrize("B,n_q,H,maxL,total,cus", [
    (1, 1, 64, 100_001, 100_001, 256),
    (32, 1, 64, 137_661, 3_269_170, 256),
    (64, 1, 64, 74_893, 1_370_066, 256),
    (16, 4, 64, 142_004, 16 * 142_004, 256),
    (2, 1, 16, 1000, 1777, 0),
    (3, 2, 16, 1, 3, 80),
    (1, 1, 64, 0, 0, 256),
])
def test_plan_covers_every_page(B, n_q, H, maxL, total, cus, dtype):
    import long_context_mla_amd as m

    pps, ms = m.mla_decode_plan(B, n_q, H, maxL, total, cus, dtype)
    pages = -(-maxL // 64)
    assert pps >= 1 and ms >= 1
    assert pps * ms >= pages
    assert pps * (ms - 1) < max(pages, 1)  # no split past the longest request
    if pages:
        # about one workgroup (a group of query rows, pages_per_split pages) per CU
        rows_groups = -(-(n_q * H) // ROWS[dtype])
        total_pages = -(-total // 64) + B
        assert pps <= max(1, -(-(total_pages * rows_groups) // (cus or 256)))


def test_plan_rejects_bad_input():
    import long_context_mla_amd as m

    with pytest.raises(m.MlaError):
        m.mla_decode_plan(1, 0, 64, 10, 10)
    with pytest.raises(m.MlaError):
        m.mla_decode_plan(1, 1, 64, -1, 10)
    with pytest.raises(m.MlaError):
        m.mla_decode_plan(1, 1, 64, 10, 10, 0, 7)  # no such cache dtype


def _model_makespan(lens, n_q, H, pps, cus, fixed=2, rows=64):
    """The planner's duration model written out: workgroup i in 1-D launch order
    on the first free compute unit of XCD i % 8, costing a fixed start plus its
    pages, working on item v = (split * B + b) * n_rg + rg: inside full block k
    of 64 workgroups (unless the batch is one request of one row group), XCD x
    takes the block's eight items of chunk (x - k) mod 8 in order; i itself
    otherwise."""
    import heapq

    pages = [-(-int(L) // 64) for L in lens]
    ms = -(-max(pages) // pps)
    n_rg = -(-(n_q * H) // rows)
    B = len(lens)
    grid = (B * ms + 7) // 8 * 8 * n_rg
    pools = [[0] * max(1, cus // 8) for _ in range(8)]
    end = 0
    full = grid // 64 * 64 if (B > 1 or n_rg > 1) else 0
    for i in range(grid):
        v = (i // 64) * 64 + ((i % 8 - i // 64) % 8) * 8 + (i // 8) % 8 if i < full else i
        u = v // n_rg
        if u >= B * ms:
            continue
        s, b = divmod(u, B)
        n = min(pages[b], s * pps + pps) - s * pps
        if n <= 0 and s != 0:
            continue
        t = heapq.heappop(pools[i & 7]) + fixed + max(n, 0)
        heapq.heappush(pools[i & 7], t)
        end = max(end, t)
    return end


def _lens(kind):
    import numpy as np

    rng = np.random.default_rng(4)
    if kind == "single":
        return [100_001]
    if kind == "uniform32":
        return list(rng.integers(60_000, 140_000, 32))
    if kind == "lognormal64":
        x = np.clip(np.exp(rng.normal(np.log(16_000), 0.8, 64)), 1000, 128_000)
        return list((x * 1.37e6 / x.sum()).astype(int))
    if kind == "spec16":
        return [142_004] * 16
    if kind == "tiny":
        return [0, 1, 63, 64, 65]
    return [0, 0]


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
@pytest.mark.parametrize("kind,n_q,H,cus", [
    ("single", 1, 64, 256), ("uniform32", 1, 64, 256), ("lognormal64", 1, 64, 256),
    ("spec16", 4, 64, 256), ("tiny", 2, 16, 80), ("empty", 1, 64, 256), ("lognormal64", 1, 64, 7),
])
def test_plan_lens(kind, n_q, H, cus, dtype):
    """mla_decode_plan_lens covers every page with at most one short split per
    request, fits its workgroups into at most four rounds when the requests
    allow it, and (under its own duration model) never does worse than the
    plan from the longest and summed lengths alone."""
    import long_context_mla_amd as m

    lens = _lens(kind)
    pps, ms = m.mla_decode_plan_lens(lens, n_q, H, cus, dtype)
    pages = [-(-int(L) // 64) for L in lens]
    assert pps >= 1 and ms >= 1
    if max(pages) == 0:
        assert (pps, ms) == (1, 1)
        return
    assert pps * ms >= max(pages) and pps * (ms - 1) < max(pages)
    n_rg = -(-(n_q * H) // ROWS[dtype])
    wgs = sum(max(1, -(-p // pps)) for p in pages) * n_rg
    if len(lens) * n_rg <= 4 * cus:
        assert wgs <= 4 * cus
    old = m.mla_decode_plan(len(lens), n_q, H, max(lens), sum(lens), cus, dtype)[0]
    rows = ROWS[dtype]
    assert _model_makespan(lens, n_q, H, pps, cus, rows=rows) <= _model_makespan(lens, n_q, H, old, cus, rows=rows)


def test_plan_lens_rejects_bad_input():
    import long_context_mla_amd as m

    with pytest.raises(m.MlaError):
        m.mla_decode_plan_lens([10, -1], 1, 64)
    with pytest.raises(m.MlaError):
        m.mla_decode_plan_lens([10], 0, 64)
