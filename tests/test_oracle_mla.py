"""Pins for the attention oracle (CPU only).

Each oracle function is checked against something other than itself:
closed forms (one visible token, equal scores, zero query, a two-token worked
example), invariants (weights sum to one, split/merge identity, physical page
permutation, causal rows), and a pure-Python loop implementation on tiny
inputs.  The mutation tests at the end plant plausible mistakes in the oracle
and check that at least one pin fails for each.
"""

import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import e4m3, mla

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SCALE = synth.SOFTMAX_SCALE


def _bf16(x):
    return synth.bf16_bits(np.asarray(x, dtype=np.float32))


def _paged_bf16(rows_bits, perm=None):
    """Put rows [T, 576] (bf16 bits) into pages; returns cache, block_table [1, n]."""
    T = rows_bits.shape[0]
    n = -(-T // 64)
    pages = np.zeros((n, 64, 576), dtype=np.uint16)
    pages.reshape(n * 64, 576)[:T] = rows_bits
    order = np.arange(n) if perm is None else np.asarray(perm)
    cache = np.zeros_like(pages)
    cache[order] = pages
    return cache, order[None, :].astype(np.int32)


# ----------------------------------------------------------------- closed forms
def check_one_token(decode=None):
    decode = decode or mla.decode_ref
    rng = np.random.default_rng(1)
    row = _bf16(rng.standard_normal((1, 576)))
    q = _bf16(rng.standard_normal((1, 1, 4, 576)))
    cache, bt = _paged_bf16(row)
    out, lse = decode(q, cache, None, bt, np.array([1], np.int32), n_q=1, H=4,
                      cache_dtype="bf16", scale_mode="none", softmax_scale=SCALE)
    V = mla.bf16_to_f64(row[0])
    assert np.array_equal(out[0, 0], np.broadcast_to(V[:512], (4, 512)))
    s = SCALE * (mla.bf16_to_f64(q[0, 0]) @ V)
    assert np.allclose(lse[0, 0], s, rtol=0, atol=1e-12)


def test_one_token_context():
    check_one_token()


def check_equal_scores(decode=None):
    """q's latent part zero and every token's rope part equal: all scores equal,
    so out = mean of the values and lse = s + ln T."""
    decode = decode or mla.decode_ref
    rng = np.random.default_rng(2)
    T, H = 150, 3
    rows = rng.standard_normal((T, 576)).astype(np.float32)
    rows[:, 512:] = rng.standard_normal(64).astype(np.float32)
    rows_b = _bf16(rows)
    q = rng.standard_normal((1, 1, H, 576)).astype(np.float32)
    q[..., :512] = 0
    qb = _bf16(q)
    cache, bt = _paged_bf16(rows_b, perm=[2, 0, 1])
    out, lse = decode(qb, cache, None, bt, np.array([T], np.int32), n_q=1, H=H,
                      cache_dtype="bf16", scale_mode="none", softmax_scale=SCALE)
    V = mla.bf16_to_f64(rows_b)
    mean = V[:, :512].mean(axis=0)
    for h in range(H):
        assert np.allclose(out[0, 0, h], mean, rtol=1e-12, atol=1e-13)
        s = SCALE * float(mla.bf16_to_f64(qb[0, 0, h]) @ V[0])
        assert abs(lse[0, 0, h] - (s + math.log(T))) < 1e-11


def test_equal_scores_give_mean_of_values():
    check_equal_scores()


def test_zero_query_lse_is_log_count():
    rng = np.random.default_rng(3)
    T = 97
    rows = _bf16(rng.standard_normal((T, 576)))
    cache, bt = _paged_bf16(rows)
    q = np.zeros((1, 1, 2, 576), np.uint16)
    out, lse = mla.decode_ref(q, cache, None, bt, np.array([T], np.int32), n_q=1, H=2,
                              cache_dtype="bf16", scale_mode="none", softmax_scale=SCALE)
    assert np.allclose(lse, math.log(T), rtol=0, atol=1e-13)
    assert np.allclose(out[0, 0, 0], mla.bf16_to_f64(rows)[:, :512].mean(0), atol=1e-13)


def check_weights_sum_to_one(decode=None):
    """With value column 0 equal to 1 on every token, out[..., 0] = sum of weights = 1."""
    decode = decode or mla.decode_ref
    rng = np.random.default_rng(4)
    T = 200
    rows = rng.standard_normal((T, 576)).astype(np.float32) * 2
    rows[:, 0] = 1.0
    rows_b = _bf16(rows)
    cache, bt = _paged_bf16(rows_b)
    q = _bf16(rng.standard_normal((1, 2, 5, 576)) * 3)
    out, lse = decode(q, cache, None, bt, np.array([T], np.int32), n_q=2, H=5,
                      cache_dtype="bf16", scale_mode="none", softmax_scale=SCALE)
    assert np.allclose(out[..., 0], 1.0, rtol=0, atol=1e-12)


def test_weights_sum_to_one():
    check_weights_sum_to_one()


def test_two_token_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "two_token_softmax.json")))
    a = g["q_scale_a"]
    # scores 0 and ln 3 with softmax_scale 1: q = a*e_0, K_0[0] = 0, K_1[0] = ln3/a
    Q = np.zeros((1, 576))
    Q[0, 0] = a
    K = np.zeros((2, 576))
    K[1, 0] = math.log(3.0) / a
    rng = np.random.default_rng(5)
    K[:, 1:512] = rng.standard_normal((2, 511))
    out, lse = mla.attend(Q, K, np.array([2]), 1.0)
    w = np.array(g["weights"])
    assert abs(lse[0] - g["lse"]) < 1e-15
    assert np.allclose(out[0], w @ K[:, :512], rtol=0, atol=1e-15)


# ----------------------------------------------------------------- brute force
def _naive_from_workload(w, q_bits, cache, scales, tensor_scale, b):
    """Gather rows with plain loops and the scalar closed-form decoder, then run
    the loop implementation."""
    L = int(w.seq_lens[b])
    k_rows = []
    for t in range(L):
        page = int(w.block_table[b][t // 64])
        slot = t % 64
        if w.cache_dtype == "bf16":
            k_rows.append([float(v) for v in mla.bf16_to_f64(cache[page, slot])])
        else:
            s = 1.0
            if w.scale_mode == "token":
                s = float(scales[page, slot])
            elif w.scale_mode == "tensor":
                s = float(tensor_scale)
            k_rows.append([e4m3.decode_value(int(c)) * s for c in cache[page, slot]])
    q_rows, vis = [], []
    for i in range(w.n_q):
        for h in range(w.H):
            q_rows.append([float(v) for v in mla.bf16_to_f64(q_bits[b, i, h])])
            vis.append(L - w.n_q + i + 1)
    return mla.decode_naive(q_rows, k_rows, w.softmax_scale, vis)


def _oracle_cache(w):
    """Oracle-side cache for a synthetic workload: quantise the pool, then append."""
    bits = w.all_page_bits()
    ts = w.tensor_scale() if w.scale_mode == "tensor" else None
    if w.cache_dtype == "bf16":
        return bits, None, None
    codes, sc = mla.fill_pages_ref(bits, w.scale_mode, ts)
    if w.n_new:
        mla.append_ref(w.new_row_bits(), codes, sc, w.block_table, w.seq_lens, w.scale_mode, ts)
    return codes, sc, ts


TINY = [
    dict(B=2, n_q=1, H=3, context_lens=(70, 130), cache_dtype="fp8", scale_mode="token"),
    dict(B=2, n_q=3, H=2, context_lens=(61, 1), cache_dtype="fp8", scale_mode="tensor"),
    dict(B=1, n_q=2, H=2, context_lens=(128,), cache_dtype="bf16"),
    dict(B=2, n_q=4, H=2, context_lens=(0, 63), cache_dtype="fp8", scale_mode="token"),
]


@pytest.mark.parametrize("cfg", TINY)
def test_vectorised_matches_loops(cfg):
    w = synth.custom("tiny", seed=11, **cfg)
    codes, sc, ts = _oracle_cache(w)
    q = w.q_bits()
    out, lse = mla.decode_ref(q, codes, sc, w.block_table, w.seq_lens, n_q=w.n_q, H=w.H,
                              cache_dtype=w.cache_dtype, scale_mode=w.scale_mode,
                              softmax_scale=w.softmax_scale, tensor_scale=ts)
    for b in range(w.B):
        o_n, l_n = _naive_from_workload(w, q, codes, sc, ts, b)
        o_n = np.array(o_n).reshape(w.n_q, w.H, 512)
        l_n = np.array(l_n).reshape(w.n_q, w.H)
        assert np.allclose(out[b], o_n, rtol=1e-12, atol=1e-14)
        assert np.allclose(lse[b], l_n, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------- invariants
def check_split_merge(attend=None, merge=None):
    attend = attend or mla.attend
    merge = merge or mla.merge_ref
    rng = np.random.default_rng(6)
    T, R = 333, 6
    Q = rng.standard_normal((R, 576))
    K = rng.standard_normal((T, 576)) * 0.5
    vis = np.array([333, 300, 64, 65, 1, 200])
    full_o, full_l = attend(Q, K, vis, SCALE)
    for trial in range(5):
        cuts = np.sort(rng.choice(np.arange(1, T), size=trial + 1, replace=False))
        bounds = [0, *cuts.tolist(), T]
        parts = [mla.partial_ref(Q, K, vis, SCALE, a, b) for a, b in zip(bounds[:-1], bounds[1:])]
        o = np.stack([p[0] for p in parts])
        l = np.stack([p[1] for p in parts])
        mo, ml = merge(o, l)
        assert np.allclose(mo, full_o, rtol=1e-11, atol=1e-13)
        assert np.allclose(ml, full_l, rtol=0, atol=1e-12)


def test_split_merge_identity():
    check_split_merge()


def test_merge_of_empty_parts():
    o = np.ones((3, 2, 512))
    l = np.full((3, 2), -np.inf)
    l[1, 1] = 0.7
    mo, ml = mla.merge_ref(o * np.arange(3)[:, None, None], l)
    assert np.all(mo[0] == 0) and ml[0] == -np.inf
    assert np.allclose(mo[1], 1.0) and ml[1] == 0.7


def test_physical_page_permutation_is_invisible():
    rng = np.random.default_rng(8)
    T = 300
    rows = _bf16(rng.standard_normal((T, 576)))
    q = _bf16(rng.standard_normal((1, 1, 4, 576)))
    res = []
    for perm in ([0, 1, 2, 3, 4], [3, 0, 4, 1, 2]):
        cache, bt = _paged_bf16(rows, perm=perm)
        res.append(mla.decode_ref(q, cache, None, bt, np.array([T], np.int32), n_q=1, H=4,
                                  cache_dtype="bf16", scale_mode="none", softmax_scale=SCALE))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])


def check_causal_rows(decode=None):
    """Query i of n_q sees exactly what a single query at length L - n_q + i + 1 sees."""
    decode = decode or mla.decode_ref
    rng = np.random.default_rng(9)
    T, n_q, H = 131, 4, 2
    rows = _bf16(rng.standard_normal((T, 576)))
    cache, bt = _paged_bf16(rows)
    q = _bf16(rng.standard_normal((1, n_q, H, 576)))
    out, lse = decode(q, cache, None, bt, np.array([T], np.int32), n_q=n_q, H=H,
                      cache_dtype="bf16", scale_mode="none", softmax_scale=SCALE)
    for i in range(n_q):
        o1, l1 = decode(q[:, i:i + 1], cache, None, bt, np.array([T - n_q + i + 1], np.int32),
                        n_q=1, H=H, cache_dtype="bf16", scale_mode="none", softmax_scale=SCALE)
        assert np.array_equal(out[0, i], o1[0, 0]) and np.array_equal(lse[0, i], l1[0, 0])
    # and the queries really differ in what they see
    assert not np.allclose(out[0, 0], mla.decode_ref(q[:, :1], cache, None, bt, np.array([T], np.int32),
                                                     n_q=1, H=H, cache_dtype="bf16", scale_mode="none",
                                                     softmax_scale=SCALE)[0][0, 0])


def test_causal_rows():
    check_causal_rows()


def test_query_subset_is_the_causal_prefix():
    """queries=[...] computes only those queries, each as a single query at
    length L - n_q + i + 1 (the causal definition, pinned above); the others
    stay NaN."""
    rng = np.random.default_rng(19)
    T, n_q, H = 200, 6, 2
    rows = _bf16(rng.standard_normal((T, 576)))
    cache, bt = _paged_bf16(rows)
    q = _bf16(rng.standard_normal((1, n_q, H, 576)))
    sel = [0, 3, 5]
    out, lse = mla.decode_ref(q, cache, None, bt, np.array([T], np.int32), n_q=n_q, H=H,
                              cache_dtype="bf16", scale_mode="none", softmax_scale=SCALE, queries=sel)
    for i in range(n_q):
        if i not in sel:
            assert np.all(np.isnan(lse[0, i]))
            continue
        o1, l1 = mla.decode_ref(q[:, i:i + 1], cache, None, bt, np.array([T - n_q + i + 1], np.int32),
                                n_q=1, H=H, cache_dtype="bf16", scale_mode="none", softmax_scale=SCALE)
        assert np.allclose(out[0, i], o1[0, 0], rtol=1e-13, atol=1e-15)
        assert np.allclose(lse[0, i], l1[0, 0], rtol=1e-13, atol=1e-13)


def test_row_with_nothing_visible():
    rng = np.random.default_rng(10)
    Q = rng.standard_normal((2, 576))
    K = rng.standard_normal((5, 576))
    o, l = mla.attend(Q, K, np.array([0, 5]), SCALE)
    assert np.all(o[0] == 0) and l[0] == -np.inf and np.isfinite(l[1])


# ----------------------------------------------------------------- FP8 append
def test_append_places_rows_and_scales():
    w = synth.custom("app", B=3, n_q=2, H=1, context_lens=(5, 64, 127), cache_dtype="fp8",
                     scale_mode="token", seed=12)
    codes = np.zeros((w.num_pages, 64, 576), np.uint8)
    sc = np.zeros((w.num_pages, 64), np.float32)
    new = w.new_row_bits()
    new[1, 0] = 0  # an all-zero row takes scale 1
    mla.append_ref(new, codes, sc, w.block_table, w.seq_lens, "token")
    touched = np.zeros((w.num_pages, 64), bool)
    for b in range(w.B):
        for j in range(2):
            p = int(w.seq_lens[b]) - 2 + j
            page, slot = int(w.block_table[b, p // 64]), p % 64
            touched[page, slot] = True
            x = mla.bf16_to_f32(new[b, j])
            amax = np.float32(np.abs(x).max())
            want = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(448.0))
            assert sc[page, slot] == want
            deq = e4m3.decode(codes[page, slot]) * float(sc[page, slot])
            err = np.abs(deq - x)
            assert np.all(err <= np.abs(x) * 2.0 ** -4 + float(sc[page, slot]) * 2.0 ** -10)
            if amax > 0:
                assert np.max(np.abs(e4m3.decode(codes[page, slot]))) == 448.0
    assert np.all(codes[~touched] == 0) and np.all(sc[~touched] == 0)


def test_per_tensor_quantisation_saturates():
    x = _bf16(np.array([[1.0] * 575 + [1000.0]]))
    c, s = mla.quantize_rows(x, "tensor", tensor_scale=np.float32(1.0))
    assert c[0, -1] == 0x7E and c[0, 0] == 0x38 and s[0] == 1.0


# ----------------------------------------------------------------- byte sizes
def test_row_sizes_from_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "kv_row_sizes.json")))
    assert synth.D == g["elements_per_row"]
    bf = synth.custom("s", B=1, H=1, context_lens=(10,), cache_dtype="bf16")
    f8 = synth.custom("s", B=1, H=1, context_lens=(10,), cache_dtype="fp8", scale_mode="tensor")
    assert bf.kv_row_bytes() == g["elements_per_row"] * g["bf16_bytes_per_element"]
    assert f8.kv_row_bytes() * 2 == bf.kv_row_bytes()
    # FP8 halves the bytes, so the same memory holds twice the tokens
    assert abs(g["capacity_tokens_fp8"] / g["capacity_tokens_bf16"] - 2.0) < 0.01
    per_token = g["elements_per_row"] * g["bf16_bytes_per_element"] * g["layers"]
    assert abs(per_token / 1000 - g["approx_kb_per_token_all_layers_bf16"]) < 2.5


# ----------------------------------------------------------------- mutations
def _mutant_attend(kind, real):
    def attend(Q, K, visible, softmax_scale):
        Q = np.array(Q, dtype=np.float64)
        K = np.array(K, dtype=np.float64)
        if kind == "drop_rope":
            Q = Q.copy()
            Q[:, 512:] = 0
        if kind == "no_scale":
            softmax_scale = 1.0
        if kind == "value_from_tail":
            K = np.concatenate([K[:, 64:], K[:, :64]], axis=1)
        if kind == "off_by_one":
            visible = np.asarray(visible) - 1
        if kind == "lse_log2":
            o, l = real(Q, K, visible, softmax_scale)
            return o, l / math.log(2)
        return real(Q, K, visible, softmax_scale)
    return attend


@pytest.mark.parametrize("kind", ["drop_rope", "no_scale", "value_from_tail", "off_by_one", "lse_log2"])
def test_pins_catch_planted_mistakes(kind, monkeypatch):
    monkeypatch.setattr(mla, "attend", _mutant_attend(kind, mla.attend))
    caught = 0
    for check in (check_one_token, check_equal_scores, check_weights_sum_to_one, check_causal_rows,
                  lambda: check_split_merge(attend=mla.attend)):
        try:
            check()
        except AssertionError:
            caught += 1
    # the two-token worked example too
    try:
        test_two_token_worked_example()
    except AssertionError:
        caught += 1
    assert caught >= 1, f"no pin caught mutation {kind}"


def test_pins_catch_wrong_page_lookup(monkeypatch):
    def bad_rows(cache, scales, block_table, b, L, cache_dtype, scale_mode, tensor_scale=None):
        n = -(-L // 64)
        raw = cache[:n].reshape(n * 64, 576)[:L]  # ignores the page map
        return mla.bf16_to_f64(raw)
    monkeypatch.setattr(mla, "request_rows", bad_rows)
    with pytest.raises(AssertionError):
        check_equal_scores()
