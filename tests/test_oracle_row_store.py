"""Pins for the oracle's row-store rules (CPU only): where the plain append
(oracle.mla.append_ref) and the decode launch carrying the page check
(oracle.integrity.append_checked_ref) put the step's new rows.

Pinned to a hand-worked case (tests/golden/in_launch_row_store_small.json): a
zero cache receives distinct rows, and exactly the slots the golden names hold
exactly those rows' codes and scales afterwards.  The mutation tests plant
plausible mistakes in the rule and check that the golden catches each."""

import json
import os

import numpy as np
import pytest

from oracle import integrity as oi
from oracle import mla as omla

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "in_launch_row_store_small.json")


def _golden():
    with open(GOLDEN) as f:
        g = json.load(f)
    arr = lambda k, t: np.asarray(g[k], dtype=t)  # noqa: E731
    return g, arr("page_tags", np.uint32), arr("block_table", np.int32), arr("expected_pages", np.int32), \
        arr("expected_tags", np.uint32), arr("seq_lens", np.int32)


def _rows(B, n_new, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, n_new, 576)).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation to bf16 bits is fine for a pin


def _written(g, bt, lens, store):
    """Run ``store(new_bits, cache, scales)`` on a zero cache; return the [B, n_new]
    mask of rows found in their own slot, after checking that nothing else changed."""
    num_pages, n_new = g["num_pages"], g["n_new"]
    B = bt.shape[0]
    new = _rows(B, n_new)
    cache = np.zeros((num_pages, 64, 576), np.uint8)
    scales = np.zeros((num_pages, 64), np.float32)
    store(new, cache, scales)
    codes, sc = omla.quantize_rows(new.reshape(-1, 576), "token")
    codes = codes.reshape(B, n_new, 576)
    sc = sc.reshape(B, n_new)
    found = np.zeros((B, n_new), dtype=int)
    for b in range(B):
        for j in range(n_new):
            p = int(lens[b]) - n_new + j
            if p < 0 or p >= bt.shape[1] * 64:
                continue
            page = int(bt[b, p // 64])
            if 0 <= page < num_pages and np.array_equal(cache[page, p % 64], codes[b, j]):
                assert scales[page, p % 64] == sc[b, j]
                found[b, j] = 1
    n_rows_written = int((cache.reshape(-1, 576) != 0).any(axis=1).sum())
    assert n_rows_written == int(found.sum()), "a row landed outside its own slot"
    assert int((scales != 0).sum()) == int(found.sum())
    return found


def test_plain_append_hand_worked():
    g, tags, bt, ep, et, lens = _golden()
    got = _written(g, bt, lens, lambda new, c, s: omla.append_ref(new, c, s, bt, lens, "token"))
    assert got.tolist() == g["stored_plain"]


def test_in_launch_store_mask_hand_worked():
    g, tags, bt, ep, et, lens = _golden()
    assert oi.stored_rows_ref(tags, bt, et, lens, g["n_new"], ep).astype(int).tolist() == g["stored_in_launch"]
    assert oi.stored_rows_ref(tags, bt, et, lens, g["n_new"], None).astype(int).tolist() == \
        g["stored_in_launch_no_page_record"]


@pytest.mark.parametrize("record", [True, False])
def test_in_launch_store_hand_worked(record):
    g, tags, bt, ep, et, lens = _golden()
    want = g["stored_in_launch" if record else "stored_in_launch_no_page_record"]
    got = _written(g, bt, lens, lambda new, c, s: oi.append_checked_ref(
        new, c, s, bt, lens, "token", None, tags, et, ep if record else None))
    assert got.tolist() == want


def test_in_launch_store_equals_plain_append_when_nothing_is_flagged():
    # a consistent history: every row the plain append stores, the in-launch form stores too
    g, tags, bt, ep, et, lens = _golden()
    ok = np.array([0, 4, 8], dtype=int)  # requests whose pages all pass and lengths fit
    status, _ = oi.check_pages_ref(tags, bt[ok], et[ok], lens[ok], ep[ok])
    assert not status.any()
    want = np.asarray(g["stored_plain"])[ok]
    assert np.array_equal(oi.stored_rows_ref(tags, bt[ok], et[ok], lens[ok], g["n_new"], ep[ok]), want == 1)


# ----------------------------------------------------------------- mutations

def _mutant_mask(kind):
    def stored(page_tags, block_table, expected_tags, seq_lens, n_new, expected_pages=None):
        B, mb = block_table.shape
        keep = np.zeros((B, n_new), dtype=bool)
        for b in range(B):
            L = int(seq_lens[b])
            if kind != "nolen" and (L < 0 or L > (mb * 64 if kind != "cap" else mb * 64 - 1)):
                continue
            for j in range(n_new):
                p = L - n_new + j + (1 if kind == "off1" else 0)
                if p < 0 and kind != "wrap":
                    continue
                k = p // 64
                if k >= mb:
                    continue
                page = int(block_table[b, k])
                if page < 0 or page >= page_tags.shape[0]:
                    continue
                if expected_pages is not None and page != int(expected_pages[b, k]) and kind != "norecord":
                    continue
                if kind != "notag" and int(page_tags[page]) != int(expected_tags[b, k]):
                    continue
                keep[b, j] = True
        return keep
    return stored


@pytest.mark.parametrize("kind", ["nolen", "cap", "off1", "wrap", "norecord", "notag"])
def test_pins_catch_planted_mistakes_in_the_store_rule(kind, monkeypatch):
    monkeypatch.setattr(oi, "stored_rows_ref", _mutant_mask(kind))
    caught = 0
    for pin in (test_in_launch_store_mask_hand_worked,):
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin caught mutation {kind}"


def _mutant_append(kind):
    def append(new_bits, cache, scales, block_table, seq_lens, scale_mode, tensor_scale=None):
        B, n_new = new_bits.shape[:2]
        codes, sc = omla.quantize_rows(new_bits.reshape(B * n_new, 576), scale_mode, tensor_scale)
        codes = codes.reshape(B, n_new, 576)
        sc = sc.reshape(B, n_new)
        cap = block_table.shape[1] * 64
        for b in range(B):
            for j in range(n_new):
                p = int(seq_lens[b]) - n_new + j
                if p < 0 and kind != "neg":
                    continue
                if p >= cap and kind != "cap":
                    continue
                if p >= cap:
                    p = cap - 1  # what a clamp would do
                page = int(block_table[b, p // 64])
                if (page < 0 or page >= cache.shape[0]) and kind != "pool":
                    continue
                cache[page, p % 64] = codes[b, j]
                scales[page, p % 64] = sc[b, j]
    return append


@pytest.mark.parametrize("kind", ["neg", "cap", "pool"])
def test_pins_catch_planted_mistakes_in_the_plain_append(kind, monkeypatch):
    monkeypatch.setattr(omla, "append_ref", _mutant_append(kind))
    with pytest.raises(AssertionError):
        test_plain_append_hand_worked()
