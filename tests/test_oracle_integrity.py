"""Pins for the page-tag check oracle (CPU only).

The oracle is pinned to a hand-worked case (tests/golden/page_tag_check_small.json)
and to allocator histories whose faults are known by construction: a consistent
history passes every request, and each planted fault flags exactly the request
it was planted in, with the bit that names it.  The mutation tests at the end
plant plausible mistakes in the oracle and check that a pin fails for each.
"""

import json
import os

import numpy as np
import pytest

from oracle import integrity as oi
from synth import integrity as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_tag_check_small.json")


def _golden():
    with open(GOLDEN) as f:
        g = json.load(f)
    arr = lambda k, t: np.asarray(g[k], dtype=t)  # noqa: E731
    return g, arr("page_tags", np.uint32), arr("block_table", np.int32), arr("expected_pages", np.int32), \
        arr("expected_tags", np.uint32), arr("seq_lens", np.int32)


def test_hand_worked_case():
    g, tags, bt, ep, et, lens = _golden()
    status, checked = oi.check_pages_ref(tags, bt, et, lens, ep)
    assert status.tolist() == g["status"]
    assert checked.tolist() == g["checked_lens"]


def test_hand_worked_case_without_page_record():
    g, tags, bt, _, et, lens = _golden()
    status, _ = oi.check_pages_ref(tags, bt, et, lens, None)
    assert status.tolist() == g["status_no_page_record"]


def _lens(rng, B, max_blocks):
    # ragged: page boundaries, one past them, short and full requests
    choices = [0, 1, 63, 64, 65, 127, 128, max_blocks * 64 - 1, max_blocks * 64]
    return [int(rng.choice(choices)) if rng.random() < 0.5 else int(rng.integers(0, max_blocks * 64 + 1))
            for _ in range(B)]


@pytest.mark.parametrize("seed", range(6))
def test_consistent_history_passes(seed):
    rng = np.random.default_rng(seed)
    B, mb = 12, 9
    lens = _lens(rng, B, mb)
    c = si.make_case(seed, lens, mb, num_pages=B * mb + 17, churn=20)
    status, checked = oi.check_pages_ref(c.page_tags, c.block_table, c.expected_tags, c.seq_lens,
                                         c.expected_pages)
    assert not status.any()
    assert checked.tolist() == list(c.seq_lens)


_BITS = {"stale": oi.STALE_TAG, "wrong": oi.WRONG_PAGE, "oob": oi.OUT_OF_RANGE, "neg": oi.OUT_OF_RANGE,
         "len": oi.BAD_LEN, "neglen": oi.BAD_LEN}


@pytest.mark.parametrize("kind", sorted(_BITS) + ["tail"])
@pytest.mark.parametrize("where", ["first", "last", "middle"])
def test_planted_fault_flags_exactly_its_request(kind, where):
    B, mb = 6, 8
    lens = [0, 64 * 3 + 1, 64 * 8, 64 * 5, 1, 64 * 2]
    victim = 2 if kind != "tail" else 3
    n = (lens[victim] + 63) // 64
    j = {"first": 0, "last": n - 1, "middle": n // 2}[where]
    if kind == "tail":
        j = {"first": n, "last": mb - 1, "middle": (n + mb) // 2}[where]
    c = si.make_case(100 + sum(map(ord, kind + where)), lens, mb, num_pages=80, faults=[(kind, victim, j)],
                     churn=5)
    status, checked = oi.check_pages_ref(c.page_tags, c.block_table, c.expected_tags, c.seq_lens,
                                         c.expected_pages)
    for b in range(B):
        if b == victim and kind != "tail":
            assert status[b] & _BITS[kind], (kind, status[b])
            if kind in ("len", "neglen"):
                assert status[b] == oi.BAD_LEN
            if kind in ("oob", "neg"):
                assert not status[b] & oi.STALE_TAG  # no tag is looked up outside the pool
            if kind == "stale":
                assert status[b] == oi.STALE_TAG
            assert checked[b] == 0
        else:
            assert status[b] == 0, (kind, where, b, status[b])
            assert checked[b] == c.seq_lens[b]


def test_stale_page_flags_only_the_old_owner():
    """A page reused by a second request: the first request's record is stale,
    the second request (which got the page with its new tag) passes."""
    c = si.make_case(7, [64 * 2, 64 * 2], 2, num_pages=8)
    p = int(c.block_table[0, 1])
    tags = c.page_tags.copy()
    bt = c.block_table.copy()
    et = c.expected_tags.copy()
    ep = c.expected_pages.copy()
    # request 1 gives its page 1 back and receives page p instead (tag changes)
    tags[p] = np.uint32(int(tags[p]) + 1)
    bt[1, 1] = p
    ep[1, 1] = p
    et[1, 1] = tags[p]
    status, _ = oi.check_pages_ref(tags, bt, et, c.seq_lens, ep)
    assert status.tolist() == [oi.STALE_TAG, 0]


def test_tag_wraps_around():
    """The tag only has to change: a counter that wraps past 2**32 - 1 still differs."""
    tags = np.array([0], np.uint32)
    status, _ = oi.check_pages_ref(tags, np.array([[0]], np.int32), np.array([[0xFFFFFFFF]], np.uint32),
                                   np.array([5], np.int32))
    assert status.tolist() == [oi.STALE_TAG]


def test_empty_batch():
    status, checked = oi.check_pages_ref(np.zeros(3, np.uint32), np.zeros((0, 4), np.int32),
                                         np.zeros((0, 4), np.uint32), np.zeros(0, np.int32))
    assert status.shape == (0,) and checked.shape == (0,)


# ----------------------------------------------------------------- mutations

def _mutant(kind):
    def check(page_tags, block_table, expected_tags, seq_lens, expected_pages=None):
        page_tags = np.asarray(page_tags, np.uint32)
        B, mb = block_table.shape
        st = np.zeros(B, np.int32)
        ck = np.zeros(B, np.int32)
        for b in range(B):
            L = int(seq_lens[b])
            s = 0
            if L < 0 or L > (mb * 64 if kind != "cap" else mb * 64 - 1):
                s = oi.BAD_LEN
            else:
                n = (L + 63) // 64 if kind != "floor" else L // 64
                for j in range(n):
                    pg = int(block_table[b, j])
                    if expected_pages is not None and pg != int(expected_pages[b, j]) and kind != "nopage":
                        s |= oi.WRONG_PAGE
                    if pg < 0 or pg >= (page_tags.shape[0] if kind != "range" else page_tags.shape[0] + 1):
                        s |= oi.OUT_OF_RANGE
                    else:
                        look = pg if kind != "recorded" else int(expected_pages[b, j]) \
                            if expected_pages is not None else pg
                        if look < page_tags.shape[0] and int(page_tags[look]) != int(expected_tags[b, j]):
                            s |= oi.STALE_TAG
            st[b] = s
            ck[b] = L if (s == 0 or kind == "keeplen") else 0
        return st, ck
    return check


@pytest.mark.parametrize("kind", ["floor", "cap", "nopage", "range", "recorded", "keeplen"])
def test_pins_catch_planted_mistakes(kind, monkeypatch):
    monkeypatch.setattr(oi, "check_pages_ref", _mutant(kind))
    pins = [test_hand_worked_case, test_hand_worked_case_without_page_record]
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    for k in sorted(_BITS):
        for where in ("first", "last", "middle"):
            try:
                test_planted_fault_flags_exactly_its_request(k, where)
            except AssertionError:
                caught += 1
    assert caught >= 1, f"no pin caught mutation {kind}"
