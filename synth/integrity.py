"""Seeded page-allocator histories for the KV page-tag check.

A toy page pool hands physical pages to requests and changes a page's tag each
time it hands the page out; each request keeps the (page, tag) pairs it was
given.  Faults are then planted into that bookkeeping the way a bug would
leave them: a page freed and handed to another request while the first still
maps it, a page-map entry overwritten with another page, an entry outside the
pool, a length beyond the map.  The pool only records what happened; the check
itself is not computed here.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PAGE = 64


@dataclass
class TagCase:
    page_tags: np.ndarray       # uint32 [num_pages]
    block_table: np.ndarray     # int32 [B, max_blocks]
    expected_pages: np.ndarray  # int32 [B, max_blocks]
    expected_tags: np.ndarray   # uint32 [B, max_blocks]
    seq_lens: np.ndarray        # int32 [B]
    planted: dict = field(default_factory=dict)  # request -> set of fault names planted into it

    @property
    def num_pages(self):
        return self.page_tags.shape[0]


class TaggedPool:
    """Pages with a tag that changes on every hand-out; the free list is shuffled."""

    def __init__(self, num_pages, rng):
        self.rng = rng
        self.tags = rng.integers(0, 2**32, size=num_pages, dtype=np.uint64).astype(np.uint32)
        self.free = list(rng.permutation(num_pages))

    def take(self, n):
        if n > len(self.free):
            raise ValueError("pool exhausted")
        pages = [int(self.free.pop()) for _ in range(n)]
        for p in pages:
            self.tags[p] = np.uint32((int(self.tags[p]) + 1) & 0xFFFFFFFF)
        return pages

    def give_back(self, pages):
        self.free.extend(int(p) for p in pages)
        self.rng.shuffle(self.free)


def make_case(seed, seq_lens, max_blocks, num_pages, faults=(), churn=0):
    """Allocate every request's pages from one pool, then plant ``faults``.

    seq_lens: lengths of the requests; max_blocks: page-map width;
    churn: requests allocated and finished first (their pages return to the
    pool, so later hand-outs change tags more than once);
    faults: (kind, request, logical page) triples, kind one of
      "stale"   the page goes back to the pool and to a new owner while the
                request still maps it (tag changes, map and record do not);
      "wrong"   the map entry is overwritten with another in-pool page;
      "oob"     the map entry is overwritten with an index outside the pool;
      "neg"     the map entry is overwritten with a negative index;
      "len"     the length is set beyond the map's capacity (page ignored);
      "neglen"  the length is set negative (page ignored);
      "tail"    an entry past the request's last page is overwritten
                (never read, so not a fault).
    """
    rng = np.random.default_rng(seed)
    pool = TaggedPool(num_pages, rng)
    for _ in range(churn):
        pool.give_back(pool.take(int(rng.integers(1, 4))))
    B = len(seq_lens)
    bt = np.full((B, max_blocks), -1, dtype=np.int32)
    # unused tail entries hold arbitrary stale numbers, as a reused map row would
    bt[:] = rng.integers(-5, num_pages + 5, size=(B, max_blocks), dtype=np.int32)
    exp_pages = bt.copy()
    exp_tags = rng.integers(0, 2**32, size=(B, max_blocks), dtype=np.uint64).astype(np.uint32)
    lens = np.asarray(seq_lens, dtype=np.int32).copy()
    for b, L in enumerate(lens):
        n = (int(L) + PAGE - 1) // PAGE
        pages = pool.take(n)
        bt[b, :n] = pages
        exp_pages[b, :n] = pages
        exp_tags[b, :n] = pool.tags[pages]
    planted = {}
    for kind, b, j in faults:
        planted.setdefault(b, set()).add(kind)
        if kind == "stale":
            p = int(bt[b, j])
            pool.give_back([p])
            # hand pages out until p comes back to someone else (its tag changes each time)
            while True:
                got = pool.take(1)
                if got[0] == p:
                    break
        elif kind == "wrong":
            other = int(rng.integers(0, num_pages - 1))
            bt[b, j] = other if other != bt[b, j] else num_pages - 1 - other
            if bt[b, j] == exp_pages[b, j]:
                bt[b, j] = (bt[b, j] + 1) % num_pages
        elif kind == "oob":
            bt[b, j] = num_pages + int(rng.integers(0, 1000))
        elif kind == "neg":
            bt[b, j] = -1 - int(rng.integers(0, 1000))
        elif kind == "len":
            lens[b] = max_blocks * PAGE + 1 + int(rng.integers(0, 100))
        elif kind == "neglen":
            lens[b] = -1 - int(rng.integers(0, 100))
        elif kind == "tail":
            bt[b, j] = num_pages + 7
        else:
            raise ValueError(kind)
    return TagCase(pool.tags.copy(), bt, exp_pages, exp_tags, lens, planted)
