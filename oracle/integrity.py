"""KV page-tag integrity check — oracle definition (test infrastructure only).

What the pages fix ("Smaller, faster, safer: running Kimi and GLM at scale",
section "Protecting a shared KV cache"):

* every physical cache page carries a tag, and the tag changes each time the
  page is handed to a new owner;
* the server keeps, for each request, the pages it expects to read and the tag
  each of them had when the request got it;
* before decode reads the cache these records are compared with the current
  state, as a batch check of its own (not inside the attention kernel);
* a request whose records do not match is aborted; it must not return data
  read from a page that is no longer its own.

Readings taken where the pages leave a step open:

* the pages a request reads are logical pages ``j < ceil(L / 64)`` of its page
  map, ``L = seq_lens[b]``; entries past them are never read and not checked;
* the record of pages may be the page map itself (``expected_pages is None``)
  or a separate copy; with a copy, every read entry must equal it;
* the tag compared is the current tag of the page the page map names, since
  that is the page decode would read;
* a length outside ``[0, max_blocks * 64]`` cannot name its pages: the request
  is flagged for its length alone and no page is looked at;
* aborting a request means its length is taken as 0 for the step, so decode
  reads none of its pages (and writes none of its new rows): its output rows
  are 0 with a log-sum-exp of -inf.

The check may also run inside the decode launch, beside the attention, instead
of in front of it (``stored_rows_ref`` / ``append_checked_ref``).  That form
reads before it checks: the attention of every request runs on the unchecked
lengths, and a flagged request is masked afterwards (rows 0, LSE -inf), so it
still returns no data.  What differs is the store of the step's new rows, which
cannot wait for the request's verdict.  Reading taken: a new row is stored iff
the page it goes to passes the check on its own -- the request's length lies in
``[0, 64 * max_blocks]``, the row's slot is at a position ``>= 0``, and the
page-map entry of that slot is inside the pool, equals the recorded page (when
a record is kept) and carries the recorded tag.  So no row ever lands in a page
that was handed to another owner; a flagged request may still store rows into
its own pages that pass.

Status bits per request (0 = the request may read the cache):
"""

from __future__ import annotations

import numpy as np

PAGE = 64

BAD_LEN = 1        # length negative or beyond the page map's capacity
OUT_OF_RANGE = 2   # a read page-map entry outside [0, num_pages)
WRONG_PAGE = 4     # a read page-map entry differs from the recorded page
STALE_TAG = 8      # the page's current tag differs from the recorded tag


def check_pages_ref(page_tags, block_table, expected_tags, seq_lens, expected_pages=None):
    """Per-request status bits and checked lengths (plain loops).

    page_tags uint32 [num_pages]; block_table int32 [B, max_blocks];
    expected_tags uint32 [B, max_blocks]; seq_lens int32 [B];
    expected_pages int32 [B, max_blocks] or None.
    Returns (status int32 [B], checked_lens int32 [B]).
    """
    page_tags = np.asarray(page_tags, dtype=np.uint32)
    block_table = np.asarray(block_table, dtype=np.int32)
    expected_tags = np.asarray(expected_tags, dtype=np.uint32)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    num_pages = page_tags.shape[0]
    B, max_blocks = block_table.shape
    status = np.zeros(B, dtype=np.int32)
    checked = np.zeros(B, dtype=np.int32)
    for b in range(B):
        L = int(seq_lens[b])
        s = 0
        if L < 0 or L > max_blocks * PAGE:
            s = BAD_LEN
        else:
            for j in range((L + PAGE - 1) // PAGE):
                page = int(block_table[b, j])
                if expected_pages is not None and page != int(expected_pages[b, j]):
                    s |= WRONG_PAGE
                if page < 0 or page >= num_pages:
                    s |= OUT_OF_RANGE
                elif int(page_tags[page]) != int(expected_tags[b, j]):
                    s |= STALE_TAG
        status[b] = s
        checked[b] = L if s == 0 else 0
    return status, checked


def stored_rows_ref(page_tags, block_table, expected_tags, seq_lens, n_new, expected_pages=None):
    """Which new rows the in-launch check lets the decode launch store.

    Row ``j`` of request ``b`` sits at ``p = seq_lens[b] - n_new + j``.  It is
    stored iff ``0 <= seq_lens[b] <= 64 * max_blocks``, ``p >= 0``, and entry
    ``e = block_table[b, p // 64]`` is in ``[0, num_pages)``, equals
    ``expected_pages[b, p // 64]`` (if a record is given) and
    ``page_tags[e] == expected_tags[b, p // 64]``.
    Returns bool [B, n_new].
    """
    page_tags = np.asarray(page_tags, dtype=np.uint32)
    block_table = np.asarray(block_table, dtype=np.int32)
    expected_tags = np.asarray(expected_tags, dtype=np.uint32)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    num_pages = page_tags.shape[0]
    B, max_blocks = block_table.shape
    keep = np.zeros((B, n_new), dtype=bool)
    for b in range(B):
        L = int(seq_lens[b])
        if L < 0 or L > max_blocks * PAGE:
            continue
        for j in range(n_new):
            p = L - n_new + j
            if p < 0:
                continue
            k = p // PAGE
            page = int(block_table[b, k])
            if page < 0 or page >= num_pages:
                continue
            if expected_pages is not None and page != int(expected_pages[b, k]):
                continue
            if int(page_tags[page]) != int(expected_tags[b, k]):
                continue
            keep[b, j] = True
    return keep


def append_checked_ref(new_bits, cache, scales, block_table, seq_lens, scale_mode, tensor_scale,
                       page_tags, expected_tags, expected_pages=None):
    """The cache after a decode launch that carries the page check: the new rows
    ``stored_rows_ref`` keeps, written in place one by one as the plain append
    (``oracle.mla.append_ref``) writes them; the others are dropped."""
    from oracle import mla as omla

    B, n_new = int(new_bits.shape[0]), int(new_bits.shape[1])
    keep = stored_rows_ref(page_tags, block_table, expected_tags, seq_lens, n_new, expected_pages)
    for b in range(B):
        for j in range(n_new):
            if keep[b, j]:
                p = int(seq_lens[b]) - n_new + j
                # one row, one request whose length ends right after it
                omla.append_ref(new_bits[b:b + 1, j:j + 1], cache, scales, block_table[b:b + 1],
                                np.asarray([p + 1], dtype=np.int32), scale_mode, tensor_scale)
    return keep
