"""One decode step over a paged latent cache: append the step's new rows (FP8
cache), split-KV attention, then the split merge, on the current stream with
buffers allocated once per batch shape.  On an FP8 cache the append rides in
the decode launch (mla_decode_paged_append); fuse_append=False issues
kv_append_fp8 and mla_decode_paged separately.  With ``page_check`` the step
starts with the KV page-tag check (kv_check_pages) and runs on the lengths it
returns, so a request whose pages fail the check reads and writes no page and
gets zero output rows (``status`` holds its reason)."""

from __future__ import annotations

import torch

from . import _lib


class DecodeStep:
    def __init__(self, B, n_q, H, max_blocks, max_seq_len, total_seq_len, device, num_cus=0,
                 pages_per_split=None, max_splits=None, fuse_append=True, seq_lens_host=None,
                 check_mode="launch", cache_dtype="fp8"):
        """seq_lens_host: the batch's lengths on the host, when known; the split
        plan is then fitted to them (mla_decode_plan_lens) instead of to the
        longest and the summed length alone.  check_mode, where the page check
        runs when a step gets ``page_check`` (and has new rows on an FP8 cache
        with more than one split; otherwise it runs in front):
          "launch"  inside the decode launch (mla_decode_paged_append_checked),
                    the combine masking flagged requests (the default);
          "front"   kv_check_pages, then the step on the checked lengths;
          "stream"  beside the decode on a second stream (see _overlapped).
        cache_dtype: "fp8" or "bf16", the cache the plan is made for."""
        self.fuse_append = fuse_append
        if pages_per_split is None or max_splits is None:
            if seq_lens_host is not None:
                pages_per_split, max_splits = _lib.mla_decode_plan_lens(seq_lens_host, n_q, H, num_cus,
                                                                        cache_dtype)
            else:
                pages_per_split, max_splits = _lib.mla_decode_plan(B, n_q, H, max_seq_len, total_seq_len,
                                                                   num_cus, cache_dtype)
        self.B, self.n_q, self.H, self.max_blocks = B, n_q, H, max_blocks
        self.pps, self.max_splits = int(pages_per_split), int(max_splits)
        self.out = torch.empty((B, n_q, H, _lib.VALUE_DIM), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((B, n_q, H), dtype=torch.float32, device=device)
        if self.max_splits > 1:
            self.o_partial = torch.empty((B, self.max_splits, n_q, H, _lib.VALUE_DIM),
                                         dtype=torch.bfloat16, device=device)
            self.lse_partial = torch.empty((B, self.max_splits, n_q, H), dtype=torch.float32,
                                           device=device)
        else:
            self.o_partial = self.lse_partial = None
        self.status = self.checked_lens = None
        if check_mode not in ("front", "launch", "stream"):
            raise ValueError(f"check_mode must be front, launch or stream, got {check_mode!r}")
        self.check_mode = check_mode

    def decode(self, q, kv_cache, kv_scale, scale_mode, block_table, seq_lens, softmax_scale,
               stream=None):
        _lib.mla_decode_paged(q, kv_cache, kv_scale, scale_mode, block_table, seq_lens,
                              softmax_scale, self.pps, self.max_splits, self.o_partial,
                              self.lse_partial, self.out, self.lse, stream=stream)

    def combine(self, seq_lens, stream=None, status=None):
        if self.max_splits > 1:
            _lib.mla_decode_combine(self.o_partial, self.lse_partial, seq_lens, self.max_blocks,
                                    self.pps, self.out, self.lse, stream=stream, status=status)

    def _check_buffers(self, device):
        if self.status is None:
            self.status = torch.empty(self.B, dtype=torch.int32, device=device)
            self.checked_lens = torch.empty(self.B, dtype=torch.int32, device=device)
            self.side = torch.cuda.Stream(device=device)

    def check(self, page_tags, block_table, expected_tags, seq_lens, expected_pages=None, stream=None):
        """kv_check_pages into this step's status / checked_lens; returns checked_lens.
        (The in-launch placement writes ``status`` only; ``checked_lens`` then keeps
        whatever an earlier check left there.)"""
        self._check_buffers(block_table.device)
        _lib.kv_check_pages(page_tags, block_table, expected_tags, seq_lens, self.status,
                            self.checked_lens, expected_pages, stream=stream)
        return self.checked_lens

    def __call__(self, q, kv_cache, kv_scale, scale_mode, block_table, seq_lens, softmax_scale,
                 new_rows=None, stream=None, page_check=None):
        """page_check: (page_tags, expected_tags, expected_pages or None) to run the
        page-tag check in this step."""
        if page_check is not None:
            page_tags, expected_tags, expected_pages = page_check
            fused = new_rows is not None and new_rows.shape[1] > 0 and self.fuse_append
            if fused and self.max_splits > 1 and self.check_mode == "stream":
                return self._overlapped(q, kv_cache, kv_scale, scale_mode, block_table, seq_lens,
                                        softmax_scale, new_rows, stream, page_tags, expected_tags,
                                        expected_pages)
            if fused and self.max_splits > 1 and self.check_mode == "launch":
                self._check_buffers(block_table.device)
                _lib.mla_decode_paged_append_checked(
                    new_rows, q, kv_cache, kv_scale, scale_mode, block_table, seq_lens, softmax_scale,
                    self.pps, self.max_splits, self.o_partial, self.lse_partial, page_tags, expected_tags,
                    self.status, expected_pages, stream=stream)
                self.combine(seq_lens, stream, status=self.status)
                return self.out, self.lse
            seq_lens = self.check(page_tags, block_table, expected_tags, seq_lens, expected_pages, stream)
        if new_rows is not None and new_rows.shape[1] > 0:
            if self.fuse_append:
                _lib.mla_decode_paged_append(new_rows, q, kv_cache, kv_scale, scale_mode, block_table,
                                             seq_lens, softmax_scale, self.pps, self.max_splits,
                                             self.o_partial, self.lse_partial, self.out, self.lse,
                                             stream=stream)
                self.combine(seq_lens, stream)
                return self.out, self.lse
            _lib.kv_append_fp8(new_rows, kv_cache, kv_scale, scale_mode, block_table, seq_lens,
                               stream=stream)
        self.decode(q, kv_cache, kv_scale, scale_mode, block_table, seq_lens, softmax_scale, stream)
        self.combine(seq_lens, stream)
        return self.out, self.lse

    def _overlapped(self, q, kv_cache, kv_scale, scale_mode, block_table, seq_lens, softmax_scale,
                    new_rows, stream, page_tags, expected_tags, expected_pages):
        """The page check off the decode's critical path.  A side stream runs
        kv_check_pages and then kv_append_fp8 on the checked lengths (only
        requests that passed store their new rows); meanwhile the decode
        attends with the new rows but stores none, and reads the unchecked
        lengths (page ids are clamped, so it stays inside the cache).  The
        combine waits for both and gives flagged requests 0 / -inf rows."""
        main = stream if stream is not None else torch.cuda.current_stream()
        self._check_buffers(block_table.device)
        side = self.side
        side.wait_stream(main)
        self.check(page_tags, block_table, expected_tags, seq_lens, expected_pages, stream=side)
        _lib.kv_append_fp8(new_rows, kv_cache, kv_scale, scale_mode, block_table, self.checked_lens,
                           stream=side)
        _lib.mla_decode_paged_append(new_rows, q, kv_cache, kv_scale, scale_mode, block_table, seq_lens,
                                     softmax_scale, self.pps, self.max_splits, self.o_partial,
                                     self.lse_partial, self.out, self.lse, stream=main, store_rows=False)
        main.wait_stream(side)
        self.combine(seq_lens, main, status=self.status)
        return self.out, self.lse
