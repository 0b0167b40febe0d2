"""ctypes binding of libmla_decode.so — argument marshalling only.

The functions carry the C names of ``include/mla_decode.h``.  They take torch
tensors, check dtype, device, contiguity and shapes, pass raw device pointers
and the current HIP stream, and raise ``MlaError`` on a non-zero status.  No
step of the computation runs here; if the library is missing, importing this
module fails.

torch is imported before the library is loaded so that the library binds to the
HIP runtime torch already loaded (one runtime per process).
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_decode.so")

HEAD_DIM = 576
VALUE_DIM = 512
PAGE_SIZE = 64

CACHE_BF16 = 0
CACHE_FP8_E4M3 = 1
SCALE_NONE = 0
SCALE_PER_TENSOR = 1
SCALE_PER_TOKEN = 2

_SCALE_NAMES = {"none": SCALE_NONE, "tensor": SCALE_PER_TENSOR, "token": SCALE_PER_TOKEN}


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python long_context_mla_amd/build.py` "
            "(hipcc, gfx950); there is no other implementation"
        )
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, L = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int64
    lib.kv_append_fp8.argtypes = [P, P, P, I, P, P, I, I, I, I, P]
    lib.mla_decode_paged.argtypes = [P, P, I, P, I, P, P, I, I, I, I, I, F, I, I, P, P, P, P, P]
    lib.mla_decode_combine.argtypes = [P, P, P, I, I, I, I, I, I, P, P, P, P]
    lib.mla_decode_paged_append.argtypes = [P, I, P, P, P, I, P, P, I, I, I, I, I, F, I, I, P, P, P, P, I, P]
    lib.mla_decode_plan.argtypes = [I, I, I, I, L, I, I, ctypes.POINTER(I), ctypes.POINTER(I)]
    lib.mla_decode_plan_lens.argtypes = [P, I, I, I, I, I, ctypes.POINTER(I), ctypes.POINTER(I)]
    lib.kv_check_pages.argtypes = [P, I, P, P, P, P, I, I, P, P, P]
    lib.mla_decode_paged_append_checked.argtypes = [P, I, P, P, P, I, P, P, I, I, I, I, I, F, I, I, P, P,
                                                    P, P, P, P, P]
    lib.mla_decode_paged_append_noalloc.argtypes = [P, I, P, P, P, I, P, P, I, I, I, I, I, F, I, I, P, P, I, P]
    lib.mla_status_string.argtypes = [I]
    lib.mla_status_string.restype = ctypes.c_char_p
    for fn in ("kv_append_fp8", "mla_decode_paged", "mla_decode_paged_append", "mla_decode_combine",
               "mla_decode_plan", "mla_decode_plan_lens", "kv_check_pages", "mla_decode_paged_append_checked",
               "mla_decode_paged_append_noalloc"):
        getattr(lib, fn).restype = I
    return lib


LIB = _load()
EXPORTS = ("kv_append_fp8", "mla_decode_paged", "mla_decode_paged_append", "mla_decode_paged_append_checked",
           "mla_decode_paged_append_noalloc", "mla_decode_combine", "mla_decode_plan", "mla_decode_plan_lens", "kv_check_pages", "mla_status_string")

NOALLOC_MAX_PARTIAL_ROWS = 32768
ERR_SCRATCH_LIMIT = 5

PAGE_OK = 0
PAGE_BAD_LEN = 1
PAGE_OUT_OF_RANGE = 2
PAGE_WRONG_PAGE = 4
PAGE_STALE_TAG = 8


def status_string(status: int) -> str:
    return LIB.mla_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# arrays the kernels move in 16-byte pieces
_ALIGN16 = ("q", "kv_cache", "kv_new", "o_partial", "out")


def _need(t, name, dtype, device=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if name in _ALIGN16 and t.data_ptr() % 16:
        raise ValueError(f"{name} must be 16-byte aligned")


def _check(fn, status):
    if status != 0:
        raise MlaError(fn, status)


def _cache_kind(kv_cache):
    if kv_cache.dtype == torch.uint8 or kv_cache.dtype == torch.float8_e4m3fn:
        return CACHE_FP8_E4M3
    if kv_cache.dtype == torch.bfloat16:
        return CACHE_BF16
    raise TypeError(f"kv_cache must be uint8/float8_e4m3fn (E4M3 codes) or bfloat16, got {kv_cache.dtype}")


def kv_append_fp8(kv_new, kv_cache, kv_scale, scale_mode, block_table, seq_lens, stream=None):
    """kv_new bf16 [B, n_new, 576]; kv_cache e4m3 codes [num_pages, 64, 576];
    kv_scale fp32 [num_pages, 64] ("token") or [1] ("tensor")."""
    mode = _SCALE_NAMES[scale_mode] if isinstance(scale_mode, str) else int(scale_mode)
    dev = kv_cache.device
    _need(kv_new, "kv_new", torch.bfloat16, dev, 3)
    if _cache_kind(kv_cache) != CACHE_FP8_E4M3 or kv_cache.dim() != 3:
        raise TypeError("kv_cache must be E4M3 codes [num_pages, 64, 576]")
    _need(kv_cache, "kv_cache", kv_cache.dtype, dev)
    _need(kv_scale, "kv_scale", torch.float32, dev)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    B, n_new, D = kv_new.shape
    num_pages = kv_cache.shape[0]
    if D != HEAD_DIM or tuple(kv_cache.shape[1:]) != (PAGE_SIZE, HEAD_DIM):
        raise ValueError("row width must be 576 and pages [64, 576]")
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_table / seq_lens batch mismatch")
    if mode == SCALE_PER_TOKEN and tuple(kv_scale.shape) != (num_pages, PAGE_SIZE):
        raise ValueError("per-token kv_scale must be [num_pages, 64]")
    if mode == SCALE_PER_TENSOR and kv_scale.numel() != 1:
        raise ValueError("per-tensor kv_scale must have one element")
    _check("kv_append_fp8", LIB.kv_append_fp8(
        _ptr(kv_new), _ptr(kv_cache), _ptr(kv_scale), mode, _ptr(block_table), _ptr(seq_lens),
        B, n_new, block_table.shape[1], num_pages, _stream(stream)))


def mla_decode_paged(q, kv_cache, kv_scale, scale_mode, block_table, seq_lens, softmax_scale,
                     pages_per_split, max_splits, o_partial=None, lse_partial=None, out=None,
                     lse=None, stream=None):
    """q bf16 [B, n_q, H, 576]; kv_cache E4M3 codes (uint8) or bf16 [num_pages, 64, 576].
    With max_splits == 1 writes out bf16 [B, n_q, H, 512] and lse fp32 [B, n_q, H];
    otherwise o_partial bf16 [B, max_splits, n_q, H, 512] and lse_partial fp32
    [B, max_splits, n_q, H]."""
    mode = _SCALE_NAMES[scale_mode] if isinstance(scale_mode, str) else int(scale_mode)
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 4)
    kind = _cache_kind(kv_cache)
    _need(kv_cache, "kv_cache", kv_cache.dtype, dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    B, n_q, H, D = q.shape
    num_pages = kv_cache.shape[0]
    if D != HEAD_DIM or tuple(kv_cache.shape[1:]) != (PAGE_SIZE, HEAD_DIM):
        raise ValueError("row width must be 576 and pages [64, 576]")
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_table / seq_lens batch mismatch")
    if mode != SCALE_NONE:
        _need(kv_scale, "kv_scale", torch.float32, dev)
        if mode == SCALE_PER_TOKEN and tuple(kv_scale.shape) != (num_pages, PAGE_SIZE):
            raise ValueError("per-token kv_scale must be [num_pages, 64]")
        if mode == SCALE_PER_TENSOR and kv_scale.numel() != 1:
            raise ValueError("per-tensor kv_scale must have one element")
    if max_splits == 1:
        _need(out, "out", torch.bfloat16, dev)
        _need(lse, "lse", torch.float32, dev)
        if tuple(out.shape) != (B, n_q, H, VALUE_DIM) or tuple(lse.shape) != (B, n_q, H):
            raise ValueError("out / lse shape mismatch")
    else:
        _need(o_partial, "o_partial", torch.bfloat16, dev)
        _need(lse_partial, "lse_partial", torch.float32, dev)
        if tuple(o_partial.shape) != (B, max_splits, n_q, H, VALUE_DIM) or \
                tuple(lse_partial.shape) != (B, max_splits, n_q, H):
            raise ValueError("o_partial / lse_partial shape mismatch")
    _check("mla_decode_paged", LIB.mla_decode_paged(
        _ptr(q), _ptr(kv_cache), kind, _ptr(kv_scale) if mode != SCALE_NONE else None, mode,
        _ptr(block_table), _ptr(seq_lens), B, n_q, H, block_table.shape[1], num_pages,
        float(softmax_scale), int(pages_per_split), int(max_splits),
        _ptr(o_partial) if max_splits > 1 else None, _ptr(lse_partial) if max_splits > 1 else None,
        _ptr(out) if max_splits == 1 else None, _ptr(lse) if max_splits == 1 else None,
        _stream(stream)))


def mla_decode_paged_append(kv_new, q, kv_cache, kv_scale, scale_mode, block_table, seq_lens,
                            softmax_scale, pages_per_split, max_splits, o_partial=None,
                            lse_partial=None, out=None, lse=None, stream=None, store_rows=True):
    """kv_append_fp8 then mla_decode_paged in one launch (E4M3 cache); kv_new bf16
    [B, n_new, 576] (n_new may be 0); the other arguments as in those two.
    store_rows=False: the new rows serve this launch only (the caller stores them)."""
    mode = _SCALE_NAMES[scale_mode] if isinstance(scale_mode, str) else int(scale_mode)
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 4)
    _need(kv_new, "kv_new", torch.bfloat16, dev, 3)
    if _cache_kind(kv_cache) != CACHE_FP8_E4M3 or kv_cache.dim() != 3:
        raise TypeError("kv_cache must be E4M3 codes [num_pages, 64, 576]")
    _need(kv_cache, "kv_cache", kv_cache.dtype, dev)
    _need(kv_scale, "kv_scale", torch.float32, dev)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    B, n_q, H, D = q.shape
    num_pages = kv_cache.shape[0]
    if D != HEAD_DIM or tuple(kv_cache.shape[1:]) != (PAGE_SIZE, HEAD_DIM):
        raise ValueError("row width must be 576 and pages [64, 576]")
    if kv_new.shape[0] != B or kv_new.shape[2] != HEAD_DIM:
        raise ValueError("kv_new must be [B, n_new, 576]")
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_table / seq_lens batch mismatch")
    if mode == SCALE_PER_TOKEN and tuple(kv_scale.shape) != (num_pages, PAGE_SIZE):
        raise ValueError("per-token kv_scale must be [num_pages, 64]")
    if mode == SCALE_PER_TENSOR and kv_scale.numel() != 1:
        raise ValueError("per-tensor kv_scale must have one element")
    if max_splits == 1:
        _need(out, "out", torch.bfloat16, dev)
        _need(lse, "lse", torch.float32, dev)
        if tuple(out.shape) != (B, n_q, H, VALUE_DIM) or tuple(lse.shape) != (B, n_q, H):
            raise ValueError("out / lse shape mismatch")
    else:
        _need(o_partial, "o_partial", torch.bfloat16, dev)
        _need(lse_partial, "lse_partial", torch.float32, dev)
        if tuple(o_partial.shape) != (B, max_splits, n_q, H, VALUE_DIM) or \
                tuple(lse_partial.shape) != (B, max_splits, n_q, H):
            raise ValueError("o_partial / lse_partial shape mismatch")
    _check("mla_decode_paged_append", LIB.mla_decode_paged_append(
        _ptr(kv_new), kv_new.shape[1], _ptr(q), _ptr(kv_cache), _ptr(kv_scale), mode,
        _ptr(block_table), _ptr(seq_lens), B, n_q, H, block_table.shape[1], num_pages,
        float(softmax_scale), int(pages_per_split), int(max_splits),
        _ptr(o_partial) if max_splits > 1 else None, _ptr(lse_partial) if max_splits > 1 else None,
        _ptr(out) if max_splits == 1 else None, _ptr(lse) if max_splits == 1 else None,
        1 if store_rows else 0, _stream(stream)))


def mla_decode_paged_append_noalloc(kv_new, q, kv_cache, kv_scale, scale_mode, block_table, seq_lens,
                                    softmax_scale, pages_per_split, max_splits, out, lse, stream=None,
                                    store_rows=True):
    """mla_decode_paged_append + mla_decode_combine with the split partials in the
    library's fixed per-GPU scratch (no allocation); out bf16 [B, n_q, H, 512] and
    lse fp32 [B, n_q, H] are written.  Calls that overlap on one GPU race."""
    mode = _SCALE_NAMES[scale_mode] if isinstance(scale_mode, str) else int(scale_mode)
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 4)
    _need(kv_new, "kv_new", torch.bfloat16, dev, 3)
    if _cache_kind(kv_cache) != CACHE_FP8_E4M3 or kv_cache.dim() != 3:
        raise TypeError("kv_cache must be E4M3 codes [num_pages, 64, 576]")
    _need(kv_cache, "kv_cache", kv_cache.dtype, dev)
    _need(kv_scale, "kv_scale", torch.float32, dev)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    _need(out, "out", torch.bfloat16, dev, 4)
    _need(lse, "lse", torch.float32, dev, 3)
    B, n_q, H, D = q.shape
    num_pages = kv_cache.shape[0]
    if D != HEAD_DIM or tuple(kv_cache.shape[1:]) != (PAGE_SIZE, HEAD_DIM):
        raise ValueError("row width must be 576 and pages [64, 576]")
    if kv_new.shape[0] != B or kv_new.shape[2] != HEAD_DIM:
        raise ValueError("kv_new must be [B, n_new, 576]")
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_table / seq_lens batch mismatch")
    if mode == SCALE_PER_TOKEN and tuple(kv_scale.shape) != (num_pages, PAGE_SIZE):
        raise ValueError("per-token kv_scale must be [num_pages, 64]")
    if mode == SCALE_PER_TENSOR and kv_scale.numel() != 1:
        raise ValueError("per-tensor kv_scale must have one element")
    if tuple(out.shape) != (B, n_q, H, VALUE_DIM) or tuple(lse.shape) != (B, n_q, H):
        raise ValueError("out / lse shape mismatch")
    _check("mla_decode_paged_append_noalloc", LIB.mla_decode_paged_append_noalloc(
        _ptr(kv_new), kv_new.shape[1], _ptr(q), _ptr(kv_cache), _ptr(kv_scale), mode,
        _ptr(block_table), _ptr(seq_lens), B, n_q, H, block_table.shape[1], num_pages,
        float(softmax_scale), int(pages_per_split), int(max_splits), _ptr(out), _ptr(lse),
        1 if store_rows else 0, _stream(stream)))


def mla_decode_combine(o_partial, lse_partial, seq_lens, max_blocks, pages_per_split, out, lse,
                       stream=None, status=None):
    """Merge the partials of mla_decode_paged into out bf16 [B, n_q, H, 512] and lse fp32 [B, n_q, H];
    status int32 [B] (kv_check_pages) or None: flagged requests get 0 / -inf rows."""
    dev = o_partial.device
    _need(o_partial, "o_partial", torch.bfloat16, dev, 5)
    _need(lse_partial, "lse_partial", torch.float32, dev, 4)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    _need(out, "out", torch.bfloat16, dev, 4)
    _need(lse, "lse", torch.float32, dev, 3)
    B, max_splits, n_q, H, DV = o_partial.shape
    if DV != VALUE_DIM or tuple(lse_partial.shape) != (B, max_splits, n_q, H):
        raise ValueError("partial shape mismatch")
    if tuple(out.shape) != (B, n_q, H, VALUE_DIM) or tuple(lse.shape) != (B, n_q, H):
        raise ValueError("out / lse shape mismatch")
    if status is not None:
        _need(status, "status", torch.int32, dev, 1)
        if status.shape[0] != B:
            raise ValueError("status must have B entries")
    _check("mla_decode_combine", LIB.mla_decode_combine(
        _ptr(o_partial), _ptr(lse_partial), _ptr(seq_lens), B, n_q, H, int(max_blocks),
        int(pages_per_split), max_splits, _ptr(out), _ptr(lse), _ptr(status), _stream(stream)))


def _dtype_code(cache_dtype):
    if isinstance(cache_dtype, str):
        return {"fp8": CACHE_FP8_E4M3, "bf16": CACHE_BF16}[cache_dtype]
    return int(cache_dtype)


def mla_decode_plan_lens(seq_lens, n_q, H, num_cus=0, cache_dtype="fp8"):
    """Host-only split plan from the batch's lengths (a host sequence of ints)
    for a cache of `cache_dtype` ("fp8" / "bf16" or CACHE_*): returns
    (pages_per_split, max_splits)."""
    import numpy as np

    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32).reshape(-1))
    pps, ms = ctypes.c_int(0), ctypes.c_int(0)
    _check("mla_decode_plan_lens", LIB.mla_decode_plan_lens(
        lens.ctypes.data if lens.size else None, int(lens.size), int(n_q), int(H), int(num_cus),
        _dtype_code(cache_dtype), ctypes.byref(pps), ctypes.byref(ms)))
    return pps.value, ms.value


def mla_decode_plan(B, n_q, H, max_seq_len, total_seq_len, num_cus=0, cache_dtype="fp8"):
    """Host-only split plan: returns (pages_per_split, max_splits)."""
    pps, ms = ctypes.c_int(0), ctypes.c_int(0)
    _check("mla_decode_plan", LIB.mla_decode_plan(int(B), int(n_q), int(H), int(max_seq_len),
                                                  int(total_seq_len), int(num_cus), _dtype_code(cache_dtype),
                                                  ctypes.byref(pps), ctypes.byref(ms)))
    return pps.value, ms.value


def _need_tags(t, name, device, ndim):
    if not isinstance(t, torch.Tensor) or t.dtype not in (torch.int32, torch.uint32):
        raise TypeError(f"{name} must be an int32 or uint32 tensor (the tag bits)")
    _need(t, name, t.dtype, device, ndim)


def kv_check_pages(page_tags, block_table, expected_tags, seq_lens, status, checked_lens,
                   expected_pages=None, stream=None):
    """page_tags [num_pages] and expected_tags [B, max_blocks] (uint32 or int32 bits);
    block_table, expected_pages (or None) int32 [B, max_blocks]; seq_lens int32 [B];
    writes status int32 [B] (PAGE_* bits) and checked_lens int32 [B] (may be seq_lens)."""
    dev = block_table.device
    _need_tags(page_tags, "page_tags", dev, 1)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need_tags(expected_tags, "expected_tags", dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    _need(status, "status", torch.int32, dev, 1)
    _need(checked_lens, "checked_lens", torch.int32, dev, 1)
    B, max_blocks = block_table.shape
    if expected_pages is not None:
        _need(expected_pages, "expected_pages", torch.int32, dev, 2)
        if tuple(expected_pages.shape) != (B, max_blocks):
            raise ValueError("expected_pages must match block_table's shape")
    if tuple(expected_tags.shape) != (B, max_blocks):
        raise ValueError("expected_tags must match block_table's shape")
    if seq_lens.shape[0] != B or status.shape[0] != B or checked_lens.shape[0] != B:
        raise ValueError("seq_lens / status / checked_lens must have B entries")
    if B and status.data_ptr() in (checked_lens.data_ptr(), seq_lens.data_ptr()):
        raise ValueError("status must not share memory with seq_lens or checked_lens")
    _check("kv_check_pages", LIB.kv_check_pages(
        _ptr(page_tags), page_tags.shape[0], _ptr(block_table), _ptr(expected_pages),
        _ptr(expected_tags), _ptr(seq_lens), B, max_blocks, _ptr(status), _ptr(checked_lens),
        _stream(stream)))


def mla_decode_paged_append_checked(kv_new, q, kv_cache, kv_scale, scale_mode, block_table, seq_lens,
                                    softmax_scale, pages_per_split, max_splits, o_partial, lse_partial,
                                    page_tags, expected_tags, status, expected_pages=None, stream=None):
    """mla_decode_paged_append (max_splits >= 2) with the page-tag check in the same launch:
    writes status int32 [B]; pass it to mla_decode_combine."""
    mode = _SCALE_NAMES[scale_mode] if isinstance(scale_mode, str) else int(scale_mode)
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 4)
    _need(kv_new, "kv_new", torch.bfloat16, dev, 3)
    if _cache_kind(kv_cache) != CACHE_FP8_E4M3 or kv_cache.dim() != 3:
        raise TypeError("kv_cache must be E4M3 codes [num_pages, 64, 576]")
    _need(kv_cache, "kv_cache", kv_cache.dtype, dev)
    _need(kv_scale, "kv_scale", torch.float32, dev)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    _need_tags(page_tags, "page_tags", dev, 1)
    _need_tags(expected_tags, "expected_tags", dev, 2)
    _need(status, "status", torch.int32, dev, 1)
    B, n_q, H, D = q.shape
    num_pages = kv_cache.shape[0]
    max_blocks = block_table.shape[1]
    if D != HEAD_DIM or tuple(kv_cache.shape[1:]) != (PAGE_SIZE, HEAD_DIM):
        raise ValueError("row width must be 576 and pages [64, 576]")
    if kv_new.shape[0] != B or kv_new.shape[2] != HEAD_DIM:
        raise ValueError("kv_new must be [B, n_new, 576]")
    if block_table.shape[0] != B or seq_lens.shape[0] != B or status.shape[0] != B:
        raise ValueError("block_table / seq_lens / status batch mismatch")
    if page_tags.shape[0] != num_pages:
        raise ValueError("page_tags must have num_pages entries")
    if tuple(expected_tags.shape) != (B, max_blocks):
        raise ValueError("expected_tags must match block_table's shape")
    if expected_pages is not None:
        _need(expected_pages, "expected_pages", torch.int32, dev, 2)
        if tuple(expected_pages.shape) != (B, max_blocks):
            raise ValueError("expected_pages must match block_table's shape")
    if mode == SCALE_PER_TOKEN and tuple(kv_scale.shape) != (num_pages, PAGE_SIZE):
        raise ValueError("per-token kv_scale must be [num_pages, 64]")
    if mode == SCALE_PER_TENSOR and kv_scale.numel() != 1:
        raise ValueError("per-tensor kv_scale must have one element")
    _need(o_partial, "o_partial", torch.bfloat16, dev)
    _need(lse_partial, "lse_partial", torch.float32, dev)
    if tuple(o_partial.shape) != (B, max_splits, n_q, H, VALUE_DIM) or \
            tuple(lse_partial.shape) != (B, max_splits, n_q, H):
        raise ValueError("o_partial / lse_partial shape mismatch")
    _check("mla_decode_paged_append_checked", LIB.mla_decode_paged_append_checked(
        _ptr(kv_new), kv_new.shape[1], _ptr(q), _ptr(kv_cache), _ptr(kv_scale), mode,
        _ptr(block_table), _ptr(seq_lens), B, n_q, H, max_blocks, num_pages,
        float(softmax_scale), int(pages_per_split), int(max_splits), _ptr(o_partial), _ptr(lse_partial),
        _ptr(page_tags), _ptr(expected_pages), _ptr(expected_tags), _ptr(status), _stream(stream)))
