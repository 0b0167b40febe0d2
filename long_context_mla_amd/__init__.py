"""Paged MLA decode attention over an FP8 (e4m3) latent KV cache on MI355X (gfx950).

The compute lives in the HIP library ``libmla_decode.so`` (C ABI in
``include/mla_decode.h``); this package only binds it.  Importing it without the
built library raises ImportError: there is no fallback implementation.
"""

from ._lib import (  # noqa: F401
    CACHE_BF16,
    CACHE_FP8_E4M3,
    LIB_PATH,
    MlaError,
    NOALLOC_MAX_PARTIAL_ROWS,
    PAGE_BAD_LEN,
    PAGE_OK,
    PAGE_OUT_OF_RANGE,
    PAGE_STALE_TAG,
    PAGE_WRONG_PAGE,
    SCALE_NONE,
    SCALE_PER_TENSOR,
    SCALE_PER_TOKEN,
    kv_append_fp8,
    kv_check_pages,
    mla_decode_combine,
    mla_decode_paged,
    mla_decode_paged_append,
    mla_decode_paged_append_noalloc,
    mla_decode_plan,
    mla_decode_plan_lens,
    status_string,
)
from .runner import DecodeStep  # noqa: F401
