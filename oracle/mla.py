"""Paged MLA decode attention — oracle definitions in fp64 (test infrastructure only).

What is computed, and where the pages fix it:

* One latent row of 576 elements per cached token serves as both key and value:
  models like Kimi have no distinct keys and values ("How to serve trillions of
  tokens for trillion-parameter coding agents", section "First, understand the
  workload"), the row is 576 elements per token per layer (same page, section
  "Tensor parallel was the best parallelism strategy for maximum
  interactivity"), and MLA compresses KV into a single latent space with one
  head ("vLLM x AgentX: Optimizing for Real-World Agentic Serving", section
  "Model-specific parallelism / Kimi K3").  Reading taken: the value is the
  first 512 (latent) elements; the last 64 (rope) are key-only; the query is
  already absorbed into the 576-d latent space.
* The cache is stored as FP8 e4m3 and converted as it is read ("Smaller,
  faster, safer: running Kimi and GLM at scale", section "Quantizing the KV
  cache"): the oracle dequantises to fp64 first and then attends.
* Physical pages reached through a per-request page map ("Smaller, faster,
  safer", section "Protecting a shared KV cache"): token ``t`` of request ``b``
  is slot ``t % 64`` of physical page ``block_table[b][t // 64]``.
* Partial attention outputs and their log-sum-exp are merged with the online
  softmax identity ("vLLM x AgentX", section "Model-specific parallelism /
  Kimi K3"): ``merge_ref``.

For request ``b`` with ``L = seq_lens[b]`` and ``n_q`` queries, query ``i``
(the ``L - n_q + i``-th position) sees tokens ``t < L - n_q + i + 1``.  For each
head ``h``: ``s_t = softmax_scale * q[b,i,h,:] . K_t``,
``lse = ln sum_t exp(s_t)``, ``out = sum_t exp(s_t - lse) * K_t[:512]``.
A row that sees no token gets ``out = 0`` and ``lse = -inf``.
"""

from __future__ import annotations

import math

import numpy as np

from . import e4m3

PAGE = 64
D = 576
DV = 512
_E4M3_MAX = 448.0


# ------------------------------------------------------------------ conversions
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


# ------------------------------------------------------------------ cache access
def request_rows(cache, scales, block_table, b, L, cache_dtype, scale_mode, tensor_scale=None):
    """Dequantised latent rows of request ``b``'s first ``L`` tokens, fp64 [L, 576].

    cache: uint8 codes [num_pages, 64, 576] (fp8) or uint16 bf16 bits (bf16).
    scales: float32 [num_pages, 64] for per-token mode, else unused.
    """
    n = -(-L // PAGE)
    pages = np.asarray(block_table[b, :n], dtype=np.int64)
    raw = cache[pages].reshape(n * PAGE, D)[:L]
    if cache_dtype == "bf16":
        return bf16_to_f64(raw)
    K = e4m3.decode(raw)
    if scale_mode == "token":
        s = scales[pages].reshape(n * PAGE)[:L].astype(np.float64)
        K = K * s[:, None]
    elif scale_mode == "tensor":
        K = K * float(np.float32(tensor_scale))
    return K


# ------------------------------------------------------------------ attention
def attend(Q: np.ndarray, K: np.ndarray, visible: np.ndarray, softmax_scale: float):
    """Softmax attention of query rows over key/value rows.

    Q fp64 [R, 576]; K fp64 [T, 576]; visible[r] = number of leading tokens row r
    sees.  Returns out fp64 [R, 512] and lse fp64 [R] (natural log).
    """
    R = Q.shape[0]
    out = np.zeros((R, DV), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    if K.shape[0] == 0:
        return out, lse
    S = (Q @ K.T) * float(softmax_scale)
    for r in range(R):
        n = int(visible[r])
        if n <= 0:
            continue
        s = S[r, :n]
        m = s.max()
        w = np.exp(s - m)
        tot = w.sum()
        lse[r] = m + math.log(tot)
        out[r] = (w / tot) @ K[:n, :DV]
    return out, lse


def decode_ref(q_bits, cache, scales, block_table, seq_lens, *, n_q, H, cache_dtype,
               scale_mode, softmax_scale, tensor_scale=None, requests=None, queries=None):
    """The attention the decode path computes, request by request.

    q_bits: bf16 bits [B, n_q, H, 576].  Query i of request b is position
    L_b - n_q + i and sees tokens t < L_b - n_q + i + 1.  Returns (out fp64
    [B, n_q, H, 512], lse fp64 [B, n_q, H]); requests not listed in
    ``requests``, and queries not listed in ``queries``, stay zero / NaN.
    """
    B = int(q_bits.shape[0])
    out = np.zeros((B, n_q, H, DV), dtype=np.float64)
    lse = np.full((B, n_q, H), np.nan, dtype=np.float64)
    todo = range(B) if requests is None else requests
    qs = np.arange(n_q) if queries is None else np.asarray(queries, dtype=np.int64)
    for b in todo:
        L = int(seq_lens[b])
        K = request_rows(cache, scales, block_table, b, L, cache_dtype, scale_mode, tensor_scale)
        Q = bf16_to_f64(q_bits[b][qs]).reshape(qs.size * H, D)
        visible = np.repeat(L - n_q + qs + 1, H)
        o, l = attend(Q, K, visible, softmax_scale)
        out[b, qs] = o.reshape(qs.size, H, DV)
        lse[b, qs] = l.reshape(qs.size, H)
    return out, lse


def partial_ref(Q: np.ndarray, K: np.ndarray, visible: np.ndarray, softmax_scale: float,
                t0: int, t1: int):
    """Attention of each row restricted to tokens in [t0, t1) it can see: the
    normalised partial output and its log-sum-exp (``-inf`` and zeros if none)."""
    vis = np.clip(np.asarray(visible) - t0, 0, max(t1 - t0, 0))
    return attend(Q, K[t0:t1], vis, softmax_scale)


def merge_ref(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge partial attentions over disjoint token sets.

    o_parts [S, ..., 512] (each normalised by its own softmax sum), lse_parts
    [S, ...].  Result: weights ``exp(lse_s - M)`` with ``M = max_s lse_s``;
    ``out = sum_s w_s o_s / sum_s w_s``; ``lse = M + ln sum_s w_s``.  Parts with
    ``lse = -inf`` carry no weight; if all do, out = 0 and lse = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    M = lse_parts.max(axis=0)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - Ms), 0.0)
    tot = w.sum(axis=0)
    safe = np.where(tot > 0, tot, 1.0)
    out = (w[..., None] * o_parts).sum(axis=0) / safe[..., None]
    out = np.where(finite[..., None], out, 0.0)
    lse = np.where(finite, Ms + np.log(safe), -np.inf)
    return out, lse


# ------------------------------------------------------------------ naive loops
def decode_naive(q_rows, k_rows, softmax_scale, visible):
    """Pure-Python attention for tiny inputs: nested loops and ``math.fsum``.

    q_rows: list of 576-float lists; k_rows: list of 576-float lists (already
    dequantised); visible: list of token counts.  Returns (out rows, lse list).
    """
    outs, lses = [], []
    for q, n in zip(q_rows, visible):
        if n <= 0:
            outs.append([0.0] * DV)
            lses.append(-math.inf)
            continue
        s = [softmax_scale * math.fsum(q[d] * k_rows[t][d] for d in range(D)) for t in range(n)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        tot = math.fsum(w)
        lses.append(m + math.log(tot))
        outs.append([math.fsum(w[t] * k_rows[t][d] for t in range(n)) / tot for d in range(DV)])
    return outs, lses


# ------------------------------------------------------------------ FP8 append
def quantize_rows(x_bits: np.ndarray, scale_mode: str, tensor_scale=None):
    """bf16 rows [N, 576] -> (codes uint8 [N, 576], scales float32 [N]).

    Per-token: ``amax = max_d |x_d|``, ``scale = fp32(amax / 448)`` (1.0 when
    amax is 0), ``code_d = e4m3(fp32(x_d / scale))``.  Per-tensor: the given
    scale.  All divisions are single-precision, correctly rounded.
    """
    x = bf16_to_f32(x_bits).reshape(-1, D)
    if scale_mode == "token":
        amax = np.abs(x).max(axis=1)
        sc = (amax / np.float32(_E4M3_MAX)).astype(np.float32)
        sc = np.where(amax == 0, np.float32(1.0), sc).astype(np.float32)
    elif scale_mode == "tensor":
        sc = np.full(x.shape[0], np.float32(tensor_scale), dtype=np.float32)
    else:
        raise ValueError(scale_mode)
    y = (x / sc[:, None]).astype(np.float32)
    return e4m3.encode(y), sc


def append_ref(new_bits, cache, scales, block_table, seq_lens, scale_mode, tensor_scale=None):
    """Write the step's new rows into the FP8 cache in place.

    Row ``j`` of request ``b`` (of ``n_new``) goes to position
    ``p = seq_lens[b] - n_new + j``: slot ``p % 64`` of page
    ``block_table[b][p // 64]``.  Per-token scales go to ``scales[page, slot]``.

    A row is written only where that slot exists: ``0 <= p < 64 * max_blocks``
    and a page id inside ``[0, num_pages)``.  Other rows are dropped (the pages
    say nothing of malformed page maps; the plainest reading is that a row with
    no slot of its own is not stored anywhere).
    """
    B, n_new = int(new_bits.shape[0]), int(new_bits.shape[1])
    num_pages = cache.shape[0]
    cap = block_table.shape[1] * PAGE
    codes, sc = quantize_rows(new_bits.reshape(B * n_new, D), scale_mode, tensor_scale)
    codes = codes.reshape(B, n_new, D)
    sc = sc.reshape(B, n_new)
    for b in range(B):
        for j in range(n_new):
            p = int(seq_lens[b]) - n_new + j
            if p < 0 or p >= cap:
                continue
            page = int(block_table[b, p // PAGE])
            if page < 0 or page >= num_pages:
                continue
            cache[page, p % PAGE] = codes[b, j]
            if scale_mode == "token":
                scales[page, p % PAGE] = sc[b, j]


def fill_pages_ref(page_bits: np.ndarray, scale_mode: str, tensor_scale=None):
    """Quantise whole pages of bf16 rows: (codes [n, 64, 576], scales [n, 64])."""
    n = page_bits.shape[0]
    codes, sc = quantize_rows(page_bits.reshape(n * PAGE, D), scale_mode, tensor_scale)
    return codes.reshape(n, PAGE, D), sc.reshape(n, PAGE)
