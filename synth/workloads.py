"""Seeded synthetic workloads for paged MLA decode attention.

The shapes follow the problem the pages describe: one compressed latent row
of 576 elements per cached token (512 latent + 64 rope), shared by every query
head ("How to serve trillions of tokens for trillion-parameter coding agents",
section "Tensor parallel was the best parallelism strategy for maximum
interactivity"; "vLLM x AgentX", section "Model-specific parallelism / Kimi
K3"), stored in physical cache pages that requests reach through a per-request
page map ("Smaller, faster, safer: running Kimi and GLM at scale", section
"Protecting a shared KV cache").

Everything here is input preparation: random draws, rounding of the draws to
bf16 (the input dtype), sequence lengths, page maps and sharing structure.  No
quantisation, attention or merge arithmetic lives here.

Random streams (numpy PCG64 through ``SeedSequence``), so that any subset of
pages can be regenerated without drawing the whole pool:

* ``[seed, 0]``          lengths and physical page permutation
* ``[seed, 1, chunk]``   latent rows of physical pages ``chunk*32 .. +32``
* ``[seed, 2, group]``   the 16 prefix-tail tokens a sharing group repeats
* ``[seed, 3]``          query rows
* ``[seed, 4]``          new latent rows written by the step's append
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

PAGE = 64  # tokens per physical cache page
D = 576  # latent row width: 512 latent + 64 rope
DV = 512  # value width (the latent part of the row)
SOFTMAX_SCALE = 192.0 ** -0.5
E4M3_MAX = 448.0  # largest finite OCP E4M3FN value (used only to calibrate a per-tensor scale)
_CHUNK = 32  # pages per random stream chunk


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 draws to bf16 (round to nearest even) and return the bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = (rounded >> np.uint32(16)).astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(list(key)))


@dataclass
class Workload:
    """One synthetic decode batch over a paged latent cache.

    ``seq_lens[b]`` counts the tokens visible to request ``b`` *after* the step
    appends its ``n_new`` rows; the ``n_q`` queries of a request are its last
    ``n_q`` positions.  ``block_table[b, j]`` is the physical page of logical
    page ``j``; entries past ``ceil(seq_lens[b]/64)`` are ``-1``.
    """

    name: str
    B: int
    n_q: int
    H: int
    seq_lens: np.ndarray  # int32 [B]
    n_new: int
    block_table: np.ndarray  # int32 [B, max_blocks]
    num_pages: int
    cache_dtype: str  # "fp8" | "bf16"
    scale_mode: str  # "none" | "tensor" | "token"
    seed: int = 0
    sigma_q: float = 1.0
    sigma_kv: float = 0.5
    softmax_scale: float = SOFTMAX_SCALE
    # physical page -> sharing group whose 16-token prefix tail fills slots 0..15
    shared_tail: dict = field(default_factory=dict)
    tail_tokens: int = 0
    # (b, token, head, gain): latent row of token := gain * q[b, 0, head]
    needles: tuple = ()
    notes: str = ""

    # ----------------------------------------------------------------- shapes
    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def rows(self) -> int:
        return self.n_q * self.H

    @property
    def context_lens(self) -> np.ndarray:
        return (self.seq_lens - self.n_new).astype(np.int32)

    def pages_of(self, b: int) -> np.ndarray:
        n = -(-int(self.seq_lens[b]) // PAGE)
        return self.block_table[b, :n]

    def unique_pages(self) -> np.ndarray:
        ids = [self.pages_of(b) for b in range(self.B)]
        return np.unique(np.concatenate(ids)) if ids else np.zeros(0, np.int32)

    # ----------------------------------------------------------------- values
    def q_bits(self) -> np.ndarray:
        """bf16 bits [B, n_q, H, 576], N(0, sigma_q) before rounding."""
        x = _rng(self.seed, 3).standard_normal((self.B, self.n_q, self.H, D), dtype=np.float32)
        return bf16_bits(x * np.float32(self.sigma_q))

    def new_row_bits(self) -> np.ndarray:
        """bf16 bits [B, n_new, 576] of the rows the step appends."""
        x = _rng(self.seed, 4).standard_normal((self.B, self.n_new, D), dtype=np.float32)
        rows = bf16_bits(x * np.float32(self.sigma_kv))
        for (b, t, h, gain) in self.needles:
            j = t - int(self.context_lens[b])
            if 0 <= j < self.n_new:
                rows[b, j] = self._needle_row(b, h, gain)
        return rows

    def _tail_bits(self, group: int) -> np.ndarray:
        x = _rng(self.seed, 2, group).standard_normal((self.tail_tokens, D), dtype=np.float32)
        return bf16_bits(x * np.float32(self.sigma_kv))

    def _needle_row(self, b: int, h: int, gain: float) -> np.ndarray:
        qb = self.q_bits()[b, 0, h].astype(np.uint32) << np.uint32(16)
        return bf16_bits(qb.view(np.float32) * np.float32(gain))

    def page_bits(self, page_ids) -> np.ndarray:
        """bf16 bits [len(page_ids), 64, 576] of the latent rows held by these physical pages.

        Slots past a request's context hold values too; they are never visible.
        """
        page_ids = np.asarray(page_ids, dtype=np.int64)
        out = np.empty((page_ids.size, PAGE, D), dtype=np.uint16)
        if page_ids.size == 0:
            return out
        chunks = np.unique(page_ids // _CHUNK)
        for c in chunks:
            x = _rng(self.seed, 1, int(c)).standard_normal((_CHUNK, PAGE, D), dtype=np.float32)
            block = bf16_bits(x * np.float32(self.sigma_kv))
            sel = np.nonzero(page_ids // _CHUNK == c)[0]
            out[sel] = block[page_ids[sel] - c * _CHUNK]
        for i, p in enumerate(page_ids):
            g = self.shared_tail.get(int(p))
            if g is not None:
                out[i, : self.tail_tokens] = self._tail_bits(g)
        for (b, t, h, gain) in self.needles:
            if t < int(self.context_lens[b]):
                phys = int(self.block_table[b, t // PAGE])
                hit = np.nonzero(page_ids == phys)[0]
                if hit.size:
                    out[hit, t % PAGE] = self._needle_row(b, h, gain)
        return out

    def all_page_bits(self) -> np.ndarray:
        return self.page_bits(np.arange(self.num_pages))

    def tensor_scale(self) -> np.float32:
        """Per-tensor scale calibrated on the data: largest |value| over the pool and
        the new rows, divided by the largest finite e4m3 value (a calibration
        recipe of this workload; the pages do not say how the scale is chosen)."""
        amax = 0.0
        for c0 in range(0, self.num_pages, 256):
            bits = self.page_bits(np.arange(c0, min(c0 + 256, self.num_pages)))
            amax = max(amax, float(np.abs((bits.astype(np.uint32) << 16).view(np.float32)).max()))
        if self.n_new:
            nb = self.new_row_bits()
            amax = max(amax, float(np.abs((nb.astype(np.uint32) << 16).view(np.float32)).max()))
        return np.float32(np.float32(amax) / np.float32(E4M3_MAX))

    # ----------------------------------------------------------------- sizes
    def kv_row_bytes(self) -> int:
        """Bytes of one cached latent row as stored (codes, plus a per-token scale)."""
        if self.cache_dtype == "bf16":
            return 2 * D
        return D + (4 if self.scale_mode == "token" else 0)

    def total_tokens(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum())

    def unique_tokens(self) -> int:
        """Tokens in distinct physical pages that some request can see."""
        seen = {}
        for b in range(self.B):
            L = int(self.seq_lens[b])
            for j, p in enumerate(self.pages_of(b)):
                seen[int(p)] = max(seen.get(int(p), 0), min(PAGE, L - j * PAGE))
        return int(sum(seen.values()))


# --------------------------------------------------------------------- builders
def _assign_pages(rng, logical: list):
    """logical: list over requests of lists of page keys (shared keys repeat).
    Returns a dict key -> physical id, drawn as a random permutation."""
    keys = []
    seen = set()
    for lst in logical:
        for k in lst:
            if k not in seen:
                seen.add(k)
                keys.append(k)
    perm = rng.permutation(len(keys)).astype(np.int32)
    return {k: int(perm[i]) for i, k in enumerate(keys)}, len(keys)


def custom(
    name="custom",
    *,
    B=1,
    n_q=1,
    H=64,
    context_lens=(100,),
    cache_dtype="fp8",
    scale_mode="token",
    permute=True,
    identity=False,
    append=None,
    seed=0,
    sigma_q=1.0,
    sigma_kv=0.5,
    share_groups=0,
    share_tokens=0,
    extra_blocks=0,
    needles=(),
) -> Workload:
    """Build a workload from explicit sizes.

    ``context_lens`` are tokens cached before the step; the step appends
    ``append`` rows per request (default ``n_q`` for an FP8 cache, 0 for bf16),
    so ``seq_lens = context_lens + append``.  ``share_groups`` groups of
    consecutive requests share the physical pages of a ``share_tokens`` prefix
    (whole pages shared; the remainder is repeated into each private page).
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    assert ctx.size == B
    if append is None:
        append = n_q if cache_dtype == "fp8" else 0
    seq = (ctx + append).astype(np.int32)
    npages = -(-seq // PAGE)
    max_blocks = int(npages.max()) + extra_blocks if B else 1
    rng = _rng(seed, 0)
    shared_pages = share_tokens // PAGE if share_groups else 0
    tail = share_tokens % PAGE if share_groups else 0
    group_of = {}
    if share_groups:
        per = B // share_groups
        for b in range(B):
            group_of[b] = b // per if b // per < share_groups else None
    logical = []
    for b in range(B):
        g = group_of.get(b)
        keys = []
        for j in range(int(npages[b])):
            if g is not None and j < shared_pages:
                keys.append(("s", g, j))
            else:
                keys.append(("p", b, j))
        logical.append(keys)
    if identity:
        assert not share_groups
        phys = {("p", b, j): b * max_blocks + j for b in range(B) for j in range(int(npages[b]))}
        num_pages = B * max_blocks
    else:
        phys, num_pages = _assign_pages(rng, logical)
        if not permute:
            order = {}
            for lst in logical:
                for k in lst:
                    order.setdefault(k, len(order))
            phys = order
    bt = np.full((B, max_blocks), -1, dtype=np.int32)
    shared_tail = {}
    for b in range(B):
        for j, k in enumerate(logical[b]):
            bt[b, j] = phys[k]
        g = group_of.get(b)
        if g is not None and tail and shared_pages < npages[b]:
            shared_tail[int(bt[b, shared_pages])] = g
    return Workload(
        name=name,
        B=B,
        n_q=n_q,
        H=H,
        seq_lens=seq,
        n_new=int(append),
        block_table=bt,
        num_pages=int(num_pages),
        cache_dtype=cache_dtype,
        scale_mode=scale_mode if cache_dtype == "fp8" else "none",
        seed=seed,
        sigma_q=sigma_q,
        sigma_kv=sigma_kv,
        shared_tail=shared_tail,
        tail_tokens=int(tail),
        needles=tuple(needles),
    )


def _lognormal_lengths(rng, n, median, sigma, lo, hi, total):
    x = rng.lognormal(mean=math.log(median), sigma=sigma, size=n)
    x = np.clip(x, lo, hi)
    x = x * (total / x.sum())
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


CONFIG_NAMES = (
    "tiny_bf16",
    "fp8_single_100k",
    "fp8_prefix_shared_b32",
    "fp8_pool_b64",
    "bf16_pool_b32",
    "fp8_spec4_b16",
)
# extend / prefill: a chunk of new tokens, causal among themselves, over a cached context
EXTEND_NAMES = (
    "bf16_extend_16k",
    "fp8_extend_16k",
)


def make(name: str, seed: int = 0) -> Workload:
    """The named workloads.

    * ``tiny_bf16``: 2 requests, 16 heads, 1 query, lengths {1000, 777}, bf16
      cache and query N(0,1), identity page map.
    * ``fp8_single_100k``: 1 request, 64 heads, 1 query, 100,000 cached tokens
      (+1 appended), e4m3 codes with one per-tensor scale, cache N(0,0.5)
      before quantisation, randomly permuted physical pages.
    * ``fp8_prefix_shared_b32``: 32 requests, lengths U[60k,140k]; 4 groups of 8
      share a 50,000-token prefix (781 whole shared pages; the 16-token
      remainder repeated in each private page); per-token scales.
    * ``fp8_pool_b64``: 64 requests, lognormal lengths (median 16k, sigma 0.8,
      clipped to [1k,128k]) rescaled to about 1.37M cached tokens; per-token
      scales.
    * ``bf16_pool_b32``: the first 32 requests of ``fp8_pool_b64`` with a bf16
      cache (the capacity comparison).
    * ``fp8_spec4_b16``: 16 requests, 4 causal query tokens each, 142,000
      cached tokens (+4 appended), per-token scales.
    * ``bf16_extend_16k``: 1 request, 64 heads, 512 new tokens (queries,
      causal among themselves) at the end of 16,896 tokens in a bf16 cache
      (the new rows already in it), randomly permuted pages.
    * ``fp8_extend_16k``: the same shape on an e4m3 cache with per-token
      scales, the 512 new rows appended by the step.
    """
    rs = _rng(seed, 0)
    if name == "tiny_bf16":
        w = custom(name, B=2, n_q=1, H=16, context_lens=(1000, 777), cache_dtype="bf16",
                   identity=True, seed=seed, sigma_q=1.0, sigma_kv=1.0)
    elif name == "fp8_single_100k":
        w = custom(name, B=1, n_q=1, H=64, context_lens=(100_000,), cache_dtype="fp8",
                   scale_mode="tensor", seed=seed)
    elif name == "fp8_prefix_shared_b32":
        ctx = rs.integers(60_000, 140_001, size=32)
        w = custom(name, B=32, n_q=1, H=64, context_lens=tuple(ctx), cache_dtype="fp8",
                   scale_mode="token", seed=seed, share_groups=4, share_tokens=50_000)
    elif name in ("fp8_pool_b64", "bf16_pool_b32"):
        ctx = _lognormal_lengths(rs, 64, 16_000, 0.8, 1_000, 128_000, 1_370_000)
        if name == "fp8_pool_b64":
            w = custom(name, B=64, n_q=1, H=64, context_lens=tuple(ctx), cache_dtype="fp8",
                       scale_mode="token", seed=seed)
        else:
            w = custom(name, B=32, n_q=1, H=64, context_lens=tuple(ctx[:32]), cache_dtype="bf16",
                       seed=seed)
    elif name == "fp8_spec4_b16":
        w = custom(name, B=16, n_q=4, H=64, context_lens=(142_000,) * 16, cache_dtype="fp8",
                   scale_mode="token", seed=seed)
    elif name == "bf16_extend_16k":
        w = custom(name, B=1, n_q=512, H=64, context_lens=(16_896,), cache_dtype="bf16", seed=seed)
    elif name == "fp8_extend_16k":
        w = custom(name, B=1, n_q=512, H=64, context_lens=(16_384,), cache_dtype="fp8",
                   scale_mode="token", seed=seed)
    else:
        raise KeyError(f"unknown workload {name!r}; known: {CONFIG_NAMES + EXTEND_NAMES}")
    w.name = name
    return w
