"""Structure of the seeded synthetic workloads (CPU only)."""

import numpy as np
import pytest

import synth


@pytest.mark.parametrize("name", synth.CONFIG_NAMES)
def test_workload_structure(name):
    w = synth.make(name)
    assert w.block_table.dtype == np.int32 and w.seq_lens.dtype == np.int32
    used = []
    for b in range(w.B):
        pages = w.pages_of(b)
        assert pages.size == -(-int(w.seq_lens[b]) // 64)
        assert np.all((pages >= 0) & (pages < w.num_pages))
        assert len(set(pages.tolist())) == pages.size  # a request never maps a page twice
        assert np.all(w.block_table[b, pages.size:] == -1)
        used.append(pages)
    if name != "tiny_bf16":  # the identity map of the tiny case leaves gaps on purpose
        assert np.unique(np.concatenate(used)).size == w.num_pages  # no unused pages


def test_named_shapes():
    assert synth.make("tiny_bf16").seq_lens.tolist() == [1000, 777]
    w = synth.make("fp8_single_100k")
    assert (w.B, w.H, w.n_q, int(w.seq_lens[0]), w.scale_mode) == (1, 64, 1, 100_001, "tensor")
    w = synth.make("fp8_spec4_b16")
    assert (w.B, w.n_q, w.H) == (16, 4, 64) and np.all(w.seq_lens == 142_004)
    w = synth.make("fp8_pool_b64")
    ctx = w.context_lens
    assert abs(int(ctx.sum()) - 1_370_000) < 200 and ctx.min() >= 1000 and ctx.max() <= 128_000
    w = synth.make("fp8_prefix_shared_b32")
    assert w.context_lens.min() >= 60_000 and w.context_lens.max() <= 140_000


def test_prefix_sharing_layout():
    w = synth.make("fp8_prefix_shared_b32")
    for g in range(4):
        members = range(8 * g, 8 * g + 8)
        first = w.block_table[8 * g, :781]
        for b in members:
            assert np.array_equal(w.block_table[b, :781], first)
    # different groups share nothing
    groups = [set(w.block_table[8 * g, :781].tolist()) for g in range(4)]
    assert all(not (groups[i] & groups[j]) for i in range(4) for j in range(i + 1, 4))
    # the 16-token remainder of the 50k prefix is repeated in each private page
    b0, b1 = 8, 9
    p0, p1 = w.block_table[b0, 781], w.block_table[b1, 781]
    assert p0 != p1
    v = w.page_bits([p0, p1])
    assert np.array_equal(v[0, :16], v[1, :16]) and not np.array_equal(v[0, 16:], v[1, 16:])
    assert w.unique_tokens() < w.total_tokens()


def test_determinism_and_page_streams():
    w1 = synth.make("fp8_pool_b64")
    w2 = synth.make("fp8_pool_b64")
    assert np.array_equal(w1.block_table, w2.block_table)
    a = w1.page_bits([5, 900, 77])
    b = w1.page_bits(np.arange(w1.num_pages))[[5, 900, 77]]
    assert np.array_equal(a, b)
    assert np.array_equal(w1.q_bits(), w2.q_bits())


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38], dtype=np.float32)
    bits = synth.bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: goes to 1 (even)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1.015625)
    assert back[3] == -2.5
