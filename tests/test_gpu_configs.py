"""GPU parity at the named workloads' full sizes, in the launch configuration the
benchmark times (planned split-KV over all 256 CUs).  The oracle recomputes every
row of a sample of requests (shortest, longest, a sharing pair, ...) one
request at a time; the tiny workload is checked whole."""

import numpy as np
import pytest

import synth

from _gpu import GpuState, compare, log, oracle_decode

pytestmark = pytest.mark.gpu


def _sample(w):
    L = w.seq_lens
    picks = {int(np.argmin(L)), int(np.argmax(L)), 0, w.B - 1}
    if w.name == "fp8_prefix_shared_b32":
        # every sharer of group 0, two members of group 1 and of group 2
        picks |= set(range(8)) | {8, 9, 16, 17}
    return sorted(picks)


@pytest.mark.parametrize("name", synth.CONFIG_NAMES)
def test_named_workload_full_size(name):
    w = synth.make(name)
    log(f"{name}: B={w.B} n_q={w.n_q} H={w.H} tokens={w.total_tokens()} pages={w.num_pages}")
    g = GpuState(w)
    log(f"{name}: cache built on the GPU")
    out, lse = g.step()
    st = g.last_step
    log(f"{name}: step done (pages_per_split={st.pps}, max_splits={st.max_splits})")
    reqs = None if name == "tiny_bf16" else _sample(w)
    ref_o, ref_l = oracle_decode(w, requests=reqs)
    log(f"{name}: oracle done for requests {reqs}")
    compare(out, lse, ref_o, ref_l, requests=reqs, tag=name)
    if name == "fp8_prefix_shared_b32":
        # requests of one group see the same prefix pages; their outputs differ
        # only through their private suffixes and queries — both must be right
        assert not np.array_equal(out[8], out[9])


@pytest.mark.parametrize("name", synth.EXTEND_NAMES)
def test_extend_workload_full_size(name):
    """A 512-token extend chunk over a 16,896-token context at full size: the
    step as the benchmark runs it, and the oracle on a sample of queries (the
    first, the last, and some between) with every head."""
    w = synth.make(name)
    log(f"{name}: B={w.B} n_q={w.n_q} H={w.H} tokens={w.total_tokens()} pages={w.num_pages}")
    g = GpuState(w)
    out, lse = g.step()
    st = g.last_step
    log(f"{name}: step done (pages_per_split={st.pps}, max_splits={st.max_splits})")
    from oracle import mla as omla
    from _gpu import oracle_state

    queries = [0, 1, 63, 64, 255, 256, 500, 510, 511]
    cache, scales, ts = oracle_state(w)
    ref_o, ref_l = omla.decode_ref(w.q_bits(), cache, scales, w.block_table, w.seq_lens, n_q=w.n_q, H=w.H,
                                   cache_dtype=w.cache_dtype, scale_mode=w.scale_mode,
                                   softmax_scale=w.softmax_scale, tensor_scale=ts, queries=queries)
    log(f"{name}: oracle done for queries {queries}")
    compare(out[:, queries], lse[:, queries], ref_o[:, queries], ref_l[:, queries], tag=name)
