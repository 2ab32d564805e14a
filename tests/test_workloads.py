"""Host checks of the seeded workload generators (no GPU): the token-budget
chunking of chunked prefill, and the layout of the budget-step workload."""
import numpy as np
import pytest

from oracle import paged as opg
from paged_kv_cache_11_amd import workloads as wl


@pytest.mark.parametrize("budget", [512, 2048, 1000])
def test_budget_chunks_cover_every_prompt_once(budget):
    """Each step takes at most the budget (exactly the budget while prompts
    remain); chunks of a prompt are contiguous and in order; over all steps
    every prompt is covered exactly once; at most one prompt is cut per
    step and it continues first in the next step."""
    lens = np.random.default_rng(budget).integers(1, 3000, size=30)
    covered = [0] * len(lens)
    step, total = 0, int(lens.sum())
    while True:
        chunks = wl.budget_chunks(lens, budget, step)
        if not chunks:
            break
        n = sum(c[2] for c in chunks)
        assert n <= budget and (n == budget or sum(covered) + n == total)
        for i, (p, first, cnt) in enumerate(chunks):
            assert first == covered[p] and cnt > 0
            covered[p] += cnt
            if i > 0:
                assert first == 0  # only the first chunk of a step continues a prompt
            if i < len(chunks) - 1:
                assert covered[p] == lens[p]  # only the last chunk may be cut
        step += 1
    assert covered == [int(x) for x in lens]
    assert step == -(-total // budget)


@pytest.mark.parametrize("budget", [512, 2048])
def test_budget_step_workload_layout(budget):
    b = wl.make(f"chunked_prefill_budget{budget}_bf16")
    qs, ends = b.chunk_query_start, b.chunk_seq_lens
    assert qs[-1] == budget == b.chunk_q.shape[0]
    assert [c[2] for c in b.chunks] == list(np.diff(qs))
    assert [c[1] + c[2] for c in b.chunks] == list(ends)
    assert b.chunks[0][1] > 0  # the step continues a prompt cut by the previous one
    # Every slot is inside the pool, used once, and at its table position.
    assert len(np.unique(b.slot_mapping)) == len(b.slot_mapping) == int(ends.sum())
    cur = 0
    for c, L in enumerate(ends):
        assert np.array_equal(b.slot_mapping[cur:cur + L], opg.slots_of(b.chunk_block_tables[c], int(L), 16))
        cur += int(L)
