"""Planted mistakes in the oracle (on the CPU only): each plausible slip —
a wrong index, a dropped term, a transposed operand, an off-by-one mask, the
wrong tie rule — must make at least one pin fail.  This is evidence that the
pins constrain the oracle rather than restate it."""
import numpy as np
import pytest

import test_oracle_attention as att
import test_oracle_block_manager as obm
import test_oracle_codecs as cod
import test_oracle_paging as pag
from oracle import block_manager, codecs, paged

_orig_attend = paged.attend
_orig_gather = paged.gather
_orig_swap = paged.swap_blocks
_orig_pairs_inside = paged._pairs_inside


def _attend_no_scale(q, K, V, scale, visible=None):
    return _orig_attend(q, K, V, 1.0, visible)


def _attend_transposed(q, K, V, scale, visible=None):
    # Weights applied to K instead of V.
    return _orig_attend(q, K, K, scale, visible)


def _attend_no_max_shift(q, K, V, scale, visible=None):
    q, K, V = (np.asarray(a, np.float64) for a in (q, K, V))
    if visible is not None:
        K, V = K[visible], V[visible]
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    with np.errstate(over="ignore", invalid="ignore"):
        p = np.exp((K @ q) * float(np.float32(scale)))
        return (p @ V) / p.sum()


def _attend_causal_off_by_one(q, K, V, scale, visible=None):
    if visible is not None:
        visible = np.roll(visible, -1)
        visible[-1] = False
    return _orig_attend(q, K, V, scale, visible)


def _gather_wrong_offset(pool, table_row, length):
    out = _orig_gather(pool, table_row, length + 1)
    return out[1:]


def _kv_head_modulo(h, num_heads, num_kv_heads):
    return h % num_kv_heads


def _merge_without_rescale(states):
    w = np.array([l for _, l, _ in states])
    o = np.stack([o for _, _, o in states])
    return (w[:, None] * o).sum(0) / w.sum()


def _encode_ties_away(x):
    x = np.asarray(x, np.float32)
    out = codecs._orig_f32_to_e4m3fn(x)
    pos = codecs.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    a = np.abs(x.astype(np.float64))
    tie = np.isin(a, mids)
    up = np.searchsorted(pos, a)
    return np.where(tie, (up | (out & 0x80)).astype(np.uint8), out)


def _swap_k_v_crossed(src_k, src_v, dst_k, dst_v, pairs):
    return _orig_swap(src_v, src_k, dst_k, dst_v, pairs)


def _swap_reversed_pairs(src_k, src_v, dst_k, dst_v, pairs):
    p = np.asarray(pairs, np.int64).reshape(-1, 2)[:, ::-1]
    return _orig_swap(src_k, src_v, dst_k, dst_v, p)


def _pairs_wrap_negative(pairs, src_blocks, dst_blocks):
    p = np.asarray(pairs, np.int64).reshape(-1, 2)
    return np.stack([p[:, 0] % src_blocks, p[:, 1] % dst_blocks], axis=1)


MUTATIONS = [
    ("attend", _attend_no_scale, [att.test_decode_matches_torch_sdpa_tiny]),
    ("attend", _attend_transposed, [att.test_decode_matches_torch_sdpa_tiny]),
    ("attend", _attend_no_max_shift, [att.test_decode_closed_forms]),
    ("attend", _attend_causal_off_by_one, [att.test_prefill_matches_sdpa_with_offset_causal_mask]),
    ("gather", _gather_wrong_offset, [pag.test_lib_worked_example_slots_and_gather]),
    ("_kv_head", _kv_head_modulo, [att.test_decode_matches_torch_sdpa_tiny]),
    ("lse_merge", _merge_without_rescale, [att.test_split_merge_equals_unsplit]),
    ("swap_blocks", _swap_k_v_crossed, [pag.test_swap_blocks_element_by_element]),
    ("swap_blocks", _swap_reversed_pairs, [pag.test_swap_out_and_in_restores_the_sequence]),
    ("_pairs_inside", _pairs_wrap_negative, [pag.test_copy_blocks_skips_pairs_outside_the_pool,
                                             pag.test_swap_blocks_element_by_element]),
]


class _LifoManager(block_manager.BlockManager):
    def _take(self):
        if not self.free:
            raise block_manager.OutOfBlocks("no free block")
        b = self.free.pop()
        self.ref[b] = 1
        return b


class _CopyFullSharedManager(block_manager.BlockManager):
    """Copies a shared last block even when it is full."""

    def append(self, sids):
        slots, pairs = [], []
        for sid in sids:
            s = self.seqs[sid]
            last = s["blocks"][-1] if s["blocks"] else None
            if last is not None and self.ref[last] > 1 and s["len"] % self.block_size == 0:
                fresh = self._take()
                self.ref[last] -= 1
                s["blocks"][-1] = fresh
                pairs.append((last, fresh))
            sl, pr = block_manager.BlockManager.append(self, [sid])
            slots += sl
            pairs += pr
        return slots, pairs


class _CowKeepsReferenceManager(block_manager.BlockManager):
    """Forgets to drop the shared block's reference on copy-on-write."""

    def append(self, sids):
        slots, pairs = block_manager.BlockManager.append(self, sids)
        for src, _ in pairs:
            self.ref[src] += 1
        return slots, pairs


class _SwapForgetsReferencesManager(block_manager.BlockManager):
    """Gives every moved block a single reference on the other side."""

    def _move(self, sids, to_host):
        pairs = block_manager.BlockManager._move(self, sids, to_host)
        ref = self.host_ref if to_host else self.ref
        for _, d in pairs:
            ref[d] = 1
        return pairs


def _hash_without_parent(parent, tokens, extra=0):
    return _orig_block_hash(0, tokens, extra)


def _hash_without_extra(parent, tokens, extra=0):
    return _orig_block_hash(parent, tokens, 0)


_orig_block_hash = block_manager.block_hash


@pytest.mark.parametrize("fn,pins", [
    (_hash_without_parent, [obm.test_system_prompt_is_shared_through_the_cache,
                            lambda: obm.test_random_prefix_cache_traces_keep_every_sequence_readable(0)]),
    (_hash_without_extra, [obm.test_block_hash_is_chained]),
])
def test_planted_prefix_hash_mistake_is_caught(monkeypatch, fn, pins):
    monkeypatch.setattr(block_manager, "block_hash", fn)
    monkeypatch.setattr(obm, "block_hash", fn)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()


class _NoTouchManager(block_manager.BlockManager):
    """Reuses cached blocks without taking them off the free list."""

    def add_prompt(self, sid, tokens, extra=0):
        free = list(self.free)
        out = block_manager.BlockManager.add_prompt(self, sid, tokens, extra)
        for b in self.seqs[sid]["blocks"]:
            if b in free and b not in self.free and self.ref[b] == 1 and b in self.cached:
                self.free.append(b)
        return out


class _SwapInKeepsCacheManager(block_manager.BlockManager):
    """Leaves a cached device block in the cache when swap-in overwrites it."""

    def _move(self, sids, to_host):
        before = dict(self.cached)
        pairs = block_manager.BlockManager._move(self, sids, to_host)
        if not to_host:
            for _, d in pairs:
                if d in before and d not in self.cached and before[d][0] not in self.table_of:
                    self.cached[d] = before[d]
                    self.table_of[before[d][0]] = d
        return pairs


@pytest.mark.parametrize("cls,pins", [
    (_LifoManager, [obm.test_deep_interleaved_figure]),
    (_CopyFullSharedManager, [obm.test_full_shared_block_is_never_copied]),
    (_SwapForgetsReferencesManager, [obm.test_swap_out_and_in_by_hand,
                                     lambda: obm.test_random_traces_with_swap_keep_every_sequence_readable(0)]),
    (_SwapInKeepsCacheManager, [lambda: [obm.test_random_prefix_cache_traces_keep_every_sequence_readable(i)
                                         for i in range(6)]]),
    (_NoTouchManager, [lambda: obm.test_random_prefix_cache_traces_keep_every_sequence_readable(1)]),
    (_CowKeepsReferenceManager, [obm.test_deep_prefix_sharing_and_copy_on_write,
                                 lambda: obm.test_random_traces_keep_every_sequence_readable(0)]),
])
def test_planted_block_manager_mistake_is_caught(monkeypatch, cls, pins):
    monkeypatch.setattr(obm, "BlockManager", cls)
    for pin in pins:
        with pytest.raises((AssertionError, block_manager.OutOfBlocks)):
            pin()


@pytest.mark.parametrize("name,fn,pins", MUTATIONS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fn, pins):
    monkeypatch.setattr(paged, name, fn)
    for pin in pins:
        with pytest.raises((AssertionError, ValueError, IndexError)):
            if pin is att.test_split_merge_equals_unsplit:
                pin(48)
            else:
                pin()


def test_planted_tie_rule_is_caught(monkeypatch):
    monkeypatch.setattr(codecs, "_orig_f32_to_e4m3fn", codecs.f32_to_e4m3fn, raising=False)
    monkeypatch.setattr(codecs, "f32_to_e4m3fn", _encode_ties_away)
    with pytest.raises(AssertionError):
        cod.test_e4m3fn_encode_ties_go_to_even_code()
