"""The library's host block manager driving the device calls end to end.

The library's manager (pa_bm_*) gives the slots, the copy-on-write pairs,
the swap pairs and the block tables; the device runs pa_copy_blocks before
pa_cache_write at every step, pa_swap_blocks to and from a pinned host pool
when sequences are preempted and resumed, and pa_decode at the end.  The
reference manager and the oracle's block copy, swap, cache write and decode
replay the same operations on the host.  Checked:

* the manager's slots and pairs equal the reference manager's at every step;
* the device pools (and the host pools) equal the oracle's bit for bit (all
  start NaN-filled, so a stray write or a missed copy shows);
* each sequence reads back, through its table, exactly the rows of its own
  tokens (prompt, then its own appended tokens: nothing of a sibling);
* pa_decode through the manager's tables matches the oracle's decode."""
import numpy as np
import pytest
import torch

import pa_gpu as G
from oracle import paged as opg
from oracle.block_manager import BlockManager as RefManager
from paged_kv_cache_11_amd import binding as pa
from paged_kv_cache_11_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _rows_bits(rows, kv_dtype, scale):
    """Raw pool words of token rows [n, Hkv, D] as the oracle's cache write
    stores them, through a pool of one-token blocks (no paging involved)."""
    n, Hkv, D = rows.shape
    kp = wl.poisoned_pool(max(n, 1), Hkv, 1, D, kv_dtype)
    vp = wl.poisoned_pool(max(n, 1), Hkv, 1, D, kv_dtype)
    bits = wl.storage_bits(wl.storage_tensor(rows, "bf16"))
    opg.cache_write(kp, vp, kv_dtype, bits, bits, "bf16", np.arange(n), scale, scale)
    return kp[:n, :, 0, :]


class Replay:
    """Both managers, the device pools (plus a pinned host pool) and the
    oracle's pools, driven by the same operations."""

    def __init__(self, kv, bs, Hq, Hkv, nb, nh=0, seed=0):
        D = 128
        self.kv, self.bs, self.Hq, self.Hkv, self.D = kv, bs, Hq, Hkv, D
        self.rng = np.random.default_rng(seed)
        self.k_scale = self.v_scale = 0.5 if kv == "fp8" else 1.0
        self.m, self.r = pa.BlockManager(nb, bs, num_host_blocks=nh), RefManager(nb, bs, num_host_blocks=nh)
        self.b = wl.PagedBatch("bm", Hq, Hkv, D, bs, nb, "bf16", "bf16", kv, 1.0 / np.sqrt(D),
                               np.zeros((1, Hq, D), np.float32), np.zeros((1, Hkv, D), np.float32),
                               np.zeros((1, Hkv, D), np.float32), np.zeros(1, np.int64),
                               np.zeros(1, np.int32), np.zeros((1, 1), np.int32),
                               k_scale=self.k_scale, v_scale=self.v_scale)
        self.kp, self.vp = G.gpu_pool(self.b)
        self.okp = wl.poisoned_pool(nb, Hkv, bs, D, kv)
        self.ovp = wl.poisoned_pool(nb, Hkv, bs, D, kv)
        if nh:
            shape = (nh, Hkv, bs, D)
            self.hk = torch.empty(shape, dtype=G.TORCH_DT[kv], pin_memory=True)
            self.hv = torch.empty(shape, dtype=G.TORCH_DT[kv], pin_memory=True)
            for t in (self.hk, self.hv):
                t.view(G.INT_VIEW[kv]).fill_(wl.POISON_BITS[kv])
            self.ohk = wl.poisoned_pool(nh, Hkv, bs, D, kv)
            self.ohv = wl.poisoned_pool(nh, Hkv, bs, D, kv)
        self.k_rows, self.v_rows = [], []  # every token ever written, in order
        self.content = {}                  # sequence id -> its token ids
        self.n_pairs = self.n_swapped = 0

    def _write(self, slots, owners):
        n = len(slots)
        k = self.rng.standard_normal((n, self.Hkv, self.D)).astype(np.float32)
        v = self.rng.standard_normal((n, self.Hkv, self.D)).astype(np.float32)
        first = len(self.k_rows)
        self.k_rows.extend(k)
        self.v_rows.extend(v)
        for i, sid in enumerate(owners):
            self.content[sid].append(first + i)
        kt, vt = wl.storage_tensor(k, "bf16"), wl.storage_tensor(v, "bf16")
        pa.pa_cache_write(kt.to(G.DEV), vt.to(G.DEV), self.kp, self.vp,
                          torch.from_numpy(np.ascontiguousarray(slots, np.int64)).to(G.DEV),
                          self.k_scale, self.v_scale)
        opg.cache_write(self.okp, self.ovp, self.kv, wl.storage_bits(kt), wl.storage_bits(vt),
                        "bf16", np.asarray(slots, np.int64), self.k_scale, self.v_scale)

    def add(self, sid, n):
        slots = self.m.add(sid, n)
        assert list(slots) == self.r.add(sid, n)
        self.content[sid] = []
        self._write(slots, [sid] * n)

    def fork(self, parent, child):
        self.m.fork(parent, child)
        self.r.fork(parent, child)
        self.content[child] = list(self.content[parent])

    def release(self, sid):
        self.m.release(sid)
        self.r.release(sid)
        del self.content[sid]

    def append(self, ids, step=None):
        slots, pairs = self.m.append(ids)
        want_slots, want_pairs = self.r.append(ids)
        assert list(slots) == want_slots and [tuple(p) for p in pairs] == want_pairs, step
        if len(pairs):
            pa.pa_copy_blocks(self.kp, self.vp, torch.from_numpy(np.ascontiguousarray(pairs)).to(G.DEV))
            opg.copy_blocks(self.okp, self.ovp, pairs)
            self.n_pairs += len(pairs)
        self._write(slots, ids)

    def swap_out(self, ids):
        pairs = self.m.swap_out(ids)
        assert [tuple(p) for p in pairs] == self.r.swap_out(ids)
        pa.pa_swap_blocks(self.kp, self.vp, self.hk, self.hv, torch.from_numpy(pairs).to(G.DEV))
        opg.swap_blocks(self.okp, self.ovp, self.ohk, self.ohv, pairs)
        self.n_swapped += len(pairs)
        # The freed device blocks are garbage from here on, on both sides.
        idx = torch.from_numpy(np.ascontiguousarray(pairs[:, 0])).to(G.DEV)
        for t, o in ((self.kp, self.okp), (self.vp, self.ovp)):
            t.view(G.INT_VIEW[self.kv])[idx] = 0
            o[pairs[:, 0]] = 0

    def swap_in(self, ids):
        pairs = self.m.swap_in(ids)
        assert [tuple(p) for p in pairs] == self.r.swap_in(ids)
        pa.pa_swap_blocks(self.hk, self.hv, self.kp, self.vp, torch.from_numpy(pairs).pin_memory())
        opg.swap_blocks(self.ohk, self.ohv, self.okp, self.ovp, pairs)
        self.n_swapped += len(pairs)

    def check(self):
        """Pools bit for bit, each live sequence's rows, and decode."""
        torch.cuda.synchronize()
        assert G.raw_equal(self.kp, self.okp), "K pool differs from the oracle's"
        assert G.raw_equal(self.vp, self.ovp), "V pool differs from the oracle's"
        if hasattr(self, "hk"):
            assert G.raw_equal(self.hk, self.ohk) and G.raw_equal(self.hv, self.ohv), "host pool"
        ids = sorted(i for i in self.content if not self.r.is_swapped(i))
        width = max(len(self.r.table(i)) for i in ids) + 2
        tables, lens = self.m.block_tables(ids, width)
        for row, ln, sid in zip(tables, lens, ids):
            assert list(row[:len(self.r.table(sid))]) == self.r.table(sid) and ln == self.r.seq_len(sid)
        gk = self.kp.cpu()
        gk = gk.view(torch.int16).numpy().view(np.uint16) if self.kv == "bf16" else gk.numpy()
        want_all = _rows_bits(np.stack(self.k_rows), self.kv, self.k_scale)
        for row, ln, sid in zip(tables, lens, ids):
            got = opg.gather(gk, row, int(ln))
            assert np.array_equal(got, want_all[self.content[sid]]), f"sequence {sid} reads foreign rows"
        q = self.rng.standard_normal((len(ids), self.Hq, self.D)).astype(np.float32)
        qt = wl.storage_tensor(q, "bf16").to(G.DEV)
        q64 = G.query_f64(qt)
        otab = np.array([self.r.table(i) + [-1] * (width - len(self.r.table(i))) for i in ids], np.int32)
        ref = opg.paged_decode(q64, self.okp, self.ovp, otab,
                               np.array([self.r.seq_len(i) for i in ids], np.int32), self.b.scale,
                               kv_dtype=self.kv, k_scale=self.k_scale, v_scale=self.v_scale)
        for ps in (pa.PA_PARTITION_BALANCED, 0):
            got = G.run_decode(self.b, self.kp, self.vp, qt, partition_size=ps, seq_lens=lens, tables=tables)
            G.assert_close(got, ref, self.kv, f"decode through the manager's tables, partition {ps}")


@pytest.mark.parametrize("kv,bs,Hq,Hkv", [
    ("bf16", 16, 32, 8), ("fp8", 32, 64, 8), ("bf16", 128, 32, 8), ("fp8", 16, 16, 2),
])
def test_sampling_and_beam_search_through_the_manager(kv, bs, Hq, Hkv):
    """Parallel sampling and beam search over two shared prompts: two
    prompts (ending inside a block) forked into 6 and 4 samples, grown token
    by token; every ninth step one sample is dropped and a survivor forked."""
    prompts = {0: 1500 + bs // 2 + 3, 1: 700 + 5}
    steps = 3 * bs + 7
    nb = sum(-(-p // bs) for p in prompts.values()) + 12 * (steps // bs + 3) + 16
    t = Replay(kv, bs, Hq, Hkv, nb, seed=bs * 10 + Hq + (kv == "fp8"))
    for sid, n in prompts.items():
        t.add(sid, n)
    next_id = 2
    for parent, copies in ((0, 5), (1, 3)):
        for _ in range(copies):
            t.fork(parent, next_id)
            next_id += 1
    for step in range(steps):
        if step % 9 == 8:
            live = sorted(t.content)
            t.release(live[int(t.rng.integers(len(live)))])
            t.fork(sorted(t.content)[int(t.rng.integers(len(t.content)))], next_id)
            next_id += 1
        t.append(sorted(t.content), step)
    assert t.n_pairs >= len(t.content) - 2, "the trace should copy shared blocks"
    G.say(f"[{kv} bs{bs} {Hq}q/{Hkv}kv] {len(t.content)} samples, {t.n_pairs} block copies, "
          f"{nb - t.m.num_free()} of {nb} blocks in use")
    t.check()


@pytest.mark.parametrize("kv,bs,Hq,Hkv", [("bf16", 16, 32, 8), ("fp8", 32, 64, 8), ("bf16", 64, 32, 8)])
def test_preemption_by_swap_through_the_manager(kv, bs, Hq, Hkv):
    """A device pool too small for everyone: four requests decode; when the
    pool runs short the newest request group (a prompt and its two samples)
    is swapped out to a pinned host pool, the others take its freed blocks,
    then one finishes and the group is swapped back in and decodes on.  The
    freed blocks are overwritten between swap-out and swap-in, so a swap
    that did not happen shows in the pools and in decode."""
    lens = {0: 300, 1: 410, 2: 5 * bs + 3}
    t = Replay(kv, bs, Hq, Hkv, nb=sum(-(-n // bs) for n in lens.values()) + 10, nh=64,
               seed=97 + bs)
    for sid, n in lens.items():
        t.add(sid, n)
    t.fork(2, 3)
    t.fork(2, 4)
    group, others = [2, 3, 4], [0, 1]
    swapped_at = resumed_at = None
    for step in range(6 * bs):
        if resumed_at is not None and step == resumed_at + bs:
            break
        ids = [i for i in sorted(t.content) if not t.r.is_swapped(i)]
        need = sum(1 for i in ids if t.r.seq_len(i) % bs == 0 or t.r.ref[t.r.table(i)[-1]] > 1)
        if swapped_at is None and need > t.r.num_free():
            t.swap_out(group)
            swapped_at = step
            G.say(f"[{kv} bs{bs}] step {step}: swapped out {group} ({t.n_swapped} blocks)")
            continue
        if swapped_at is not None and resumed_at is None and step == swapped_at + 2 * bs:
            t.release(others[0])
            t.swap_in(group[::-1])
            resumed_at = step
            G.say(f"[{kv} bs{bs}] step {step}: released {others[0]}, swapped in {group[::-1]}")
            continue
        t.append(ids, step)
    assert swapped_at is not None and resumed_at is not None, (swapped_at, resumed_at)
    t.check()


def _prefix_rows(keys, Hkv, D, salt):
    """K or V rows of tokens whose whole context is named by ``keys``: each
    row is drawn from a generator seeded by its context key, so equal
    prefixes give equal rows and any other prefix gives other rows."""
    return np.stack([np.random.default_rng([salt, int(k)]).standard_normal((Hkv, D)).astype(np.float32)
                     for k in keys]) if len(keys) else np.zeros((0, Hkv, D), np.float32)


def _context_keys(tokens, extra):
    """A running key per position naming (extra, tokens[0..t])."""
    keys, k = [], (int(extra) * 1000003 + 17) % (1 << 61)
    for t in tokens:
        k = (k * 1000003 + int(t) + 1) % (1 << 61)
        keys.append(k)
    return keys


@pytest.mark.parametrize("kv,bs,Hq,Hkv", [("bf16", 16, 32, 8), ("fp8", 32, 64, 8)])
def test_prefix_cache_through_the_manager(kv, bs, Hq, Hkv):
    """Automatic prefix caching end to end.  Requests share a 2000-token
    system prompt (one with another adapter, one sharing only its first
    half); each writes K/V only past its cached prefix; some decode with
    token ids (filling blocks that enter the cache), some finish, and new
    requests reuse their released cached blocks.  Decode of every live
    sequence through the manager's tables is compared with attention over
    its own context computed without any paging, from rows that depend on
    the whole prefix — a wrong cache hit cannot pass."""
    D = 128
    rng = np.random.default_rng(41 + bs)
    nb = 420 if bs == 16 else 220
    ks = vs = 0.5 if kv == "fp8" else 1.0
    m = pa.BlockManager(nb, bs, prefix_caching=True)
    r = RefManager(nb, bs, prefix_caching=True)
    b = wl.PagedBatch("apc", Hq, Hkv, D, bs, nb, "bf16", "bf16", kv, 1.0 / np.sqrt(D),
                      np.zeros((1, Hq, D), np.float32), np.zeros((1, Hkv, D), np.float32),
                      np.zeros((1, Hkv, D), np.float32), np.zeros(1, np.int64), np.zeros(1, np.int32),
                      np.zeros((1, 1), np.int32), k_scale=ks, v_scale=vs)
    kp, vp = G.gpu_pool(b)
    system = rng.integers(0, 32000, 2000).tolist()
    seqs = {}  # id -> (tokens, extra)

    def write(keys, slots):
        if not len(keys):
            return
        k, v = _prefix_rows(keys, Hkv, D, 1), _prefix_rows(keys, Hkv, D, 2)
        pa.pa_cache_write(wl.storage_tensor(k, "bf16").to(G.DEV), wl.storage_tensor(v, "bf16").to(G.DEV),
                          kp, vp, torch.from_numpy(np.ascontiguousarray(slots, np.int64)).to(G.DEV),
                          ks, vs)

    def add(sid, tokens, extra=0):
        slots, nc = m.add_prompt(sid, tokens, extra)
        want_slots, want_nc = r.add_prompt(sid, tokens, extra)
        assert list(slots) == want_slots and nc == want_nc
        write(_context_keys(tokens, extra)[nc:], slots[nc:])  # the cached prefix is in the pool
        seqs[sid] = (list(tokens), extra)
        return nc

    assert add(0, system + rng.integers(0, 32000, 150).tolist()) == 0
    assert add(1, system + rng.integers(0, 32000, 301).tolist()) == 2000 // bs * bs
    assert add(2, system + rng.integers(0, 32000, 77).tolist(), extra=7) == 0
    half = system[:1000] + rng.integers(0, 32000, 500).tolist()
    assert add(3, half) == 1000 // bs * bs
    for step in range(2 * bs + 3):  # decode: blocks fill and enter the cache
        ids = sorted(seqs)
        toks = rng.integers(0, 32000, len(ids)).tolist()
        slots, pairs = m.append_tokens(ids, toks)
        want_slots, want_pairs = r.append_tokens(ids, toks)
        assert list(slots) == want_slots and [tuple(p) for p in pairs] == want_pairs == []
        keys = []
        for sid, t in zip(ids, toks):
            seqs[sid][0].append(t)
            keys.append(_context_keys(*seqs[sid])[-1])
        write(keys, slots)
    cached_before = m.num_cached_blocks()
    # 0 finishes; a new request continuing 0's whole text reuses all of its
    # full blocks from the free list (touch), and one more system-prompt
    # request shares the prompt again.
    full0 = list(seqs[0][0])
    m.release(0)
    r.release(0)
    del seqs[0]
    n0 = add(10, full0 + rng.integers(0, 32000, 40).tolist())
    assert n0 == len(full0) // bs * bs
    assert add(11, system + [5, 6, 7]) == 2000 // bs * bs
    assert m.num_cached_blocks() >= cached_before
    G.say(f"[apc {kv} bs{bs}] {len(seqs)} live, {m.num_cached_blocks()} cached blocks, "
          f"{nb - m.num_free()} of {nb} in use")

    ids = sorted(seqs)
    width = max(len(r.table(i)) for i in ids) + 1
    tables, lens = m.block_tables(ids, width)
    q = rng.standard_normal((len(ids), Hq, D)).astype(np.float32)
    qt = wl.storage_tensor(q, "bf16").to(G.DEV)
    q64 = G.query_f64(qt)
    ref = np.zeros((len(ids), Hq, D))
    for i, sid in enumerate(ids):
        tokens, extra = seqs[sid]
        keys = _context_keys(tokens, extra)
        Kb = _rows_bits(_prefix_rows(keys, Hkv, D, 1), kv, ks)
        Vb = _rows_bits(_prefix_rows(keys, Hkv, D, 2), kv, vs)
        K, V = opg.pool_values(Kb, kv, ks), opg.pool_values(Vb, kv, vs)
        for h in range(Hq):
            g = h // (Hq // Hkv)
            ref[i, h] = opg.attend(q64[i, h], K[:, g], V[:, g], b.scale)
    for ps in (pa.PA_PARTITION_BALANCED, 0):
        got = G.run_decode(b, kp, vp, qt, partition_size=ps, seq_lens=lens, tables=tables)
        G.assert_close(got, ref, kv, f"decode over cached prefixes, partition {ps}")
