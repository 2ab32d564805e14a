"""Pins of the reference block manager (oracle/block_manager.py) to the
pages' figures and to invariants checked by brute force."""
import random

import pytest

from conftest import load_golden
from oracle.block_manager import BlockManager, OutOfBlocks


def test_deep_interleaved_figure():
    """Two requests growing token by token into a 9-block pool reproduce the
    figure of "vLLM 深度解析" §3.1: R1 (41 tokens) in blocks [1, 3, 5], R2
    (56 tokens) in [0, 2, 4, 6], blocks 7 and 8 free.  The interleaving
    (R2's block before R1's at every block boundary) and the first-in
    first-out free list are what make the physical picture."""
    g = load_golden("deep_two_requests.json")
    bs = g["printed"]["block_size"]
    m = BlockManager(g["printed"]["num_physical_blocks"], bs)
    m.add("R2", 0)
    m.add("R1", 0)
    lens = g["derived_by_hand"]["seq_lens"]
    last = {}
    for t in range(max(lens.values())):
        ids = [r for r in ("R2", "R1") if t < lens[r]]
        slots, pairs = m.append(ids)
        assert pairs == []
        for r, s in zip(ids, slots):
            last[r] = s
    for r in ("R1", "R2"):
        assert m.table(r) == g["printed"]["requests"][r]["block_table"]
        assert m.seq_len(r) == lens[r]
        assert last[r] == g["derived_by_hand"]["last_token_slot"][r]
        assert len(m.table(r)) * bs - m.seq_len(r) == g["derived_by_hand"]["waste_tokens"][r]
    owner = g["printed"]["physical_owner"]
    for b, o in enumerate(owner):
        if o == "FREE":
            assert m.ref[b] == 0 and b in m.free
        else:
            r, i = o.split("-")
            assert m.table(r)[int(i)] == b and m.ref[b] == 1


def test_lib_worked_example():
    """A 50-token sequence at block size 16 takes 4 blocks; with the free
    list starting 102, 205, 78, 33 its table is the page's [102, 205, 78, 33]
    and its slots are the hand-derived ranges."""
    g = load_golden("lib_block_table_example.json")
    p, d = g["printed"], g["derived_by_hand"]
    order = p["block_table"] + [b for b in range(256) if b not in p["block_table"]]
    m = BlockManager(256, p["block_size"], free_order=order)
    slots = m.add("S", p["seq_len"])
    assert m.table("S") == p["block_table"]
    ranges = [[slots[i * 16], slots[min(i * 16 + 15, p["seq_len"] - 1)]] for i in range(p["num_blocks"])]
    assert ranges == d["slot_ranges"]
    assert p["seq_len"] - (p["num_blocks"] - 1) * p["block_size"] == d["last_block_fill"]
    assert p["num_blocks"] * p["block_size"] - p["seq_len"] == d["waste_tokens"]


def test_deep_prefix_sharing_and_copy_on_write():
    """A 20-token system prompt (blocks 0 and 1) shared by A, B, C: both
    blocks are held three times.  The first own token of A and of B lands in
    a shared, partly filled block, so each copies it first; C, by then the
    block's only holder, writes in place.  Block 0 (full) is never copied."""
    g = load_golden("deep_prefix_sharing.json")
    bs = g["printed"]["block_size"]
    m = BlockManager(16, bs)
    m.add("A", g["printed"]["system_prompt_tokens"])
    m.fork("A", "B")
    m.fork("A", "C")
    assert m.table("A") == g["printed"]["shared"]
    assert [m.ref[b] for b in g["printed"]["shared"]] == [3, 3]
    slots, pairs = m.append(["A", "B", "C"])
    assert pairs == [(1, 2), (1, 3)]
    assert m.table("A") == [0, 2] and m.table("B") == [0, 3] and m.table("C") == [0, 1]
    assert slots == [2 * bs + 4, 3 * bs + 4, 1 * bs + 4]
    assert m.ref[0] == 3 and m.ref[1] == 1
    # Filling A's copied block and opening the next never copies again.
    for _ in range(12):
        _, pairs = m.append(["A"])
        assert pairs == []
    assert m.table("A") == [0, 2, 4]


def test_full_shared_block_is_never_copied():
    """Append copies only the block it writes into ([EVAL] fork / append /
    free: only the block that changes is copied).  A prompt that ends on a
    block edge, forked three ways: every sample's first own token opens a
    fresh block and the full prompt blocks stay shared by all four."""
    m = BlockManager(16, 4)
    m.add("P", 8)
    for c in ("a", "b", "c"):
        m.fork("P", c)
    slots, pairs = m.append(["P", "a", "b", "c"])
    assert pairs == []
    assert [m.ref[b] for b in (0, 1)] == [4, 4]
    assert [m.table(s)[-1] for s in ("P", "a", "b", "c")] == [2, 3, 4, 5]
    assert slots == [8, 12, 16, 20]


def _check_content(m, mem, content):
    """Every live sequence reads back exactly its tokens through its table."""
    bs = m.block_size
    for sid, toks in content.items():
        tbl = m.table(sid)
        assert len(toks) == m.seq_len(sid)
        assert len(tbl) == -(-len(toks) // bs)
        for t, tok in enumerate(toks):
            assert mem[tbl[t // bs] * bs + t % bs] == tok, (sid, t)


def _check_counts(m):
    held = [0] * m.num_blocks
    for sid in m.seqs:
        for b in m.table(sid):
            held[b] += 1
    assert held == m.ref
    assert len(set(m.free)) == len(m.free)
    assert sorted(m.free) == [b for b in range(m.num_blocks) if m.ref[b] == 0]


@pytest.mark.parametrize("seed", range(6))
def test_random_traces_keep_every_sequence_readable(seed):
    """Random add / fork / append / free traces over a small pool, with a
    brute-force token memory: block copies are applied as the pairs say,
    writes go to the returned slots, and every live sequence must read back
    its own tokens; reference counts equal table occurrences and the free
    list is exactly the unreferenced blocks.  Out-of-blocks requests must
    leave everything unchanged."""
    rng = random.Random(seed)
    bs = rng.choice([2, 4, 16])
    m = BlockManager(rng.randint(8, 40), bs)
    mem = [None] * (m.num_blocks * bs)
    content = {}
    next_id, next_tok = 0, 0
    for _ in range(400):
        op = rng.random()
        live = list(content)
        try:
            if op < 0.2 or not live:
                n = rng.randint(0, 3 * bs)
                slots = m.add(next_id, n)
                toks = list(range(next_tok, next_tok + n))
                next_tok += n
                for s, tok in zip(slots, toks):
                    mem[s] = tok
                content[next_id] = toks
                next_id += 1
            elif op < 0.35:
                p = rng.choice(live)
                m.fork(p, next_id)
                content[next_id] = list(content[p])
                next_id += 1
            elif op < 0.85:
                ids = rng.sample(live, rng.randint(1, len(live)))
                before = (list(m.free), list(m.ref), {k: dict(v, blocks=list(v["blocks"])) for k, v in m.seqs.items()})
                try:
                    slots, pairs = m.append(ids)
                except OutOfBlocks:
                    assert (m.free, m.ref, m.seqs) == before
                    continue
                for src, dst in pairs:  # the block copy happens before the writes
                    mem[dst * bs:(dst + 1) * bs] = mem[src * bs:(src + 1) * bs]
                for sid, s in zip(ids, slots):
                    mem[s] = next_tok
                    content[sid].append(next_tok)
                    next_tok += 1
            else:
                sid = rng.choice(live)
                m.release(sid)
                del content[sid]
        except OutOfBlocks:
            pass
        _check_counts(m)
        _check_content(m, mem, content)


def test_out_of_blocks_changes_nothing():
    m = BlockManager(3, 4)
    m.add("a", 4)
    m.add("b", 4)
    m.fork("a", "c")
    # a and c share a full block: appending to all three needs 3 new blocks.
    before = (list(m.free), list(m.ref), {k: dict(v, blocks=list(v["blocks"])) for k, v in m.seqs.items()})
    with pytest.raises(OutOfBlocks):
        m.append(["a", "b", "c"])
    assert (m.free, m.ref, m.seqs) == before
    with pytest.raises(OutOfBlocks):
        m.add("d", 5)
    assert m.num_free() == 1


def test_swap_out_and_in_by_hand():
    """A 6-block device pool, 4 host blocks, block size 4.  A (6 tokens) is
    forked into C; B holds its own blocks.  Swapping out A alone is refused
    (C shares its blocks); A and C together move their two blocks once each;
    the freed device blocks serve a new request; A and C come back into
    other blocks once the device has room."""
    m = BlockManager(6, 4, num_host_blocks=4)
    m.add("A", 6)
    m.add("B", 5)
    m.fork("A", "C")
    with pytest.raises(ValueError):
        m.swap_out(["A"])
    assert m.swap_out(["A", "C"]) == [(0, 0), (1, 1)]
    assert m.free == [4, 5, 0, 1] and m.host_ref == [2, 2, 0, 0] and m.ref[:2] == [0, 0]
    assert m.table("A") == m.table("C") == [0, 1] and m.is_swapped("C")
    with pytest.raises(KeyError):
        m.append(["A"])
    with pytest.raises(KeyError):
        m.fork("C", "E")
    assert m.add("D", 9)[:1] == [16]  # blocks 4, 5, 0
    with pytest.raises(OutOfBlocks):
        m.swap_in(["A", "C"])
    m.release("D")  # its blocks come back last block first
    assert m.free == [1, 0, 5, 4]
    assert m.swap_in(["C", "A"]) == [(0, 1), (1, 0)]
    assert m.table("A") == m.table("C") == [1, 0] and m.ref[1] == m.ref[0] == 2
    assert m.host_free == [2, 3, 0, 1]
    slots, pairs = m.append(["A"])  # the shared partial block is copied first
    assert pairs == [(0, 5)] and slots == [5 * 4 + 2]


def _groups(m, swapped: bool):
    """Sets of sequences that hold their blocks alone: connected components
    of the sharing relation among sequences on one side."""
    ids = [s for s in m.seqs if m.is_swapped(s) == swapped]
    owner, comp = {}, {s: s for s in ids}

    def root(x):
        while comp[x] != x:
            x = comp[x]
        return x
    for s in ids:
        for b in m.table(s):
            if b in owner:
                comp[root(s)] = root(owner[b])
            else:
                owner[b] = s
    out = {}
    for s in ids:
        out.setdefault(root(s), []).append(s)
    return list(out.values())


@pytest.mark.parametrize("seed", range(6))
def test_random_traces_with_swap_keep_every_sequence_readable(seed):
    """Random traces with swap-out and swap-in of whole sharing groups over
    a brute-force device memory and host memory: the pairs are applied as
    the swap kernel would, and every sequence reads back its own tokens from
    the side it lives on; reference counts equal table occurrences on both
    sides and each free list is exactly that side's unreferenced blocks."""
    rng = random.Random(50 + seed)
    bs = rng.choice([2, 4, 16])
    m = BlockManager(rng.randint(8, 40), bs, num_host_blocks=rng.randint(4, 40))
    dev = [None] * (m.num_blocks * bs)
    host = [None] * (m.num_host_blocks * bs)
    content, next_id, next_tok = {}, 0, 0
    swaps = 0
    for _ in range(500):
        op = rng.random()
        live = [s for s in content if not m.is_swapped(s)]
        out = [s for s in content if m.is_swapped(s)]
        try:
            if op < 0.15 or not content:
                n = rng.randint(0, 3 * bs)
                slots = m.add(next_id, n)
                content[next_id] = list(range(next_tok, next_tok + n))
                for s, tok in zip(slots, content[next_id]):
                    dev[s] = tok
                next_tok += n
                next_id += 1
            elif op < 0.27 and live:
                p = rng.choice(live)
                m.fork(p, next_id)
                content[next_id] = list(content[p])
                next_id += 1
            elif op < 0.6 and live:
                ids = rng.sample(live, rng.randint(1, len(live)))
                slots, pairs = m.append(ids)
                for src, dst in pairs:
                    dev[dst * bs:(dst + 1) * bs] = dev[src * bs:(src + 1) * bs]
                for sid, s in zip(ids, slots):
                    dev[s] = next_tok
                    content[sid].append(next_tok)
                    next_tok += 1
            elif op < 0.72 and live:
                group = rng.choice(_groups(m, False))
                pairs = m.swap_out(group)
                for d, h in pairs:
                    host[h * bs:(h + 1) * bs] = dev[d * bs:(d + 1) * bs]
                    dev[d * bs:(d + 1) * bs] = [None] * bs  # the device block is reused
                swaps += 1
            elif op < 0.84 and out:
                group = rng.choice(_groups(m, True))
                rng.shuffle(group)
                pairs = m.swap_in(group)
                for h, d in pairs:
                    dev[d * bs:(d + 1) * bs] = host[h * bs:(h + 1) * bs]
                swaps += 1
            else:
                sid = rng.choice(list(content))
                m.release(sid)
                del content[sid]
        except OutOfBlocks:
            pass
        for side, mem, ref, free, nb in ((False, dev, m.ref, m.free, m.num_blocks),
                                         (True, host, m.host_ref, m.host_free, m.num_host_blocks)):
            held = [0] * nb
            for sid, toks in content.items():
                if m.is_swapped(sid) != side:
                    continue
                tbl = m.table(sid)
                assert len(tbl) == -(-len(toks) // bs)
                for b in tbl:
                    held[b] += 1
                for t, tok in enumerate(toks):
                    assert mem[tbl[t // bs] * bs + t % bs] == tok, (sid, t, side)
            assert held == ref
            assert sorted(free) == [b for b in range(nb) if ref[b] == 0] and len(set(free)) == len(free)
    assert swaps > 10


# -- prefix caching -------------------------------------------------------------
from oracle.block_manager import block_hash, fnv1a64  # noqa: E402


def test_fnv1a64_published_vectors():
    """Test vectors of 64-bit FNV-1a published with its definition."""
    assert fnv1a64(b"") == 0xCBF29CE484222325
    assert fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fnv1a64(b"foobar") == 0x85944171F73967E8


def test_block_hash_is_chained():
    """hash(parent, tokens, extra): equal for equal inputs, different when
    any of the three differs, so one block's hash names its whole prefix."""
    a = block_hash(0, [1, 2, 3, 4])
    assert a == block_hash(0, [1, 2, 3, 4]) and a == fnv1a64(
        bytes(8) + b"".join(t.to_bytes(4, "little") for t in (1, 2, 3, 4)) + bytes(8))
    assert len({a, block_hash(0, [1, 2, 3, 5]), block_hash(a, [1, 2, 3, 4]),
                block_hash(0, [1, 2, 3, 4], extra=7), block_hash(0, [4, 3, 2, 1])}) == 5
    # The same block after two different first blocks hashes differently.
    b1 = block_hash(block_hash(0, [9, 9, 9, 9]), [5, 6, 7, 8])
    b2 = block_hash(block_hash(0, [9, 9, 9, 8]), [5, 6, 7, 8])
    assert b1 != b2


def test_system_prompt_is_shared_through_the_cache():
    """The page's use case: requests that start with the same system prompt.
    A (system prompt of 2 full blocks + 3 own tokens) commits its 2 full
    blocks; B with the same system prompt hits both (8 cached tokens, 2
    references each) and takes one block for its own tail; C with another
    adapter (extra hash) hits nothing; D differing in the prompt's second
    block hits only the first."""
    bs = 4
    m = BlockManager(16, bs, prefix_caching=True)
    sys_prompt = [11, 12, 13, 14, 15, 16, 17, 18]
    slots_a, ca = m.add_prompt("A", sys_prompt + [1, 2, 3])
    assert ca == 0 and m.table("A") == [0, 1, 2] and m.num_cached_blocks() == 2
    slots_b, cb = m.add_prompt("B", sys_prompt + [4, 5])
    assert cb == 8 and m.table("B") == [0, 1, 3] and m.ref[:2] == [2, 2]
    assert slots_b[:8] == slots_a[:8] and slots_b[8:] == [12, 13]
    _, cc = m.add_prompt("C", sys_prompt + [4, 5], extra=99)
    assert cc == 0 and m.table("C") == [4, 5, 6] and m.num_cached_blocks() == 4
    _, cd = m.add_prompt("D", sys_prompt[:4] + [0, 0, 0, 0] + [7])
    assert cd == 4 and m.table("D") == [0, 7, 8] and m.ref[0] == 3
    # G starts with the tokens of the prompt's second block: that block's K/V
    # belong after the first block, so nothing is reused.
    _, cg = m.add_prompt("G", sys_prompt[4:] + [1])
    assert cg == 0 and m.table("G") == [9, 10]
    m.release("G")
    # A fills its third block during decode: it enters the cache, and a new
    # request with A's whole prompt plus that token hits all three blocks.
    _, pairs = m.append_tokens(["A"], [9])
    assert pairs == [] and m.num_cached_blocks() == 7  # A: 0 1 2, C: 4 5, D: 7, G: 9
    _, ce = m.add_prompt("E", sys_prompt + [1, 2, 3, 9, 10])
    assert ce == 12 and m.table("E")[:3] == [0, 1, 2]


def test_eviction_is_lru_and_leaf_first():
    """Released cached blocks wait in the free list: a later request takes
    never-used blocks first, then evicts the least recently released, and
    within one release the chain's last block before its first."""
    bs = 2
    m = BlockManager(6, bs, prefix_caching=True)
    m.add_prompt("X", [1, 1, 2, 2, 3, 3])   # blocks 0, 1, 2, all cached
    m.add_prompt("Y", [7, 7])               # block 3, cached
    m.release("X")                          # free: 4, 5, 2, 1, 0 (X's leaf first)
    m.release("Y")                          # ... then 3
    assert m.free == [4, 5, 2, 1, 0, 3] and m.num_cached_blocks() == 4
    m.add_prompt("Z", [8, 8, 9, 9, 6, 6])   # 3 misses: takes 4, 5 (unused), then evicts 2
    assert m.table("Z") == [4, 5, 2] and m.num_cached_blocks() == 3 + 3
    # X's first two blocks survived the eviction of its leaf.
    _, c = m.add_prompt("X2", [1, 1, 2, 2, 3, 3])
    assert c == 4 and m.table("X2")[:2] == [0, 1]


@pytest.mark.parametrize("seed", range(6))
def test_random_prefix_cache_traces_keep_every_sequence_readable(seed):
    """Prompts drawn from a few shared prefixes, with adapters, decode steps
    with token ids, forks, frees and plain adds over a small pool, against a
    brute-force memory whose value at a slot names the whole prefix up to
    that token and the adapter (as K/V depend on the whole context): the
    caller writes only the tokens past num_cached, so a wrong hit shows as a
    wrong value.  Reference counts equal table occurrences; the free list is
    exactly the unreferenced blocks; every cached block holds what its hash
    names."""
    rng = random.Random(700 + seed)
    bs = rng.choice([2, 4])
    m = BlockManager(rng.randint(12, 40), bs, prefix_caching=True, num_host_blocks=rng.randint(4, 24))
    mem = [None] * (m.num_blocks * bs)
    host = [None] * (m.num_host_blocks * bs)
    prefixes = [[rng.randint(0, 3) for _ in range(rng.randint(0, 4 * bs))] for _ in range(4)]
    content, next_id, hits = {}, 0, 0

    def value(toks, t, extra):
        return (tuple(toks[:t + 1]), extra)

    for _ in range(500):
        op = rng.random()
        try:
            if op < 0.3 or not content:
                toks = rng.choice(prefixes) + [rng.randint(0, 3) for _ in range(rng.randint(0, 2 * bs))]
                extra = rng.choice([0, 0, 0, 5])
                slots, nc = m.add_prompt(next_id, toks, extra)
                assert nc % bs == 0 and nc <= len(toks)
                for t in range(nc):  # cached: already in the pool
                    assert mem[slots[t]] == value(toks, t, extra)
                for t in range(nc, len(toks)):
                    mem[slots[t]] = value(toks, t, extra)
                content[next_id] = (list(toks), extra)
                hits += nc
                next_id += 1
            elif op < 0.4:
                p = rng.choice(list(content))
                if m.is_swapped(p):
                    continue
                m.fork(p, next_id)
                content[next_id] = (list(content[p][0]), content[p][1])
                next_id += 1
            elif op < 0.5:
                live = [i for i in content if not m.is_swapped(i)]
                out = [i for i in content if m.is_swapped(i)]
                if rng.random() < 0.5 and live:
                    for d, h in m.swap_out(rng.choice(_groups(m, False))):
                        host[h * bs:(h + 1) * bs] = mem[d * bs:(d + 1) * bs]
                        mem[d * bs:(d + 1) * bs] = [None] * bs  # reused from now on
                elif out:
                    for h, d in m.swap_in(rng.choice(_groups(m, True))):
                        mem[d * bs:(d + 1) * bs] = host[h * bs:(h + 1) * bs]
            elif op < 0.75:
                live = [i for i in content if not m.is_swapped(i)]
                if not live:
                    continue
                ids = rng.sample(live, rng.randint(1, len(live)))
                toks = [rng.randint(0, 3) for _ in ids]
                slots, pairs = m.append_tokens(ids, toks)
                for src, dst in pairs:
                    mem[dst * bs:(dst + 1) * bs] = mem[src * bs:(src + 1) * bs]
                for sid, s, t in zip(ids, slots, toks):
                    seq, extra = content[sid]
                    seq.append(t)
                    mem[s] = value(seq, len(seq) - 1, extra)
            else:
                sid = rng.choice(list(content))
                m.release(sid)
                del content[sid]
        except OutOfBlocks:
            pass
        held = [0] * m.num_blocks
        for sid, (toks, extra) in content.items():
            tbl = m.table(sid)
            side = host if m.is_swapped(sid) else mem
            for b in ([] if m.is_swapped(sid) else tbl):
                held[b] += 1
            for t in range(len(toks)):
                assert side[tbl[t // bs] * bs + t % bs] == value(toks, t, extra), (sid, t)
        assert held == m.ref
        assert sorted(m.free) == [b for b in range(m.num_blocks) if m.ref[b] == 0]
        for b, (h, toks, extra) in m.cached.items():
            assert m.table_of[h] == b
            assert [mem[b * bs + i][0][-1] for i in range(bs)] == list(toks)
            assert all(mem[b * bs + i][1] == extra for i in range(bs))
    assert hits > 0
