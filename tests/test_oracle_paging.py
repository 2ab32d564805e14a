"""Pins of the oracle's paging semantics: the pages' worked block-table
examples (tests/golden), the paging invariants (relabelling physical blocks,
sharing prefix blocks), and the cache-write / block-copy definitions."""
import numpy as np
import pytest

from conftest import load_golden
from oracle import codecs, paged
from paged_kv_cache_11_amd import workloads


def _empty_pool(nb, Hkv, bs, D):
    return np.full((nb, Hkv, bs, D), np.nan)


def _write(kp, vp, K, V, slots):
    """Write float64 rows into float64 pools through the oracle's cache write
    (float64 pools are handled as 'f32'-typed words of a matching dtype)."""
    paged.cache_write(kp, vp, "f64", K, V, "f64", slots)


def test_lib_worked_example_slots_and_gather():
    g = load_golden("lib_block_table_example.json")
    p, d = g["printed"], g["derived_by_hand"]
    L, bs, table = p["seq_len"], p["block_size"], np.array(p["block_table"])
    assert -(-L // bs) == p["num_blocks"] == len(table)
    slots = paged.slots_of(table, L, bs)
    expect = np.concatenate([np.arange(a, b + 1) for a, b in d["slot_ranges"]])
    assert np.array_equal(slots, expect)
    assert L - (len(table) - 1) * bs == d["last_block_fill"]
    assert len(table) * bs - L == d["waste_tokens"] < bs
    # Write a 50-token sequence through those slots into a 256-block pool and
    # gather it back: the paged copy equals the contiguous one, and only the
    # four listed blocks changed.
    rng = np.random.default_rng(0)
    Hkv, D, nb = 2, 8, 256
    K, V = rng.standard_normal((L, Hkv, D)), rng.standard_normal((L, Hkv, D))
    kp, vp = _empty_pool(nb, Hkv, bs, D), _empty_pool(nb, Hkv, bs, D)
    _write(kp, vp, K, V, slots)
    assert np.array_equal(paged.gather(kp, table, L), K)
    assert np.array_equal(paged.gather(vp, table, L), V)
    touched = sorted(set(np.nonzero(~np.isnan(kp).all(axis=(1, 2, 3)))[0].tolist()))
    assert touched == sorted(table.tolist())
    # The two used slots of the last block are written; its other 14 are not.
    assert not np.isnan(kp[33, :, :2]).any() and np.isnan(kp[33, :, 2:]).all()


def test_deep_two_interleaved_requests():
    g = load_golden("deep_two_requests.json")
    p, d = g["printed"], g["derived_by_hand"]
    bs, nb = p["block_size"], p["num_physical_blocks"]
    rng = np.random.default_rng(1)
    Hkv, D = 1, 4
    kp, vp = _empty_pool(nb, Hkv, bs, D), _empty_pool(nb, Hkv, bs, D)
    data = {}
    for name, r in p["requests"].items():
        L = r["tokens"][1] - r["tokens"][0] + 1
        assert L == d["seq_lens"][name]
        table = np.array(r["block_table"])
        slots = paged.slots_of(table, L, bs)
        assert slots[-1] == d["last_token_slot"][name]
        assert len(table) * bs - L == d["waste_tokens"][name] < bs
        K = rng.standard_normal((L, Hkv, D))
        V = rng.standard_normal((L, Hkv, D))
        _write(kp, vp, K, V, slots)
        data[name] = (table, L, K, V)
    # Physical view: block i holds logical block j of the request printed for it.
    for i, owner in enumerate(p["physical_owner"]):
        if owner == "FREE":
            assert np.isnan(kp[i]).all()
            continue
        name, j = owner.split("-")
        table, L, K, _ = data[name]
        assert table[int(j)] == i
        n = min(bs, L - int(j) * bs)
        assert np.array_equal(kp[i, :, :n], K[int(j) * bs:int(j) * bs + n].transpose(1, 0, 2))
    # Attention through the tables equals attention over the contiguous rows.
    q = rng.standard_normal((2, 2, D))
    for s, name in enumerate(("R1", "R2")):
        table, L, K, V = data[name]
        out = paged.paged_decode(q[s][None], kp, vp, table[None], np.array([L]), 0.5)
        for h in range(2):
            np.testing.assert_array_equal(out[0, h], paged.attend(q[s, h], K[:, 0], V[:, 0], 0.5))


def test_deep_prefix_sharing_with_copy_on_write():
    g = load_golden("deep_prefix_sharing.json")
    p = g["printed"]
    bs, P = p["block_size"], p["system_prompt_tokens"]
    tables = {k: np.array(v) for k, v in p["block_tables"].items()}
    # Reference counts implied by the printed tables.
    refs = {}
    for t in tables.values():
        for b in t:
            refs[int(b)] = refs.get(int(b), 0) + 1
    assert {b for b, c in refs.items() if c > 1} == set(p["shared"]) and refs[0] == refs[1] == 3
    # Reading (fixture 'reading'): dense tables, block 1 copied before each
    # request's first own token.
    rng = np.random.default_rng(2)
    Hkv, D, nb = 2, 8, 12
    own = {"A": 20, "B": 13, "C": 5}
    private = {"A": [5, 6], "B": [7, 8], "C": [9]}
    KP, VP = rng.standard_normal((P, Hkv, D)), rng.standard_normal((P, Hkv, D))
    kp, vp = _empty_pool(nb, Hkv, bs, D), _empty_pool(nb, Hkv, bs, D)
    _write(kp, vp, KP, VP, paged.slots_of(np.array([0, 1]), P, bs))
    paged.copy_blocks(kp, vp, [(1, private[r][0]) for r in ("A", "B", "C")])
    seqs = {}
    for r in ("A", "B", "C"):
        L = P + own[r]
        table = np.array([0] + private[r])
        assert -(-L // bs) == len(table)
        K = np.concatenate([KP, rng.standard_normal((own[r], Hkv, D))])
        V = np.concatenate([VP, rng.standard_normal((own[r], Hkv, D))])
        _write(kp, vp, K[P:], V[P:], paged.slots_of(table, L, bs)[P:])
        seqs[r] = (table, L, K, V)
    # Shared block 0 is untouched by the appends, the copied prompt tail
    # survives in each private block, and the original block 1 is unchanged.
    assert np.array_equal(kp[0], KP[:16].transpose(1, 0, 2))
    assert np.array_equal(kp[1, :, :4], KP[16:20].transpose(1, 0, 2)) and np.isnan(kp[1, :, 4:]).all()
    q = rng.standard_normal((3, 4, D))
    for s, r in enumerate(("A", "B", "C")):
        table, L, K, V = seqs[r]
        assert np.array_equal(paged.gather(kp, table, L), K)
        out = paged.paged_decode(q[s][None], kp, vp, table[None], np.array([L]), 0.3)
        # Same request with a fully private copy of every block.
        kq, vq = _empty_pool(4, Hkv, bs, D), _empty_pool(4, Hkv, bs, D)
        priv = np.arange(len(table))
        _write(kq, vq, K, V, paged.slots_of(priv, L, bs))
        ref = paged.paged_decode(q[s][None], kq, vq, priv[None], np.array([L]), 0.3)
        np.testing.assert_array_equal(out, ref)


def test_relabelling_physical_blocks_leaves_outputs_unchanged():
    b = workloads.tiny_decode()
    nb, Hkv, bs, D = b.num_blocks, b.num_kv_heads, b.block_size, b.head_size
    kp, vp = _empty_pool(nb, Hkv, bs, D), _empty_pool(nb, Hkv, bs, D)
    _write(kp, vp, b.k.astype(np.float64), b.v.astype(np.float64), b.slot_mapping)
    out = paged.paged_decode(b.q.astype(np.float64), kp, vp, b.block_tables, b.seq_lens, b.scale)
    perm = np.random.default_rng(4).permutation(nb)        # old id -> new id
    kq, vq = np.empty_like(kp), np.empty_like(vp)
    kq[perm], vq[perm] = kp, vp
    tables = np.where(b.block_tables >= 0, perm[np.maximum(b.block_tables, 0)], -1)
    out2 = paged.paged_decode(b.q.astype(np.float64), kq, vq, tables, b.seq_lens, b.scale)
    np.testing.assert_array_equal(out, out2)


def test_waste_is_below_one_block_per_sequence():
    rng = np.random.default_rng(6)
    for bs in (16, 32, 64, 128):
        L = rng.integers(1, 10000, 500)
        waste = (-(-L // bs)) * bs - L
        assert waste.min() >= 0 and waste.max() <= bs - 1


def test_cache_write_skips_padding_and_touches_nothing_else():
    nb, Hkv, bs, D = 6, 2, 4, 8
    rng = np.random.default_rng(8)
    k = rng.integers(0, 2 ** 16, (5, Hkv, D)).astype(np.uint16)
    v = rng.integers(0, 2 ** 16, (5, Hkv, D)).astype(np.uint16)
    kp = np.full((nb, Hkv, bs, D), 0xABCD, np.uint16)
    vp = kp.copy()
    slots = np.array([3, -1, 17, 8, -5])
    paged.cache_write(kp, vp, "bf16", k, v, "bf16", slots)
    for t, sl in enumerate(slots):
        if sl >= 0:
            assert np.array_equal(kp[sl // bs, :, sl % bs], k[t])
            assert np.array_equal(vp[sl // bs, :, sl % bs], v[t])
    mask = np.ones((nb, bs), bool)
    for sl in (3, 17, 8):
        mask[sl // bs, sl % bs] = False
    assert (kp.transpose(0, 2, 1, 3)[mask] == 0xABCD).all()
    with pytest.raises(ValueError):
        paged.cache_write(kp, vp, "bf16", k[:2], v[:2], "bf16", np.array([5, 5]))
    with pytest.raises(ValueError):
        paged.cache_write(kp, vp, "bf16", k[:1], v[:1], "bf16", np.array([nb * bs]))


def test_cache_write_fp8_quantises_per_tensor():
    rng = np.random.default_rng(10)
    nb, Hkv, bs, D = 4, 2, 8, 16
    kf = rng.standard_normal((6, Hkv, D)).astype(np.float32) * 3
    vf = rng.standard_normal((6, Hkv, D)).astype(np.float32)
    ks, vs = np.float32(np.abs(kf).max() / 448), np.float32(np.abs(vf).max() / 448)
    kp = np.full((nb, Hkv, bs, D), 0x7F, np.uint8)
    vp = kp.copy()
    slots = np.array([0, 9, 10, 31, 17, 2])
    paged.cache_write(kp, vp, "fp8", kf.view(np.uint32), vf.view(np.uint32), "f32", slots, ks, vs)
    for t, sl in enumerate(slots):
        got = codecs.e4m3fn_to_f64(kp[sl // bs, :, sl % bs]) * float(ks)
        np.testing.assert_allclose(got, kf[t], rtol=2 ** -4, atol=float(ks) * 2 ** -9)
    # The largest magnitude maps to the largest code exactly.
    t, h, d = np.unravel_index(np.abs(kf).argmax(), kf.shape)
    assert kp[slots[t] // bs, h, slots[t] % bs, d] & 0x7F == 0x7E


def test_copy_blocks_semantics():
    rng = np.random.default_rng(12)
    kp = rng.integers(0, 255, (8, 2, 4, 8)).astype(np.uint8)
    vp = rng.integers(0, 255, (8, 2, 4, 8)).astype(np.uint8)
    k0, v0 = kp.copy(), vp.copy()
    paged.copy_blocks(kp, vp, [(1, 5), (1, 6), (3, 0)])
    for s, d in ((1, 5), (1, 6), (3, 0)):
        assert np.array_equal(kp[d], k0[s]) and np.array_equal(vp[d], v0[s])
    for b in (1, 2, 3, 4, 7):
        assert np.array_equal(kp[b], k0[b]) and np.array_equal(vp[b], v0[b])
    paged.copy_blocks(kp, vp, np.zeros((0, 2), np.int64))   # no pairs: a no-op
    with pytest.raises(ValueError):
        paged.copy_blocks(kp, vp, [(1, 2), (3, 2)])
    with pytest.raises(ValueError):
        paged.copy_blocks(kp, vp, [(1, 2), (2, 3)])


def test_copy_blocks_skips_pairs_outside_the_pool():
    rng = np.random.default_rng(13)
    kp = rng.integers(0, 255, (6, 2, 4, 8)).astype(np.uint8)
    vp = kp[::-1].copy()
    k0, v0 = kp.copy(), vp.copy()
    paged.copy_blocks(kp, vp, [(-1, 2), (6, 3), (1, 6), (0, -2), (4, 5)])
    assert np.array_equal(kp[5], k0[4]) and np.array_equal(vp[5], v0[4])
    assert np.array_equal(kp[:5], k0[:5]) and np.array_equal(vp[:5], v0[:5])


def test_swap_blocks_element_by_element():
    """Brute force on a tiny case: every word of every destination block is
    the source word at the same (head, offset, dim); all else is untouched."""
    rng = np.random.default_rng(14)
    dev_k = rng.integers(0, 1 << 16, (5, 2, 3, 4)).astype(np.uint16)
    dev_v = rng.integers(0, 1 << 16, (5, 2, 3, 4)).astype(np.uint16)
    host_k = np.full((7, 2, 3, 4), 0x7FC1, np.uint16)
    host_v = np.full((7, 2, 3, 4), 0x7FC1, np.uint16)
    pairs = [(4, 0), (0, 6), (2, 3), (9, 1), (1, 7)]  # the last two name no block
    paged.swap_blocks(dev_k, dev_v, host_k, host_v, pairs)
    moved = {0: 4, 6: 0, 3: 2}
    for b in range(7):
        for h in range(2):
            for o in range(3):
                for d in range(4):
                    if b in moved:
                        assert host_k[b, h, o, d] == dev_k[moved[b], h, o, d]
                        assert host_v[b, h, o, d] == dev_v[moved[b], h, o, d]
                    else:
                        assert host_k[b, h, o, d] == 0x7FC1 == host_v[b, h, o, d]
    with pytest.raises(ValueError):
        paged.swap_blocks(dev_k, dev_v, host_k, host_v, [(0, 1), (2, 1)])
    with pytest.raises(ValueError):
        paged.swap_blocks(dev_k, dev_v, host_k[:, :1].copy(), host_v[:, :1].copy(), [(0, 0)])


def test_swap_out_and_in_restores_the_sequence():
    """A sequence's blocks swapped out to arbitrary host blocks and back into
    other device blocks: its gathered K/V is unchanged, and equals the same
    move done by the block copy within one pool."""
    rng = np.random.default_rng(15)
    bs, nb = 4, 12
    kp = rng.standard_normal((nb, 2, bs, 8))
    vp = rng.standard_normal((nb, 2, bs, 8))
    table, L = [7, 2, 9], 10
    K0, V0 = paged.gather(kp, table, L), paged.gather(vp, table, L)
    hk, hv = np.zeros((5, 2, bs, 8)), np.zeros((5, 2, bs, 8))
    paged.swap_blocks(kp, vp, hk, hv, [(7, 3), (2, 0), (9, 4)])
    kp[table] = np.nan  # the device blocks are reused meanwhile
    vp[table] = np.nan
    back = [1, 11, 5]
    paged.swap_blocks(hk, hv, kp, vp, [(3, 1), (0, 11), (4, 5)])
    assert np.array_equal(paged.gather(kp, back, L), K0)
    assert np.array_equal(paged.gather(vp, back, L), V0)
    kq, vq = kp.copy(), vp.copy()
    paged.swap_blocks(kp, vp, kp, vp, [(1, 0), (11, 3)])
    paged.copy_blocks(kq, vq, [(1, 0), (11, 3)])
    assert np.array_equal(kp, kq, equal_nan=True) and np.array_equal(vp, vq, equal_nan=True)
