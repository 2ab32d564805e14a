"""Reference block manager (test infrastructure, not part of the product path).

What the pages describe and this models, step by step:

* a pool of physical blocks of ``block_size`` token slots, preallocated at
  start, handed out from a free list in O(1) ("vLLM：大语言模型推理与服务库"
  §4.2 item 3, block pool; "vLLM 深度解析" §3.1);
* one block table per sequence: logical block i of the sequence is physical
  block ``table[i]``, token t lives in logical block t // block_size at
  offset t % block_size, so its slot is ``table[t // bs] * bs + t % bs``
  ("vLLM：大语言模型推理与服务库" §4.2 item 2 and its worked example);
* a new token goes into the sequence's last block; when that block is full
  a new block is taken from the free list first (§4.3 item 2 of the same
  page);
* fork / append / free over shared blocks ("vLLM 高性能大语言模型推理引擎深度
  技术评估与分布式架构展望", the fork / append / free primitives; "vLLM 深度
  解析" §3.1 prefix sharing and copy-on-write): fork gives the child the
  parent's table and adds a reference to every block; appending into a
  last block that is shared and not full first copies that block into a
  fresh one (copy-on-write: the pair (shared, fresh) is what the block copy
  kernel moves) and drops one reference from the shared block; free drops
  one reference from each block and returns blocks that reach zero to the
  free list.

Readings where the pages are silent or disagree:

* free-list order: blocks are taken from the front and returned to the back
  (first in, first out).  One page's code pops from the back, the other's
  from the front; the front is what reproduces the interleaved 9-block
  figure of "vLLM 深度解析" §3.1 (request tables [1, 3, 5] and
  [0, 2, 4, 6]);
* a full shared last block is left shared: the new token opens a new block
  and nothing is copied;
* a batch append either succeeds for every sequence or, when the free list
  cannot cover it, changes nothing and raises ``OutOfBlocks``;
* a freed sequence returns its blocks last block first (so that with prefix
  caching the leaf end of a chain is reused before its root).

Swap (the SWAP mode of preemption: [EVAL], its section on preemption;
"vLLM 深度解析" §3.2, preemption strategies): a preempted sequence's blocks
move to a pool of host blocks and come back when it resumes.  Readings:

* sequences are swapped as a set that holds its blocks alone (a block
  shared with a sequence outside the set cannot move; sampling and beam
  search siblings go together);
* each distinct block moves once, in order of first appearance (sequences in
  the given order, each table front to back), to a block taken from the
  front of the destination's free list; its reference count moves with it
  and the source block returns to the back of its free list;
* a swapped-out sequence can be freed, not appended to or forked;
* a swap the destination cannot hold changes nothing (out of blocks);
* with prefix caching, blocks that move drop out of the cache.

Prefix caching ([EVAL], its section on automatic prefix caching): every
block filled with tokens gets a chained hash of (the previous block's hash,
the block's token ids, extra hashes such as an adapter id); a table maps
hashes to physical blocks.  A new prompt looks up its chain block by block
(stopping at the first miss) and points its table at the blocks it finds
(lookup), adding a reference to each and taking unreferenced ones off the
free list (touch); blocks it fills itself, and blocks that fill later during
decode, enter the table (commit); when a block must be taken from the free
list and the one in front is still cached, it leaves the table (eviction).
Unreferenced cached blocks wait in the free list, so eviction is least
recently released first and, within one release, last block first: the
leaves of long chains go before the blocks near the root.  Readings:

* the hash is 64-bit FNV-1a (its published definition) over the bytes of
  the parent hash (8, little endian; 0 for the first block), the block's
  token ids (4 each, little endian) and the extra hash (8, little endian);
* a hit also compares the block's stored token ids and extra hash, so a
  collision within one block cannot alias it;
* the first block committed under a hash keeps it; a later block with the
  same hash stays uncached;
* the caller writes the K/V of tokens from ``num_cached`` on; hits need no
  write;
* only full blocks are cached; a partly filled block is never shared
  through the cache.

Plain lists and dicts, no performance intent.
"""
from __future__ import annotations

import copy


class OutOfBlocks(RuntimeError):
    """The free list cannot cover the request (the pages' OOM)."""


FNV64_OFFSET = 0xCBF29CE484222325
FNV64_PRIME = 0x100000001B3


def fnv1a64(data: bytes) -> int:
    """64-bit FNV-1a: for each byte, xor it into the state, then multiply by
    the FNV prime modulo 2**64 (Fowler, Noll and Vo's published definition)."""
    h = FNV64_OFFSET
    for byte in data:
        h ^= byte
        h = (h * FNV64_PRIME) % (1 << 64)
    return h


def block_hash(parent: int, tokens, extra: int = 0) -> int:
    """Chained hash of one full block: hash(parent hash, token ids, extra)."""
    data = int(parent).to_bytes(8, "little")
    for t in tokens:
        data += int(t).to_bytes(4, "little", signed=True)
    data += int(extra).to_bytes(8, "little")
    return fnv1a64(data)


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None, num_host_blocks: int = 0,
                 prefix_caching: bool = False):
        if num_blocks <= 0 or block_size <= 0 or num_host_blocks < 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.prefix_caching = prefix_caching
        self.table_of = {}      # hash -> cached block
        self.cached = {}        # cached block -> (hash, token ids, extra)
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        self.ref = [0] * num_blocks
        self.num_host_blocks = num_host_blocks
        self.host_free = list(range(num_host_blocks))
        self.host_ref = [0] * num_host_blocks
        self.seqs = {}  # seq id -> {"blocks": [...], "len": tokens, "swapped": bool}

    # -- helpers ------------------------------------------------------------
    def _take(self) -> int:
        if not self.free:
            raise OutOfBlocks("no free block")
        b = self.free.pop(0)
        if b in self.cached:  # eviction: the block leaves the cache
            del self.table_of[self.cached.pop(b)[0]]
        self.ref[b] = 1
        return b

    def _commit(self, b: int, h: int, tokens, extra: int) -> None:
        if h not in self.table_of:
            self.table_of[h] = b
            self.cached[b] = (h, tuple(int(t) for t in tokens), int(extra))

    def _hit(self, h: int, tokens, extra: int):
        b = self.table_of.get(h)
        if b is None or self.cached[b][1:] != (tuple(int(t) for t in tokens), int(extra)):
            return None
        return b

    def _slot(self, block: int, offset: int) -> int:
        return block * self.block_size + offset

    # -- primitives ---------------------------------------------------------
    def add(self, sid: int, num_tokens: int) -> list:
        """A new sequence with num_tokens tokens (its prompt); returns their slots."""
        if sid in self.seqs:
            raise KeyError(f"sequence {sid} exists")
        if num_tokens < 0:
            raise ValueError("negative length")
        need = -(-num_tokens // self.block_size)
        if need > len(self.free):
            raise OutOfBlocks(f"{need} blocks needed, {len(self.free)} free")
        blocks = [self._take() for _ in range(need)]
        self.seqs[sid] = {"blocks": blocks, "len": num_tokens, "swapped": False, "tokens": None}
        return [self._slot(blocks[t // self.block_size], t % self.block_size) for t in range(num_tokens)]

    def _append_one(self, sid):
        """One token for one sequence: (its slot, the copy-on-write pair or None)."""
        s = self.seqs[sid]
        if s["swapped"]:
            raise KeyError(f"sequence {sid} is swapped out")
        off = s["len"] % self.block_size
        pair = None
        if off == 0:  # last block full (or none yet): open a new one
            s["blocks"].append(self._take())
        else:
            last = s["blocks"][-1]
            if self.ref[last] > 1:  # shared and not full: copy on write
                fresh = self._take()
                self.ref[last] -= 1
                s["blocks"][-1] = fresh
                pair = (last, fresh)
        s["len"] += 1
        return self._slot(s["blocks"][-1], off), pair

    def _batch(self, sids, tokens):
        saved = copy.deepcopy((self.free, self.ref, self.seqs, self.table_of, self.cached))
        try:
            slots, pairs = [], []
            for i, sid in enumerate(sids):
                slot, pair = self._append_one(sid)
                slots.append(slot)
                if pair:
                    pairs.append(pair)
                t = self.seqs[sid]["tokens"]
                if tokens is None or t is None:
                    self.seqs[sid]["tokens"] = None  # token ids unknown: no more commits
                    continue
                t["partial"].append(int(tokens[i]))
                if len(t["partial"]) == self.block_size:  # the block is full: commit
                    h = block_hash(t["hashes"][-1] if t["hashes"] else 0, t["partial"], t["extra"])
                    self._commit(self.seqs[sid]["blocks"][-1], h, t["partial"], t["extra"])
                    t["hashes"].append(h)
                    t["partial"] = []
            return slots, pairs
        except (OutOfBlocks, KeyError):
            self.free, self.ref, self.seqs, self.table_of, self.cached = saved
            raise

    def append(self, sids) -> tuple:
        """One new token for each listed sequence, in order.  Returns (slots,
        copy-on-write pairs (src, dst) in the order they were made)."""
        return self._batch(list(sids), None)

    def fork(self, parent: int, child: int) -> None:
        if child in self.seqs:
            raise KeyError(f"sequence {child} exists")
        p = self.seqs[parent]
        if p["swapped"]:
            raise KeyError(f"sequence {parent} is swapped out")
        for b in p["blocks"]:
            self.ref[b] += 1
        self.seqs[child] = copy.deepcopy(p)

    def release(self, sid: int) -> None:
        """Free a sequence: one reference less on each block, blocks at zero
        go back to the free list in table order."""
        s = self.seqs.pop(sid)
        ref, free = (self.host_ref, self.host_free) if s["swapped"] else (self.ref, self.free)
        for b in reversed(s["blocks"]):
            ref[b] -= 1
            if ref[b] == 0:
                free.append(b)

    # -- prefix caching -----------------------------------------------------
    def add_prompt(self, sid, tokens, extra: int = 0) -> tuple:
        """A new sequence with these prompt token ids, reusing cached blocks
        of its longest cached prefix of full blocks.  Returns (the slot of
        every token, num_cached: tokens whose K/V is already in the pool)."""
        if not self.prefix_caching:
            raise ValueError("prefix caching is off")
        if sid in self.seqs:
            raise KeyError(f"sequence {sid} exists")
        bs, tokens = self.block_size, [int(t) for t in tokens]
        n, nfull = len(tokens), len(tokens) // bs
        hashes, h = [], 0
        for i in range(nfull):
            h = block_hash(h, tokens[i * bs:(i + 1) * bs], extra)
            hashes.append(h)
        hits = []
        for i in range(nfull):
            b = self._hit(hashes[i], tokens[i * bs:(i + 1) * bs], extra)
            if b is None:
                break
            hits.append(b)
        need = -(-n // bs) - len(hits)
        if need > len(self.free) - sum(1 for b in hits if self.ref[b] == 0):
            raise OutOfBlocks(f"{need} blocks needed")
        for b in hits:  # touch
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
        blocks = list(hits)
        for i in range(len(hits), -(-n // bs)):
            b = self._take()
            blocks.append(b)
            if i < nfull:
                self._commit(b, hashes[i], tokens[i * bs:(i + 1) * bs], extra)
        self.seqs[sid] = {"blocks": blocks, "len": n, "swapped": False,
                          "tokens": {"hashes": hashes, "partial": tokens[nfull * bs:], "extra": int(extra)}}
        return [self._slot(blocks[t // bs], t % bs) for t in range(n)], len(hits) * bs

    def append_tokens(self, sids, tokens) -> tuple:
        """``append`` with the new token ids: a block filled by its last token
        is committed to the cache."""
        if len(tokens) != len(sids):
            raise ValueError("one token per listed sequence")
        return self._batch(list(sids), list(tokens))

    def num_cached_blocks(self) -> int:
        return len(self.table_of)

    def _move(self, sids, to_host: bool) -> list:
        sids = list(sids)
        if len(set(sids)) != len(sids):
            raise ValueError("a sequence is listed twice")
        for sid in sids:
            if self.seqs[sid]["swapped"] == to_host:
                raise KeyError(f"sequence {sid} is already {'out' if to_host else 'in'}")
        src_ref, src_free = (self.ref, self.free) if to_host else (self.host_ref, self.host_free)
        dst_ref, dst_free = (self.host_ref, self.host_free) if to_host else (self.ref, self.free)
        order, held = [], {}
        for sid in sids:
            for b in self.seqs[sid]["blocks"]:
                if b not in held:
                    order.append(b)
                    held[b] = 0
                held[b] += 1
        if any(held[b] != src_ref[b] for b in order):
            raise ValueError("a block is shared with a sequence outside the set")
        if len(order) > len(dst_free):
            raise OutOfBlocks(f"{len(order)} blocks needed, {len(dst_free)} free")
        where = {}
        for b in order:
            if to_host and b in self.cached:
                del self.table_of[self.cached.pop(b)[0]]
            d = dst_free.pop(0)
            if not to_host and d in self.cached:  # eviction: the block will be overwritten
                del self.table_of[self.cached.pop(d)[0]]
            dst_ref[d], src_ref[b] = src_ref[b], 0
            where[b] = d
        src_free.extend(order)
        for sid in sids:
            s = self.seqs[sid]
            s["blocks"] = [where[b] for b in s["blocks"]]
            s["swapped"] = to_host
        return [(b, where[b]) for b in order]

    def swap_out(self, sids) -> list:
        """Move the blocks of these sequences to host blocks; returns the
        (device block, host block) pairs the block swap moves."""
        return self._move(sids, True)

    def swap_in(self, sids) -> list:
        """Move swapped-out sequences back; returns (host block, device block) pairs."""
        return self._move(sids, False)

    # -- views --------------------------------------------------------------
    def table(self, sid: int) -> list:
        return list(self.seqs[sid]["blocks"])

    def seq_len(self, sid: int) -> int:
        return self.seqs[sid]["len"]

    def num_free(self) -> int:
        return len(self.free)

    def num_free_host(self) -> int:
        return len(self.host_free)

    def is_swapped(self, sid: int) -> bool:
        return self.seqs[sid]["swapped"]
