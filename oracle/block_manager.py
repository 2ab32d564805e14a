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

Readings where the pages are silent or disagree (listed in the design doc):

* free-list order: blocks are taken from the front and returned to the back
  (first in, first out).  One page's code pops from the back, the other's
  from the front; the front is what reproduces the interleaved 9-block
  figure of "vLLM 深度解析" §3.1 (request tables [1, 3, 5] and
  [0, 2, 4, 6]);
* a full shared last block is left shared: the new token opens a new block
  and nothing is copied;
* a batch append either succeeds for every sequence or, when the free list
  cannot cover it, changes nothing and raises ``OutOfBlocks``;
* a freed sequence returns its blocks in table order.

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
* a swap the destination cannot hold changes nothing (out of blocks).

Plain lists and dicts, no performance intent.
"""
from __future__ import annotations

import copy


class OutOfBlocks(RuntimeError):
    """The free list cannot cover the request (the pages' OOM)."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None, num_host_blocks: int = 0):
        if num_blocks <= 0 or block_size <= 0 or num_host_blocks < 0:
            raise ValueError("num_blocks and block_size must be positive")
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
        self.ref[b] = 1
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
        self.seqs[sid] = {"blocks": blocks, "len": num_tokens, "swapped": False}
        return [self._slot(blocks[t // self.block_size], t % self.block_size) for t in range(num_tokens)]

    def append(self, sids) -> tuple:
        """One new token for each listed sequence, in order.  Returns (slots,
        copy-on-write pairs (src, dst) in the order they were made)."""
        saved = copy.deepcopy((self.free, self.ref, self.seqs))
        try:
            slots, pairs = [], []
            for sid in sids:
                s = self.seqs[sid]
                if s["swapped"]:
                    raise KeyError(f"sequence {sid} is swapped out")
                off = s["len"] % self.block_size
                if off == 0:  # last block full (or none yet): open a new one
                    s["blocks"].append(self._take())
                else:
                    last = s["blocks"][-1]
                    if self.ref[last] > 1:  # shared and not full: copy on write
                        fresh = self._take()
                        self.ref[last] -= 1
                        s["blocks"][-1] = fresh
                        pairs.append((last, fresh))
                slots.append(self._slot(s["blocks"][-1], off))
                s["len"] += 1
            return slots, pairs
        except (OutOfBlocks, KeyError):
            self.free, self.ref, self.seqs = saved
            raise

    def fork(self, parent: int, child: int) -> None:
        if child in self.seqs:
            raise KeyError(f"sequence {child} exists")
        p = self.seqs[parent]
        if p["swapped"]:
            raise KeyError(f"sequence {parent} is swapped out")
        for b in p["blocks"]:
            self.ref[b] += 1
        self.seqs[child] = {"blocks": list(p["blocks"]), "len": p["len"], "swapped": False}

    def release(self, sid: int) -> None:
        """Free a sequence: one reference less on each block, blocks at zero
        go back to the free list in table order."""
        s = self.seqs.pop(sid)
        ref, free = (self.host_ref, self.host_free) if s["swapped"] else (self.ref, self.free)
        for b in s["blocks"]:
            ref[b] -= 1
            if ref[b] == 0:
                free.append(b)

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
            d = dst_free.pop(0)
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
