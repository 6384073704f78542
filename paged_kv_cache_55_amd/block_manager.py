"""Host-side block manager and admission ledger for a paged KV pool.

This is the bookkeeping that produces the integer inputs of the device
calls: block tables, slot numbers for new tokens, and (src, dst) pairs for
copy-on-write. It never touches KV values.

* One pool of fixed-size blocks is allocated up front; a sequence takes a
  block from the free list only when its last block is full, and its blocks
  need not be neighbours [cs2680 Lecture 10, §10.3].
* Blocks are reference counted; a fork shares every block, and the first
  write into a shared block copies it to a fresh block first (copy-on-write:
  the writer gets the copy with refcount 1, the original loses one
  reference) [cs2680 Lecture 10, §10.4 and its instructor notes;
  llm-serving.xyz "KV-cache systems", copy-on-write paragraph].
* Ownership is a ledger separate from device memory: freeing a block only
  returns it to the free list [inferenceinterviews.com "Reserve the page a
  request has not written yet", "Separate the pool from its owners"].
* Admission reserves whole pages for the full declared output, and charges a
  trust group's complete shared-prefix pages once [same page, "Pick a
  reservation policy you can explain" and "Charge shared pages once"].
"""

from __future__ import annotations

from collections import deque

import numpy as np


class OutOfBlocks(RuntimeError):
    """The free list cannot satisfy an allocation."""


def _ceil_div(a: int, b: int) -> int:
    return -(-int(a) // int(b))


class BlockManager:
    """Free list, per-sequence block tables and reference counts."""

    def __init__(self, num_blocks: int, block_size: int = 16,
                 free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = range(num_blocks) if free_order is None else list(free_order)
        if sorted(int(b) for b in order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the block ids")
        self._free = deque(int(b) for b in order)
        self.refcount = np.zeros(num_blocks, dtype=np.int64)
        self.tables: dict = {}
        self.lens: dict = {}

    # -- pool -------------------------------------------------------------
    @property
    def num_free(self) -> int:
        return len(self._free)

    def _take(self) -> int:
        if not self._free:
            raise OutOfBlocks("no free block")
        blk = self._free.popleft()
        self.refcount[blk] = 1
        return blk

    def _release(self, blk: int) -> None:
        self.refcount[blk] -= 1
        if self.refcount[blk] < 0:
            raise AssertionError(f"refcount of block {blk} went negative")
        if self.refcount[blk] == 0:
            self._free.append(blk)

    # -- sequences ----------------------------------------------------------
    def add_sequence(self, seq, num_tokens: int, prefix_from=None,
                     prefix_blocks: int = 0) -> list:
        """Create a sequence of ``num_tokens`` tokens.

        With ``prefix_from`` the first ``prefix_blocks`` blocks are shared
        with that sequence (each gains a reference); the rest are fresh.
        Nothing is allocated unless the whole request fits.
        """
        if seq in self.tables:
            raise KeyError(f"sequence {seq!r} exists")
        need = _ceil_div(num_tokens, self.block_size)
        shared = []
        if prefix_from is not None:
            parent = self.tables[prefix_from]
            if prefix_blocks > len(parent) or prefix_blocks > need:
                raise ValueError("prefix_blocks exceeds the parent or the request")
            if prefix_blocks * self.block_size > num_tokens:
                raise ValueError("a shared prefix block must be complete")
            shared = parent[:prefix_blocks]
        fresh = need - len(shared)
        if fresh > self.num_free:
            raise OutOfBlocks(f"need {fresh} blocks, {self.num_free} free")
        for blk in shared:
            self.refcount[blk] += 1
        table = list(shared) + [self._take() for _ in range(fresh)]
        self.tables[seq] = table
        self.lens[seq] = int(num_tokens)
        return table

    def fork(self, parent, child) -> list:
        """Child shares every block of the parent (parallel sampling)."""
        if child in self.tables:
            raise KeyError(f"sequence {child!r} exists")
        table = list(self.tables[parent])
        for blk in table:
            self.refcount[blk] += 1
        self.tables[child] = table
        self.lens[child] = self.lens[parent]
        return table

    def append_token(self, seq):
        """Reserve the slot of the sequence's next token.

        Returns ``(slot, cow)``: ``slot = block * block_size + offset`` is
        where the new token's K/V go, and ``cow`` is ``(src, dst)`` when the
        target block was shared and had to be copied first, else ``None``.
        """
        pos = self.lens[seq]
        table = self.tables[seq]
        cow = None
        if pos % self.block_size == 0:
            table.append(self._take())
        else:
            last = table[-1]
            if self.refcount[last] > 1:
                dst = self._take()
                self.refcount[last] -= 1
                table[-1] = dst
                cow = (last, dst)
        self.lens[seq] = pos + 1
        slot = table[pos // self.block_size] * self.block_size \
            + pos % self.block_size
        return slot, cow

    def free_sequence(self, seq) -> None:
        for blk in self.tables.pop(seq):
            self._release(blk)
        del self.lens[seq]

    # -- device inputs --------------------------------------------------------
    def table_array(self, seqs, max_blocks: int, pad: int) -> np.ndarray:
        """int32 [len(seqs), max_blocks]; unused entries hold ``pad``."""
        out = np.full((len(seqs), max_blocks), pad, dtype=np.int32)
        for i, s in enumerate(seqs):
            t = self.tables[s]
            if len(t) > max_blocks:
                raise ValueError(f"sequence {s!r} has {len(t)} blocks > {max_blocks}")
            out[i, :len(t)] = t
        return out

    def len_array(self, seqs) -> np.ndarray:
        return np.array([self.lens[s] for s in seqs], dtype=np.int32)


class AdmissionLedger:
    """Page reservations promised to admitted requests.

    Each request reserves ceil((prompt + max_output) / block) pages up front.
    Within one trust group the complete pages of a shared prefix are charged
    once, to the group, while it has members; every request pays its own
    private pages. A request that does not fit is refused and nothing is
    charged.
    """

    def __init__(self, pool_pages: int, block_size: int = 16):
        self.pool_pages = int(pool_pages)
        self.block_size = int(block_size)
        self.reserved = 0
        self._private: dict = {}      # request -> (group, private pages)
        self._groups: dict = {}       # group -> [shared pages, member set]

    @property
    def free_pages(self) -> int:
        return self.pool_pages - self.reserved

    def _split(self, prompt_tokens, max_output_tokens, group,
               shared_prefix_tokens):
        total = _ceil_div(prompt_tokens + max_output_tokens, self.block_size)
        if group is None or not shared_prefix_tokens:
            return 0, total
        shared = int(shared_prefix_tokens) // self.block_size
        return shared, total - shared

    def pages_needed(self, prompt_tokens: int, max_output_tokens: int,
                     group=None, shared_prefix_tokens: int = 0) -> int:
        shared, private = self._split(prompt_tokens, max_output_tokens, group,
                                      shared_prefix_tokens)
        if group in self._groups:
            shared = 0
        return shared + private

    def reserve(self, request_id, prompt_tokens: int, max_output_tokens: int,
                group=None, shared_prefix_tokens: int = 0) -> bool:
        if request_id in self._private:
            raise KeyError(f"request {request_id!r} already admitted")
        shared, private = self._split(prompt_tokens, max_output_tokens, group,
                                      shared_prefix_tokens)
        new_group = shared > 0 and group not in self._groups
        need = private + (shared if new_group else 0)
        if need > self.free_pages:
            return False
        self.reserved += need
        if new_group:
            self._groups[group] = [shared, set()]
        if group in self._groups:
            self._groups[group][1].add(request_id)
            self._private[request_id] = (group, private)
        else:
            self._private[request_id] = (None, private)
        return True

    def release(self, request_id) -> None:
        group, private = self._private.pop(request_id)
        self.reserved -= private
        if group is not None:
            shared, members = self._groups[group]
            members.discard(request_id)
            if not members:
                self.reserved -= shared
                del self._groups[group]
