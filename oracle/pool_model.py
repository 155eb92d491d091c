"""Reference model of the refcounted KV block pool with copy-on-write.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix:
  * the cache is cut into fixed-size blocks (16 tokens by default); a block
    table per sequence maps logical block j to a physical block, and new
    blocks are appended as tokens are generated
    [IV §PagedAttention: What the OS Figured Out Decades Ago];
  * blocks are claimed on demand and released as soon as a sequence finishes
    [IV §PagedAttention ...], [RW §How PagedAttention Works];
  * sequences branched from one prompt share its blocks through reference
    counts; only when a branch writes a new token is *that* block copied, the
    rest stays shared [IV §Copy-on-Write Makes Beam Search Cheap],
    [RW §How PagedAttention Works], [TG §How PagedAttention Reclaims GPU
    Memory];
  * the allocator acts as the page-frame table of the pool [IV §Python LLM
    Inference Optimization with vLLM: Parameters That Actually Matter].

Readings where the pages are silent (stated, and shared with the library only
as a specification, not as code):
  * the free list is a LIFO stack; its initial order is a Fisher-Yates shuffle
    of [0, N) driven by SplitMix64(seed) (seed 0: identity).  Allocation takes
    order[0] first; a freed block goes on top and is the next one handed out;
  * ``append`` is all-or-nothing: if the free blocks cannot cover every new
    block plus the copy-on-write copy, nothing changes and it reports ENOMEM;
  * a copy-on-write copy happens exactly when a token is appended into a
    partially filled last block whose refcount is above one; the sequence
    gets a fresh block, the pair (old, new) is reported for the device copy,
    and the old block loses one reference;
  * ``free`` drops one reference from every block in table order; blocks that
    reach zero are pushed in that order (the last one ends on top);
  * sequence ids count up from 1.
"""
from __future__ import annotations

from .splitmix64 import shuffled_order


class PoolError(Exception):
    def __init__(self, code: str, msg: str = ""):
        super().__init__(f"{code}: {msg}")
        self.code = code


class PoolModel:
    def __init__(self, num_blocks: int, block_size: int, seed: int = 0):
        if num_blocks <= 0 or block_size <= 0:
            raise PoolError("EINVAL", "num_blocks and block_size must be > 0")
        self.N = num_blocks
        self.B = block_size
        order = shuffled_order(num_blocks, seed)
        self.stack = list(reversed(order))   # top of the stack = end of list
        self.ref = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.ntok: dict[int, int] = {}
        self.next_id = 1

    # -- queries ---------------------------------------------------------
    def num_free(self) -> int:
        return len(self.stack)

    def refcount(self, block: int) -> int:
        return self.ref[block] if 0 <= block < self.N else -1

    def block_table(self, seq: int):
        self._check(seq)
        return list(self.tables[seq]), self.ntok[seq]

    # -- operations ------------------------------------------------------
    def seq_create(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.tables[sid] = []
        self.ntok[sid] = 0
        return sid

    def seq_fork(self, parent: int) -> int:
        self._check(parent)
        sid = self.next_id
        self.next_id += 1
        self.tables[sid] = list(self.tables[parent])
        self.ntok[sid] = self.ntok[parent]
        for b in self.tables[sid]:
            self.ref[b] += 1
        return sid

    def seq_append(self, seq: int, n_tokens: int):
        """Returns (slot_mapping [n_tokens], cow_pairs [(src, dst)])."""
        self._check(seq)
        if n_tokens < 0:
            raise PoolError("EINVAL", "negative token count")
        table = self.tables[seq]
        n0 = self.ntok[seq]
        B = self.B
        need_cow = (n_tokens > 0 and n0 % B != 0 and self.ref[table[-1]] > 1)
        blocks_after = -(-(n0 + n_tokens) // B)
        need_new = blocks_after - len(table) + (1 if need_cow else 0)
        if need_new > len(self.stack):
            raise PoolError("ENOMEM", f"need {need_new} blocks, "
                                      f"{len(self.stack)} free")
        cow = []
        slots = []
        for _ in range(n_tokens):
            n = self.ntok[seq]
            if n % B == 0:
                b = self.stack.pop()
                self.ref[b] = 1
                table.append(b)
            elif self.ref[table[-1]] > 1:
                src = table[-1]
                dst = self.stack.pop()
                self.ref[dst] = 1
                self.ref[src] -= 1
                table[-1] = dst
                cow.append((src, dst))
            slots.append(table[-1] * B + n % B)
            self.ntok[seq] = n + 1
        return slots, cow

    def seq_free(self, seq: int) -> None:
        self._check(seq)
        for b in self.tables.pop(seq):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.stack.append(b)
        del self.ntok[seq]

    def _check(self, seq: int) -> None:
        if seq not in self.tables:
            raise PoolError("EINVAL", f"unknown sequence {seq}")
