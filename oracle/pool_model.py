"""Reference model of the refcounted KV block pool with copy-on-write.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix:
  * the cache is cut into fixed-size blocks (16 tokens by default); a block
    table per sequence maps logical block j to a physical block, and new
    blocks are appended as tokens are generated
    [IV §PagedAttention: What the OS Figured Out Decades Ago];
  * blocks are claimed on demand and released as soon as a sequence finishes
    [IV §PagedAttention ...], [RW §How PagedAttention Works];
  * branches of one prompt hold its blocks by reference count, and a block
    is duplicated for a branch only at the moment that branch writes into
    it; every other block stays common [IV §Copy-on-Write Makes Beam Search Cheap],
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

Prefix caching (optional, ``prefix_caching=True``).  The pages fix: the
content of each full block is hashed, and a new request whose leading tokens
hash-match blocks already computed reuses those physical blocks instead of
recomputing them [IV §PagedAttention in a Python RAG Application, and its
question "How does prefix caching work in vLLM and when does it actually
help?"]; cached prefixes skip their prefill [TG §Tuning Batching, Prefill,
and Cache].  Readings where the pages are silent:
  * a block's content is its 16 token ids *and* everything before them, so
    the key of a full block is (key of the block before it, its token ids);
    keys are exact (compared in full), never a lossy hash, and each distinct
    key gets a content id the first time it is registered, kept for good;
  * a block is registered when its last slot is appended, if its tokens are
    known (appended with ids) and the block before it is registered (or it is
    the first block); if its content id already maps to a live block it
    stays unregistered (a duplicate);
  * ``append_tokens`` looks up whole blocks only, starting at a block
    boundary, from the sequence's current last block, and stops at the first
    miss or at ``max_hit_tokens``; reused tokens get slot -1 (nothing to
    write) and count as cached for prefill;
  * a registered block whose references drop to zero is not freed but moves
    to the tail of an evictable list (least recently released first); a hit
    takes it back out; allocation uses the free stack first and then evicts
    the head of that list (unmapping its content id);
  * ``append``/``append_tokens`` stay all-or-nothing over the free stack plus
    the evictable list (less the evictable blocks the call itself reuses).

Swapping (optional, ``num_host_blocks > 0``).  The pages fix: under memory
pressure a sequence's blocks can be moved to CPU memory and brought back
later, at the cost of host-link bandwidth [IV §Python LLM Inference
Optimization with vLLM: Parameters That Actually Matter].  Readings:
  * host swap space is its own pool of host blocks, handed out from a LIFO
    stack whose initial order is the identity (host block 0 first);
  * ``swap_out`` moves a whole sequence: for each of its blocks in table
    order it takes a host block, reports (device, host), and drops the
    device block's reference (a shared block stays with its other holders;
    one that reaches zero is released as by ``free``).  All-or-nothing over
    the host free stack.  The sequence then holds host blocks only and
    cannot append or fork until swapped in;
  * ``swap_in`` takes a device block per host block (free stack, then
    eviction), in table order, reports (host, device), and returns the host
    blocks to their stack in that order.  All-or-nothing over free plus
    evictable device blocks.  The new device blocks are not registered for
    prefix caching (their content ids are not carried over);
  * ``free`` of a swapped sequence returns its host blocks in table order.
"""
from __future__ import annotations

from .splitmix64 import shuffled_order


class PoolError(Exception):
    def __init__(self, code: str, msg: str = ""):
        super().__init__(f"{code}: {msg}")
        self.code = code


class PoolModel:
    def __init__(self, num_blocks: int, block_size: int, seed: int = 0,
                 prefix_caching: bool = False, num_host_blocks: int = 0):
        if num_blocks <= 0 or block_size <= 0:
            raise PoolError("EINVAL", "num_blocks and block_size must be > 0")
        self.N = num_blocks
        self.B = block_size
        order = shuffled_order(num_blocks, seed)
        self.stack = list(reversed(order))   # top of the stack = end of list
        self.ref = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.ntok: dict[int, int] = {}
        self.toks: dict[int, list] = {}      # token ids per sequence (None: unknown)
        self.next_id = 1
        self.caching = prefix_caching
        self.evictable: list[int] = []       # head = least recently released
        self.content_of_block = [-1] * num_blocks
        self.block_of_content: dict[int, int] = {}
        self.content_ids: dict[tuple, int] = {}   # (previous content id, tokens) -> id
        self.host_stack = list(range(num_host_blocks - 1, -1, -1))   # top = end: host block 0 first
        self.host_tables: dict[int, list[int]] = {}   # sequences that are swapped out

    # -- queries ---------------------------------------------------------
    def num_free(self) -> int:
        return len(self.stack)

    def num_free_host(self) -> int:
        return len(self.host_stack)

    def num_cached(self) -> int:
        """Registered blocks with no reference, kept for reuse."""
        return len(self.evictable)

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
        self.toks[sid] = []
        return sid

    def seq_fork(self, parent: int) -> int:
        self._check(parent)
        self._resident(parent)
        sid = self.next_id
        self.next_id += 1
        self.tables[sid] = list(self.tables[parent])
        self.ntok[sid] = self.ntok[parent]
        self.toks[sid] = list(self.toks[parent])
        for b in self.tables[sid]:
            self.ref[b] += 1
        return sid

    def seq_append(self, seq: int, n_tokens: int):
        """Returns (slot_mapping [n_tokens], cow_pairs [(src, dst)])."""
        self._check(seq)
        self._resident(seq)
        if n_tokens < 0:
            raise PoolError("EINVAL", "negative token count")
        slots, cow, _ = self._append(seq, [None] * n_tokens, 0)
        return slots, cow

    def seq_append_tokens(self, seq: int, tokens, max_hit_tokens: int):
        """Append tokens with known ids.  Returns (slot_mapping, cow_pairs,
        n_hit): the first n_hit tokens reuse cached blocks (slot -1)."""
        self._check(seq)
        self._resident(seq)
        return self._append(seq, [int(x) for x in tokens], max(0, int(max_hit_tokens)))

    def seq_swap_out(self, seq: int):
        """Returns [(device block, host block)] in table order."""
        self._check(seq)
        self._resident(seq)
        table = self.tables[seq]
        if len(table) > len(self.host_stack):
            raise PoolError("ENOMEM", f"need {len(table)} host blocks, {len(self.host_stack)} free")
        pairs, host = [], []
        for b in table:
            h = self.host_stack.pop()
            pairs.append((b, h))
            host.append(h)
            self._release(b)
        self.tables[seq] = []
        self.host_tables[seq] = host
        return pairs

    def seq_swap_in(self, seq: int):
        """Returns [(host block, device block)] in table order."""
        self._check(seq)
        if seq not in self.host_tables:
            raise PoolError("EINVAL", f"sequence {seq} is not swapped out")
        host = self.host_tables[seq]
        if len(host) > len(self.stack) + len(self.evictable):
            raise PoolError("ENOMEM", f"need {len(host)} blocks, "
                                      f"{len(self.stack) + len(self.evictable)} available")
        pairs = []
        for h in host:
            d = self._take()
            pairs.append((h, d))
            self.tables[seq].append(d)
            self.host_stack.append(h)
        del self.host_tables[seq]
        return pairs

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if self.content_of_block[b] >= 0:
                self.evictable.append(b)
            else:
                self.stack.append(b)

    def _resident(self, seq: int) -> None:
        if seq in self.host_tables:
            raise PoolError("EINVAL", f"sequence {seq} is swapped out")

    def _append(self, seq: int, tokens: list, max_hit: int):
        table = self.tables[seq]
        n0 = self.ntok[seq]
        n_tokens = len(tokens)
        B = self.B
        # Whole-block hits along the content chain, not applied yet.
        # The chain starts at the root (empty sequence) or at a registered
        # last block; an unregistered last block has no known content.
        hits = []
        if self.caching and n0 % B == 0 and (not table or self.content_of_block[table[-1]] >= 0):
            prev = self.content_of_block[table[-1]] if table else -1
            while (len(hits) + 1) * B <= min(n_tokens, max_hit):
                blk_toks = tokens[len(hits) * B:(len(hits) + 1) * B]
                if any(t is None for t in blk_toks):
                    break
                cid = self.content_ids.get((prev, tuple(blk_toks)))
                if cid is None or cid not in self.block_of_content:
                    break
                hits.append(self.block_of_content[cid])
                prev = cid
        n_hit = len(hits) * B
        rest = n_tokens - n_hit
        need_cow = (rest > 0 and n0 % B != 0 and self.ref[table[-1]] > 1)
        blocks_after = -(-(n0 + n_tokens) // B)
        need_new = blocks_after - len(table) - len(hits) + (1 if need_cow else 0)
        reused_idle = sum(1 for b in hits if self.ref[b] == 0)
        avail = len(self.stack) + len(self.evictable) - reused_idle
        if need_new > avail:
            raise PoolError("ENOMEM", f"need {need_new} blocks, {avail} available")
        slots, cow = [], []
        for b in hits:
            if self.ref[b] == 0:
                self.evictable.remove(b)
            self.ref[b] += 1
            table.append(b)
        for t in tokens[:n_hit]:
            self.toks[seq].append(t)
        slots += [-1] * n_hit
        self.ntok[seq] = n0 + n_hit
        for t in tokens[n_hit:]:
            n = self.ntok[seq]
            if n % B == 0:
                table.append(self._take())
            elif self.ref[table[-1]] > 1:
                src = table[-1]
                dst = self._take()
                self.ref[src] -= 1
                table[-1] = dst
                cow.append((src, dst))
            slots.append(table[-1] * B + n % B)
            self.toks[seq].append(t)
            self.ntok[seq] = n + 1
            if (n + 1) % B == 0:
                self._register(seq, len(table) - 1)
        return slots, cow, n_hit

    def _take(self) -> int:
        if self.stack:
            b = self.stack.pop()
        else:
            b = self.evictable.pop(0)
            del self.block_of_content[self.content_of_block[b]]
            self.content_of_block[b] = -1
        self.ref[b] = 1
        return b

    def _register(self, seq: int, j: int) -> None:
        if not self.caching:
            return
        table, B = self.tables[seq], self.B
        prev = self.content_of_block[table[j - 1]] if j > 0 else -1
        if j > 0 and prev == -1:
            return
        blk_toks = self.toks[seq][j * B:(j + 1) * B]
        if any(t is None for t in blk_toks):
            return
        key = (prev, tuple(blk_toks))
        cid = self.content_ids.setdefault(key, len(self.content_ids))
        if cid in self.block_of_content:
            return
        self.block_of_content[cid] = table[j]
        self.content_of_block[table[j]] = cid

    def seq_free(self, seq: int) -> None:
        self._check(seq)
        for b in self.tables.pop(seq):
            self._release(b)
        for h in self.host_tables.pop(seq, []):
            self.host_stack.append(h)
        del self.ntok[seq]
        del self.toks[seq]

    def _check(self, seq: int) -> None:
        if seq not in self.tables:
            raise PoolError("EINVAL", f"unknown sequence {seq}")
