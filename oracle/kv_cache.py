"""Bit-exact reference for the KV write path and copy-on-write block copies.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[IV §PagedAttention: What the OS Figured Out Decades Ago]: as tokens are
generated their keys/values are appended, and new blocks are added to the
sequence's block table.  Each new token therefore goes to one *slot*:
``slot = physical_block * B + offset``.  A negative slot means "no write"
(padding tokens).

[IV §Copy-on-Write Makes Beam Search Cheap], [RW §How PagedAttention Works]:
when a branch writes into a shared block, that block is copied first; the copy
is a whole-block duplicate of K and V for every KV head.

Operates in place on raw 16-bit patterns (numpy uint16 or float16), so the
result is compared bit for bit.  Storage format (the library's documented
one): k_cache [N, Hkv, D/32, B, 32] (element d of the key in slot s at
[.., d // 32, s, d % 32]), v_cache [N, Hkv, B/4, D, 4] (groups of four
slots, dim-major within a group: element d of the value in slot s at
[.., s // 4, d, s % 4]).
"""
from __future__ import annotations

import numpy as np


def write_kv(k_cache: np.ndarray, v_cache: np.ndarray, k: np.ndarray,
             v: np.ndarray, slot_mapping, block_size: int) -> None:
    """For each token i with slot_mapping[i] >= 0 store k[i], v[i] (each
    [Hkv, D]) into the slot; tokens are applied in index order."""
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), block_size)
        H, D = k[i].shape
        k_cache[blk, :, :, off, :] = k[i].reshape(H, D // 32, 32)
        v_cache[blk, :, off // 4, :, off % 4] = v[i]


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, pairs) -> None:
    """Apply (src, dst) whole-block copies in order, K and V, all heads."""
    for src, dst in np.asarray(pairs).reshape(-1, 2).tolist():
        k_cache[dst] = k_cache[src]
        v_cache[dst] = v_cache[src]


def swap_blocks(dev_k: np.ndarray, dev_v: np.ndarray, host_k: np.ndarray, host_v: np.ndarray,
                pairs, direction: int) -> None:
    """Whole-block copies between the device caches and host swap space of
    the same layout, in pair order: direction 0 copies device block src to
    host block dst, direction 1 host block src to device block dst; a pair
    with an id outside its side's range is skipped.  Moving a sequence's
    blocks to CPU memory and back ("Inside vLLM ...", section "Python LLM
    Inference Optimization with vLLM: Parameters That Actually Matter")."""
    src_k, src_v, dst_k, dst_v = ((dev_k, dev_v, host_k, host_v) if direction == 0
                                  else (host_k, host_v, dev_k, dev_v))
    for src, dst in np.asarray(pairs).reshape(-1, 2).tolist():
        if 0 <= src < src_k.shape[0] and 0 <= dst < dst_k.shape[0]:
            dst_k[dst] = src_k[src]
            dst_v[dst] = src_v[src]
