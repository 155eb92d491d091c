"""The pages' closed form for KV-cache size, and paged-pool accounting.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[IV §The Real Reason Your GPU Memory Is "Full" When It Isn't]: per sequence,
KV memory is 2 (K and V) x layers x sequence length x hidden size x bytes per
element.  With grouped KV heads the "hidden" term is the KV width
num_kv_heads x head_dim, which equals the model's hidden size when every
query head has its own KV head.

[RW §How PagedAttention Works]: with fixed-size blocks the only waste is the
unfilled part of each sequence's last block.
"""
from __future__ import annotations


def kv_bytes(num_layers: int, seq_len: int, hidden: int, dtype_bytes: int) -> int:
    """Live KV bytes of one sequence: 2 * layers * seq_len * hidden * bytes."""
    return 2 * num_layers * seq_len * hidden * dtype_bytes


def kv_bytes_gqa(num_layers: int, seq_len: int, num_kv_heads: int,
                 head_dim: int, dtype_bytes: int) -> int:
    return kv_bytes(num_layers, seq_len, num_kv_heads * head_dim, dtype_bytes)


def paged_bytes(num_layers: int, seq_len: int, hidden: int, dtype_bytes: int,
                block_size: int) -> int:
    """Pool bytes held by one sequence: whole blocks, ceil(L / B) of them."""
    n_blocks = -(-seq_len // block_size)
    return kv_bytes(num_layers, n_blocks * block_size, hidden, dtype_bytes)


def paged_waste_fraction(seq_lens, block_size: int) -> float:
    """Fraction of held slots that hold no token, over a batch."""
    held = sum(-(-L // block_size) * block_size for L in seq_lens)
    used = sum(seq_lens)
    return (held - used) / held if held else 0.0


def reserved_waste_fraction(seq_lens, max_len: int) -> float:
    """Same fraction when every sequence reserves max_len contiguous slots
    up front (the pre-paging allocator the pages describe)."""
    held = len(seq_lens) * max_len
    return (held - sum(seq_lens)) / held if held else 0.0
