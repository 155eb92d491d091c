"""Workload definitions and seeded input draws (no attention arithmetic)."""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16


def torch_dtype(dtype: str):
    import torch
    return {"fp16": torch.float16, "bf16": torch.bfloat16}[dtype]


def normal_tensor(shape, dtype: str, gen):
    """N(0, 1) values drawn by ``gen`` (a torch.Generator) on its device,
    stored in the 16-bit format ``dtype``."""
    import torch
    return torch.randn(*shape, generator=gen, device=gen.device,
                       dtype=torch.float32).to(torch_dtype(dtype))


def _scatter_layout(lens, block_size, bt_stride, rng, pool_blocks=None,
                    pool_factor=1.2, extra_seqs_blocks=()):
    """Random physical placement: a seeded permutation of the pool, handed out
    in sequence order.  Unused block-table entries point at ``pad_block``, an
    unused block (so any stray read stays inside the pool)."""
    nb = [-(-int(L) // block_size) for L in lens] + list(extra_seqs_blocks)
    demand = int(sum(nb))
    if pool_blocks is None:
        pool_blocks = int(np.ceil(pool_factor * demand))
    if pool_blocks < demand:
        raise ValueError("pool smaller than demand")
    perm = rng.permutation(pool_blocks).astype(np.int32)
    if pool_blocks > demand:
        pad_block, n_total = int(perm[demand]), pool_blocks
    else:
        pad_block, n_total = pool_blocks, pool_blocks + 1
    bt = np.full((len(nb), bt_stride), pad_block, dtype=np.int32)
    at = 0
    for s, n in enumerate(nb):
        if n > bt_stride:
            raise ValueError("sequence longer than the block table")
        bt[s, :n] = perm[at:at + n]
        at += n
    return bt, n_total, pad_block


@dataclass
class DecodeWorkload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    context_lens: np.ndarray          # int32 [S]
    block_tables: np.ndarray          # int32 [S, bt_stride]
    num_blocks: int                   # physical blocks in the pool
    pad_block: int                    # block that unused table entries name
    partition_size: int = 0           # 0: library default
    max_model_len: int = 2048
    block_size: int = BLOCK_SIZE

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.head_dim)))

    @property
    def kv_bytes(self) -> int:
        """Bytes of K and V the step must read: sum_s L_s * 2 * Hkv * D * 2."""
        return int(self.context_lens.astype(np.int64).sum()) * 2 * \
            self.num_kv_heads * self.head_dim * 2

    def cache_shapes(self):
        """K [N, Hkv, D/32, B, 32] (32-dim chunks) and V [N, Hkv, B/4, D, 4]
        (groups of four slots, dim-major within a group)."""
        N, H, B, D = self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim
        return (N, H, D // 32, B, 32), (N, H, B // 4, D, 4)

    def make_tensors(self, device="cpu", seed_offset=0):
        """q [S, Hq, D], k_cache [N, Hkv, D/32, B, 32], v_cache [N, Hkv, B/4, D, 4]."""
        import torch
        g = torch.Generator(device=device)
        g.manual_seed(self.seed + seed_offset)
        kshape, vshape = self.cache_shapes()
        q = normal_tensor((self.num_seqs, self.num_q_heads, self.head_dim), self.dtype, g)
        k = normal_tensor(kshape, self.dtype, g)
        v = normal_tensor(vshape, self.dtype, g)
        return q, k, v


def tiny(seed: int = 4221) -> DecodeWorkload:
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.array([1, 17, 33, 100], dtype=np.int32)
    bt, n, pad = _scatter_layout(lens, BLOCK_SIZE, 8, rng, pool_blocks=64)
    return DecodeWorkload("tiny", seed, 4, 4, 64, "fp16", lens, bt, n, pad,
                          max_model_len=128)


def llama7b(seed: int = 4222, num_seqs: int = 64) -> DecodeWorkload:
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(128, 2048 + 1, size=num_seqs).astype(np.int32)
    bt, n, pad = _scatter_layout(lens, BLOCK_SIZE, 128, rng)
    return DecodeWorkload("llama7b", seed, 32, 32, 128, "fp16", lens, bt, n, pad,
                          max_model_len=2048)


def llama8b_gqa(seed: int = 4224, num_seqs: int = 256) -> DecodeWorkload:
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(512, 4096 + 1, size=num_seqs).astype(np.int32)
    bt, n, pad = _scatter_layout(lens, BLOCK_SIZE, 256, rng)
    return DecodeWorkload("llama8b_gqa", seed, 32, 8, 128, "bf16", lens, bt, n, pad,
                          partition_size=512, max_model_len=4096)


def llama8b_long(seed: int = 4226, num_seqs: int = 32) -> DecodeWorkload:
    """Long contexts, 8192 to 32768 tokens: each is longer than one
    partition's block table (4096 tokens), so every sequence is split into
    partitions whose states the second pass merges."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(8192, 32768 + 1, size=num_seqs).astype(np.int32)
    bt, n, pad = _scatter_layout(lens, BLOCK_SIZE, 2048, rng)
    return DecodeWorkload("llama8b_long", seed, 32, 8, 128, "bf16", lens, bt, n, pad,
                          max_model_len=32768)


# ---------------------------------------------------------------------------
# prefix sharing (copy-on-write) workload: logical description only.  The
# physical layout is produced by whoever lays it out (the block pool, or a
# private copy per sequence).
# ---------------------------------------------------------------------------

@dataclass
class SharedWorkload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    context_lens: np.ndarray        # int32 [S]
    group_size: int
    prefix_lens: np.ndarray         # int32 [S // group_size]
    token_rows: list = field(default_factory=list)  # per seq: int64 [L_s]
    num_token_rows: int = 0
    num_blocks: int = 0             # pool size: 1.2 x private demand (+1 pad)
    bt_stride: int = 128
    block_size: int = BLOCK_SIZE
    max_model_len: int = 2048

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.head_dim)))

    @property
    def kv_bytes(self) -> int:
        """Logical bytes: every sequence reads its whole context."""
        return int(self.context_lens.astype(np.int64).sum()) * 2 * \
            self.num_kv_heads * self.head_dim * 2

    @property
    def unique_kv_bytes(self) -> int:
        """Distinct token rows (shared prefixes counted once)."""
        return self.num_token_rows * 2 * self.num_kv_heads * self.head_dim * 2

    def make_tensors(self, device="cpu"):
        """q [S, Hq, D], k_tok / v_tok [num_token_rows, Hkv, D]."""
        import torch
        g = torch.Generator(device=device)
        g.manual_seed(self.seed)
        q = normal_tensor((self.num_seqs, self.num_q_heads, self.head_dim), self.dtype, g)
        k = normal_tensor((self.num_token_rows, self.num_kv_heads, self.head_dim), self.dtype, g)
        v = normal_tensor((self.num_token_rows, self.num_kv_heads, self.head_dim), self.dtype, g)
        return q, k, v


def llama13b_shared(seed: int = 4223, num_seqs: int = 128, num_heads: int = 40,
                    max_len: int = 2048) -> SharedWorkload:
    if num_seqs % 4:
        raise ValueError("groups of 4")
    rng = np.random.Generator(np.random.PCG64(seed))
    raw = rng.lognormal(mean=np.log(400.0), sigma=1.0, size=num_seqs)
    lens = np.clip(np.rint(raw), 1, max_len).astype(np.int32)
    G = 4
    prefix = np.array([int(lens[k * G:(k + 1) * G].min()) // 2
                       for k in range(num_seqs // G)], dtype=np.int32)
    rows = []
    at = 0
    for k in range(num_seqs // G):
        P = int(prefix[k])
        pre = np.arange(at, at + P, dtype=np.int64)
        at += P
        for s in range(k * G, (k + 1) * G):
            own = int(lens[s]) - P
            rows.append(np.concatenate([pre, np.arange(at, at + own, dtype=np.int64)]))
            at += own
    demand = sum(-(-int(L) // BLOCK_SIZE) for L in lens)
    return SharedWorkload("llama13b_shared", seed, num_heads, num_heads, 128, "fp16",
                          lens, G, prefix, rows, at,
                          num_blocks=int(np.ceil(1.2 * demand)) + 1,
                          bt_stride=-(-max_len // BLOCK_SIZE), max_model_len=max_len)


# ---------------------------------------------------------------------------
# mixed step: slot-mapped write of 8192 new tokens, 2 prefill chunks, 4096
# decode sequences, all at the 8B GQA shape.
# ---------------------------------------------------------------------------

@dataclass
class MixedWorkload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    decode_lens: np.ndarray          # int32 [S_dec], includes the new token
    decode_bt: np.ndarray            # int32 [S_dec, bt_stride]
    prefill_cached: int              # tokens already cached per chunk
    prefill_chunk: int               # query tokens per chunk
    prefill_bt: np.ndarray           # int32 [n_chunks, bt_stride]
    slot_mapping: np.ndarray         # int64 [T]: decode tokens, then chunks
    num_blocks: int
    pad_block: int
    partition_size: int = 0           # 0: library default
    max_model_len: int = 4096
    block_size: int = BLOCK_SIZE

    @property
    def num_decode(self) -> int:
        return int(self.decode_lens.shape[0])

    @property
    def num_chunks(self) -> int:
        return int(self.prefill_bt.shape[0])

    @property
    def num_new_tokens(self) -> int:
        return int(self.slot_mapping.shape[0])

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.head_dim)))

    @property
    def q_start_loc(self) -> np.ndarray:
        return (np.arange(self.num_chunks + 1) * self.prefill_chunk).astype(np.int32)

    @property
    def prefill_seq_lens(self) -> np.ndarray:
        return np.full(self.num_chunks, self.prefill_cached + self.prefill_chunk, np.int32)

    @property
    def decode_kv_bytes(self) -> int:
        return int(self.decode_lens.astype(np.int64).sum()) * 2 * \
            self.num_kv_heads * self.head_dim * 2

    @property
    def prefill_flops(self) -> int:
        """Causal QK^T + PV multiply-adds x 2: Hq * 4 * D * sum_j (n_cached + j + 1)."""
        n, c = self.prefill_chunk, self.prefill_cached
        keys = n * c + n * (n + 1) // 2
        return self.num_chunks * self.num_q_heads * 4 * self.head_dim * keys

    @property
    def write_bytes(self) -> int:
        """New K and V read once and written once."""
        return self.num_new_tokens * 2 * self.num_kv_heads * self.head_dim * 2 * 2

    def cache_shapes(self):
        """K [N, Hkv, D/32, B, 32] (32-dim chunks) and V [N, Hkv, B/4, D, 4]
        (groups of four slots, dim-major within a group)."""
        N, H, B, D = self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim
        return (N, H, D // 32, B, 32), (N, H, B // 4, D, 4)

    def make_tensors(self, device="cpu"):
        """Pre-step caches, new k/v [T, Hkv, D], decode q [S_dec, Hq, D],
        prefill q [n_chunks * chunk, Hq, D]."""
        import torch
        g = torch.Generator(device=device)
        g.manual_seed(self.seed)
        kshape, vshape = self.cache_shapes()
        H, Hq, D = self.num_kv_heads, self.num_q_heads, self.head_dim
        kc = normal_tensor(kshape, self.dtype, g)
        vc = normal_tensor(vshape, self.dtype, g)
        k_new = normal_tensor((self.num_new_tokens, H, D), self.dtype, g)
        v_new = normal_tensor((self.num_new_tokens, H, D), self.dtype, g)
        q_dec = normal_tensor((self.num_decode, Hq, D), self.dtype, g)
        q_pre = normal_tensor((self.num_chunks * self.prefill_chunk, Hq, D), self.dtype, g)
        return kc, vc, k_new, v_new, q_dec, q_pre


def _slot_of(bt_row, pos: int, block_size: int) -> int:
    """Storage address of logical position ``pos``: block * B + offset."""
    return int(bt_row[pos // block_size]) * block_size + pos % block_size


def mixed(seed: int = 4225, num_decode: int = 4096, num_chunks: int = 2,
          chunk: int = 2048, cached: int = 1024, lmin: int = 256,
          lmax: int = 4096) -> MixedWorkload:
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(lmin, lmax + 1, size=num_decode).astype(np.int32)
    pre_blocks = -(-(cached + chunk) // BLOCK_SIZE)
    stride = -(-lmax // BLOCK_SIZE)
    bt, n, pad = _scatter_layout(lens, BLOCK_SIZE, max(stride, pre_blocks), rng,
                                 extra_seqs_blocks=[pre_blocks] * num_chunks)
    dec_bt, pre_bt = bt[:num_decode], bt[num_decode:]
    slots = [_slot_of(dec_bt[s], int(lens[s]) - 1, BLOCK_SIZE) for s in range(num_decode)]
    for c in range(num_chunks):
        slots += [_slot_of(pre_bt[c], p, BLOCK_SIZE) for p in range(cached, cached + chunk)]
    return MixedWorkload("mixed", seed, 32, 8, 128, "bf16", lens, dec_bt, cached, chunk,
                         pre_bt, np.array(slots, dtype=np.int64), n, pad,
                         max_model_len=lmax)


WORKLOADS = {
    "tiny": tiny,
    "llama7b": llama7b,
    "llama13b_shared": llama13b_shared,
    "llama8b_gqa": llama8b_gqa,
    "llama8b_long": llama8b_long,
    "mixed": mixed,
}


def make_workload(name: str, **kw):
    return WORKLOADS[name](**kw)
