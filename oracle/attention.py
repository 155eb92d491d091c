"""fp64 reference for paged decode, chunked prefill and the split-KV merge.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Page citations use the tags defined in ``oracle/__init__.py``:
[IV] Inside vLLM ..., [RW] vLLM PagedAttention: Reducing KV Cache Memory
Waste, [TG] PagedAttention in vLLM: A Throughput Settings Guide.

Storage format read here (the library's documented cache format; the pages fix
only "fixed-size blocks" of 16 tokens by default, [IV §PagedAttention: What the
OS Figured Out Decades Ago]):

    k_cache[block, kv_head, dim // 32, slot, dim % 32]   shape [N, Hkv, D/32, B, 32]
    v_cache[block, kv_head, slot // 4, dim, slot % 4]    shape [N, Hkv, B/4, D, 4]

Token t of a sequence with block-table row ``bt`` lives in block
``bt[t // B]`` at slot ``t % B``.

Values arrive as raw 16-bit patterns (fp16 or bf16) and are widened exactly to
float64 before any arithmetic.  Readings of points the pages leave open:

  * scale: 1/sqrt(D) passed explicitly as a float32; used as
    float64(float32(scale)).
  * query head h reads KV head h // (Hq / Hkv) (contiguous grouping).
  * a context of length 0 yields a zero output row.
  * the context length counts every key attended, including the newest token.
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# exact widening of 16-bit storage formats
# --------------------------------------------------------------------------

def widen(x, dtype: str) -> np.ndarray:
    """Exact conversion of fp16 / bf16 storage to float64.

    fp16: IEEE binary16, widened by numpy.  bf16: the top 16 bits of an IEEE
    binary32, so the pattern shifted left by 16 *is* the float32 value.
    """
    a = np.asarray(x)
    if dtype == "fp16":
        if a.dtype != np.float16:
            a = a.view(np.float16)
        return a.astype(np.float64)
    if dtype == "bf16":
        u = a.view(np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# gather through the block table  ([IV §PagedAttention ...], [RW §How
# PagedAttention Works]: a block table maps logical block j of a sequence to a
# physical block; non-contiguous blocks read as one contiguous sequence)
# --------------------------------------------------------------------------

def gather_kv(k_cache: np.ndarray, v_cache: np.ndarray, bt_row, n_tokens: int,
              kv_head: int, block_size: int, dtype: str):
    """Contiguous K [n_tokens, D] and V [n_tokens, D] (float64) of one
    sequence and KV head, read from raw 16-bit caches.

    Token t is read from physical block bt_row[t // B], slot t % B; only the
    gathered elements are widened.
    """
    n_blocks = -(-n_tokens // block_size)
    phys = np.asarray(bt_row[:n_blocks], dtype=np.int64)
    D = v_cache.shape[3]
    k_raw = k_cache[phys, kv_head].transpose(0, 2, 1, 3).reshape(len(phys), block_size, D)
    # [nb, D/32, B, 32] -> [nb, B, D/32, 32] -> [nb, B, D]
    v_raw = v_cache[phys, kv_head].transpose(0, 1, 3, 2).reshape(len(phys), block_size, D)
    # [nb, B/4, D, 4] -> [nb, B/4, 4, D] -> [nb, B, D]
    K = widen(np.ascontiguousarray(k_raw), dtype).reshape(-1, D)[:n_tokens]
    V = widen(np.ascontiguousarray(v_raw), dtype).reshape(-1, D)[:n_tokens]
    return K, V


# --------------------------------------------------------------------------
# dense attention for one query row (the definition)
# --------------------------------------------------------------------------

def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
           return_probs: bool = False):
    """softmax(scale * K q) V for one query row, in float64.

    ``q`` [D], ``K``/``V`` [L, D].  L == 0 gives a zero row.
    """
    L, D = V.shape
    if L == 0:
        out = np.zeros(D, dtype=np.float64)
        return (out, np.zeros(0)) if return_probs else out
    z = float(scale) * (K @ q)
    z = z - z.max()
    e = np.exp(z)
    p = e / e.sum()
    out = p @ V
    return (out, p) if return_probs else out


def scale64(scale: float) -> float:
    """The float32 scale the kernels receive, widened exactly."""
    return float(np.float64(np.float32(scale)))


# --------------------------------------------------------------------------
# decode: one query token per sequence against its whole context
# --------------------------------------------------------------------------

def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float,
           dtype: str, block_size: int = 16, num_kv_heads: int | None = None,
           seqs=None) -> np.ndarray:
    """Paged decode attention, fp64, unrounded.

    q [S, Hq, D], caches in the storage format above (raw 16-bit),
    block_tables [S, >= ceil(L/B)], context_lens [S].  Returns [S, Hq, D]
    float64 (rows of sequences not listed in ``seqs`` are left at zero when
    ``seqs`` restricts the work to a sample).
    """
    qf = widen(q, dtype)
    S, Hq, D = qf.shape
    Hkv = k_cache.shape[1] if num_kv_heads is None else num_kv_heads
    G = Hq // Hkv
    sc = scale64(scale)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        L = int(context_lens[s])
        for g in range(Hkv):
            K, V = gather_kv(k_cache, v_cache, block_tables[s], L, g,
                             block_size, dtype)
            for h in range(g * G, (g + 1) * G):
                out[s, h] = attend(qf[s, h], K, V, sc)
    return out


def decode_logical(q, K_seqs, V_seqs, scale: float, dtype: str) -> np.ndarray:
    """Decode attention on logical (already contiguous) per-sequence K/V.

    ``K_seqs[s]`` / ``V_seqs[s]``: [L_s, Hkv, D] raw 16-bit.  This is the
    paging-free definition the paged result must equal.
    """
    qf = widen(q, dtype)
    S, Hq, D = qf.shape
    sc = scale64(scale)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        K = widen(K_seqs[s], dtype)
        V = widen(V_seqs[s], dtype)
        Hkv = K.shape[1]
        G = Hq // Hkv
        for h in range(Hq):
            out[s, h] = attend(qf[s, h], K[:, h // G, :], V[:, h // G, :], sc)
    return out


# --------------------------------------------------------------------------
# chunked prefill ([TG §Tuning Batching, Prefill, and Cache]: the scheduler
# serves decode first and fills the rest of the token budget with prefill
# chunks).  A chunk continues its own sequence: row j of a chunk of length n
# over a sequence that now holds ``seq_len`` keys sits at absolute position
# seq_len - n + j and attends keys 0 .. seq_len - n + j (causal, inclusive).
# --------------------------------------------------------------------------

def prefill(q, k_cache, v_cache, block_tables, q_start_loc, seq_lens,
            scale: float, dtype: str, block_size: int = 16,
            rows=None, heads=None) -> np.ndarray:
    """Causal chunked-prefill attention over paged K/V, fp64, unrounded.

    q [T, Hq, D] packed; chunk c owns rows q_start_loc[c] .. q_start_loc[c+1]
    and block-table row c.  ``rows`` optionally restricts the work to a list
    of packed row indices, ``heads`` to a list of query heads (the rest stay
    zero); the restriction selects work and changes no arithmetic.
    """
    qf = widen(q, dtype)
    T, Hq, D = qf.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    sc = scale64(scale)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    want = None if rows is None else set(int(r) for r in rows)
    want_h = None if heads is None else set(int(h) for h in heads)
    n_chunks = len(seq_lens)
    for c in range(n_chunks):
        r0, r1 = int(q_start_loc[c]), int(q_start_loc[c + 1])
        n = r1 - r0
        n_keys = int(seq_lens[c])
        n_cached = n_keys - n
        for g in range(Hkv):
            hs = [h for h in range(g * G, (g + 1) * G) if want_h is None or h in want_h]
            if not hs:
                continue
            K, V = gather_kv(k_cache, v_cache, block_tables[c], n_keys, g,
                             block_size, dtype)
            for j in range(n):
                r = r0 + j
                if want is not None and r not in want:
                    continue
                lim = n_cached + j + 1
                for h in hs:
                    out[r, h] = attend(qf[r, h], K[:lim], V[:lim], sc)
    return out


# --------------------------------------------------------------------------
# split of a long context into partitions, merged by log-sum-exp.  Not on the
# pages: this is the library's way to spread one long sequence over many
# workgroups.  In exact arithmetic the merge equals the unsplit softmax.
# --------------------------------------------------------------------------

def partition_state(q, K, V, scale: float):
    """(m, l, acc) of one partition: m = max z, l = sum e^{z-m},
    acc = sum e^{z-m} V_t, with z = scale * K q (float64)."""
    z = float(scale) * (K @ q)
    m = z.max()
    e = np.exp(z - m)
    return m, e.sum(), e @ V


def merge_partitions(states):
    """Merge [(m_p, l_p, acc_p)]: m = max m_p, l = sum l_p e^{m_p-m},
    o = (sum acc_p e^{m_p-m}) / l."""
    m = max(s[0] for s in states)
    l = sum(s[1] * np.exp(s[0] - m) for s in states)
    acc = sum(s[2] * np.exp(s[0] - m) for s in states)
    return acc / l


def attend_partitioned(q, K, V, scale: float, partition: int):
    """Decode row computed partition by partition and merged."""
    L = K.shape[0]
    if L == 0:
        return np.zeros(V.shape[1])
    states = [partition_state(q, K[a:a + partition], V[a:a + partition], scale)
              for a in range(0, L, partition)]
    return merge_partitions(states)
