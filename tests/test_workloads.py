"""The seeded generators are deterministic and draw the stated shapes."""
import numpy as np

from workloads import llama7b, llama8b_gqa, llama8b_long, llama13b_shared, mixed, tiny


def _valid_layout(w):
    used = []
    for s, L in enumerate(w.context_lens):
        nb = -(-int(L) // 16)
        row = w.block_tables[s]
        used += list(row[:nb])
        assert np.all(row[nb:] == w.pad_block)
    assert len(set(used)) == len(used)          # no block is used twice
    assert w.pad_block not in used
    assert max(used) < w.num_blocks and min(used) >= 0


def test_tiny():
    w = tiny()
    assert list(w.context_lens) == [1, 17, 33, 100]
    assert w.num_blocks == 64 and w.head_dim == 64 and w.dtype == "fp16"
    _valid_layout(w)
    assert w.kv_bytes == 151 * 2 * 4 * 64 * 2 == 154_624


def test_llama7b_deterministic_and_in_range():
    a, b = llama7b(), llama7b()
    assert np.array_equal(a.context_lens, b.context_lens)
    assert np.array_equal(a.block_tables, b.block_tables)
    assert a.context_lens.min() >= 128 and a.context_lens.max() <= 2048
    assert a.num_seqs == 64 and a.num_q_heads == a.num_kv_heads == 32
    demand = sum(-(-int(L) // 16) for L in a.context_lens)
    assert a.num_blocks == int(np.ceil(1.2 * demand))
    _valid_layout(a)


def test_llama8b_gqa():
    w = llama8b_gqa()
    assert (w.num_q_heads, w.num_kv_heads, w.dtype, w.partition_size) == (32, 8, "bf16", 512)
    assert w.context_lens.min() >= 512 and w.context_lens.max() <= 4096
    assert w.block_tables.shape == (256, 256)
    _valid_layout(w)


def test_llama8b_long():
    w = llama8b_long()
    assert (w.num_seqs, w.num_q_heads, w.num_kv_heads, w.dtype, w.partition_size) == (32, 32, 8, "bf16", 0)
    assert w.context_lens.min() >= 8192 and w.context_lens.max() <= 32768
    assert w.block_tables.shape == (32, 2048) and w.max_model_len == 32768
    _valid_layout(w)


def test_llama13b_shared_groups():
    w = llama13b_shared()
    assert w.num_seqs == 128 and w.context_lens.max() <= 2048 and w.context_lens.min() >= 1
    for k in range(32):
        P = int(w.prefix_lens[k])
        rows = [w.token_rows[s] for s in range(4 * k, 4 * k + 4)]
        for r in rows:
            assert np.array_equal(r[:P], rows[0][:P])
        owns = np.concatenate([r[P:] for r in rows])
        assert len(set(owns.tolist())) == len(owns)
    assert w.unique_kv_bytes < w.kv_bytes


def test_mixed_small():
    w = mixed(num_decode=64, chunk=64, cached=32, lmax=512)
    assert w.num_new_tokens == 64 + 2 * 64
    sl = w.slot_mapping
    assert len(set(sl.tolist())) == len(sl)
    for s in range(w.num_decode):
        L = int(w.decode_lens[s])
        assert sl[s] == w.decode_bt[s, (L - 1) // 16] * 16 + (L - 1) % 16
    assert list(w.q_start_loc) == [0, 64, 128]
    assert list(w.prefill_seq_lens) == [96, 96]
