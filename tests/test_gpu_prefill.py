"""Chunked-prefill parity against the fp64 oracle, and the mixed step
(slot-mapped write, prefill chunks, decode) end to end."""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_422_amd as pa
from oracle import attention as A
from oracle import kv_cache as KC
from tests.gpu_util import DEV, assert_close, bits, dtype_name, run_decode, set_v_slots
from workloads import mixed

pytestmark = pytest.mark.gpu


def prefill_case(chunks, Hq, Hkv, D, dtype, seed=0):
    """chunks: list of (n_cached, n).  Scattered layout, NaN in unused slots."""
    rng = np.random.default_rng(seed)
    lens = [c + n for c, n in chunks]
    nb = [-(-L // 16) for L in lens]
    N = sum(nb) + 3
    perm = rng.permutation(N).astype(np.int32)
    stride = max(nb) + 1
    bt = np.full((len(chunks), stride), int(perm[-1]), np.int32)
    at = 0
    for c, n in enumerate(nb):
        bt[c, :n] = perm[at:at + n]
        at += n
    g = torch.Generator(device=DEV).manual_seed(seed)
    T = sum(n for _, n in chunks)
    q = torch.randn(T, Hq, D, generator=g, device=DEV).to(dtype)
    kc = torch.randn(pa.k_cache_shape(N, Hkv, D), generator=g, device=DEV).to(dtype)
    vc = torch.randn(pa.v_cache_shape(N, Hkv, D), generator=g, device=DEV).to(dtype)
    for c, L in enumerate(lens):
        if L % 16:
            kc[int(bt[c, nb[c] - 1]), :, :, L % 16:, :] = float("nan")
            set_v_slots(vc, int(bt[c, nb[c] - 1]), L % 16, float("nan"))
    for b in perm[at:]:
        kc[int(b)] = float("nan")
        vc[int(b)] = float("nan")
    qsl = np.concatenate([[0], np.cumsum([n for _, n in chunks])]).astype(np.int32)
    return q, kc, vc, bt, qsl, np.asarray(lens, np.int32)


def run_prefill(q, kc, vc, bt, qsl, lens, scale):
    out = torch.full_like(q, float("nan"))
    n_max = int(np.max(np.diff(qsl)))
    pa.prefill_chunk(out, q, kc, vc, torch.from_numpy(bt).to(DEV), torch.from_numpy(qsl).to(DEV),
                     torch.from_numpy(lens).to(DEV), n_max, int(lens.max()), scale)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (4, 4, 64), (8, 2, 64), (12, 4, 128), (3, 1, 128)])
def test_prefill_shapes(dtype, Hq, Hkv, D):
    chunks = [(0, 1), (0, 45), (17, 64), (1024 - 40, 97), (5, 200), (33, 16)]
    print(f"prefill dtype={dtype} Hq={Hq} Hkv={Hkv} D={D}", flush=True)
    q, kc, vc, bt, qsl, lens = prefill_case(chunks, Hq, Hkv, D, dtype, seed=Hq * D)
    scale = 1 / math.sqrt(D)
    out = run_prefill(q, kc, vc, bt, qsl, lens, scale)
    want = A.prefill(bits(q), bits(kc), bits(vc), bt, qsl, lens, scale, dtype_name(q))
    assert_close(out, want, what=f"prefill Hq={Hq} Hkv={Hkv} D={D}")


@pytest.mark.parametrize("Hq,Hkv,D,dtype", [(4, 2, 128, torch.bfloat16), (16, 8, 64, torch.float16),
                                            (16, 2, 128, torch.float16), (32, 2, 64, torch.bfloat16),
                                            (32, 1, 128, torch.bfloat16), (24, 1, 128, torch.float16),
                                            (12, 4, 64, torch.bfloat16)],
                         ids=["g2", "g2-D64", "g8", "g16-D64", "g32", "g24", "g3-D64"])
def test_prefill_group_sizes(Hq, Hkv, D, dtype):
    """Query-head groups of 2, 8, 16 and 32 per KV head: a workgroup then
    covers 2 heads x 4 row tiles or 4 heads x 2 row tiles, and a KV group
    spans several workgroups."""
    chunks = [(0, 3), (31, 70), (200, 129), (7, 33)]
    print(f"prefill groups Hq={Hq} Hkv={Hkv} D={D} {dtype}", flush=True)
    q, kc, vc, bt, qsl, lens = prefill_case(chunks, Hq, Hkv, D, dtype, seed=Hq * 7 + D)
    scale = 1 / math.sqrt(D)
    out = run_prefill(q, kc, vc, bt, qsl, lens, scale)
    want = A.prefill(bits(q), bits(kc), bits(vc), bt, qsl, lens, scale, dtype_name(q))
    assert_close(out, want, what=f"prefill Hq={Hq} Hkv={Hkv} D={D}")


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_prefill_long_context(dtype):
    """Cached context past 1024 blocks (16384 keys), so tiles take block ids
    from beyond the kernel's on-chip copy of the table."""
    chunks = [(20000 - 70, 70), (16384 - 16, 33), (300, 5)]
    print(f"prefill long dtype={dtype}", flush=True)
    q, kc, vc, bt, qsl, lens = prefill_case(chunks, 4, 2, 64, dtype, seed=77)
    out = run_prefill(q, kc, vc, bt, qsl, lens, 0.125)
    want = A.prefill(bits(q), bits(kc), bits(vc), bt, qsl, lens, 0.125, dtype_name(q))
    assert_close(out, want, what="prefill long context")


@pytest.mark.parametrize("scale", [-0.09, 0.0, 3.0])
def test_prefill_scale_sign_and_size(scale):
    """A negative scale (carried by Q's sign), a zero scale (uniform weights
    over the visible keys) and a large one (peaked weights, frequent moves of
    the running maximum)."""
    chunks = [(0, 33), (40, 70), (0, 1), (100, 130)]
    print(f"prefill scale={scale}", flush=True)
    q, kc, vc, bt, qsl, lens = prefill_case(chunks, 8, 2, 128, torch.bfloat16, seed=5)
    out = run_prefill(q, kc, vc, bt, qsl, lens, scale)
    want = A.prefill(bits(q), bits(kc), bits(vc), bt, qsl, lens, scale, dtype_name(q))
    assert_close(out, want, what=f"prefill scale={scale}")


def test_prefill_bf16_values_beyond_fp16_range():
    """bf16 V values the fp16 P.V cannot hold (2e5) in one sequence, and the
    largest bf16 value it can (65280) in another: both match the oracle."""
    chunks = [(40, 90), (300, 70)]
    print("prefill wide bf16 values", flush=True)
    q, kc, vc, bt, qsl, lens = prefill_case(chunks, 8, 2, 128, torch.bfloat16, seed=8)
    for c, val in ((0, 2.0e5), (1, 65280.0)):
        for pos in (3, 57, int(lens[c]) - 2):
            blk = int(bt[c, pos // 16])
            vc[blk, :, (pos % 16) // 4, 5:9, pos % 4] = val
            vc[blk, :, (pos % 16) // 4, 100, pos % 4] = -val
    out = run_prefill(q, kc, vc, bt, qsl, lens, 0.088)
    want = A.prefill(bits(q), bits(kc), bits(vc), bt, qsl, lens, 0.088, dtype_name(q))
    assert_close(out, want, what="prefill wide values")


def test_prefill_chunking_and_decode_agree():
    """Rows computed as one chunk, as two chunks, and the last row as a
    decode step all agree within tolerance of the oracle."""
    dtype, Hq, Hkv, D, L = torch.bfloat16, 32, 8, 128, 300
    q, kc, vc, bt, qsl, lens = prefill_case([(0, L)], Hq, Hkv, D, dtype, seed=21)
    scale = 1 / math.sqrt(D)
    want = A.prefill(bits(q), bits(kc), bits(vc), bt, qsl, lens, scale, "bf16")
    one = run_prefill(q, kc, vc, bt, qsl, lens, scale)
    assert_close(one, want, what="one chunk")
    cut = 111
    first = run_prefill(q[:cut].contiguous(), kc, vc, bt, np.array([0, cut], np.int32),
                        np.array([cut], np.int32), scale)
    second = run_prefill(q[cut:].contiguous(), kc, vc, bt, np.array([0, L - cut], np.int32),
                         np.array([L], np.int32), scale)
    assert_close(torch.cat([first, second]), want, what="two chunks")
    dec = run_decode(q[-1:].contiguous(), kc, vc, bt, np.array([L], np.int32), L, scale, 0)
    assert_close(dec, want[-1:], what="decode of the last row")


def _mixed_step(w, kc, vc, k_new, v_new, q_dec, q_pre):
    """write_kv -> prefill chunks -> decode, on the current stream."""
    sm = torch.from_numpy(w.slot_mapping).to(DEV)
    pa.write_kv(k_new, v_new, kc, vc, sm)
    out_pre = torch.full_like(q_pre, float("nan"))
    pa.prefill_chunk(out_pre, q_pre, kc, vc, torch.from_numpy(w.prefill_bt).to(DEV),
                     torch.from_numpy(w.q_start_loc).to(DEV),
                     torch.from_numpy(w.prefill_seq_lens).to(DEV), w.prefill_chunk,
                     w.prefill_cached + w.prefill_chunk, w.scale)
    out_dec = torch.full_like(q_dec, float("nan"))
    pa.decode(out_dec, q_dec, kc, vc, torch.from_numpy(w.decode_bt).to(DEV),
              torch.from_numpy(w.decode_lens).to(DEV), w.max_model_len, w.scale, w.partition_size)
    torch.cuda.synchronize()
    return out_pre, out_dec


def _oracle_mixed(w, kc0, vc0, k_new, v_new, q_dec, q_pre, dec_seqs, pre_rows):
    """Oracle on host copies of the pre-step caches: apply the write, then
    attention for the sampled decode sequences and prefill rows."""
    kh, vh = kc0.copy(), vc0.copy()
    KC.write_kv(kh, vh, bits(k_new), bits(v_new), w.slot_mapping, 16)
    pre = A.prefill(bits(q_pre), kh, vh, w.prefill_bt, w.q_start_loc, w.prefill_seq_lens,
                    w.scale, w.dtype, rows=pre_rows)
    dec = A.decode(bits(q_dec), kh, vh, w.decode_bt, w.decode_lens, w.scale, w.dtype,
                   seqs=dec_seqs)
    return pre, dec


def test_mixed_step_small():
    w = mixed(num_decode=96, chunk=300, cached=77, lmin=1, lmax=1200)
    print(f"mixed small: blocks={w.num_blocks}", flush=True)
    kc, vc, k_new, v_new, q_dec, q_pre = w.make_tensors(DEV)
    kc0, vc0 = bits(kc), bits(vc)
    out_pre, out_dec = _mixed_step(w, kc, vc, k_new, v_new, q_dec, q_pre)
    pre, dec = _oracle_mixed(w, kc0, vc0, k_new, v_new, q_dec, q_pre, None, None)
    assert_close(out_pre, pre, what="mixed prefill")
    assert_close(out_dec, dec, what="mixed decode")


def test_mixed_step_full_size_sampled():
    """The full 8192-token step (44 GB pool).  The oracle takes every row of
    both 2048-row chunks for the four query heads of one KV group (so every
    prefill workgroup of that group is compared), and 256 seeded decode
    sequences with all their heads, on copies of only the blocks they read."""
    w = mixed()
    print(f"mixed full: blocks={w.num_blocks}", flush=True)
    kc, vc, k_new, v_new, q_dec, q_pre = w.make_tensors(DEV)
    rng = np.random.default_rng(99)
    dec_seqs = sorted(rng.choice(w.num_decode, 256, replace=False).tolist())
    G = w.num_q_heads // w.num_kv_heads
    g = int(rng.integers(w.num_kv_heads))
    heads = list(range(g * G, (g + 1) * G))
    need = set()
    for s in dec_seqs:
        need.update(w.decode_bt[s, :-(-int(w.decode_lens[s]) // 16)].tolist())
    for c in range(w.num_chunks):
        need.update(w.prefill_bt[c, :-(-int(w.prefill_seq_lens[c]) // 16)].tolist())
    need = np.array(sorted(need), dtype=np.int64)
    remap = np.zeros(w.num_blocks, dtype=np.int64)       # unused entries read block 0
    remap[need] = np.arange(len(need))
    idx = torch.from_numpy(need).to(DEV)
    kc_s, vc_s = bits(kc[idx]), bits(vc[idx])          # pre-step copies of the needed blocks
    out_pre, out_dec = _mixed_step(w, kc, vc, k_new, v_new, q_dec, q_pre)
    print(f"  kernels done; oracle on {len(need)} blocks, KV group {g}", flush=True)
    # Re-express the workload over the compacted block set for the oracle:
    # slots outside it are skipped, table entries map to their copies.
    in_set = np.zeros(w.num_blocks, dtype=bool)
    in_set[need] = True
    blk = w.slot_mapping // 16
    sm = np.where(in_set[blk], remap[blk] * 16 + w.slot_mapping % 16, -1).astype(np.int64)
    dbt = remap[w.decode_bt].astype(np.int32)
    pbt = remap[w.prefill_bt].astype(np.int32)
    kh, vh = kc_s.copy(), vc_s.copy()
    KC.write_kv(kh, vh, bits(k_new), bits(v_new), sm, 16)
    pre = A.prefill(bits(q_pre), kh, vh, pbt, w.q_start_loc, w.prefill_seq_lens, w.scale,
                    w.dtype, heads=heads)
    dec = A.decode(bits(q_dec), kh, vh, dbt, w.decode_lens, w.scale, w.dtype, seqs=dec_seqs)
    assert_close(out_pre[:, heads], pre[:, heads], what=f"full mixed prefill (all rows, KV group {g})")
    assert_close(out_dec[dec_seqs], dec[dec_seqs], what="full mixed decode (256 sequences)")


def test_prefill_chunk_longer_than_max_q_len():
    """A chunk with more rows than max_q_len gets NaN in every row the grid
    covers and leaves the rows beyond untouched; the other chunks of the call
    are unaffected."""
    chunks = [(10, 40), (5, 100), (0, 30)]
    q, kc, vc, bt, qsl, lens = prefill_case(chunks, 8, 2, 128, torch.float16, seed=4)
    out = torch.full_like(q, 7.0)
    pa.prefill_chunk(out, q, kc, vc, torch.from_numpy(bt).to(DEV), torch.from_numpy(qsl).to(DEV),
                     torch.from_numpy(lens).to(DEV), 64, int(lens.max()), 0.088)
    torch.cuda.synchronize()
    covered = 64           # 8 waves over 4 query heads: two 32-row tiles per workgroup, one row block
    r0 = int(qsl[1])
    assert torch.isnan(out[r0:r0 + covered].float()).all()
    assert (out[r0 + covered:int(qsl[2])].float() == 7.0).all()
    want = A.prefill(bits(q), bits(kc), bits(vc), bt, qsl, lens, 0.088, "fp16")
    for c in (0, 2):
        a, b = int(qsl[c]), int(qsl[c + 1])
        assert_close(out[a:b], want[a:b], what=f"chunk {c} beside an over-long chunk")
