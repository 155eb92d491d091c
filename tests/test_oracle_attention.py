"""Pins for the fp64 attention oracle against things other than itself.

Each test names what fixes the expected value: brute force on tiny inputs,
a library routine on the special case that reduces to it (identity block
table = dense attention), closed forms, and invariants the pages state
(blocks "appear contiguous" to the attention kernel, so any physical
placement gives the same result; shared prefix blocks read exactly like
private copies).
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import kv_cache as KC

B = 16


# ---------------------------------------------------------------------------
# helpers that build inputs (no attention arithmetic)
# ---------------------------------------------------------------------------

def rand_bits(rng, shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    if dtype == "fp16":
        return x.astype(np.float16)
    return (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation: still a valid bf16


def kshape(N, Hkv, D):
    """K cache shape in the library's storage format: 32-dim chunks, slot-major within a chunk."""
    return (N, Hkv, D // 32, B, 32)


def vshape(N, Hkv, D):
    """V cache shape in the library's storage format: groups of four slots, dim-major within a group."""
    return (N, Hkv, B // 4, D, 4)


def paged_layout(rng, lens, Hkv, D, dtype, extra=3):
    """Random scattered cache holding per-sequence logical K/V."""
    nb = [-(-L // B) for L in lens]
    N = sum(nb) + extra
    perm = rng.permutation(N)
    kc = rand_bits(rng, kshape(N, Hkv, D), dtype)
    vc = rand_bits(rng, vshape(N, Hkv, D), dtype)
    bt = np.zeros((len(lens), max(max(nb), 1)), dtype=np.int32)
    at = 0
    for s, n in enumerate(nb):
        bt[s, :n] = perm[at:at + n]
        at += n
    return kc, vc, bt


def brute_attend(q, K, V, scale):
    """Pure-Python triple loop: scores, max-shifted exponentials, weighted sum."""
    L = len(K)
    D = len(q)
    if L == 0:
        return [0.0] * D
    z = []
    for t in range(L):
        acc = 0.0
        for d in range(D):
            acc += q[d] * K[t][d]
        z.append(scale * acc)
    m = max(z)
    e = [math.exp(zt - m) for zt in z]
    den = sum(e)
    out = []
    for d in range(D):
        acc = 0.0
        for t in range(L):
            acc += e[t] * V[t][d]
        out.append(acc / den)
    return out


def brute_decode(q, kc, vc, bt, lens, scale, dtype, Hkv):
    """Gather element by element through the block table, then brute force."""
    qf = A.widen(q, dtype)
    kf = A.widen(kc, dtype)
    vf = A.widen(vc, dtype)
    S, Hq, D = qf.shape
    G = Hq // Hkv
    out = np.zeros((S, Hq, D))
    for s in range(S):
        for h in range(Hq):
            g = h // G
            K = [[kf[bt[s][t // B], g, d // 32, t % B, d % 32] for d in range(D)] for t in range(lens[s])]
            V = [[vf[bt[s][t // B], g, (t % B) // 4, d, t % 4] for d in range(D)] for t in range(lens[s])]
            out[s, h] = brute_attend(list(qf[s, h]), K, V, A.scale64(scale))
    return out


# ---------------------------------------------------------------------------
# exact widening of the storage formats (IEEE binary16 / bfloat16 definitions)
# ---------------------------------------------------------------------------

def test_widen_known_patterns():
    bf = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F80, 0x0001], dtype=np.uint16)
    got = A.widen(bf, "bf16")
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 1.0 + 2.0 ** -7
    assert got[3] == 0.0 and math.copysign(1, got[4]) == -1.0 and got[5] == math.inf
    assert got[6] == 2.0 ** -133  # smallest bf16 subnormal
    hf = np.array([0x3C00, 0x3C01, 0xC000, 0x0001, 0x7BFF], dtype=np.uint16)
    got = A.widen(hf, "fp16")
    assert list(got) == [1.0, 1.0 + 2.0 ** -10, -2.0, 2.0 ** -24, 65504.0]


# ---------------------------------------------------------------------------
# P5: brute force on tiny inputs (includes the tiny workload's shape)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("case", [
    dict(lens=[1, 17, 33, 40], Hq=4, Hkv=4, D=32),
    dict(lens=[5, 16, 32], Hq=4, Hkv=2, D=64),
    dict(lens=[0, 3, 31], Hq=2, Hkv=1, D=32),
])
def test_decode_matches_brute_force(dtype, case):
    rng = np.random.default_rng(7)
    kc, vc, bt = paged_layout(rng, case["lens"], case["Hkv"], case["D"], dtype)
    q = rand_bits(rng, (len(case["lens"]), case["Hq"], case["D"]), dtype)
    scale = 1.0 / math.sqrt(case["D"])
    got = A.decode(q, kc, vc, bt, case["lens"], scale, dtype)
    want = brute_decode(q, kc, vc, bt, case["lens"], scale, dtype, case["Hkv"])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_tiny_workload_shape_brute_force():
    """The tiny workload itself (4 seqs, L = 1, 17, 33, 100, 4 heads, D = 64),
    with inputs drawn the same way the tests draw them."""
    from workloads import tiny
    w = tiny()
    q, k, v = w.make_tensors("cpu")
    qn, kn, vn = q.numpy(), k.numpy(), v.numpy()
    got = A.decode(qn, kn, vn, w.block_tables, w.context_lens, w.scale, "fp16")
    want = brute_decode(qn, kn, vn, w.block_tables, list(w.context_lens), w.scale,
                        "fp16", w.num_kv_heads)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# library special case: identity block table == dense attention, compared with
# torch's scaled_dot_product_attention in float64 on the CPU
# ---------------------------------------------------------------------------

def _dense_from_identity(kc, vc, L, g, dtype):
    nb = -(-L // B)
    D = vc.shape[3]
    # K [nb, D/32, B, 32]: key (block j, slot t), dim 32c + e sits at [j, c, t, e]
    K = A.widen(np.ascontiguousarray(np.swapaxes(kc[:nb, g], 1, 2)), dtype).reshape(-1, D)[:L]
    # V [nb, B/4, D, 4]: value (block j, slot 4u + r), dim d sits at [j, u, d, r]
    V = A.widen(np.ascontiguousarray(np.swapaxes(vc[:nb, g], 2, 3)), dtype).reshape(-1, D)[:L]
    return K, V


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_decode_identity_table_equals_sdpa(dtype):
    rng = np.random.default_rng(11)
    Hq, Hkv, D, L = 8, 2, 64, 77
    nb = -(-L // B)
    kc = rand_bits(rng, kshape(nb, Hkv, D), dtype)
    vc = rand_bits(rng, vshape(nb, Hkv, D), dtype)
    q = rand_bits(rng, (1, Hq, D), dtype)
    bt = np.arange(nb, dtype=np.int32)[None]
    scale = 1.0 / math.sqrt(D)
    got = A.decode(q, kc, vc, bt, [L], scale, dtype)
    qf = torch.from_numpy(A.widen(q, dtype))  # [1, Hq, D]
    for h in range(Hq):
        K, V = _dense_from_identity(kc, vc, L, h // (Hq // Hkv), dtype)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qf[:, h:h + 1, :], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
            scale=A.scale64(scale))
        np.testing.assert_allclose(got[0, h], ref[0, 0].numpy(), rtol=0, atol=1e-13)


def test_prefill_identity_table_equals_sdpa_with_causal_mask():
    """Chunk of n rows over n_cached already-cached keys: row j may see keys
    0..n_cached+j.  torch gets the same rule as an explicit boolean mask."""
    rng = np.random.default_rng(12)
    dtype, Hq, Hkv, D, n_cached, n = "bf16", 4, 2, 64, 21, 30
    L = n_cached + n
    nb = -(-L // B)
    kc = rand_bits(rng, kshape(nb, Hkv, D), dtype)
    vc = rand_bits(rng, vshape(nb, Hkv, D), dtype)
    q = rand_bits(rng, (n, Hq, D), dtype)
    bt = np.arange(nb, dtype=np.int32)[None]
    scale = 1.0 / math.sqrt(D)
    got = A.prefill(q, kc, vc, bt, [0, n], [L], scale, dtype)
    mask = torch.tensor([[t <= n_cached + j for t in range(L)] for j in range(n)])
    qf = torch.from_numpy(A.widen(q, dtype))
    for h in range(Hq):
        K, V = _dense_from_identity(kc, vc, L, h // 2, dtype)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qf[:, h, :][None], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
            attn_mask=mask[None], scale=A.scale64(scale))
        np.testing.assert_allclose(got[:, h], ref[0].numpy(), rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def test_two_key_closed_form_fixes_scale_and_sign():
    """Two keys, q = e0: z = scale * (a, b), p0 = 1 / (1 + exp(scale (b - a)))."""
    D = 4
    q = np.zeros(D); q[0] = 1.0
    K = np.zeros((2, D)); K[0, 0], K[1, 0] = 3.0, -1.0
    V = np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0]])
    scale = 0.5
    o = A.attend(q, K, V, scale)
    p0 = 1.0 / (1.0 + math.exp(scale * (-1.0 - 3.0)))
    np.testing.assert_allclose(o, [p0, 1 - p0, 0, 0], rtol=0, atol=1e-15)


def test_single_key_returns_that_value_exactly():
    rng = np.random.default_rng(3)
    for dtype in ("fp16", "bf16"):
        kc, vc, bt = paged_layout(rng, [1], 2, 32, dtype)
        q = rand_bits(rng, (1, 2, 32), dtype)
        o = A.decode(q, kc, vc, bt, [1], 0.3, dtype)
        v0 = A.widen(vc[bt[0, 0], :, 0, :, 0], dtype)
        assert np.array_equal(o[0], v0)


def test_zero_keys_give_mean_of_values():
    rng = np.random.default_rng(4)
    L, D = 37, 8
    K = np.zeros((L, D))
    V = rng.standard_normal((L, D))
    o = A.attend(rng.standard_normal(D), K, V, 0.125)
    np.testing.assert_allclose(o, V.mean(axis=0), rtol=0, atol=1e-14)


def test_dominant_logit_selects_its_value():
    rng = np.random.default_rng(5)
    L, D = 50, 8
    K = rng.standard_normal((L, D)) * 0.01
    q = np.ones(D)
    K[17] = 100.0
    V = rng.standard_normal((L, D))
    o = A.attend(q, K, V, 1.0)
    np.testing.assert_allclose(o, V[17], rtol=0, atol=1e-12)


def test_empty_context_is_zero_row():
    rng = np.random.default_rng(6)
    kc, vc, bt = paged_layout(rng, [0, 3], 1, 32, "fp16")
    q = rand_bits(rng, (2, 1, 32), "fp16")
    o = A.decode(q, kc, vc, bt, [0, 3], 0.5, "fp16")
    assert np.all(o[0] == 0.0) and np.all(np.isfinite(o))


def test_gqa_head_mapping_contiguous_groups():
    """KV head g holds V == g + 1 everywhere, so query head h must return
    h // (Hq / Hkv) + 1 in every coordinate."""
    rng = np.random.default_rng(8)
    Hq, Hkv, D, L = 8, 2, 32, 20
    kc, vc, bt = paged_layout(rng, [L], Hkv, D, "fp16")
    for g in range(Hkv):
        vc[:, g] = np.float16(g + 1)
    q = rand_bits(rng, (1, Hq, D), "fp16")
    o = A.decode(q, kc, vc, bt, [L], 0.5, "fp16")
    for h in range(Hq):
        np.testing.assert_allclose(o[0, h], h // (Hq // Hkv) + 1, rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# invariants the pages state
# ---------------------------------------------------------------------------

def test_softmax_rows_sum_to_one_and_unit_values_give_unit_output():
    rng = np.random.default_rng(9)
    K = rng.standard_normal((300, 16)) * 3
    q = rng.standard_normal(16)
    o, p = A.attend(q, K, np.ones((300, 16)), 0.25, return_probs=True)
    assert abs(p.sum() - 1.0) < 1e-12 and np.all(p >= 0)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-12)


def test_block_permutation_invariance():
    """Attention reads a sequence's scattered blocks as one run of tokens
    (Inside vLLM, section "PagedAttention: What the OS Figured Out Decades
    Ago"), so relabelling the physical blocks changes nothing."""
    rng = np.random.default_rng(10)
    lens = [40, 1, 64, 17]
    kc, vc, bt = paged_layout(rng, lens, 2, 32, "bf16", extra=5)
    q = rand_bits(rng, (4, 4, 32), "bf16")
    base = A.decode(q, kc, vc, bt, lens, 0.35, "bf16")
    pi = rng.permutation(kc.shape[0])
    kc2 = np.empty_like(kc); vc2 = np.empty_like(vc)
    kc2[pi] = kc; vc2[pi] = vc
    bt2 = pi[bt].astype(np.int32)
    again = A.decode(q, kc2, vc2, bt2, lens, 0.35, "bf16")
    assert np.array_equal(base, again)


def test_shared_prefix_reads_like_private_copies():
    """Copy-on-write sharing (Inside vLLM, section 'Copy-on-Write Makes Beam
    Search Cheap'): sequences pointing at the same prefix blocks give exactly
    the result of sequences owning private copies."""
    rng = np.random.default_rng(13)
    Hkv, D, P = 2, 32, 37                     # prefix ends inside block 2
    lens = [P + 5, P + 20, P]
    prefix_k = rand_bits(rng, (P, Hkv, D), "fp16")
    prefix_v = rand_bits(rng, (P, Hkv, D), "fp16")
    K_seqs, V_seqs = [], []
    for L in lens:
        K_seqs.append(np.concatenate([prefix_k, rand_bits(rng, (L - P, Hkv, D), "fp16")]))
        V_seqs.append(np.concatenate([prefix_v, rand_bits(rng, (L - P, Hkv, D), "fp16")]))
    q = rand_bits(rng, (3, 4, D), "fp16")
    want = A.decode_logical(q, K_seqs, V_seqs, 0.4, "fp16")

    # shared layout: full prefix blocks shared, partial last prefix block
    # copied for every sequence that writes past the prefix.
    N = 40
    kc = np.zeros(kshape(N, Hkv, D), np.float16); vc = np.zeros(vshape(N, Hkv, D), np.float16)
    shared = [0, 1]                           # holds tokens 0..31
    nxt = 2
    bt = np.zeros((3, 8), np.int32)
    for s, L in enumerate(lens):
        row = list(shared)
        for j in range(2, -(-L // B)):
            row.append(nxt); nxt += 1
        bt[s, :len(row)] = row
    slots = {}
    for s, L in enumerate(lens):
        for t in range(L):
            slots.setdefault(s, []).append(int(bt[s, t // B]) * B + t % B)
    for s in range(3):
        KC.write_kv(kc, vc, K_seqs[s], V_seqs[s], slots[s], B)
    got = A.decode(q, kc, vc, bt, lens, 0.4, "fp16")
    assert np.array_equal(got, want)


def test_decode_is_last_row_of_prefill_and_chunking_is_invisible():
    rng = np.random.default_rng(14)
    dtype, Hq, Hkv, D, L = "bf16", 4, 2, 32, 45
    kc, vc, bt = paged_layout(rng, [L], Hkv, D, dtype)
    q = rand_bits(rng, (L, Hq, D), dtype)
    one = A.prefill(q, kc, vc, bt, [0, L], [L], 0.3, dtype)
    # decode of the last position == last row of the prefill
    dec = A.decode(q[-1:], kc, vc, bt, [L], 0.3, dtype)
    assert np.array_equal(dec[0], one[-1])
    # the same rows computed as three chunks over growing caches
    cuts = [0, 10, 29, L]
    for a, b in zip(cuts[:-1], cuts[1:]):
        part = A.prefill(q[a:b], kc, vc, bt, [0, b - a], [b], 0.3, dtype)
        assert np.array_equal(part, one[a:b])


def test_partitioned_merge_equals_unsplit():
    rng = np.random.default_rng(15)
    L, D = 1300, 32
    K = rng.standard_normal((L, D)) * 2
    V = rng.standard_normal((L, D))
    q = rng.standard_normal(D)
    want = A.attend(q, K, V, 0.2)
    for P in (16, 256, 512, 1299, 1300, 4096):
        np.testing.assert_allclose(A.attend_partitioned(q, K, V, 0.2, P), want,
                                   rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# planted mistakes: each plausible slip in the oracle must trip a pin above.
# The slip is planted in the oracle (monkeypatched, on the CPU) and the pin
# must then fail.
# ---------------------------------------------------------------------------

_good_attend = A.attend
_good_gather = A.gather_kv


def _no_scale(q, K, V, scale, return_probs=False):
    return _good_attend(q, K, V, 1.0, return_probs)


def _flipped_sign(q, K, V, scale, return_probs=False):
    return _good_attend(q, K, V, -scale, return_probs)


def _drops_last_key(q, K, V, scale, return_probs=False):
    if len(K) > 1:
        K, V = K[:-1], V[:-1]
    return _good_attend(q, K, V, scale, return_probs)


def _values_read_slot_major(k_cache, v_cache, bt_row, n_tokens, kv_head, block_size, dtype):
    K, _ = _good_gather(k_cache, v_cache, bt_row, n_tokens, kv_head, block_size, dtype)
    nb = -(-n_tokens // block_size)
    phys = np.asarray(bt_row[:nb], dtype=np.int64)
    raw = np.ascontiguousarray(v_cache[phys, kv_head])  # read [B/4, D, 4] as if [B, D]
    V = A.widen(raw, dtype).reshape(-1, v_cache.shape[3])[:n_tokens]
    return K, V


def _keys_read_slot_major(k_cache, v_cache, bt_row, n_tokens, kv_head, block_size, dtype):
    _, V = _good_gather(k_cache, v_cache, bt_row, n_tokens, kv_head, block_size, dtype)
    nb = -(-n_tokens // block_size)
    phys = np.asarray(bt_row[:nb], dtype=np.int64)
    raw = np.ascontiguousarray(k_cache[phys, kv_head])  # read [D/32, B, 32] as if [B, D]
    K = A.widen(raw, dtype).reshape(-1, v_cache.shape[3])[:n_tokens]
    return K, V


def _wrong_kv_head(k_cache, v_cache, bt_row, n_tokens, kv_head, block_size, dtype):
    H = k_cache.shape[1]
    return _good_gather(k_cache, v_cache, bt_row, n_tokens, (kv_head + 1) % H,
                        block_size, dtype)


def _wrong_slot(k_cache, v_cache, bt_row, n_tokens, kv_head, block_size, dtype):
    # reads the logical block order reversed inside the table
    nb = -(-n_tokens // block_size)
    row = np.asarray(bt_row).copy()
    row[:nb] = row[:nb][::-1]
    return _good_gather(k_cache, v_cache, row, n_tokens, kv_head, block_size, dtype)


@pytest.mark.parametrize("name,target,bad,pin", [
    ("dropped scale", "attend", _no_scale, lambda: test_decode_identity_table_equals_sdpa("bf16")),
    ("dropped scale (closed form)", "attend", _no_scale, test_two_key_closed_form_fixes_scale_and_sign),
    ("flipped sign", "attend", _flipped_sign, lambda: test_decode_identity_table_equals_sdpa("fp16")),
    ("off-by-one context", "attend", _drops_last_key, lambda: test_decode_matches_brute_force(
        "bf16", dict(lens=[5, 16, 32], Hq=4, Hkv=2, D=64))),
    ("off-by-one causal (prefill)", "attend", _drops_last_key, test_prefill_identity_table_equals_sdpa_with_causal_mask),
    ("V storage read slot-major", "gather_kv", _values_read_slot_major, test_shared_prefix_reads_like_private_copies),
    ("K chunks read as slot-major rows", "gather_kv", _keys_read_slot_major, lambda: test_decode_identity_table_equals_sdpa("fp16")),
    ("K chunks read as slot-major rows (brute force)", "gather_kv", _keys_read_slot_major, lambda: test_decode_matches_brute_force(
        "bf16", dict(lens=[5, 16, 32], Hq=4, Hkv=2, D=64))),
    ("wrong KV head", "gather_kv", _wrong_kv_head, test_gqa_head_mapping_contiguous_groups),
    ("block table order", "gather_kv", _wrong_slot, lambda: test_decode_matches_brute_force(
        "fp16", dict(lens=[1, 17, 33, 40], Hq=4, Hkv=4, D=32))),
])
def test_planted_mistake_trips_a_pin(monkeypatch, name, target, bad, pin):
    monkeypatch.setattr(A, target, bad)
    with pytest.raises(AssertionError):
        pin()
