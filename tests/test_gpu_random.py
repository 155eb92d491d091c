"""Seeded random shapes against the fp64 oracle: decode over random head
groups, head dims, dtypes, context lengths and partition sizes (including
batches large enough for the single pass, and 2048-token partitions of short
contexts that run on half the waves), and prefill over random groups and
chunk layouts.  Each case prints its parameters before it runs."""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_422_amd as pa
from oracle import attention as A
from tests.gpu_util import DEV, assert_close, bits, dtype_name, run_decode, set_v_slots

pytestmark = pytest.mark.gpu

GROUPS = [1, 2, 3, 4, 5, 6, 8, 12, 16, 20, 24, 32]


def scattered(lens, Hkv, D, dtype, rng, gen):
    """K/V caches with each sequence's blocks scattered; unused slots and
    spare blocks hold NaN.  Returns (kc, vc, block table)."""
    nb = [-(-int(L) // 16) for L in lens]
    N = sum(nb) + 2
    perm = rng.permutation(N).astype(np.int32)
    bt = np.full((len(lens), max(max(nb), 1) + 1), int(perm[-1]), np.int32)
    at = 0
    for s, n in enumerate(nb):
        bt[s, :n] = perm[at:at + n]
        at += n
    kc = torch.randn(pa.k_cache_shape(N, Hkv, D), generator=gen, device=DEV).to(dtype)
    vc = torch.randn(pa.v_cache_shape(N, Hkv, D), generator=gen, device=DEV).to(dtype)
    for s, L in enumerate(lens):
        if L % 16:
            kc[int(bt[s, nb[s] - 1]), :, :, int(L) % 16:, :] = float("nan")
            set_v_slots(vc, int(bt[s, nb[s] - 1]), int(L) % 16, float("nan"))
    for b in perm[at:]:
        kc[int(b)] = float("nan")
        vc[int(b)] = float("nan")
    return kc, vc, bt


def decode_case(i):
    rng = np.random.default_rng(9000 + i)
    G = int(rng.choice(GROUPS))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    while G * Hkv > 64:
        Hkv //= 2
    D = int(rng.choice([64, 128]))
    dtype = [torch.float16, torch.bfloat16][int(rng.integers(2))]
    big = i % 6 == 5                                   # >= 1024 (sequence, KV head) items
    S = -(-1024 // Hkv) if big else int(rng.integers(1, 25))
    max_len = int(rng.choice([3000, 4096] if big else [64, 384, 2048, 3000, 4096]))
    lens = rng.integers(1, max_len + 1, S)
    lens[rng.random(S) < 0.1] = 0
    P = int(rng.choice([512, 1024, 2048] if big else [0, 16, 64, 256, 512, 1024, 2048, 4096]))
    return G * Hkv, Hkv, D, dtype, lens, max_len, P


@pytest.mark.parametrize("i", range(30))
def test_random_decode(i):
    Hq, Hkv, D, dtype, lens, max_len, P = decode_case(i)
    S = len(lens)
    print(f"random decode {i}: S={S} Hq={Hq} Hkv={Hkv} D={D} {dtype_name(torch.empty(0, dtype=dtype))} "
          f"max_len={max_len} P={P} plan={pa.decode_plan(S, Hq, Hkv, D, max_len, P)}", flush=True)
    rng = np.random.default_rng(1 + i)
    gen = torch.Generator(device=DEV).manual_seed(1 + i)
    kc, vc, bt = scattered(lens, Hkv, D, dtype, rng, gen)
    q = torch.randn(S, Hq, D, generator=gen, device=DEV).to(dtype)
    scale = 1 / math.sqrt(D)
    out = run_decode(q, kc, vc, bt, lens.astype(np.int32), max_len, scale, P)
    seqs = list(range(S)) if S <= 32 else [int(x) for x in rng.choice(S, 32, replace=False)]
    want = A.decode(bits(q), bits(kc), bits(vc), bt, lens.astype(np.int32), scale, dtype_name(q), seqs=seqs)
    assert_close(out[seqs], want[seqs], what=f"random decode {i}")


@pytest.mark.parametrize("i", range(12))
def test_random_prefill(i):
    rng = np.random.default_rng(7000 + i)
    G = int(rng.choice(GROUPS))
    Hkv = int(rng.choice([1, 2, 4]))
    while G * Hkv > 32:
        Hkv //= 2
    Hq = G * Hkv
    D = int(rng.choice([64, 128]))
    dtype = [torch.float16, torch.bfloat16][int(rng.integers(2))]
    chunks = [(int(rng.integers(0, 600)), int(rng.integers(1, 260))) for _ in range(int(rng.integers(1, 5)))]
    print(f"random prefill {i}: Hq={Hq} Hkv={Hkv} D={D} {dtype_name(torch.empty(0, dtype=dtype))} "
          f"chunks={chunks}", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(100 + i)
    lens = np.asarray([c + n for c, n in chunks], np.int32)
    kc, vc, bt = scattered(lens, Hkv, D, dtype, rng, gen)
    T = sum(n for _, n in chunks)
    q = torch.randn(T, Hq, D, generator=gen, device=DEV).to(dtype)
    qsl = np.concatenate([[0], np.cumsum([n for _, n in chunks])]).astype(np.int32)
    scale = 1 / math.sqrt(D)
    out = torch.full_like(q, float("nan"))
    pa.prefill_chunk(out, q, kc, vc, torch.from_numpy(bt).to(DEV), torch.from_numpy(qsl).to(DEV),
                     torch.from_numpy(lens).to(DEV), int(np.max(np.diff(qsl))), int(lens.max()), scale)
    torch.cuda.synchronize()
    want = A.prefill(bits(q), bits(kc), bits(vc), bt, qsl, lens, scale, dtype_name(q))
    assert_close(out, want, what=f"random prefill {i}")
