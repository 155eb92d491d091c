"""Swapping: pa_swap_blocks copies whole blocks between the device caches
and pinned host memory bit for bit in both directions, and a sequence
swapped out (its device blocks reused meanwhile) and back in decodes exactly
as before."""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_422_amd as pa
from oracle import kv_cache as KC
from tests.gpu_util import DEV, bits, run_decode

pytestmark = pytest.mark.gpu


def _pinned_like(n, shape_tail, dtype):
    return torch.zeros((n, *shape_tail), dtype=dtype).pin_memory()


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("H,D", [(8, 128), (3, 64)])
def test_swap_blocks_bit_exact_both_ways(dtype, H, D):
    print(f"swap dtype={dtype} H={H} D={D}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(12)
    N, NH = 20, 9
    kc = torch.randn(pa.k_cache_shape(N, H, D), generator=g, device=DEV).to(dtype)
    vc = torch.randn(pa.v_cache_shape(N, H, D), generator=g, device=DEV).to(dtype)
    hk, hv = _pinned_like(NH, pa.k_cache_shape(NH, H, D)[1:], dtype), _pinned_like(NH, pa.v_cache_shape(NH, H, D)[1:], dtype)
    want_dk, want_dv, want_hk, want_hv = bits(kc), bits(vc), bits(hk), bits(hv)
    out_pairs = np.array([[3, 0], [17, 8], [0, 4], [5, 11], [25, 1]], dtype=np.int32)   # last two skipped
    pa.swap_blocks(kc, vc, hk, hv, torch.from_numpy(out_pairs).to(DEV), pa.PA_SWAP_OUT)
    torch.cuda.synchronize()
    KC.swap_blocks(want_dk, want_dv, want_hk, want_hv, out_pairs, 0)
    assert np.array_equal(bits(hk), want_hk) and np.array_equal(bits(hv), want_hv)
    in_pairs = np.array([[0, 19], [8, 2], [4, 3], [9, 0]], dtype=np.int32)               # last skipped
    pa.swap_blocks(kc, vc, hk, hv, torch.from_numpy(in_pairs).to(DEV), pa.PA_SWAP_IN)
    torch.cuda.synchronize()
    KC.swap_blocks(want_dk, want_dv, want_hk, want_hv, in_pairs, 1)
    assert np.array_equal(bits(kc), want_dk) and np.array_equal(bits(vc), want_dv)


def test_swap_blocks_rejects_unpinned_host_memory():
    kc = torch.zeros(pa.k_cache_shape(4, 1, 64), dtype=torch.float16, device=DEV)
    vc = torch.zeros(pa.v_cache_shape(4, 1, 64), dtype=torch.float16, device=DEV)
    host = np.zeros((4, 1, 2, 16, 32), dtype=np.float16)       # ordinary pageable memory, one block per K tile
    pairs = torch.tensor([[0, 0]], dtype=torch.int32, device=DEV)
    st_ = pa._lib.pa_swap_blocks(kc.data_ptr(), vc.data_ptr(), 4, host.ctypes.data, host.ctypes.data, 4,
                                 pairs.data_ptr(), 1, pa.PA_SWAP_OUT, 1, 64, 16, pa.PA_FP16, None)
    assert st_ == pa.PA_EINVAL and "pinned" in pa.last_error()


def test_sequence_swapped_out_and_in_decodes_identically():
    print("swap round trip decode", flush=True)
    N, NH, H, Hq, D, dtype = 40, 16, 4, 16, 128, torch.bfloat16
    pool = pa.BlockPool(N, 16, 21, num_host_blocks=NH)
    g = torch.Generator(device=DEV).manual_seed(21)
    kc = torch.full(pa.k_cache_shape(N, H, D), float("nan"), dtype=dtype, device=DEV)
    vc = torch.full(pa.v_cache_shape(N, H, D), float("nan"), dtype=dtype, device=DEV)
    hk, hv = _pinned_like(NH, pa.k_cache_shape(NH, H, D)[1:], dtype), _pinned_like(NH, pa.v_cache_shape(NH, H, D)[1:], dtype)

    def grow(sid, n):
        slots, cow = pool.append(sid, n)
        assert not cow
        k = torch.randn(n, H, D, generator=g, device=DEV).to(dtype)
        v = torch.randn(n, H, D, generator=g, device=DEV).to(dtype)
        pa.write_kv(k, v, kc, vc, torch.tensor(slots, dtype=torch.int64, device=DEV))

    a = pool.create()
    grow(a, 150)
    q = torch.randn(1, Hq, D, generator=g, device=DEV).to(dtype)
    tab, L = pool.block_table(a)
    before = run_decode(q, kc, vc, np.array([tab], np.int32), np.array([L], np.int32), L, 0.09)

    pairs = pool.swap_out(a)
    pa.swap_blocks(kc, vc, hk, hv, torch.tensor(pairs, dtype=torch.int32, device=DEV), pa.PA_SWAP_OUT)
    other = pool.create()
    grow(other, 16 * (N - 2))                   # reuses every freed device block
    pool.free(other)
    pairs = pool.swap_in(a)
    pa.swap_blocks(kc, vc, hk, hv, torch.tensor(pairs, dtype=torch.int32, device=DEV), pa.PA_SWAP_IN)
    tab2, L2 = pool.block_table(a)
    assert L2 == L and tab2 != tab
    after = run_decode(q, kc, vc, np.array([tab2], np.int32), np.array([L], np.int32), L, 0.09)
    assert torch.equal(before.view(torch.int16), after.view(torch.int16))
