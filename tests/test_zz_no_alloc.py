"""pa_decode_static, the decode entry point that allocates nothing: its
two-pass partition states go to the library's static per-device scratch.
Called through the C ABI and compared with pa_decode (same kernels, so bit
for bit) and with the fp64 oracle, on two calls in a row, the second with a
smaller input than the first."""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_422_amd as pa
from oracle import attention as A
from tests.gpu_util import DEV, assert_close, bits, dtype_name
from tests.test_gpu_decode import small_case

pytestmark = pytest.mark.gpu


def _static_and_workspace(q, kc, vc, bt, ctx, max_ctx, scale, P):
    """(output of pa_decode_static, output of pa_decode with a workspace)."""
    bt_t = torch.as_tensor(bt, dtype=torch.int32).to(DEV)
    ctx_t = torch.as_tensor(ctx, dtype=torch.int32).to(DEV)
    got = torch.full_like(q, float("nan"))
    pa.decode_static(got, q, kc, vc, bt_t, ctx_t, max_ctx, scale, P)
    ref = torch.full_like(q, float("nan"))
    pa.decode(ref, q, kc, vc, bt_t, ctx_t, max_ctx, scale, P)
    torch.cuda.synchronize()
    return got, ref


def _case(S, Hq, Hkv, D, dtype, lens, P, seed):
    print(f"decode_static S={S} Hq={Hq} Hkv={Hkv} D={D} {dtype} P={P} max_len={max(lens)}", flush=True)
    q, kc, vc, bt, ctx = small_case(S, Hq, Hkv, D, dtype, lens, seed=seed)
    max_ctx = max(lens)
    scale = 1 / math.sqrt(D)
    # the two-pass merge, so the scratch is in use
    assert pa.decode_plan(S, Hq, Hkv, D, max_ctx, P)[1] == pa.MERGE_TWO_PASS
    need = pa.decode_workspace_size(S, Hq, D, max_ctx, P, Hkv)
    assert 0 < need <= pa.DECODE_STATIC_SCRATCH_BYTES
    got, ref = _static_and_workspace(q, kc, vc, bt, ctx, max_ctx, scale, P)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    want = A.decode(bits(q), bits(kc), bits(vc), bt, ctx, scale, dtype_name(q))
    assert_close(got, want, what=f"decode_static S={S}")


def test_two_calls_second_smaller():
    rng = np.random.default_rng(7)
    # First call: 24 sequences of up to 1500 tokens in 64-token partitions,
    # bf16 GQA (2.4 MB of partition states); contexts 0 and 1 included.
    lens1 = [0, 1, 16, 64, 65, 1500] + rng.integers(2, 1500, 18).tolist()
    _case(24, 8, 2, 128, torch.bfloat16, lens1, 64, seed=11)
    # Second call, smaller: 5 sequences, fp16 MHA at head_dim 64, 32-token
    # partitions.  Stale states of the first call stay in the scratch.
    lens2 = [3, 33, 100, 250, 300]
    _case(5, 4, 4, 64, torch.float16, lens2, 32, seed=12)


def test_single_pass_and_unsplit_need_no_scratch():
    """A batch whose partitions merge on chip, and one with a single partition
    per sequence, give pa_decode's bits as well."""
    rng = np.random.default_rng(8)
    lens = rng.integers(1, 2048, 128).tolist()
    q, kc, vc, bt, ctx = small_case(128, 32, 8, 128, torch.bfloat16, lens, seed=13)
    for P in (512, 0):
        merge = pa.decode_plan(128, 32, 8, 128, 2048, P)[1]
        assert merge in (pa.MERGE_ON_CHIP, pa.MERGE_NONE)
        got, ref = _static_and_workspace(q, kc, vc, bt, ctx, 2048, 1 / math.sqrt(128), P)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), P
