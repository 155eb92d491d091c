"""CPU-side checks of the C ABI: the library loads, exports everything the
header declares, validates arguments before launching anything, and its host
block pool matches the pool model bit for bit (slots, copy-on-write pairs,
block tables, refcounts, ENOMEM behaviour)."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_422_amd as pa
from tests import pool_suites


class _PoolAbi:
    """The product library's host half, as the shared pool checks see it."""
    BlockPool = pa.BlockPool
    PAError = pa.PAError
    PA_OK, PA_EINVAL, PA_ENOMEM, PA_ENOTSUP = pa.PA_OK, pa.PA_EINVAL, pa.PA_ENOMEM, pa.PA_ENOTSUP
    lib = pa._lib
    last_error = staticmethod(pa.last_error)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "pa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert "pa_decode" in names and "pa_write_kv" in names and "pa_prefill_chunk" in names
    for n in names:
        assert hasattr(pa._lib, n), n
    assert set(names) == set(pa.EXPORTED)


def test_version():
    assert "gfx950" in pa.version()


def test_decode_plan_reports_the_merge_path():
    """The single pass is chosen exactly when the batch alone fills the GPU
    (>= 1024 sequence-KV-head items), a head group has at most 8 query heads,
    contexts fit 4096 tokens and the partitions fit the kernel's LDS; a call
    with one partition per sequence needs no merge at all."""
    # (num_seqs, Hq, Hkv, D, max_ctx, P) -> (partition, merge, waves)
    cases = [
        ((256, 32, 8, 128, 4096, 512), (512, pa.MERGE_ON_CHIP, 4)),     # 8B GQA workload
        ((1, 32, 8, 128, 4096, 512), (512, pa.MERGE_TWO_PASS, 4)),      # same sizes, one sequence
        ((127, 32, 8, 128, 4096, 512), (512, pa.MERGE_TWO_PASS, 4)),    # 1016 items: below the threshold
        ((128, 32, 8, 128, 4096, 2048), (2048, pa.MERGE_ON_CHIP, 8)),   # long partitions: 8 waves
        ((64, 32, 32, 128, 2048, 2048), (2048, pa.MERGE_NONE, 8)),      # 7B workload: no split
        ((128, 64, 8, 64, 4096, 1024), (1024, pa.MERGE_ON_CHIP, 4)),    # 8-head groups, head_dim 64
        ((128, 128, 8, 128, 4096, 512), (512, pa.MERGE_TWO_PASS, 4)),   # 16-head groups: two passes
        ((1024, 8, 8, 128, 8192, 4096), (4096, pa.MERGE_TWO_PASS, 8)),  # contexts beyond 4096 tokens
        ((256, 32, 8, 128, 4096, 16), (16, pa.MERGE_TWO_PASS, 4)),      # 256 partitions: beyond LDS
        ((256, 32, 8, 128, 4096, 256), (256, pa.MERGE_TWO_PASS, 4)),    # 16 partitions: beyond the 78 KB form
        ((128, 64, 8, 128, 4096, 512), (512, pa.MERGE_ON_CHIP, 4)),     # 8-head groups keep 150 KB: 8 fit
    ]
    for args, want in cases:
        assert pa.decode_plan(*args) == want, args
    P = pa.default_partition_size(4, 32, 8, 128, 4096)
    assert pa.decode_plan(4, 32, 8, 128, 4096) == (P, pa.MERGE_TWO_PASS, 4 if P < 2048 else 8)
    for bad, code in (((4, 33, 8, 128, 4096, 0), pa.PA_EINVAL), ((4, 32, 8, 96, 4096, 0), pa.PA_ENOTSUP),
                      ((4, 32, 8, 128, 4096, 40), pa.PA_ENOTSUP), ((-1, 32, 8, 128, 4096, 0), pa.PA_EINVAL)):
        with pytest.raises(pa.PAError) as e:
            pa.decode_plan(*bad)
        assert e.value.status == code


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), pa.PA_ENOTSUP),
    (dict(block_size=32), pa.PA_ENOTSUP),
    (dict(dtype=7), pa.PA_ENOTSUP),
    (dict(num_q_heads=33), pa.PA_EINVAL),
    (dict(partition_size=40), pa.PA_ENOTSUP),
    (dict(partition_size=8192), pa.PA_ENOTSUP),
    (dict(num_seqs=-1), pa.PA_EINVAL),
    (dict(bt_stride=0), pa.PA_EINVAL),
    (dict(), pa.PA_EINVAL),                         # null pointers
])
def test_decode_rejects_before_launch(kw, code):
    a = dict(num_seqs=4, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
             bt_stride=16, partition_size=0, dtype=pa.PA_BF16)
    a.update(kw)
    st_ = pa._lib.pa_decode(None, None, None, None, 100, None, a["bt_stride"], None, a["num_seqs"],
                            a["num_q_heads"], a["num_kv_heads"], a["head_dim"], a["block_size"],
                            256, 0.1, a["partition_size"], None, 0, a["dtype"], None)
    assert st_ == code, pa.last_error()
    assert pa.last_error()


def test_decode_rejects_small_workspace_and_misalignment():
    # Fake, never-dereferenced pointers: validation must fail before any launch.
    fake = ctypes.c_void_p(0x1000)
    st_ = pa._lib.pa_decode(fake, fake, fake, fake, 100, fake, 16, fake, 4, 8, 8, 64, 16, 1024,
                            0.1, 256, None, 0, pa.PA_FP16, None)
    assert st_ == pa.PA_EINVAL and "workspace" in pa.last_error()
    odd = ctypes.c_void_p(0x1002)
    st_ = pa._lib.pa_decode(odd, fake, fake, fake, 100, fake, 16, fake, 4, 8, 8, 64, 16, 16,
                            0.1, 0, None, 0, pa.PA_FP16, None)
    assert st_ == pa.PA_ENOTSUP


def test_decode_rejects_a_grid_beyond_the_dispatch_limit():
    # 2048-token partitions run 8-wave (512 work-item) workgroups: 3 x 65535 x 64
    # of them are 6.4e9 work-items, past the dispatch packet's 32 bits (at 256
    # work-items per workgroup they would still fit).
    # No workspace is passed, so without the check the call would still stop
    # at the workspace test, before any launch.
    fake = ctypes.c_void_p(0x1000)
    _, _, waves = pa.decode_plan(65535, 64, 64, 128, 3 * 2048, 2048)
    assert waves == 8
    st_ = pa._lib.pa_decode(fake, fake, fake, fake, 100, fake, 384, fake, 65535, 64, 64, 128, 16, 3 * 2048,
                            0.1, 2048, None, 0, pa.PA_FP16, None)
    assert st_ == pa.PA_ENOTSUP and "work items" in pa.last_error()
    # The same grid with one partition fewer fits.
    st_ = pa._lib.pa_decode(fake, fake, fake, fake, 100, fake, 384, fake, 65535, 64, 64, 128, 16, 2 * 2048,
                            0.1, 2048, None, 0, pa.PA_FP16, None)
    assert st_ == pa.PA_EINVAL and "workspace" in pa.last_error()
    # 16-head groups at 1024-token partitions: the partition kernel's 2 x 65535 x 128
    # workgroups of 256 fit, the merge pass's 65535 x 2048 waves do not.
    st_ = pa._lib.pa_decode(fake, fake, fake, fake, 100, fake, 384, fake, 65535, 2048, 128, 128, 16, 2 * 1024,
                            0.1, 1024, None, 0, pa.PA_FP16, None)
    assert st_ == pa.PA_ENOTSUP and "work items" in pa.last_error()


def test_zero_sized_calls_are_noops():
    assert pa._lib.pa_write_kv(None, None, 0, None, None, 0, None, 0, 8, 128, 16, 0, None) == pa.PA_OK
    assert pa._lib.pa_copy_blocks(None, None, 0, None, 0, 8, 128, 16, 0, None) == pa.PA_OK
    assert pa._lib.pa_decode(None, None, None, None, 0, None, 1, None, 0, 8, 8, 64, 16, 0, 1.0, 0,
                             None, 0, 0, None) == pa.PA_OK


def test_write_kv_rejects_bad_stride():
    fake = ctypes.c_void_p(0x1000)
    assert pa._lib.pa_write_kv(fake, fake, 12, fake, fake, 10, fake, 3, 1, 64, 16, 0, None) == pa.PA_EINVAL
    assert pa._lib.pa_write_kv(fake, fake, 68, fake, fake, 10, fake, 3, 1, 64, 16, 0, None) == pa.PA_ENOTSUP


def test_workspace_size_formula():
    # [S][Hq][ceil(L/P)][D + 2] fp32; zero when no sequence can need 2 partitions
    assert pa.decode_workspace_size(64, 32, 128, 2048, 512, 32) == 64 * 32 * 4 * 130 * 4
    assert pa.decode_workspace_size(64, 32, 128, 512, 512, 32) == 0
    assert pa.decode_workspace_size(3, 4, 64, 100, 16, 4) == 3 * 4 * 7 * 66 * 4
    assert pa.default_partition_size(64, 32, 8, 128, 4096) % 16 == 0


def test_default_partition_follows_available_parallelism():
    # enough (sequence, KV head) rows: one partition per sequence (capped at 4096)
    assert pa.default_partition_size(64, 32, 32, 128, 2048) == 2048
    assert pa.default_partition_size(256, 32, 8, 128, 4096) == 4096
    assert pa.default_partition_size(4096, 32, 8, 128, 8192) == 4096
    # few rows: split until about 1024 items, never below 256 tokens
    assert pa.default_partition_size(1, 32, 8, 128, 32768) == 256
    assert pa.default_partition_size(8, 32, 8, 128, 32768) == 2048
    assert pa.default_partition_size(4, 4, 4, 64, 128) == 256


# ---------------------------------------------------------------------------
# host pool vs the pool model
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), pa.PA_ENOTSUP),
    (dict(block_size=8), pa.PA_ENOTSUP),
    (dict(num_q_heads=12, num_kv_heads=8), pa.PA_EINVAL),
    (dict(bt_stride=0), pa.PA_EINVAL),
    (dict(num_chunks=-1), pa.PA_EINVAL),
    (dict(), pa.PA_EINVAL),                          # null pointers with work to do
    (dict(aligned=False), pa.PA_ENOTSUP),
    (dict(num_chunks=70000), pa.PA_ENOTSUP),
])
def test_prefill_rejects_before_launch(kw, code):
    a = dict(num_chunks=2, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, bt_stride=8,
             aligned=True, fake=True)
    a.update(kw)
    if code == pa.PA_EINVAL and not kw:
        p = [None] * 7
    else:
        f = ctypes.c_void_p(0x1000 if a["aligned"] else 0x1004)
        p = [f] * 7
    st_ = pa._lib.pa_prefill_chunk(p[0], p[1], p[2], p[3], 100, p[4], a["bt_stride"], p[5], p[6],
                                   a["num_chunks"], 64, 1024, a["num_q_heads"], a["num_kv_heads"],
                                   a["head_dim"], a["block_size"], 0.1, pa.PA_BF16, None)
    assert st_ == code, pa.last_error()


def test_prefill_rejects_a_grid_beyond_the_dispatch_limit():
    # 2^30 rows per chunk need 2^24 workgroups of 512 work-items in the grid's
    # first dimension, past the dispatch packet's 32 bits.  Null pointers: a
    # call that got past this check would still stop at the pointer test.
    st_ = pa._lib.pa_prefill_chunk(None, None, None, None, 100, None, 8, None, None, 2, 1 << 30, 1 << 30,
                                   32, 8, 128, 16, 0.1, pa.PA_BF16, None)
    assert st_ == pa.PA_ENOTSUP and "max_q_len" in pa.last_error()
    st_ = pa._lib.pa_prefill_chunk(None, None, None, None, 100, None, 8, None, None, 2, 1 << 20, 1 << 20,
                                   32, 8, 128, 16, 0.1, pa.PA_BF16, None)
    assert st_ == pa.PA_EINVAL and "null" in pa.last_error()


def test_decode_and_prefill_reject_an_empty_pool_with_work():
    """Both kernels read block 0 for a bad block id (and decode for a prefetch
    past a sequence's end), so a call with work needs at least one block."""
    f = ctypes.c_void_p(0x1000)
    st_ = pa._lib.pa_decode(f, f, f, f, 0, f, 16, f, 4, 32, 8, 128, 16, 256, 0.1, 0, f, 1 << 20,
                            pa.PA_BF16, None)
    assert st_ == pa.PA_EINVAL and "num_blocks" in pa.last_error()
    st_ = pa._lib.pa_prefill_chunk(f, f, f, f, 0, f, 8, f, f, 2, 64, 1024, 32, 8, 128, 16, 0.1,
                                   pa.PA_BF16, None)
    assert st_ == pa.PA_EINVAL and "num_blocks" in pa.last_error()
    # no sequences: nothing to read, still fine
    assert pa._lib.pa_decode(None, None, None, None, 0, None, 16, None, 0, 32, 8, 128, 16, 256, 0.1, 0,
                             None, 0, pa.PA_BF16, None) == pa.PA_OK


def test_cache_shape_helpers_and_mismatch_rejected():
    """K is [N, Hkv, D/32, B, 32] and V [N, Hkv, B/4, D, 4]; the binding reads
    N, Hkv, D, B from V and rejects a K tensor of any other shape (the old
    slot-major [N, Hkv, B, D] included), and a V tensor that is not in groups
    of four slots (the old dim-major [N, Hkv, D, B]), before calling the
    library."""
    import torch
    assert pa.k_cache_shape(10, 8, 128) == (10, 8, 4, 16, 32)
    assert pa.v_cache_shape(10, 8, 128) == (10, 8, 4, 128, 4)
    vc = torch.zeros(pa.v_cache_shape(10, 8, 128), dtype=torch.float16)
    good = torch.zeros(pa.k_cache_shape(10, 8, 128), dtype=torch.float16)
    assert pa._cache_dims(good, vc) == (10, 8, 16, 128)
    for bad in (torch.zeros(10, 8, 16, 128, dtype=torch.float16),
                torch.zeros(pa.k_cache_shape(10, 8, 64), dtype=torch.float16),
                torch.zeros(pa.k_cache_shape(11, 8, 128), dtype=torch.float16)):
        with pytest.raises(pa.PAError):
            pa.copy_blocks(bad, vc, torch.zeros((0, 2), dtype=torch.int32))
    q = torch.zeros(1, 8, 128, dtype=torch.float16)
    with pytest.raises(pa.PAError):
        pa.decode(q.clone(), q, torch.zeros(10, 8, 16, 128, dtype=torch.float16), vc,
                  torch.zeros(1, 1, dtype=torch.int32), torch.zeros(1, dtype=torch.int32), 16, 0.1)
    with pytest.raises(pa.PAError):
        pa.copy_blocks(good, torch.zeros(10, 8, 128, 16, dtype=torch.float16),
                       torch.zeros((0, 2), dtype=torch.int32))


def test_prefill_and_swap_zero_work_are_noops():
    assert pa._lib.pa_prefill_chunk(None, None, None, None, 0, None, 1, None, None, 0, 0, 0, 8, 8, 64, 16,
                                    0.1, pa.PA_FP16, None) == pa.PA_OK
    assert pa._lib.pa_swap_blocks(None, None, 0, None, None, 0, None, 0, pa.PA_SWAP_OUT, 8, 128, 16,
                                  pa.PA_BF16, None) == pa.PA_OK


@pytest.mark.parametrize("direction,aligned,code", [(2, True, pa.PA_EINVAL), (pa.PA_SWAP_IN, False, pa.PA_ENOTSUP)])
def test_swap_blocks_rejects_before_launch(direction, aligned, code):
    f = ctypes.c_void_p(0x1000 if aligned else 0x1008)
    st_ = pa._lib.pa_swap_blocks(f, f, 10, f, f, 10, f, 3, direction, 8, 128, 16, pa.PA_BF16, None)
    assert st_ == code, pa.last_error()


def test_decode_static_rejects_before_launch():
    """pa_decode_static checks everything pa_decode does, and refuses a call
    whose two-pass partition states would not fit its static scratch, before
    touching the device (so these run without one)."""
    m = re.search(r"#define PA_DECODE_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)",
                  open(os.path.join(ROOT, "include", "pa.h")).read())
    assert m and int(m.group(1)) << int(m.group(2)) == pa.DECODE_STATIC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)
    # 4096 sequences x 32 heads x 64 partitions of 16 tokens: 4096*32*64*130*4 bytes
    st_ = pa._lib.pa_decode_static(fake, fake, fake, fake, 100, fake, 64, fake, 4096, 32, 8, 128, 16,
                                   1024, 0.1, 16, pa.PA_BF16, None)
    assert st_ == pa.PA_ENOTSUP and "static scratch" in pa.last_error()
    assert pa._lib.pa_decode_static(None, None, None, None, 100, None, 16, None, 4, 32, 8, 128, 16, 256,
                                    0.1, 0, pa.PA_BF16, None) == pa.PA_EINVAL
    assert pa._lib.pa_decode_static(None, None, None, None, 0, None, 1, None, 0, 8, 8, 64, 16, 0, 1.0, 0,
                                    0, None) == pa.PA_OK
    assert pa._lib.pa_decode_static(fake, fake, fake, fake, 100, fake, 16, fake, 4, 8, 8, 96, 16, 16,
                                    0.1, 0, pa.PA_FP16, None) == pa.PA_ENOTSUP

# The pool-against-model checks, shared with the sanitizer run of the host half.
_POOL = pool_suites.suites(_PoolAbi)


def test_pool_rejects_bad_arguments():
    _POOL["pool_rejects_bad_arguments"]()


def test_pool_initial_order_matches_model():
    _POOL["pool_initial_order_matches_model"]()


def test_pool_matches_model_bit_for_bit():
    _POOL["pool_matches_model_bit_for_bit"]()


def test_prefix_cached_pool_matches_model_bit_for_bit():
    _POOL["prefix_cached_pool_matches_model_bit_for_bit"]()


def test_pool_create_ex_rejects_unknown_flags():
    _POOL["pool_create_ex_rejects_unknown_flags"]()


def test_swapping_pool_matches_model_bit_for_bit():
    _POOL["swapping_pool_matches_model_bit_for_bit"]()


def test_append_many_is_appends_in_order():
    _POOL["append_many_is_appends_in_order"]()


def test_fork_many_and_free_many_equal_single_calls():
    _POOL["fork_many_and_free_many_equal_single_calls"]()


def header_signatures():
    """name -> number of parameters, from the declarations in include/pa.h."""
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "pa.h")).read(), flags=re.S)
    sigs = {}
    for m in re.finditer(r"\b(pa_[a-z0-9_]+)\s*\(([^;{)]*)\)\s*;", src):
        params = m.group(2).strip()
        sigs[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    return sigs


def test_binding_argument_counts_match_the_header():
    """Each call's ctypes signature takes exactly the parameters pa.h
    declares, so no argument is dropped or shifted between the two."""
    sigs = header_signatures()
    assert set(sigs) == set(pa.EXPORTED)
    table = {**pa._abi.HOST_SIGS, **pa._SIGS}
    for name, n in sigs.items():
        assert len(table[name][1]) == n, (name, len(table[name][1]), n)
    # the calls whose argument lists this library adds to or changes
    assert sigs["pa_decode_workspace_size"] == 7 and sigs["pa_prefill_chunk"] == 19
    assert sigs["pa_decode"] == 20 and sigs["pa_write_kv"] == 13
