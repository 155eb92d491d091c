"""Thin Python binding over libpa.so (paged KV-cache attention for MI355X).

Argument marshalling only: tensors become raw device pointers, the current
torch stream becomes the hipStream_t, and every step of the hot path runs in
the library's HIP kernels.  There is no fallback: if libpa.so is missing the
import fails loudly (build it with ``python __graft_entry__.py``, which
calls ``__graft_entry__.build()``).

Function names and arguments follow include/pa.h.  Cache tensors use the
library's storage format (``k_cache_shape`` / ``v_cache_shape``):
    k_cache [num_blocks, num_kv_heads, head_dim // 32, 16, 32]
    v_cache [num_blocks, num_kv_heads, 4, head_dim, 4]
Element d of a key sits in 32-dim chunk d // 32 at position d % 32; element
d of the value in slot s sits at [s // 4, d, s % 4].
"""
from __future__ import annotations

import ctypes
import os

# One HIP runtime per process: torch brings its own libamdhip64, and libpa
# must bind to that same runtime (it shares torch's memory and streams), so
# torch is loaded before libpa.so resolves its HIP dependency.
import torch  # noqa: F401  (load order matters)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libpa.so not found at {LIB_PATH}; build it first "
                      "(python __graft_entry__.py)")
_lib = ctypes.CDLL(LIB_PATH)

from . import _abi
from ._abi import (PA_EHIP, PA_EINVAL, PA_ENOMEM, PA_ENOTSUP, PA_OK,  # noqa: F401
                   PA_POOL_PREFIX_CACHING, BlockPool, PAError)
from ._abi import c_f32, c_i32, c_i64, c_sz, c_vp, P_i32

PA_SWAP_OUT, PA_SWAP_IN = 0, 1      # pa_swap_blocks directions
PA_FP16, PA_BF16 = 0, 1
DECODE_STATIC_SCRATCH_BYTES = 16 << 20   # PA_DECODE_STATIC_SCRATCH_BYTES

_SIGS = {
    "pa_write_kv": (c_i32, [c_vp, c_vp, c_i64, c_vp, c_vp, c_i64, c_vp, c_i32, c_i32, c_i32,
                            c_i32, c_i32, c_vp]),
    "pa_copy_blocks": (c_i32, [c_vp, c_vp, c_i64, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp]),
    "pa_default_partition_size": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32]),
    "pa_decode_workspace_size": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                         ctypes.POINTER(c_sz)]),
    "pa_decode_plan": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, P_i32, P_i32, P_i32]),
    "pa_decode": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_i32, c_vp, c_i32, c_i32, c_i32,
                          c_i32, c_i32, c_i32, c_f32, c_i32, c_vp, c_sz, c_i32, c_vp]),
    "pa_decode_static": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_i32, c_vp, c_i32, c_i32, c_i32,
                                 c_i32, c_i32, c_i32, c_f32, c_i32, c_i32, c_vp]),
    "pa_prefill_chunk": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_i32, c_vp, c_vp, c_i32,
                                 c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_f32, c_i32, c_vp]),
    "pa_swap_blocks": (c_i32, [c_vp, c_vp, c_i64, c_vp, c_vp, c_i64, c_vp, c_i32, c_i32, c_i32, c_i32,
                               c_i32, c_i32, c_vp]),
}
_abi.bind(_lib, _abi.HOST_SIGS, default=True)
_abi.bind(_lib, _SIGS)

EXPORTED = tuple(_abi.HOST_SIGS) + tuple(_SIGS)


def _check(status: int):
    _abi._check(_lib, status)


def last_error() -> str:
    return _lib.pa_last_error().decode()


def version() -> str:
    return _lib.pa_version().decode()


# ---------------------------------------------------------------------------
# device entry points (torch tensors in, launches on the current stream)
# ---------------------------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return PA_FP16
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise PAError(PA_ENOTSUP, f"unsupported dtype {t.dtype} (fp16 or bf16)")


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def k_cache_shape(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int = 16):
    """Shape of a K cache tensor: 32-dim chunks of each key, slot-major within a chunk."""
    return (num_blocks, num_kv_heads, head_dim // 32, block_size, 32)


def v_cache_shape(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int = 16):
    """Shape of a V cache tensor: groups of four slots, dim-major within a group."""
    return (num_blocks, num_kv_heads, block_size // 4, head_dim, 4)


def _fail(msg):
    raise PAError(PA_EINVAL, msg)


def _on_device(fn, **tensors):
    """Every named tensor lives on the GPU (the library takes device pointers)."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            _fail(f"{fn}: {name} must be a device (cuda) tensor, got one on {t.device}")


def _int_vector(fn, name, t, dtype, n=None):
    """A contiguous integer vector (or [n, ...] array) of the given dtype."""
    if t.dtype != dtype:
        _fail(f"{fn}: {name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        _fail(f"{fn}: {name} must be contiguous")
    if n is not None and t.shape[0] != n:
        _fail(f"{fn}: {name} has {t.shape[0]} rows, expected {n}")


def _same_16bit(fn, **tensors):
    """fp16 / bf16 tensors of one dtype, contiguous."""
    dts = {t.dtype for t in tensors.values()}
    if len(dts) != 1:
        _fail(f"{fn}: " + ", ".join(f"{k} is {t.dtype}" for k, t in tensors.items()) + " (one dtype needed)")
    for name, t in tensors.items():
        _dtype_code(t)
        if not t.is_contiguous():
            _fail(f"{fn}: {name} must be contiguous")


def _cache_dims(k_cache, v_cache):
    """(num_blocks, num_kv_heads, block_size, head_dim) of a K/V cache pair."""
    if v_cache.dim() != 5 or v_cache.shape[4] != 4:
        raise PAError(PA_EINVAL, f"v_cache shape {tuple(v_cache.shape)} is not "
                                 "[num_blocks, num_kv_heads, block_size // 4, head_dim, 4]")
    N, H, G, D, _ = v_cache.shape
    B = 4 * G
    if D % 32 or tuple(k_cache.shape) != k_cache_shape(N, H, D, B):
        raise PAError(PA_EINVAL, f"k_cache shape {tuple(k_cache.shape)} does not match "
                                 f"v_cache {tuple(v_cache.shape)}: expected {k_cache_shape(N, H, D, B)}")
    return N, H, B, D


def write_kv(k, v, k_cache, v_cache, slot_mapping, stream=None):
    """k, v [T, Hkv, D] (token stride may exceed Hkv*D); slot_mapping int64 [T]."""
    import torch
    fn = "write_kv"
    T, H, D = k.shape
    if v.shape != k.shape or v.stride() != k.stride():
        _fail(f"{fn}: k and v must have one shape and one stride")
    if k.stride(2) != 1 or k.stride(1) != D:
        _fail(f"{fn}: each token's heads must be contiguous ([T, Hkv, D] with a token stride)")
    if k.dtype != v.dtype:
        _fail(f"{fn}: k is {k.dtype}, v is {v.dtype}")
    _same_16bit(fn, k_cache=k_cache, v_cache=v_cache)
    if k.dtype != k_cache.dtype:
        _fail(f"{fn}: new tokens are {k.dtype}, the cache is {k_cache.dtype}")
    _int_vector(fn, "slot_mapping", slot_mapping, torch.int64, T)
    N, Hc, B, Dc = _cache_dims(k_cache, v_cache)
    if (Hc, Dc) != (H, D):
        _fail(f"{fn}: tokens have {H} heads of {D}, the cache {Hc} of {Dc}")
    _on_device(fn, k=k, v=v, k_cache=k_cache, v_cache=v_cache, slot_mapping=slot_mapping)
    _check(_lib.pa_write_kv(_ptr(k), _ptr(v), k.stride(0), _ptr(k_cache), _ptr(v_cache),
                            N, _ptr(slot_mapping), T, H, D, B,
                            _dtype_code(k), _stream(stream)))


def copy_blocks(k_cache, v_cache, pairs, stream=None):
    """pairs int32 [n, 2] device tensor of (src, dst)."""
    import torch
    _same_16bit("copy_blocks", k_cache=k_cache, v_cache=v_cache)
    _int_vector("copy_blocks", "pairs", pairs, torch.int32)
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        _fail(f"copy_blocks: pairs must be [n, 2], got {tuple(pairs.shape)}")
    _on_device("copy_blocks", k_cache=k_cache, v_cache=v_cache, pairs=pairs)
    N, H, B, D = _cache_dims(k_cache, v_cache)
    _check(_lib.pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), N, _ptr(pairs), pairs.shape[0],
                               H, D, B, _dtype_code(k_cache), _stream(stream)))


def swap_blocks(k_cache, v_cache, host_k, host_v, pairs, direction, stream=None):
    """Whole-block copies between the device caches and pinned host tensors of
    the same layout (pin_memory=True).  pairs int32 [n, 2] device tensor:
    (device, host) for PA_SWAP_OUT, (host, device) for PA_SWAP_IN."""
    import torch
    _same_16bit("swap_blocks", k_cache=k_cache, v_cache=v_cache, host_k=host_k, host_v=host_v)
    _int_vector("swap_blocks", "pairs", pairs, torch.int32)
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        _fail(f"swap_blocks: pairs must be [n, 2], got {tuple(pairs.shape)}")
    N, H, B, D = _cache_dims(k_cache, v_cache)
    if _cache_dims(host_k, host_v)[1:] != (H, B, D):
        _fail("swap_blocks: host and device caches differ in heads, block size or head_dim")
    _on_device("swap_blocks", k_cache=k_cache, v_cache=v_cache, pairs=pairs)
    if not (host_k.is_pinned() and host_v.is_pinned()):
        raise PAError(PA_EINVAL, "swap_blocks: host tensors must be pinned")
    _check(_lib.pa_swap_blocks(_ptr(k_cache), _ptr(v_cache), N, host_k.data_ptr(), host_v.data_ptr(),
                               host_k.shape[0], _ptr(pairs), pairs.shape[0], direction, H, D, B,
                               _dtype_code(k_cache), _stream(stream)))


def default_partition_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           max_context_len: int) -> int:
    return int(_lib.pa_default_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                              max_context_len))


def decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len,
                          partition_size=0, num_kv_heads=1) -> int:
    out = c_sz(0)
    _check(_lib.pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len,
                                         partition_size, num_kv_heads, ctypes.byref(out)))
    return int(out.value)


MERGE_NONE, MERGE_ON_CHIP, MERGE_TWO_PASS = 0, 1, 2


def decode_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_size=0):
    """(partition size, merge kind, waves per partition) that decode would use."""
    part, merge, waves = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    _check(_lib.pa_decode_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                               partition_size, ctypes.byref(part), ctypes.byref(merge),
                               ctypes.byref(waves)))
    return int(part.value), int(merge.value), int(waves.value)


def _check_decode(fn, out, q, k_cache, v_cache, block_tables, context_lens):
    """Shapes, dtypes and placement of a decode call; returns (S, Hq, D)."""
    import torch
    _same_16bit(fn, out=out, q=q, k_cache=k_cache, v_cache=v_cache)
    if q.dim() != 3 or out.shape != q.shape:
        _fail(f"{fn}: q and out must both be [S, Hq, D], got {tuple(q.shape)} and {tuple(out.shape)}")
    S, Hq, D = q.shape
    _int_vector(fn, "context_lens", context_lens, torch.int32, S)
    _int_vector(fn, "block_tables", block_tables, torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] < S:
        _fail(f"{fn}: block_tables must be [>= {S}, stride], got {tuple(block_tables.shape)}")
    if _cache_dims(k_cache, v_cache)[3] != D:
        _fail(f"{fn}: q has head_dim {D}, the cache {_cache_dims(k_cache, v_cache)[3]}")
    _on_device(fn, out=out, q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
               context_lens=context_lens)
    return S, Hq, D


def decode(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
           partition_size=0, workspace=None, stream=None):
    """q/out [S, Hq, D]; block_tables int32 [S, stride]; context_lens int32 [S].
    ``workspace``: uint8 device tensor of decode_workspace_size() bytes."""
    import torch
    S, Hq, D = _check_decode("decode", out, q, k_cache, v_cache, block_tables, context_lens)
    if workspace is not None:
        _on_device("decode", workspace=workspace)
        if not workspace.is_contiguous():
            _fail("decode: workspace must be contiguous")
    N, Hkv, B, _ = _cache_dims(k_cache, v_cache)
    need = decode_workspace_size(S, Hq, D, max_context_len, partition_size, Hkv)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.pa_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), N,
                          _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), S, Hq,
                          Hkv, D, B, max_context_len, scale, partition_size, _ptr(workspace),
                          ws_bytes, _dtype_code(q), _stream(stream)))
    return out


def decode_static(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                  partition_size=0, stream=None):
    """decode() without a workspace: two-pass partition states go to the
    library's static per-device scratch (PA_DECODE_STATIC_SCRATCH_BYTES);
    nothing is allocated.  Calls that overlap on one device race."""
    S, Hq, D = _check_decode("decode_static", out, q, k_cache, v_cache, block_tables, context_lens)
    N, Hkv, B, _ = _cache_dims(k_cache, v_cache)
    _check(_lib.pa_decode_static(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), N,
                                 _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), S, Hq,
                                 Hkv, D, B, max_context_len, scale, partition_size, _dtype_code(q),
                                 _stream(stream)))
    return out


def prefill_chunk(out, q, k_cache, v_cache, block_tables, q_start_loc, seq_lens, max_q_len,
                  max_seq_len, scale, stream=None):
    """q/out [T, Hq, D] packed; q_start_loc int32 [n+1]; seq_lens int32 [n]."""
    import torch
    fn = "prefill_chunk"
    _same_16bit(fn, out=out, q=q, k_cache=k_cache, v_cache=v_cache)
    if q.dim() != 3 or out.shape != q.shape:
        _fail(f"{fn}: q and out must both be [T, Hq, D], got {tuple(q.shape)} and {tuple(out.shape)}")
    T, Hq, D = q.shape
    n = seq_lens.shape[0]
    _int_vector(fn, "seq_lens", seq_lens, torch.int32)
    _int_vector(fn, "q_start_loc", q_start_loc, torch.int32, n + 1)
    _int_vector(fn, "block_tables", block_tables, torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] < n:
        _fail(f"{fn}: block_tables must be [>= {n}, stride], got {tuple(block_tables.shape)}")
    N, Hkv, B, Dc = _cache_dims(k_cache, v_cache)
    if Dc != D:
        _fail(f"{fn}: q has head_dim {D}, the cache {Dc}")
    _on_device(fn, out=out, q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
               q_start_loc=q_start_loc, seq_lens=seq_lens)
    _check(_lib.pa_prefill_chunk(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), N,
                                 _ptr(block_tables), block_tables.shape[1], _ptr(q_start_loc),
                                 _ptr(seq_lens), seq_lens.shape[0], max_q_len, max_seq_len, Hq,
                                 Hkv, D, B, scale, _dtype_code(q), _stream(stream)))
    return out
