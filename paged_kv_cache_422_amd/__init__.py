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

PA_OK, PA_EINVAL, PA_ENOMEM, PA_EHIP, PA_ENOTSUP = range(5)
PA_POOL_PREFIX_CACHING = 1          # pa_pool_create_ex flag
PA_SWAP_OUT, PA_SWAP_IN = 0, 1      # pa_swap_blocks directions
PA_FP16, PA_BF16 = 0, 1
DECODE_STATIC_SCRATCH_BYTES = 16 << 20   # PA_DECODE_STATIC_SCRATCH_BYTES
_STATUS = {1: "EINVAL", 2: "ENOMEM", 3: "EHIP", 4: "ENOTSUP"}

c_i32, c_i64, c_u64, c_f32, c_sz, c_vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                          ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p)
P_i32 = ctypes.POINTER(ctypes.c_int32)
P_i64 = ctypes.POINTER(ctypes.c_int64)

_SIGS = {
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_version": (ctypes.c_char_p, []),
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
    "pa_pool_create": (c_i32, [c_i32, c_i32, c_u64, ctypes.POINTER(c_vp)]),
    "pa_pool_create_ex": (c_i32, [c_i32, c_i32, c_u64, ctypes.c_uint32, c_i32, ctypes.POINTER(c_vp)]),
    "pa_pool_num_cached": (c_i32, [c_vp]),
    "pa_pool_num_free_host": (c_i32, [c_vp]),
    "pa_seq_swap_out": (c_i32, [c_vp, c_i64, P_i32, c_i32, P_i32]),
    "pa_seq_swap_in": (c_i32, [c_vp, c_i64, P_i32, c_i32, P_i32]),
    "pa_swap_blocks": (c_i32, [c_vp, c_vp, c_i64, c_vp, c_vp, c_i64, c_vp, c_i32, c_i32, c_i32, c_i32,
                               c_i32, c_i32, c_vp]),
    "pa_pool_destroy": (None, [c_vp]),
    "pa_pool_num_free": (c_i32, [c_vp]),
    "pa_pool_num_blocks": (c_i32, [c_vp]),
    "pa_block_refcount": (c_i32, [c_vp, c_i32]),
    "pa_seq_create": (c_i32, [c_vp, P_i64]),
    "pa_seq_fork": (c_i32, [c_vp, c_i64, P_i64]),
    "pa_seq_append": (c_i32, [c_vp, c_i64, c_i32, P_i64, P_i32, c_i32, P_i32]),
    "pa_seq_append_many": (c_i32, [c_vp, P_i64, P_i32, c_i32, P_i64, P_i32, c_i32, P_i32, P_i32]),
    "pa_seq_fork_many": (c_i32, [c_vp, P_i64, c_i32, P_i64, P_i32]),
    "pa_seq_free_many": (c_i32, [c_vp, P_i64, c_i32, P_i32]),
    "pa_seq_append_tokens": (c_i32, [c_vp, c_i64, P_i32, c_i32, c_i32, P_i64, P_i32, c_i32, P_i32,
                                     P_i32]),
    "pa_seq_free": (c_i32, [c_vp, c_i64]),
    "pa_seq_block_table": (c_i32, [c_vp, c_i64, P_i32, c_i32, P_i32, P_i32]),
    "pa_seq_block_tables": (c_i32, [c_vp, P_i64, c_i32, P_i32, c_i32, c_i32, P_i32]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


class PAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


def _check(status: int):
    if status != PA_OK:
        raise PAError(status, _lib.pa_last_error().decode())


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
    raise TypeError(f"unsupported dtype {t.dtype}")


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
    T, H, D = k.shape
    assert v.shape == k.shape and v.stride() == k.stride()
    assert k.stride(2) == 1 and k.stride(1) == D
    N, _, B, _ = _cache_dims(k_cache, v_cache)
    _check(_lib.pa_write_kv(_ptr(k), _ptr(v), k.stride(0), _ptr(k_cache), _ptr(v_cache),
                            N, _ptr(slot_mapping), T, H, D, B,
                            _dtype_code(k), _stream(stream)))


def copy_blocks(k_cache, v_cache, pairs, stream=None):
    """pairs int32 [n, 2] device tensor of (src, dst)."""
    N, H, B, D = _cache_dims(k_cache, v_cache)
    _check(_lib.pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), N, _ptr(pairs), pairs.shape[0],
                               H, D, B, _dtype_code(k_cache), _stream(stream)))


def swap_blocks(k_cache, v_cache, host_k, host_v, pairs, direction, stream=None):
    """Whole-block copies between the device caches and pinned host tensors of
    the same layout (pin_memory=True).  pairs int32 [n, 2] device tensor:
    (device, host) for PA_SWAP_OUT, (host, device) for PA_SWAP_IN."""
    N, H, B, D = _cache_dims(k_cache, v_cache)
    _cache_dims(host_k, host_v)
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


def decode(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
           partition_size=0, workspace=None, stream=None):
    """q/out [S, Hq, D]; block_tables int32 [S, stride]; context_lens int32 [S].
    ``workspace``: uint8 device tensor of decode_workspace_size() bytes."""
    import torch
    S, Hq, D = q.shape
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
    S, Hq, D = q.shape
    N, Hkv, B, _ = _cache_dims(k_cache, v_cache)
    _check(_lib.pa_decode_static(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), N,
                                 _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), S, Hq,
                                 Hkv, D, B, max_context_len, scale, partition_size, _dtype_code(q),
                                 _stream(stream)))
    return out


def prefill_chunk(out, q, k_cache, v_cache, block_tables, q_start_loc, seq_lens, max_q_len,
                  max_seq_len, scale, stream=None):
    """q/out [T, Hq, D] packed; q_start_loc int32 [n+1]; seq_lens int32 [n]."""
    T, Hq, D = q.shape
    N, Hkv, B, _ = _cache_dims(k_cache, v_cache)
    _check(_lib.pa_prefill_chunk(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), N,
                                 _ptr(block_tables), block_tables.shape[1], _ptr(q_start_loc),
                                 _ptr(seq_lens), seq_lens.shape[0], max_q_len, max_seq_len, Hq,
                                 Hkv, D, B, scale, _dtype_code(q), _stream(stream)))
    return out


# ---------------------------------------------------------------------------
# host block pool
# ---------------------------------------------------------------------------

class BlockPool:
    """Refcounted block pool with copy-on-write (host side, ids only)."""

    def __init__(self, num_blocks: int, block_size: int = 16, seed: int = 0,
                 prefix_caching: bool = False, num_host_blocks: int = 0):
        h = c_vp()
        flags = PA_POOL_PREFIX_CACHING if prefix_caching else 0
        _check(_lib.pa_pool_create_ex(num_blocks, block_size, seed, flags, num_host_blocks,
                                      ctypes.byref(h)))
        self._h = h
        self.block_size = block_size

    def close(self):
        # At interpreter exit the module globals may already be gone.
        if getattr(self, "_h", None) and _lib is not None:
            _lib.pa_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    @property
    def num_free(self) -> int:
        return int(_lib.pa_pool_num_free(self._h))

    @property
    def num_blocks(self) -> int:
        return int(_lib.pa_pool_num_blocks(self._h))

    @property
    def num_cached(self) -> int:
        return int(_lib.pa_pool_num_cached(self._h))

    @property
    def num_free_host(self) -> int:
        return int(_lib.pa_pool_num_free_host(self._h))

    def _swap(self, fn, seq: int):
        nb, nt = c_i32(), c_i32()
        cap = self.num_blocks + 1
        buf = (c_i32 * (2 * cap))()
        n = c_i32(0)
        _check(fn(self._h, seq, buf, cap, ctypes.byref(n)))
        return [(buf[2 * i], buf[2 * i + 1]) for i in range(n.value)]

    def swap_out(self, seq: int):
        """[(device block, host block)] in table order."""
        return self._swap(_lib.pa_seq_swap_out, seq)

    def swap_in(self, seq: int):
        """[(host block, device block)] in table order."""
        return self._swap(_lib.pa_seq_swap_in, seq)

    def refcount(self, block: int) -> int:
        return int(_lib.pa_block_refcount(self._h, block))

    def create(self) -> int:
        sid = c_i64()
        _check(_lib.pa_seq_create(self._h, ctypes.byref(sid)))
        return sid.value

    def fork(self, parent: int) -> int:
        sid = c_i64()
        _check(_lib.pa_seq_fork(self._h, parent, ctypes.byref(sid)))
        return sid.value

    def append(self, seq: int, n_tokens: int):
        """Returns (slots: list[int], cow: list[(src, dst)])."""
        slots = (c_i64 * max(n_tokens, 1))()
        cow = (c_i32 * 2)()
        n_cow = c_i32(0)
        _check(_lib.pa_seq_append(self._h, seq, n_tokens, slots, cow, 1, ctypes.byref(n_cow)))
        return list(slots[:n_tokens]), ([(cow[0], cow[1])] if n_cow.value else [])

    def fork_many(self, parents):
        """Forks each parent in order; returns the children's ids."""
        import numpy as np
        ids = np.ascontiguousarray(parents, dtype=np.int64)
        out = np.empty(max(len(ids), 1), dtype=np.int64)
        done = c_i32(0)
        _check(_lib.pa_seq_fork_many(self._h, ids.ctypes.data_as(P_i64), len(ids), out.ctypes.data_as(P_i64),
                                     ctypes.byref(done)))
        return out[:len(ids)].tolist()

    def free_many(self, seqs):
        import numpy as np
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        done = c_i32(0)
        _check(_lib.pa_seq_free_many(self._h, ids.ctypes.data_as(P_i64), len(ids), ctypes.byref(done)))

    def append_many(self, seqs, n_tokens):
        """Appends n_tokens[i] tokens to seqs[i], in order, in one call.
        Returns (slots int64 numpy array, cow pairs list).  On failure raises
        PAError with .n_done = the sequences already applied."""
        import numpy as np
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        cnt = np.ascontiguousarray(n_tokens, dtype=np.int32)
        n = len(ids)
        slots = np.empty(max(int(cnt.clip(min=0).sum()), 1), dtype=np.int64)
        cow = np.empty((max(n, 1), 2), dtype=np.int32)
        n_cow, n_done = c_i32(0), c_i32(0)
        st_ = _lib.pa_seq_append_many(self._h, ids.ctypes.data_as(P_i64), cnt.ctypes.data_as(P_i32), n,
                                      slots.ctypes.data_as(P_i64), cow.ctypes.data_as(P_i32), max(n, 1),
                                      ctypes.byref(n_cow), ctypes.byref(n_done))
        if st_ != PA_OK:
            err = PAError(st_, last_error())
            err.n_done = n_done.value
            raise err
        return slots[:int(cnt.clip(min=0).sum())], [tuple(x) for x in cow[:n_cow.value].tolist()]

    def append_tokens(self, seq: int, tokens, max_hit_tokens: int):
        """Returns (slots, cow, n_hit); the first n_hit tokens reuse cached
        blocks and have slot -1."""
        n = len(tokens)
        ids = (c_i32 * max(n, 1))(*[int(t) for t in tokens])
        slots = (c_i64 * max(n, 1))()
        cow = (c_i32 * 2)()
        n_cow, n_hit = c_i32(0), c_i32(0)
        _check(_lib.pa_seq_append_tokens(self._h, seq, ids, n, max_hit_tokens, slots, cow, 1,
                                         ctypes.byref(n_cow), ctypes.byref(n_hit)))
        return list(slots[:n]), ([(cow[0], cow[1])] if n_cow.value else []), n_hit.value

    def free(self, seq: int):
        _check(_lib.pa_seq_free(self._h, seq))

    def block_table(self, seq: int):
        nb, nt = c_i32(), c_i32()
        _check(_lib.pa_seq_block_table(self._h, seq, None, 0, ctypes.byref(nb), ctypes.byref(nt)))
        buf = (c_i32 * max(nb.value, 1))()
        _check(_lib.pa_seq_block_table(self._h, seq, buf, nb.value, ctypes.byref(nb),
                                       ctypes.byref(nt)))
        return list(buf[:nb.value]), nt.value

    def block_tables(self, seqs, stride: int, pad: int = 0):
        """int32 numpy [len(seqs), stride] block tables and int32 context lengths."""
        import numpy as np
        n = len(seqs)
        ids = np.asarray(seqs, dtype=np.int64)
        out = np.empty((n, stride), dtype=np.int32)
        ctx = np.empty(n, dtype=np.int32)
        _check(_lib.pa_seq_block_tables(self._h, ids.ctypes.data_as(P_i64), n,
                                        out.ctypes.data_as(P_i32), stride, pad,
                                        ctx.ctypes.data_as(P_i32)))
        return out, ctx
