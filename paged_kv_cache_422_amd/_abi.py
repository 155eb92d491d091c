"""Host half of the libpa binding: status codes, errors and the refcounted
block pool (include/pa.h, pool calls).  Needs only ctypes and numpy, not
torch, so it can drive any build of the library's host half, such as the
one compiled with the address and undefined-behaviour sanitizers.
Argument marshalling only: every pool operation runs in the library.
"""
from __future__ import annotations

import ctypes

PA_OK, PA_EINVAL, PA_ENOMEM, PA_EHIP, PA_ENOTSUP = range(5)
PA_POOL_PREFIX_CACHING = 1          # pa_pool_create_ex flag
_STATUS = {1: "EINVAL", 2: "ENOMEM", 3: "EHIP", 4: "ENOTSUP"}

c_i32, c_i64, c_u64, c_f32, c_sz, c_vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                          ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p)
P_i32 = ctypes.POINTER(ctypes.c_int32)
P_i64 = ctypes.POINTER(ctypes.c_int64)

# Signatures of the calls the host half exports.
HOST_SIGS = {
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_version": (ctypes.c_char_p, []),
    "pa_pool_create": (c_i32, [c_i32, c_i32, c_u64, ctypes.POINTER(c_vp)]),
    "pa_pool_create_ex": (c_i32, [c_i32, c_i32, c_u64, ctypes.c_uint32, c_i32, ctypes.POINTER(c_vp)]),
    "pa_pool_num_cached": (c_i32, [c_vp]),
    "pa_pool_num_free_host": (c_i32, [c_vp]),
    "pa_seq_swap_out": (c_i32, [c_vp, c_i64, P_i32, c_i32, P_i32]),
    "pa_seq_swap_in": (c_i32, [c_vp, c_i64, P_i32, c_i32, P_i32]),
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

_default_lib = None


def bind(lib, sigs, default: bool = False):
    """Set the ctypes signatures of `sigs` on `lib`; with default=True,
    BlockPool uses `lib` when constructed without one."""
    global _default_lib
    for name, (res, args) in sigs.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if default:
        _default_lib = lib
    return lib


class PAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


def _check(lib, status: int):
    if status != PA_OK:
        raise PAError(status, lib.pa_last_error().decode())


class BlockPool:
    """Refcounted block pool with copy-on-write (host side, ids only)."""

    def __init__(self, num_blocks: int, block_size: int = 16, seed: int = 0,
                 prefix_caching: bool = False, num_host_blocks: int = 0, lib=None):
        self._lib = _default_lib if lib is None else lib
        h = c_vp()
        flags = PA_POOL_PREFIX_CACHING if prefix_caching else 0
        _check(self._lib, self._lib.pa_pool_create_ex(num_blocks, block_size, seed, flags, num_host_blocks,
                                      ctypes.byref(h)))
        self._h = h
        self.block_size = block_size

    def close(self):
        # At interpreter exit the module globals may already be gone.
        if getattr(self, "_h", None) and getattr(self, "_lib", None) is not None:
            self._lib.pa_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    @property
    def num_free(self) -> int:
        return int(self._lib.pa_pool_num_free(self._h))

    @property
    def num_blocks(self) -> int:
        return int(self._lib.pa_pool_num_blocks(self._h))

    @property
    def num_cached(self) -> int:
        return int(self._lib.pa_pool_num_cached(self._h))

    @property
    def num_free_host(self) -> int:
        return int(self._lib.pa_pool_num_free_host(self._h))

    def _swap(self, fn, seq: int):
        cap = self.num_blocks + 1
        buf = (c_i32 * (2 * cap))()
        n = c_i32(0)
        _check(self._lib, fn(self._h, seq, buf, cap, ctypes.byref(n)))
        return [(buf[2 * i], buf[2 * i + 1]) for i in range(n.value)]

    def swap_out(self, seq: int):
        """[(device block, host block)] in table order."""
        return self._swap(self._lib.pa_seq_swap_out, seq)

    def swap_in(self, seq: int):
        """[(host block, device block)] in table order."""
        return self._swap(self._lib.pa_seq_swap_in, seq)

    def refcount(self, block: int) -> int:
        return int(self._lib.pa_block_refcount(self._h, block))

    def create(self) -> int:
        sid = c_i64()
        _check(self._lib, self._lib.pa_seq_create(self._h, ctypes.byref(sid)))
        return sid.value

    def fork(self, parent: int) -> int:
        sid = c_i64()
        _check(self._lib, self._lib.pa_seq_fork(self._h, parent, ctypes.byref(sid)))
        return sid.value

    def append(self, seq: int, n_tokens: int):
        """Returns (slots: list[int], cow: list[(src, dst)])."""
        slots = (c_i64 * max(n_tokens, 1))()
        cow = (c_i32 * 2)()
        n_cow = c_i32(0)
        _check(self._lib, self._lib.pa_seq_append(self._h, seq, n_tokens, slots, cow, 1, ctypes.byref(n_cow)))
        return list(slots[:n_tokens]), ([(cow[0], cow[1])] if n_cow.value else [])

    def fork_many(self, parents):
        """Forks each parent in order; returns the children's ids."""
        import numpy as np
        ids = np.ascontiguousarray(parents, dtype=np.int64)
        out = np.empty(max(len(ids), 1), dtype=np.int64)
        done = c_i32(0)
        _check(self._lib, self._lib.pa_seq_fork_many(self._h, ids.ctypes.data_as(P_i64), len(ids), out.ctypes.data_as(P_i64),
                                     ctypes.byref(done)))
        return out[:len(ids)].tolist()

    def free_many(self, seqs):
        import numpy as np
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        done = c_i32(0)
        _check(self._lib, self._lib.pa_seq_free_many(self._h, ids.ctypes.data_as(P_i64), len(ids), ctypes.byref(done)))

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
        st_ = self._lib.pa_seq_append_many(self._h, ids.ctypes.data_as(P_i64), cnt.ctypes.data_as(P_i32), n,
                                      slots.ctypes.data_as(P_i64), cow.ctypes.data_as(P_i32), max(n, 1),
                                      ctypes.byref(n_cow), ctypes.byref(n_done))
        if st_ != PA_OK:
            err = PAError(st_, self._lib.pa_last_error().decode())
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
        _check(self._lib, self._lib.pa_seq_append_tokens(self._h, seq, ids, n, max_hit_tokens, slots, cow, 1,
                                         ctypes.byref(n_cow), ctypes.byref(n_hit)))
        return list(slots[:n]), ([(cow[0], cow[1])] if n_cow.value else []), n_hit.value

    def free(self, seq: int):
        _check(self._lib, self._lib.pa_seq_free(self._h, seq))

    def block_table(self, seq: int):
        nb, nt = c_i32(), c_i32()
        _check(self._lib, self._lib.pa_seq_block_table(self._h, seq, None, 0, ctypes.byref(nb), ctypes.byref(nt)))
        buf = (c_i32 * max(nb.value, 1))()
        _check(self._lib, self._lib.pa_seq_block_table(self._h, seq, buf, nb.value, ctypes.byref(nb),
                                       ctypes.byref(nt)))
        return list(buf[:nb.value]), nt.value

    def block_tables(self, seqs, stride: int, pad: int = 0):
        """int32 numpy [len(seqs), stride] block tables and int32 context lengths."""
        import numpy as np
        n = len(seqs)
        ids = np.asarray(seqs, dtype=np.int64)
        out = np.empty((n, stride), dtype=np.int32)
        ctx = np.empty(n, dtype=np.int32)
        _check(self._lib, self._lib.pa_seq_block_tables(self._h, ids.ctypes.data_as(P_i64), n,
                                        out.ctypes.data_as(P_i32), stride, pad,
                                        ctx.ctypes.data_as(P_i32)))
        return out, ctx
