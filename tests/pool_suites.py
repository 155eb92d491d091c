"""The host pool's checks against the pool model (oracle/pool_model.py),
bit for bit, written once and run against any build of the library's host
half: the product library (tests/test_abi.py) and the build with the
address and undefined-behaviour sanitizers (tests/test_host_sanitizers.py).
Needs numpy, hypothesis and the oracle, not torch.

``abi`` provides BlockPool, PAError, the PA_* status codes, ``lib`` (the
ctypes handle, for calls the BlockPool wrapper does not make) and
last_error().
"""
import ctypes

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle.pool_model import PoolError, PoolModel


def suites(abi):
    """Name -> zero-argument check (the hypothesis ones draw their own cases)."""
    Pool = abi.BlockPool

    def pool_rejects_bad_arguments():
        with pytest.raises(abi.PAError):
            Pool(0)
        p = Pool(4, 16, 1)
        with pytest.raises(abi.PAError) as e:
            p.fork(99)
        assert e.value.status == abi.PA_EINVAL
        with pytest.raises(abi.PAError):
            p.free(99)
        assert p.refcount(-1) == -1 and p.refcount(4) == -1

    def pool_initial_order_matches_model():
        for seed in (0, 1, 4223, 2 ** 63 + 5):
            p, m = Pool(37, 16, seed), PoolModel(37, 16, seed)
            a, b = p.create(), m.seq_create()
            slots, cow = p.append(a, 37 * 16)
            want = m.seq_append(b, 37 * 16)
            assert slots == want[0] and cow == want[1] == []
            assert p.block_table(a)[0] == m.block_table(b)[0]
            assert p.num_free == 0

    @settings(max_examples=80, deadline=None, suppress_health_check=[HealthCheck.too_slow])
    @given(st.lists(st.tuples(st.integers(0, 3), st.integers(0, 40), st.integers(0, 7)),
                    min_size=1, max_size=80),
           st.integers(0, 2 ** 64 - 1))
    def pool_matches_model_bit_for_bit(ops, seed):
        N = 24
        p, m = Pool(N, 16, seed), PoolModel(N, 16, seed)
        seqs = []   # (lib id, model id)
        for op, n, pick in ops:
            if op == 0 or not seqs:
                seqs.append((p.create(), m.seq_create()))
            elif op == 1:
                a, b = seqs[pick % len(seqs)]
                seqs.append((p.fork(a), m.seq_fork(b)))
            elif op == 2:
                a, b = seqs[pick % len(seqs)]
                try:
                    want = m.seq_append(b, n)
                except PoolError as e:
                    assert e.code == "ENOMEM"
                    with pytest.raises(abi.PAError) as err:
                        p.append(a, n)
                    assert err.value.status == abi.PA_ENOMEM
                else:
                    slots, cow = p.append(a, n)
                    assert slots == want[0] and cow == want[1]
            else:
                a, b = seqs.pop(pick % len(seqs))
                p.free(a)
                m.seq_free(b)
            assert p.num_free == m.num_free()
            for a, b in seqs:
                assert p.block_table(a) == m.block_table(b)
            for blk in range(N):
                assert p.refcount(blk) == m.refcount(blk)
        ids = [a for a, _ in seqs]
        if ids:
            tabs, ctx = p.block_tables(ids, stride=64, pad=-7)
            for i, (a, b) in enumerate(seqs):
                t, n = m.block_table(b)
                assert list(tabs[i, :len(t)]) == t and np.all(tabs[i, len(t):] == -7)
                assert ctx[i] == n

    @settings(max_examples=80, deadline=None, suppress_health_check=[HealthCheck.too_slow])
    @given(st.lists(st.tuples(st.integers(0, 4), st.integers(0, 40), st.integers(0, 7), st.integers(0, 3)),
                    min_size=1, max_size=80),
           st.integers(0, 2 ** 64 - 1))
    def prefix_cached_pool_matches_model_bit_for_bit(ops, seed):
        N, B = 24, 16
        p, m = Pool(N, B, seed, prefix_caching=True), PoolModel(N, B, seed, prefix_caching=True)
        prompts = [[7] * 64, list(range(64)), [1, 2] * 32, [3] * 16 + [4] * 48]
        seqs = []
        for op, n, pick, which in ops:
            if op == 0 or not seqs:
                seqs.append((p.create(), m.seq_create()))
            elif op == 1:
                a, b = seqs[pick % len(seqs)]
                seqs.append((p.fork(a), m.seq_fork(b)))
            elif op in (2, 3):
                a, b = seqs[pick % len(seqs)]
                k = m.ntok[b]
                toks = [prompts[which][(k + i) % 64] for i in range(n)]
                try:
                    want = m.seq_append_tokens(b, toks, n - pick) if op == 2 else (*m.seq_append(b, n), 0)
                except PoolError as e:
                    assert e.code == "ENOMEM"
                    with pytest.raises(abi.PAError) as err:
                        p.append_tokens(a, toks, n - pick) if op == 2 else p.append(a, n)
                    assert err.value.status == abi.PA_ENOMEM
                else:
                    got = p.append_tokens(a, toks, n - pick) if op == 2 else (*p.append(a, n), 0)
                    assert tuple(got) == tuple(want)
            else:
                a, b = seqs.pop(pick % len(seqs))
                p.free(a)
                m.seq_free(b)
            assert p.num_free == m.num_free() and p.num_cached == m.num_cached()
            for a, b in seqs:
                assert p.block_table(a) == m.block_table(b)
            for blk in range(N):
                assert p.refcount(blk) == m.refcount(blk)

    def pool_create_ex_rejects_unknown_flags():
        h = ctypes.c_void_p()
        assert abi.lib.pa_pool_create_ex(4, 16, 0, 6, 0, ctypes.byref(h)) == abi.PA_EINVAL
        assert not h.value and "flags" in abi.last_error()
        assert abi.lib.pa_pool_create_ex(4, 16, 0, 0, -1, ctypes.byref(h)) == abi.PA_EINVAL
        assert abi.lib.pa_pool_num_cached(None) == -1
        p = Pool(4, 16, 0)
        assert p.num_cached == 0
        s = p.create()
        assert p.append_tokens(s, list(range(20)), 19)[2] == 0    # caching off: never reuses

    @settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
    @given(st.lists(st.tuples(st.integers(0, 5), st.integers(0, 40), st.integers(0, 7)),
                    min_size=1, max_size=80),
           st.integers(0, 2 ** 64 - 1), st.booleans())
    def swapping_pool_matches_model_bit_for_bit(ops, seed, caching):
        N, B, H = 24, 16, 10
        p = Pool(N, B, seed, prefix_caching=caching, num_host_blocks=H)
        m = PoolModel(N, B, seed, prefix_caching=caching, num_host_blocks=H)
        seqs = []
        for op, n, pick in ops:
            if op == 0 or not seqs:
                seqs.append((p.create(), m.seq_create()))
                continue
            a, b = seqs[pick % len(seqs)]
            if op == 1:
                calls = (lambda: p.fork(a), lambda: m.seq_fork(b))
            elif op == 2:
                toks = [(m.ntok[b] + i) % 5 for i in range(n)]
                calls = (lambda: p.append_tokens(a, toks, n), lambda: m.seq_append_tokens(b, toks, n))
            elif op == 3:
                calls = (lambda: p.swap_out(a), lambda: m.seq_swap_out(b))
            elif op == 4:
                calls = (lambda: p.swap_in(a), lambda: m.seq_swap_in(b))
            else:
                seqs.pop(pick % len(seqs))
                p.free(a)
                m.seq_free(b)
                calls = None
            if calls:
                try:
                    want = calls[1]()
                except PoolError as e:
                    with pytest.raises(abi.PAError) as err:
                        calls[0]()
                    assert err.value.status == {"ENOMEM": abi.PA_ENOMEM, "EINVAL": abi.PA_EINVAL}[e.code]
                else:
                    got = calls[0]()
                    if op == 1:
                        seqs.append((got, want))
                    else:
                        assert (tuple(got) if op == 2 else got) == (tuple(want) if op == 2 else want)
            assert (p.num_free, p.num_cached, p.num_free_host) == (m.num_free(), m.num_cached(), m.num_free_host())
            for a, b in seqs:
                assert p.block_table(a) == m.block_table(b)
            for blk in range(N):
                assert p.refcount(blk) == m.refcount(blk)

    @settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
    @given(st.lists(st.tuples(st.integers(0, 7), st.integers(0, 20)), min_size=1, max_size=30),
           st.integers(0, 2 ** 64 - 1))
    def append_many_is_appends_in_order(batch, seed):
        """One batched call equals the same appends one by one, including where
        it stops when the pool runs dry."""
        N, B = 20, 16
        p, m = Pool(N, B, seed), PoolModel(N, B, seed)
        ids = []
        for i in range(4):
            a, b = p.create(), m.seq_create()
            p.append(a, 9 * i)
            m.seq_append(b, 9 * i)
            ids.append((a, b))
        a0, b0 = ids[0]
        ids += [(p.fork(a0), m.seq_fork(b0)), (p.fork(ids[2][0]), m.seq_fork(ids[2][1]))]
        seqs = [ids[i % len(ids)] for i, _ in batch]
        counts = [n for _, n in batch]
        want_slots, want_cow, done = [], [], 0
        for (a, b), n in zip(seqs, counts):
            try:
                sl, cow = m.seq_append(b, n)
            except PoolError:
                break
            want_slots += sl
            want_cow += cow
            done += 1
        try:
            slots, cow = p.append_many([a for a, _ in seqs], counts)
            assert done == len(seqs)
        except abi.PAError as e:
            assert e.status == abi.PA_ENOMEM and e.n_done == done
        else:
            assert slots.tolist() == want_slots and cow == want_cow
        for a, b in ids:
            assert p.block_table(a) == m.block_table(b)

    def fork_many_and_free_many_equal_single_calls():
        p, m = Pool(30, 16, 3), PoolModel(30, 16, 3)
        a, b = p.create(), m.seq_create()
        p.append(a, 40)
        m.seq_append(b, 40)
        kids = p.fork_many([a, a, a])
        mk = [m.seq_fork(b) for _ in range(3)]
        for x, y in zip(kids, mk):
            assert p.block_table(x) == m.block_table(y)
        p.free_many([kids[0], kids[2]])
        m.seq_free(mk[0])
        m.seq_free(mk[2])
        assert p.num_free == m.num_free() and p.refcount(p.block_table(a)[0][0]) == 2
        with pytest.raises(abi.PAError):
            p.free_many([kids[1], 999])
        assert p.num_free == m.num_free() + 0 and p.block_table(a)[0]   # kids[1] freed before the failure
        m.seq_free(mk[1])
        assert p.num_free == m.num_free()

    return {n: f for n, f in list(locals().items()) if callable(f) and n not in ("Pool", "abi")}
