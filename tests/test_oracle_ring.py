"""Pins for ring (sliding-window) paging in the oracle (CPU only).

Sources: [P2] "Module 04: KV cache and memory arithmetic", section 4
("Capacity-cache") and the kv_cache.py listing (KVCache.write/read,
ring_demo with its printed output), and Task 04.1, requirement 2.
"""
import numpy as np
import pytest

from oracle import pkv_oracle as O

BS = 16


def bf16_bits(x):
    b = np.asarray(x, np.float32).view(np.uint32)
    assert np.all(b & 0xFFFF == 0)
    return (b >> 16).astype(np.uint16)


def check_ring_demo_printed():
    """ring_demo: capacity 8, 12 writes of k = position, read(12) returns
    positions [4..11] and K[:, 0, 0] = [4.0 .. 11.0] (the page's printed
    output; block size 4 so the ring is two pages)."""
    bs, cap = 4, 8
    pool = np.full((4, bs, 1, 4), 0x7FC0, np.uint16)
    table = [3, 1]
    for t in range(12):
        k = bf16_bits(np.full((1, 1, 4), float(t), np.float32))
        slots = O.ring_slot_ref([table], [0, 1], [t + 1], cap, block_size=bs)
        pool, _ = O.append_ref(pool, pool, k, k, slots, block_size=bs)
    rows, pos = O.ring_read_ref(pool, table, 12, cap, block_size=bs)
    assert pos.tolist() == [4, 5, 6, 7, 8, 9, 10, 11]
    assert O.bf16_to_f64(rows[:, 0, 0]).tolist() == [4.0, 5.0, 6.0, 7.0, 8.0, 9.0, 10.0, 11.0]


def _random_setup(rng, n_seqs, W, nb, Hq=4, Hkv=2, D=8):
    pool_k = bf16_bits(rng.integers(-24, 25, (nb, BS, Hkv, D)) / 8.0)
    pool_v = bf16_bits(rng.integers(-24, 25, (nb, BS, Hkv, D)) / 8.0)
    perm = rng.permutation(nb)
    tables = [perm[i * (W // BS):(i + 1) * (W // BS)].tolist() for i in range(n_seqs)]
    return pool_k, pool_v, tables


def check_ring_equals_plain_paging_before_wrap():
    """While n <= W the ring is ordinary paging: same slots, same decode and
    prefill as the plain oracle."""
    rng = np.random.default_rng(60)
    W, nb = 64, 16
    pk, pv, tables = _random_setup(rng, 2, W, nb)
    ctx, cu = [37, 64], [0, 5, 9]
    assert O.ring_slot_ref(tables, cu, ctx, W) == O.slot_ref(tables, cu, ctx)
    q = bf16_bits(rng.integers(-8, 9, (2, 4, 8)) / 8.0)
    assert np.allclose(O.ring_decode_ref(q, pk, pv, tables, ctx, W, 0.3),
                       O.decode_ref(q, pk, pv, tables, ctx, 0.3), atol=1e-12)
    qp = bf16_bits(rng.integers(-8, 9, (9, 4, 8)) / 8.0)
    assert np.allclose(O.ring_prefill_ref(qp, cu, pk, pv, tables, ctx, W, 0.3),
                       O.prefill_ref(qp, cu, pk, pv, tables, ctx, 0.3), atol=1e-12)


def check_decode_is_a_sliding_window():
    """Write n > W tokens one at a time; decode at n equals attention over the
    last W tokens of the naive (unbounded) list, by brute force."""
    rng = np.random.default_rng(61)
    W, nb, n, Hq, Hkv, D = 32, 4, 75, 4, 2, 8
    pool_k = np.full((nb, BS, Hkv, D), 0x7FC0, np.uint16)
    pool_v = pool_k.copy()
    table = [2, 0]
    ks = bf16_bits(rng.integers(-24, 25, (n, Hkv, D)) / 8.0)
    vs = bf16_bits(rng.integers(-24, 25, (n, Hkv, D)) / 8.0)
    for t in range(n):
        slots = O.ring_slot_ref([table], [0, 1], [t + 1], W)
        pool_k, pool_v = O.append_ref(pool_k, pool_v, ks[t:t + 1], vs[t:t + 1], slots)
    q = bf16_bits(rng.integers(-8, 9, (1, Hq, D)) / 8.0)
    got = O.ring_decode_ref(q, pool_k, pool_v, [table], [n], W, 0.25)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        K = O.bf16_to_f64(ks[n - W:, g]); V = O.bf16_to_f64(vs[n - W:, g])
        s = K @ O.bf16_to_f64(q[0, h]) * 0.25
        w = np.exp(s - s.max()); w /= w.sum()
        assert np.allclose(got[0, h], w @ V, atol=1e-12)


def check_chunk_sees_ring_contents_up_to_its_position():
    """A chunk of T rows written into a ring of W < n: row t sees exactly the
    keys at absolute positions max(0, n - W) .. its own (brute force over the
    naive list)."""
    rng = np.random.default_rng(62)
    W, nb, Hq, Hkv, D = 48, 6, 2, 1, 8
    n_pre, T = 70, 20
    n = n_pre + T
    pool_k = np.full((nb, BS, Hkv, D), 0x7FC0, np.uint16)
    pool_v = pool_k.copy()
    table = [5, 1, 3]
    ks = bf16_bits(rng.integers(-24, 25, (n, Hkv, D)) / 8.0)
    vs = bf16_bits(rng.integers(-24, 25, (n, Hkv, D)) / 8.0)
    slots = O.ring_slot_ref([table], [0, n_pre], [n_pre], W)
    pool_k, pool_v = O.append_ref(pool_k, pool_v, ks[:n_pre], vs[:n_pre], slots)
    slots = O.ring_slot_ref([table], [0, T], [n], W)
    pool_k, pool_v = O.append_ref(pool_k, pool_v, ks[n_pre:], vs[n_pre:], slots)
    q = bf16_bits(rng.integers(-8, 9, (T, Hq, D)) / 8.0)
    got = O.ring_prefill_ref(q, [0, T], pool_k, pool_v, [table], [n], W, 0.25)
    for t in range(T):
        qpos = n_pre + t
        keys = range(n - W, qpos + 1)
        for h in range(Hq):
            K = O.bf16_to_f64(ks[list(keys), 0]); V = O.bf16_to_f64(vs[list(keys), 0])
            s = K @ O.bf16_to_f64(q[t, h]) * 0.25
            w = np.exp(s - s.max()); w /= w.sum()
            assert np.allclose(got[t, h], w @ V, atol=1e-12), (t, h)


PINS = [check_ring_demo_printed, check_ring_equals_plain_paging_before_wrap,
        check_decode_is_a_sliding_window, check_chunk_sees_ring_contents_up_to_its_position]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def _mutants():
    orig_read = O.ring_read_ref
    orig_slot = O.ring_slot_ref

    def read_in_buffer_order(cache, row, end, window, block_size=BS):
        # rows in ring-index order with positions taken as buffer indices (the
        # pitfall the page warns about: masking by buffer index)
        rows, pos = orig_read(cache, row, end, window, block_size)
        order = np.argsort(pos % window, kind="stable")
        return rows[order], np.arange(end - len(pos), end)

    def slot_without_wrap(tables, cu, ctx, window, block_size=BS):
        return O.slot_ref(tables, cu, ctx, block_size)

    return {
        "mask by buffer index": ("ring_read_ref", read_in_buffer_order),
        "no wrap-around": ("ring_slot_ref", slot_without_wrap),
    }


@pytest.mark.parametrize("name", sorted(_mutants()))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = _mutants()[name]
    monkeypatch.setattr(O, attr, fn)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except Exception:
            failed += 1
    assert failed, f"mutant '{name}' passes every pin"
