"""Pins for the CPU oracle: each check ties the oracle to something other than
itself -- brute force written independently, closed forms, invariants the
pages state, and the byte counts the pages print.  The last test plants
plausible mistakes in the oracle and shows each one fails at least one pin.

Pages: [P1] "Module 12: Final project - mini inference engine";
[P2] "Module 04: KV cache and memory arithmetic"; [P3] "Inference
Optimization" (AI Engineering from Scratch).
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import pkv_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
BS = O.BLOCK_SIZE


# ---------------------------------------------------------------------------
# test-side input builders (exactly representable values, pure layout)
# ---------------------------------------------------------------------------

def bits(x):
    """float values that are exactly bf16-representable -> uint16 patterns."""
    a = np.asarray(x, dtype=np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def rand_exact(rng, shape, lim=24):
    """Random multiples of 1/8 in [-lim/8, lim/8]: exact in bf16."""
    return rng.integers(-lim, lim + 1, size=shape).astype(np.float64) / 8.0


def build_paged(rng, naive_k, naive_v, num_blocks, Hkv, D, shuffle=True):
    """Place per-sequence token lists (NaiveKVCache) into a page pool, walking
    pages and their slots.  Unused slots hold bf16 NaN.  Returns
    (k_pool, v_pool, tables)."""
    kp = np.full((num_blocks, BS, Hkv, D), 0x7FC0, dtype=np.uint16)
    vp = kp.copy()
    order = rng.permutation(num_blocks) if shuffle else np.arange(num_blocks)
    nxt = 0
    tables = []
    for ks, vs in zip(naive_k, naive_v):
        n = len(ks)
        npg = (n + BS - 1) // BS
        row = [int(p) for p in order[nxt:nxt + npg]]
        nxt += npg
        for j, page in enumerate(row):
            for r in range(BS):
                pos = j * BS + r
                if pos < n:
                    kp[page, r] = bits(ks[pos])
                    vp[page, r] = bits(vs[pos])
        tables.append(row + [-1] * 4)
    return kp, vp, tables


def brute_attention(q_row, keys, vals, src_head, scale):
    """Pure-Python softmax attention of one query row over explicit lists."""
    scores = []
    for k in keys:
        s = 0.0
        for a, b in zip(q_row, k[src_head]):
            s += a * b
        scores.append(s * scale)
    mx = max(scores)
    e = [math.exp(s - mx) for s in scores]
    tot = sum(e)
    D = len(q_row)
    return [sum(e[p] * vals[p][src_head][d] for p in range(len(keys))) / tot for d in range(D)]


def repeated_heads(Hq, Hkv):
    """[P2] attend: each KV head repeated n_rep = Hq/Hkv times along the head
    axis (np.repeat) -> source KV head of every query head."""
    return list(np.repeat(np.arange(Hkv), Hq // Hkv))


def tiny_case(seed, B=3, Hq=4, Hkv=2, D=8, lens=None, num_blocks=12):
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = [int(x) for x in rng.integers(1, 41, size=B)]
    naive_k = [rand_exact(rng, (n, Hkv, D)) for n in lens]
    naive_v = [rand_exact(rng, (n, Hkv, D)) for n in lens]
    kp, vp, tables = build_paged(rng, naive_k, naive_v, num_blocks, Hkv, D)
    return rng, lens, naive_k, naive_v, kp, vp, tables


# ---------------------------------------------------------------------------
# pins: decode
# ---------------------------------------------------------------------------

def check_decode_brute_force(seed=0, Hq=4, Hkv=2):
    rng, lens, nk, nv, kp, vp, tables = tiny_case(seed, Hq=Hq, Hkv=Hkv)
    B, D = len(lens), 8
    q = rand_exact(rng, (B, Hq, D))
    scale = 1.0 / math.sqrt(D)
    got = O.decode_ref(bits(q), kp, vp, tables, lens, scale)
    src = repeated_heads(Hq, Hkv)
    for b in range(B):
        for h in range(Hq):
            want = brute_attention(list(q[b, h]), list(nk[b]), list(nv[b]), src[h], scale)
            assert np.allclose(got[b, h], want, rtol=0, atol=1e-12), (b, h)


@pytest.mark.parametrize("seed,Hq,Hkv", [(0, 4, 2), (1, 4, 1), (2, 2, 2), (3, 4, 4)])
def test_decode_matches_brute_force(seed, Hq, Hkv):
    """Paged oracle == pure-Python attention over per-sequence token lists:
    the NaiveKVCache-equals-PagedKVCache invariant of [P1] ("Component ->
    course module": the naive cache must satisfy the paged protocol)."""
    check_decode_brute_force(seed, Hq, Hkv)


def check_hand_example():
    """Two keys, D=4, scale 1/sqrt(4)=0.5: q=(2,0,0,0), k0=0, k1=(1,0,0,0)
    give scores 0 and 1, weights 1/(1+e) and e/(1+e); with v0=(1,0,0,0) and
    v1=(0,1,0,0) the output is (1/(1+e), e/(1+e), 0, 0)."""
    Hq = Hkv = 1
    D = 4
    k = np.zeros((2, 1, D)); k[1, 0, 0] = 1.0
    v = np.zeros((2, 1, D)); v[0, 0, 0] = 1.0; v[1, 0, 1] = 1.0
    rng = np.random.default_rng(0)
    kp, vp, tables = build_paged(rng, [k], [v], 4, Hkv, D)
    q = np.zeros((1, Hq, D)); q[0, 0, 0] = 2.0
    got = O.decode_ref(bits(q), kp, vp, tables, [2], O.default_scale(D))
    e = math.e
    want = [1 / (1 + e), e / (1 + e), 0.0, 0.0]
    assert np.allclose(got[0, 0], want, rtol=0, atol=1e-15), got


def test_hand_example_closed_form():
    check_hand_example()


def check_ctx1_returns_v0(seed=5):
    rng, lens, nk, nv, kp, vp, tables = tiny_case(seed, lens=[1, 1, 1])
    q = rand_exact(rng, (3, 4, 8))
    got = O.decode_ref(bits(q), kp, vp, tables, lens, 0.3535)
    src = repeated_heads(4, 2)
    for b in range(3):
        for h in range(4):
            assert np.array_equal(got[b, h], nv[b][0][src[h]])


def test_ctx1_returns_the_only_value_row():
    """softmax over one key is 1, so the output is that key's V row exactly."""
    check_ctx1_returns_v0()


def check_zero_query_gives_mean(seed=6):
    rng, lens, nk, nv, kp, vp, tables = tiny_case(seed)
    q = np.zeros((3, 4, 8))
    got = O.decode_ref(bits(q), kp, vp, tables, lens, 0.3535)
    src = repeated_heads(4, 2)
    for b in range(3):
        for h in range(4):
            assert np.allclose(got[b, h], nv[b][:, src[h], :].mean(axis=0), atol=1e-12)


def test_zero_query_gives_mean_of_values():
    check_zero_query_gives_mean()


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(7)
    n, Hkv, D = 37, 2, 8
    krow = rand_exact(rng, (1, Hkv, D))
    k = np.repeat(krow, n, axis=0)
    v = rand_exact(rng, (n, Hkv, D))
    kp, vp, tables = build_paged(rng, [k], [v], 6, Hkv, D)
    q = rand_exact(rng, (1, 4, D))
    got = O.decode_ref(bits(q), kp, vp, tables, [n], 0.25)
    src = repeated_heads(4, 2)
    for h in range(4):
        assert np.allclose(got[0, h], v[:, src[h], :].mean(axis=0), atol=1e-12)


def check_dominant_key(seed=8):
    """One key equal to c*q with large c takes all the weight: out -> its V."""
    rng = np.random.default_rng(seed)
    n, D = 21, 8
    q = np.zeros((1, 1, D)); q[0, 0, :] = 1.0
    k = rand_exact(rng, (n, 1, D), lim=2)
    k[13, 0, :] = 16.0                      # score 0.5*16*8 = 64 above the rest
    v = rand_exact(rng, (n, 1, D))
    kp, vp, tables = build_paged(rng, [k], [v], 4, 1, D)
    got = O.decode_ref(bits(q), kp, vp, tables, [n], 0.5)
    assert np.allclose(got[0, 0], v[13, 0], atol=1e-20 + 1e-15)


def test_dominant_key_takes_all_weight():
    check_dominant_key()


def check_rows_sum_to_one(seed=9):
    rng, lens, nk, nv, kp, vp, tables = tiny_case(seed)
    q = bits(rand_exact(rng, (3, 4, 8)))
    for b in range(3):
        for h in range(4):
            w = O.decode_weights_ref(q[b, h], kp, tables[b], lens[b], O.kv_head_of(h, 4, 2), 0.3)
            assert abs(w.sum() - 1.0) < 1e-12 and np.all(w >= 0)


def test_softmax_rows_sum_to_one():
    check_rows_sum_to_one()


def test_context_zero_gives_zeros():
    rng, lens, nk, nv, kp, vp, tables = tiny_case(10)
    q = bits(rand_exact(rng, (3, 4, 8)))
    got = O.decode_ref(q, kp, vp, tables, [lens[0], 0, lens[2]], 0.3)
    assert np.all(got[1] == 0)


def check_placement_permutation(seed=11):
    """Relabelling physical pages (and the tables with them) changes nothing
    ([P3] "Paged Attention": pages may sit anywhere in memory; the page table
    maps logical positions to physical pages)."""
    rng, lens, nk, nv, kp, vp, tables = tiny_case(seed)
    q = bits(rand_exact(rng, (3, 4, 8)))
    a = O.decode_ref(q, kp, vp, tables, lens, 0.3)
    perm = rng.permutation(kp.shape[0])
    kp2 = np.empty_like(kp); vp2 = np.empty_like(vp)
    kp2[perm] = kp; vp2[perm] = vp
    t2 = [[int(perm[p]) if p >= 0 else -1 for p in row] for row in tables]
    b = O.decode_ref(q, kp2, vp2, t2, lens, 0.3)
    assert np.array_equal(a, b)


def test_placement_permutation_invariance():
    check_placement_permutation()


def check_gqa_equals_repeated_mha(seed=12):
    """GQA with Hkv heads == MHA over the KV heads repeated Hq/Hkv times
    ([P2] attend: np.repeat of k and v along the head axis)."""
    rng, lens, nk, nv, kp, vp, tables = tiny_case(seed, Hq=4, Hkv=2)
    q = bits(rand_exact(rng, (3, 4, 8)))
    a = O.decode_ref(q, kp, vp, tables, lens, 0.3)
    kr = np.repeat(kp, 2, axis=2)
    vr = np.repeat(vp, 2, axis=2)
    b = O.decode_ref(q, kr, vr, tables, lens, 0.3)
    assert np.allclose(a, b, atol=1e-13)


def test_gqa_equals_repeated_mha():
    check_gqa_equals_repeated_mha()


def test_pages_style_gqa_einsum_agrees():
    """[P1] forward groups heads without materialising repeats
    (einsum 'thgd,lhd->hgtl' on q viewed [T, n_kv, group, D]); the oracle's
    per-head loop must agree with that grouped formulation."""
    rng, lens, nk, nv, kp, vp, tables = tiny_case(13, Hq=4, Hkv=2)
    B, Hq, Hkv, D = 3, 4, 2, 8
    q = rand_exact(rng, (B, Hq, D))
    got = O.decode_ref(bits(q), kp, vp, tables, lens, 0.3)
    for b in range(B):
        K, V = nk[b], nv[b]
        sc = np.einsum("thgd,lhd->hgtl", q[b].reshape(1, Hkv, Hq // Hkv, D), K) * 0.3
        sc = sc - sc.max(axis=-1, keepdims=True)
        p = np.exp(sc); p = p / p.sum(axis=-1, keepdims=True)
        o = np.einsum("hgtl,lhd->thgd", p, V).reshape(Hq, D)
        assert np.allclose(got[b], o, atol=1e-12)


# ---------------------------------------------------------------------------
# pins: causal prefill
# ---------------------------------------------------------------------------

def check_prefill_brute_force(seed=20):
    rng = np.random.default_rng(seed)
    Hq, Hkv, D = 4, 2, 8
    lens = [19, 33]
    news = [5, 33]          # the last T_b positions of each context are queries
    nk = [rand_exact(rng, (n, Hkv, D)) for n in lens]
    nv = [rand_exact(rng, (n, Hkv, D)) for n in lens]
    kp, vp, tables = build_paged(rng, nk, nv, 8, Hkv, D)
    cu = [0, news[0], news[0] + news[1]]
    q = rand_exact(rng, (cu[-1], Hq, D))
    got = O.prefill_ref(bits(q), cu, kp, vp, tables, lens, 0.3)
    src = repeated_heads(Hq, Hkv)
    for b in range(2):
        for t in range(news[b]):
            qpos = lens[b] - news[b] + t
            for h in range(Hq):
                want = brute_attention(list(q[cu[b] + t, h]), list(nk[b][:qpos + 1]),
                                       list(nv[b][:qpos + 1]), src[h], 0.3)
                assert np.allclose(got[cu[b] + t, h], want, atol=1e-12), (b, t, h)


def test_prefill_matches_brute_force():
    check_prefill_brute_force()


def check_causal_hand_example():
    """Two queries over two keys at positions 0, 1: row 0 sees key 0 only, so
    it returns V0 exactly; row 1 weighs both keys."""
    D = 4
    k = np.zeros((2, 1, D)); k[1, 0, 0] = 1.0
    v = np.zeros((2, 1, D)); v[0, 0, 0] = 1.0; v[1, 0, 1] = 1.0
    rng = np.random.default_rng(1)
    kp, vp, tables = build_paged(rng, [k], [v], 3, 1, D)
    q = np.zeros((2, 1, D)); q[:, 0, 0] = 2.0
    got = O.prefill_ref(bits(q), [0, 2], kp, vp, tables, [2], 0.5)
    e = math.e
    assert np.array_equal(got[0, 0], [1.0, 0, 0, 0])
    assert np.allclose(got[1, 0], [1 / (1 + e), e / (1 + e), 0, 0], atol=1e-15)


def test_causal_hand_example():
    check_causal_hand_example()


def p3_sdpa(query, keys, values):
    """[P3] "Step 2: attention with KV cache": scores / sqrt(head_dim), then for
    more than one query an additive -1e9 mask from triu(ones, k=Lk-Lq+1)
    (the query block sits at the end of the keys), softmax, @ values.
    query [H, Lq, D], keys/values [H, Lk, D]."""
    hd = query.shape[-1]
    scores = np.matmul(query, np.swapaxes(keys, -1, -2)) / np.sqrt(hd)
    lq, lk = scores.shape[-2], scores.shape[-1]
    if lq > 1:
        scores = scores + np.triu(np.ones((lq, lk)), k=lk - lq + 1) * (-1e9)
    scores = scores - scores.max(axis=-1, keepdims=True)
    w = np.exp(scores)
    return np.matmul(w / w.sum(axis=-1, keepdims=True), values)


def check_mask_equivalence(seed=21):
    """The absolute-position mask (kpos <= qpos, [P1] forward; [P2] section 4
    pitfall 2) equals [P3]'s bottom-right triu mask when the queries are the
    last Lq keys."""
    rng = np.random.default_rng(seed)
    Hq = Hkv = 2
    D, n, T = 8, 29, 11
    nk = [rand_exact(rng, (n, Hkv, D))]
    nv = [rand_exact(rng, (n, Hkv, D))]
    kp, vp, tables = build_paged(rng, nk, nv, 4, Hkv, D)
    q = rand_exact(rng, (T, Hq, D))
    got = O.prefill_ref(bits(q), [0, T], kp, vp, tables, [n], 1 / math.sqrt(D))
    ref = p3_sdpa(np.transpose(q, (1, 0, 2)), np.transpose(nk[0], (1, 0, 2)),
                  np.transpose(nv[0], (1, 0, 2)))
    assert np.allclose(got, np.transpose(ref, (1, 0, 2)), atol=1e-12)


def test_mask_equivalence_with_triu_formulation():
    check_mask_equivalence()


def test_p2_attend_with_repeat_and_large_negative_mask():
    """[P2] attend: np.repeat of KV heads, scores / sqrt(dh), masked entries set
    to -1e30, softmax: same numbers as the oracle's causal prefill."""
    rng = np.random.default_rng(22)
    Hq, Hkv, D, n, T = 4, 2, 8, 26, 9
    nk = [rand_exact(rng, (n, Hkv, D))]
    nv = [rand_exact(rng, (n, Hkv, D))]
    kp, vp, tables = build_paged(rng, nk, nv, 4, Hkv, D)
    q = rand_exact(rng, (T, Hq, D))
    got = O.prefill_ref(bits(q), [0, T], kp, vp, tables, [n], 1 / np.sqrt(D))
    k = np.repeat(nk[0], Hq // Hkv, axis=1)
    v = np.repeat(nv[0], Hq // Hkv, axis=1)
    qpos = np.arange(n - T, n)
    mask = np.arange(n)[None, :] <= qpos[:, None]
    sc = np.einsum("thd,shd->hts", q, k) / np.sqrt(D)
    sc = np.where(mask, sc, -1e30)
    sc = sc - sc.max(axis=-1, keepdims=True)
    p = np.exp(sc); p /= p.sum(axis=-1, keepdims=True)
    want = np.einsum("hts,shd->thd", p, v)
    assert np.allclose(got, want, atol=1e-12)


def check_chunking_invariance(seed=23):
    """Chunked prefill (each chunk after its own append) gives the same rows as
    one call over the whole prompt ([P1] "Why chunked prefill": the total work
    is the same; [P2] section 3.4)."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, n = 4, 2, 8, 45
    nk = [rand_exact(rng, (n, Hkv, D))]
    nv = [rand_exact(rng, (n, Hkv, D))]
    kp, vp, tables = build_paged(rng, nk, nv, 5, Hkv, D)
    q = bits(rand_exact(rng, (n, Hq, D)))
    whole = O.prefill_ref(q, [0, n], kp, vp, tables, [n], 0.3)
    for lo, hi in [(0, 16), (16, 32), (32, 45)]:
        part = O.prefill_ref(q[lo:hi], [0, hi - lo], kp, vp, tables, [hi], 0.3)
        assert np.array_equal(part, whole[lo:hi])


def test_chunking_invariance():
    check_chunking_invariance()


def test_decode_is_last_prefill_row():
    rng, lens, nk, nv, kp, vp, tables = tiny_case(24)
    q = bits(rand_exact(rng, (3, 4, 8)))
    dec = O.decode_ref(q, kp, vp, tables, lens, 0.3)
    for b in range(3):
        pre = O.prefill_ref(q[b:b + 1], [0, 1], kp, vp, [tables[b]], [lens[b]], 0.3)
        assert np.array_equal(pre[0], dec[b])


# ---------------------------------------------------------------------------
# pins: slot mapping and append
# ---------------------------------------------------------------------------

def load_golden(name):
    with open(os.path.join(HERE, "golden", name)) as f:
        return json.load(f)


def check_reserve20_example():
    ex = load_golden("slot_examples.json")["reserve20"]
    slots = O.slot_ref([ex["block_table"]], [0, ex["n_tokens"]], [ex["n_tokens"]])
    pages = [s // BS for s in slots]
    offs = [s % BS for s in slots]
    assert pages == ex["expected_pages"] and offs == ex["expected_offsets"]


def test_slot_mapping_printed_example():
    check_reserve20_example()


def check_decode_slots_follow_context():
    """A decode step appends one token at position context_len-1 (start_pos is
    the committed length, [P1] forward / SequenceCache.commit); a chunk of T
    rows takes the last T positions of its context."""
    tables = [[7, 3, 9], [2, 5, -1]]
    # seq 0: position 39 -> logical page 2 (physical 9), offset 7
    # seq 1: position 16 -> logical page 1 (physical 5), offset 0
    assert O.slot_ref(tables, [0, 1, 2], [40, 17]) == [9 * BS + 7, 5 * BS + 0]
    # 4 rows ending a 20-token context on table [4, 6]: positions 16..19
    assert O.slot_ref([[4, 6]], [0, 4], [20]) == [6 * BS + 0, 6 * BS + 1, 6 * BS + 2, 6 * BS + 3]


def test_decode_and_chunk_slots():
    check_decode_slots_follow_context()


def test_write_read_printed_example():
    """[P1] Task 12.1: write two positions through blocks [0, 1], read back
    length 2 -> [2, Hkv, D], length 17 -> [17, Hkv, D]."""
    ex = load_golden("slot_examples.json")["write_read"]
    Hkv, D = 2, 4
    pool = np.zeros((4, BS, Hkv, D), dtype=np.uint16)
    rng = np.random.default_rng(30)
    k_new = bits(rand_exact(rng, (2, Hkv, D)))
    slots = [ex["block_table"][p // BS] * BS + p % BS for p in range(ex["written"])]
    kc, _ = O.append_ref(pool, pool, k_new, k_new, slots)
    for n in ex["read_lengths"]:
        assert O.gather_ref(kc, ex["block_table"], n).shape == (n, Hkv, D)
    assert np.array_equal(O.gather_ref(kc, ex["block_table"], 2), k_new)


def test_append_is_a_bit_copy():
    """Scatter copies bit patterns (NaN payloads, -0.0), skips negative slots,
    leaves every other slot untouched; a repeated slot keeps the last write
    (the page's loop writes tokens in order)."""
    Hkv, D, nb = 2, 4, 3
    rng = np.random.default_rng(31)
    pool_k = rng.integers(0, 1 << 16, size=(nb, BS, Hkv, D), dtype=np.uint16)
    pool_v = rng.integers(0, 1 << 16, size=(nb, BS, Hkv, D), dtype=np.uint16)
    k_new = rng.integers(0, 1 << 16, size=(5, Hkv, D), dtype=np.uint16)
    v_new = rng.integers(0, 1 << 16, size=(5, Hkv, D), dtype=np.uint16)
    k_new[0, 0, 0] = 0x8000   # -0.0
    k_new[1, 0, 0] = 0x7FC1   # NaN with payload
    slots = [5, 40, -1, 17, 40]
    kc, vc = O.append_ref(pool_k, pool_v, k_new, v_new, slots)
    want_k = pool_k.copy(); want_v = pool_v.copy()
    for t, s in enumerate(slots):
        if s >= 0:
            want_k[s // BS, s % BS] = k_new[t]
            want_v[s // BS, s % BS] = v_new[t]
    assert np.array_equal(kc, want_k) and np.array_equal(vc, want_v)
    assert kc[0, 5, 0, 0] == 0x8000 and kc[2, 8, 0, 0] == k_new[4, 0, 0]
    assert np.array_equal(pool_k, pool_k)  # inputs unchanged (copies returned)
    with pytest.raises(IndexError):
        O.append_ref(pool_k, pool_v, k_new[:1], v_new[:1], [nb * BS])


def test_append_then_decode_equals_naive_with_new_token():
    """Appending the step's K/V and attending over the post-append context is
    the pages' order (read prefix, concatenate current k/v, attend, write)."""
    rng = np.random.default_rng(32)
    Hq, Hkv, D = 4, 2, 8
    lens_pre = [15, 16, 0]
    nk = [rand_exact(rng, (n + 1, Hkv, D)) for n in lens_pre]
    nv = [rand_exact(rng, (n + 1, Hkv, D)) for n in lens_pre]
    kp, vp, tables = build_paged(rng, [k[:-1] for k in nk], [v[:-1] for v in nv], 8, Hkv, D)
    # give each sequence room for one more page
    free = [p for p in range(8) if all(p not in row for row in tables)]
    for b, n in enumerate(lens_pre):
        if n % BS == 0:
            tables[b][n // BS] = free.pop()
    ctx = [n + 1 for n in lens_pre]
    slots = O.slot_ref(tables, [0, 1, 2, 3], ctx)
    k_new = bits(np.stack([k[-1] for k in nk]))
    v_new = bits(np.stack([v[-1] for v in nv]))
    kc, vc = O.append_ref(kp, vp, k_new, v_new, slots)
    q = rand_exact(rng, (3, Hq, D))
    got = O.decode_ref(bits(q), kc, vc, tables, ctx, 0.3)
    src = repeated_heads(Hq, Hkv)
    for b in range(3):
        for h in range(Hq):
            want = brute_attention(list(q[b, h]), list(nk[b]), list(nv[b]), src[h], 0.3)
            assert np.allclose(got[b, h], want, atol=1e-12)


# ---------------------------------------------------------------------------
# pins: byte formula ([P1] "Memory"; [P2] sections 2.1-2.4 and the listing's
# expected output)
# ---------------------------------------------------------------------------

UNITS = {"B": 1, "KiB": 1 << 10, "MiB": 1 << 20, "GiB": 1 << 30, "MB": 10 ** 6, "GB": 10 ** 9}


def check_printed_bytes():
    g = load_golden("kv_bytes.json")
    for e in g["per_token"]:
        got = O.kv_bytes_per_token(e["L"], e["Hkv"], e["D"], e["b"])
        assert got == e["printed"] * UNITS[e["unit"]], e
    for e in g["totals"]:
        got = O.kv_bytes(e["L"], e["Hkv"], e["D"], e["ctx"], e["b"]) / UNITS[e["unit"]]
        tol = 0.006 if e["unit"] == "MB" else 1e-12
        assert abs(got - e["printed"]) <= tol, (e, got)
    for name, L, Hkv, D, Hq, ctx, f16, i8, mha in g["kv_table_printed"]["rows"]:
        for cell, (heads, b) in zip((f16, i8, mha), ((Hkv, 2), (Hkv, 1), (Hq, 2))):
            if cell is None:      # contradicts the page itself; see the fixture's note
                continue
            val, unit = cell
            got = O.kv_bytes(L, heads, D, ctx, b) / UNITS[unit]
            if unit == "MiB":
                assert abs(got - val) <= 1e-3 * val, (name, ctx, val, got)
            else:
                assert abs(got - val) <= 0.05 + 1e-9, (name, ctx, val, got)
    for gpu_gb, params, ctx, n_req, mb in g["capacity_printed"]["rows"]:
        per_req_gb = O.kv_bytes(36, 8, 128, ctx, 2) / 1e9
        free = gpu_gb - params * 2 / 1e9 - 0.6
        assert int(free // per_req_gb) == n_req
        assert round(per_req_gb * 1000) == mb


def test_byte_formula_matches_printed_values():
    check_printed_bytes()


def test_f_full_scales_linearly():
    """[P2] section 5.4: only a fraction f_full of layers keeps a full cache."""
    assert O.kv_bytes(36, 8, 128, 4096, 2, f_full=0.25) == O.kv_bytes(9, 8, 128, 4096, 2)


def test_pool_bytes_of_the_0p6b_engine():
    """[P1] "Memory": a 512-block pool over 28 layers is 896 MiB; the same
    number as 512 pages of 16 tokens x 112 KiB."""
    per_layer_page = 2 * BS * 8 * 128 * 2          # K and V of one page, one layer
    assert 512 * per_layer_page * 28 == 896 * (1 << 20)


def check_copy_on_write_scenario():
    """[P1] test_copy_on_write (block size 4, one layer, one KV head, D 8):
    sequence a writes 4 zero rows into its block; b forks from a, whose last
    block is copied to a fresh block (fork_from); b then writes 4 rows of
    ones into its next block.  The fork's block holds a's rows, a's block is
    unchanged, and the write went to a block a does not use."""
    bs, nb = 4, 8
    pool = np.full((1, nb, bs, 1, 8), 0x7FC0, dtype=np.uint16)    # [L][blocks][slot][Hkv][D]
    zeros = np.zeros((4, 1, 8), dtype=np.uint16)                   # bf16 +0.0
    ones = np.full((4, 1, 8), 0x3F80, dtype=np.uint16)             # bf16 1.0
    a_blocks = [2]
    slots = O.slot_ref([a_blocks], [0, 4], [4], block_size=bs)
    pool[0], _ = O.append_ref(pool[0], pool[0], zeros, zeros, slots, block_size=bs)
    b_blocks = [5]                                                 # fork: tail copied (COW)
    pool = O.copy_blocks_ref(pool, [a_blocks[-1]], [b_blocks[-1]])
    assert np.array_equal(pool[0, 5], pool[0, 2])
    b_blocks.append(6)                                             # b.reserve(4)
    slots = O.slot_ref([b_blocks], [0, 4], [8], block_size=bs)
    pool[0], _ = O.append_ref(pool[0], pool[0], ones, ones, slots, block_size=bs)
    assert b_blocks[-1] != a_blocks[-1]
    assert np.all(pool[0, 2] == 0) and np.all(pool[0, 5] == 0) and np.all(pool[0, 6] == 0x3F80)
    assert np.all(pool[0, [0, 1, 3, 4, 7]] == 0x7FC0)


def check_copy_blocks_bits_all_layers():
    """Every layer's destination block becomes the source's bits (NaN
    payloads, -0.0); sources and other blocks are untouched; pairs run in
    order (a chain 1->3, 3->4 leaves block 4 equal to block 1)."""
    rng = np.random.default_rng(40)
    pool = rng.integers(0, 1 << 16, size=(3, 6, BS, 2, 4), dtype=np.uint16)
    pool[1, 1, 0, 0, 0] = 0x7FC1
    pool[2, 1, 3, 1, 2] = 0x8000
    out = O.copy_blocks_ref(pool, [1, 3, 0], [3, 4, 5])
    assert np.array_equal(out[:, 3], pool[:, 1]) and np.array_equal(out[:, 4], pool[:, 1])
    assert np.array_equal(out[:, 5], pool[:, 0])
    assert np.array_equal(out[:, :3], pool[:, :3])
    with pytest.raises(IndexError):
        O.copy_blocks_ref(pool, [6], [0])


def test_copy_on_write_scenario():
    check_copy_on_write_scenario()


def test_copy_blocks_bits_all_layers():
    check_copy_blocks_bits_all_layers()


# ---------------------------------------------------------------------------
# planted mistakes: each one must fail at least one pin above
# ---------------------------------------------------------------------------

PINS = [check_decode_brute_force, check_hand_example, check_ctx1_returns_v0,
        check_zero_query_gives_mean, check_dominant_key, check_rows_sum_to_one,
        check_gqa_equals_repeated_mha, check_prefill_brute_force, check_causal_hand_example,
        check_mask_equivalence, check_reserve20_example, check_decode_slots_follow_context,
        check_copy_on_write_scenario, check_copy_blocks_bits_all_layers]


def _mutants():
    orig_attend = O.attend_one
    orig_gather = O.gather_ref
    orig_slot = O.slot_ref

    def gather_reversed_offsets(cache, row, n, block_size=BS):
        rows = [cache[int(row[p // block_size]), block_size - 1 - p % block_size] for p in range(n)]
        return np.stack(rows) if rows else orig_gather(cache, row, n, block_size)

    def gather_wrapped_pages(cache, row, n, block_size=BS):
        used = (n + block_size - 1) // block_size
        rows = [cache[int(row[(p // block_size + 1) % used]), p % block_size] for p in range(n)]
        return np.stack(rows) if rows else orig_gather(cache, row, n, block_size)

    def slot_off_by_one(tables, cu, ctx, block_size=BS):
        return orig_slot(tables, cu, [c + 1 for c in ctx], block_size)

    def prefill_exclusive(q, cu, kc, vc, tables, ctx, scale, block_size=BS):
        # mask kpos < qpos instead of kpos <= qpos (keeping at least one key)
        out = np.zeros(q.shape)
        Hq, Hkv = q.shape[1], kc.shape[2]
        for b in range(len(ctx)):
            lo, hi = cu[b], cu[b + 1]
            T, n = hi - lo, ctx[b]
            K = O.bf16_to_f64(orig_gather(kc, tables[b], n, block_size))
            V = O.bf16_to_f64(orig_gather(vc, tables[b], n, block_size))
            for t in range(T):
                qp = max(n - T + t, 1)
                for h in range(Hq):
                    g = h // (Hq // Hkv)
                    out[lo + t, h] = orig_attend(O.bf16_to_f64(q[lo + t, h]), K[:qp, g], V[:qp, g], scale)
        return out

    orig_copy = O.copy_blocks_ref

    def copy_first_layer_only(pool, src, dst):
        out = np.array(pool, copy=True)
        out[:1] = orig_copy(pool[:1], src, dst)
        return out

    return {
        "block copy of layer 0 only": ("copy_blocks_ref", copy_first_layer_only),
        "head map h % Hkv": ("kv_head_of", lambda h, Hq, Hkv: h % Hkv),
        "scale dropped": ("attend_one", lambda q, K, V, s: orig_attend(q, K, V, 1.0)),
        "scale applied twice": ("attend_one", lambda q, K, V, s: orig_attend(q, K, V, s * s)),
        "K and V swapped": ("attend_one", lambda q, K, V, s: orig_attend(q, V, K, s)),
        "last key dropped": ("attend_one", lambda q, K, V, s: orig_attend(q, K[:-1], V[:-1], s)),
        "softmax not normalised": ("softmax_weights", lambda s: np.exp(s - np.max(s))),
        "offsets reversed within a page": ("gather_ref", gather_reversed_offsets),
        "logical pages shifted": ("gather_ref", gather_wrapped_pages),
        "start position off by one": ("slot_ref", slot_off_by_one),
        "causal mask exclusive": ("prefill_ref", prefill_exclusive),
    }


@pytest.mark.parametrize("name", sorted(_mutants()))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = _mutants()[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"planted mistake '{name}' passed every pin"
