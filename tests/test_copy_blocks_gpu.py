"""Copy-on-write / fork block copy on the GPU, through the C ABI, against the
oracle's copy ([P1] paged.py: SequenceCache._cow_copy and fork_from).  Bit
exact; pools of several layers, strided layers, bf16 and int8 page formats,
and the copy-on-write scenario end to end (fork, append, decode)."""
import numpy as np
import pytest
import torch

from oracle import pkv_oracle as O
from paged_kv_gqa_pkv_amd import binding as bd
from paged_kv_gqa_pkv_amd import step as ST
from paged_kv_gqa_pkv_amd import synth as S

pytestmark = pytest.mark.gpu


def bits(t):
    """Any tensor's raw bytes as a uint8 numpy array with a block axis kept."""
    t = t.detach().contiguous().cpu()
    return t.view(torch.uint8).numpy() if t.element_size() == 1 else \
        t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


def ids(xs):
    return torch.tensor(xs, dtype=torch.int32, device="cuda")


def test_copy_layered_bf16_pools():
    L, nb, Hkv, D = 3, 24, 8, 128
    k = S.randn_bf16((L, nb, 16, Hkv, D), 501).cuda()
    v = S.randn_bf16((L, nb, 16, Hkv, D), 502).cuda()
    k.view(torch.int16)[1, 7, 0, 0, 0] = 0x7FC1                 # NaN payload
    k.view(torch.int16)[2, 2, 5, 3, 9] = -32768                  # -0.0
    src, dst = [2, 7, 11], [20, 3, 15]
    want_k = O.copy_blocks_ref(bits(k), src, dst)
    want_v = O.copy_blocks_ref(bits(v), src, dst)
    bd.pkv_copy_blocks(ids(src), ids(dst), k, v, layered=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(k), want_k) and np.array_equal(bits(v), want_v)


def test_copy_strided_layers_leave_padding_untouched():
    """Layers that are further apart than their blocks (a view of a larger
    allocation): only the viewed blocks move; the padding between layers keeps
    its bits."""
    L, nb, Hkv, D = 2, 10, 2, 128
    full = S.randn_bf16((L, nb + 3, 16, Hkv, D), 503).cuda()
    before = bits(full)
    view = full[:, :nb]
    bd.pkv_copy_blocks(ids([1, 4]), ids([9, 0]), view, layered=True)
    torch.cuda.synchronize()
    after = bits(full)
    want = O.copy_blocks_ref(before[:, :nb], [1, 4], [9, 0])
    assert np.array_equal(after[:, :nb], want)
    assert np.array_equal(after[:, nb:], before[:, nb:])


def test_copy_int8_codes_and_scales():
    w = S.workload("c2")
    t = S.make_tables(w)
    d = S.make_layer_int8(w, t, 0, device="cuda")
    src, dst = [5, 17, 300], [511, 0, 64]
    want_kc = O.copy_blocks_ref(bits(d.k_codes)[None], src, dst)[0]
    want_vc = O.copy_blocks_ref(bits(d.v_codes)[None], src, dst)[0]
    want_ks = O.copy_blocks_ref(bits(d.k_scales)[None], src, dst)[0]
    want_vs = O.copy_blocks_ref(bits(d.v_scales)[None], src, dst)[0]
    bd.pkv_copy_blocks(ids(src), ids(dst), d.k_codes, d.v_codes)
    bd.pkv_copy_blocks(ids(src), ids(dst), d.k_scales, d.v_scales)
    torch.cuda.synchronize()
    assert np.array_equal(bits(d.k_codes), want_kc) and np.array_equal(bits(d.v_codes), want_vc)
    assert np.array_equal(bits(d.k_scales), want_ks) and np.array_equal(bits(d.v_scales), want_vs)


def test_copy_skips_pairs_outside_the_pool():
    nb = 6
    k = S.randn_bf16((nb, 16, 2, 128), 504).cuda()
    before = bits(k)
    bd.pkv_copy_blocks(ids([1, 99, -1, 2]), ids([3, 4, 5, 200]), k)
    torch.cuda.synchronize()
    assert np.array_equal(bits(k), O.copy_blocks_ref(before[None], [1], [3])[0])


def test_copy_on_write_fork_then_append_and_decode():
    """Sequence a holds 40 tokens (pages p0, p1 full, p2 partial).  b forks
    from a: p0 and p1 are shared by reference, the partial tail p2 is copied
    to a fresh page (fork_from).  Both then append one token at position 40
    and decode.  a's pages keep their bits except the slot a wrote; each
    output matches the oracle on its own table."""
    Hq, Hkv, D, nb = 16, 8, 128, 12
    k = S.randn_bf16((nb, 16, Hkv, D), 505).cuda()
    v = S.randn_bf16((nb, 16, Hkv, D), 506).cuda()
    ta, tb = [4, 9, 2], [4, 9, 7]                     # page 7 <- copy of a's tail page 2
    bd.pkv_copy_blocks(ids([2]), ids([7]), k, v)
    torch.cuda.synchronize()
    shared_before = bits(k)[[4, 9]].copy()
    tables = torch.tensor([ta, tb], dtype=torch.int32)
    ctx = torch.tensor([41, 41], dtype=torch.int32)
    cu = torch.tensor([0, 1, 2], dtype=torch.int32)
    slots = O.slot_ref(tables.tolist(), cu.tolist(), ctx.tolist())
    assert slots == [2 * 16 + 8, 7 * 16 + 8]
    kn = S.randn_bf16((2, Hkv, D), 507).cuda()
    vn = S.randn_bf16((2, Hkv, D), 508).cuda()
    pages_k = lambda: bits(k).view(np.uint16)
    pages_v = lambda: bits(v).view(np.uint16)
    kc0, vc0 = pages_k(), pages_v()
    sm = torch.empty(2, dtype=torch.int32, device="cuda")
    bd.pkv_slot_mapping(sm, tables.cuda(), cu.cuda(), ctx.cuda())
    bd.pkv_append(kn, vn, sm, k, v)
    q = S.randn_bf16((2, Hq, D), 509).cuda()
    out = torch.empty_like(q)
    bd.pkv_attn_decode(out, q, k, v, tables.cuda(), ctx.cuda(), 41, 128 ** -0.5)
    torch.cuda.synchronize()
    assert sm.cpu().tolist() == slots
    assert np.array_equal(bits(k)[[4, 9]], shared_before), "shared pages changed"
    u16 = lambda t: t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    kc, vc = O.append_ref(kc0, vc0, u16(kn), u16(vn), slots)
    assert np.array_equal(pages_k(), kc) and np.array_equal(pages_v(), vc)
    want = O.decode_ref(u16(q), kc, vc, tables.tolist(), ctx.tolist(), 128 ** -0.5)
    got = O.bf16_to_f64(u16(out))
    err = np.abs(got - want)
    print(f"cow fork decode: max abs {err.max():.3e} mean abs {err.mean():.3e}", flush=True)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    # the fork's copy differs from a's page only in the slot each one wrote
    ka, kb = kc[2], kc[7]
    diff = np.any(ka != kb, axis=(1, 2))             # per slot
    assert diff.tolist() == [i == 8 for i in range(16)]
