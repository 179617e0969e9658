"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Acceptance: slot mapping and append are bit-exact over the whole pool
(shared prefix pages and canary pages included); attention outputs from
bf16 inputs with fp32 accumulation are within max abs 2e-2 and mean abs
2e-3 of the oracle run on the same bf16 inputs, and finite (the NaN
canaries in unwritten slots and unused pages would poison any stray read).
"""
import math

import numpy as np
import pytest
import torch

from oracle import pkv_oracle as O
from paged_kv_gqa_pkv_amd import binding as bd
from paged_kv_gqa_pkv_amd import step as ST
from paged_kv_gqa_pkv_amd import synth as S

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def as_f64(t: torch.Tensor) -> np.ndarray:
    return O.bf16_to_f64(u16(t))


def assert_close(got: torch.Tensor, want: np.ndarray, what: str):
    g = as_f64(got)
    assert np.all(np.isfinite(g)), f"{what}: non-finite outputs"
    err = np.abs(g - want)
    print(f"{what}: max abs {err.max():.3e} mean abs {err.mean():.3e}", flush=True)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (what, err.max(), err.mean())


def oracle_step(w, t, d):
    """Slot mapping, append, prefill and decode on the CPU for one layer."""
    bt = t.block_tables.numpy().tolist()
    ctx = t.context_lens.numpy().tolist()
    slots = O.slot_ref(bt, t.cu_new.numpy().tolist(), ctx)
    kc, vc = O.append_ref(u16(d.k_cache), u16(d.v_cache), u16(d.k_new),
                          u16(d.v_new), slots)
    scale = O.default_scale(w.D)
    npre = len(w.prefill_seqs)
    dec = pre = None
    if w.decode_seqs:
        dec = O.decode_ref(u16(d.q_decode), kc, vc, bt[npre:], ctx[npre:], scale)
    if w.prefill_seqs:
        pre = O.prefill_ref(u16(d.q_prefill), S.prefill_cu(w).numpy().tolist(), kc, vc,
                            bt[:npre], ctx[:npre], scale)
    return slots, kc, vc, dec, pre


def gpu_step(w, t, d, fused=True):
    plan = ST.plan_step(w, t, fused=fused)
    dev = {k: getattr(d, k).cuda() if getattr(d, k) is not None else None
           for k in ("k_cache", "v_cache", "k_new", "v_new", "q_decode", "q_prefill")}
    out_dec = torch.empty_like(dev["q_decode"]) if w.decode_seqs else None
    out_pre = torch.empty_like(dev["q_prefill"]) if w.prefill_seqs else None
    ST.slot_mapping(plan)
    ST.layer(plan, dev["k_cache"], dev["v_cache"], dev["k_new"], dev["v_new"],
             dev["q_decode"], out_dec, dev["q_prefill"], out_pre)
    torch.cuda.synchronize()
    return plan, dev, out_dec, out_pre


def check_workload(w, layer=0, fused=True):
    """A decode-only step runs fused (pkv_attn_decode_append) unless fused is
    False (pkv_append, then pkv_attn_decode)."""
    print(f"[parity] {w.name} layer {layer} fused={fused}: {w.description}", flush=True)
    t = S.make_tables(w)
    d = S.make_layer(w, t, layer)
    plan, dev, out_dec, out_pre = gpu_step(w, t, d, fused)
    slots, kc, vc, dec, pre = oracle_step(w, t, d)
    assert plan.slot_mapping.cpu().numpy().tolist() == slots, "slot mapping differs"
    assert np.array_equal(u16(dev["k_cache"]), kc), "K pool after append differs"
    assert np.array_equal(u16(dev["v_cache"]), vc), "V pool after append differs"
    if dec is not None:
        assert_close(out_dec, dec, f"{w.name} decode")
    if pre is not None:
        assert_close(out_pre, pre, f"{w.name} prefill")
    return plan, dev, out_dec, out_pre


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_decode_configs(name, fused):
    check_workload(S.workload(name), fused=fused)


def test_c3_another_layer_and_shared_pages_untouched():
    w = S.workload("c3")
    plan, dev, _, _ = check_workload(w, layer=27)
    t = S.make_tables(w)
    d = S.make_layer(w, t, 27)
    shared = t.block_tables[0, :13].long()
    assert torch.equal(dev["k_cache"].cpu()[shared].view(torch.int16),
                       d.k_cache[shared].view(torch.int16))


@pytest.mark.parametrize("chunk_step", range(6))
def test_mixed_step_configs(chunk_step):
    check_workload(S.workload("c5", chunk_step))


def _seqs_decode(ctxs):
    return [S.SeqSpec(c - 1, 1, False) for c in ctxs]


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_group_sizes_and_ragged_lengths(G):
    Hkv = 2
    ctxs = [1, 15, 16, 17, 31, 33, 200, 515]
    w = S.custom_workload(f"ragged_G{G}", _seqs_decode(ctxs), Hq=Hkv * G, Hkv=Hkv, D=128,
                          num_blocks=96, base_seed=70 + G)
    check_workload(w, fused=False)


def test_decode_long_context_many_splits():
    w = S.custom_workload("long_small_batch", _seqs_decode([5000, 777, 3]), Hq=32, Hkv=8, D=128,
                          num_blocks=400, base_seed=80)
    assert bd.pkv_decode_num_splits(3, 32, 8, 128, 5000) > 1
    check_workload(w)


@pytest.mark.parametrize("fused", [True, False])
def test_decode_group_size_8_heads_of_a_large_model_with_splits(fused):
    """G = 8 (64 query heads over 8 KV heads, the bf16 policy on the matrix
    cores) with a context long enough for splits, a page boundary, a partial
    page and a one-token context, every output row compared."""
    ctxs = [4500, 2048, 1025, 17, 1]
    w = S.custom_workload("g8_splits", _seqs_decode(ctxs), Hq=64, Hkv=8, D=128,
                          num_blocks=520, base_seed=83)
    assert bd.pkv_decode_num_splits(len(ctxs), 64, 8, 128, 4500) > 1
    check_workload(w, fused=fused)


def test_decode_single_pass_large_batch():
    ctxs = [int(x) for x in np.random.default_rng(81).integers(1, 90, size=160)]
    w = S.custom_workload("wide_batch", _seqs_decode(ctxs), Hq=16, Hkv=8, D=128,
                          num_blocks=1200, base_seed=81)
    assert bd.pkv_decode_num_splits(160, 16, 8, 128, max(ctxs)) == 1
    check_workload(w)


def test_prefill_varlen_batch():
    seqs = [S.SeqSpec(0, 37, True), S.SeqSpec(100, 1, True), S.SeqSpec(60, 200, True),
            S.SeqSpec(16, 16, True), S.SeqSpec(3, 1, False), S.SeqSpec(90, 1, False)]
    for G, Hkv in ((1, 4), (2, 4), (4, 2), (8, 1)):
        w = S.custom_workload(f"varlen_G{G}", seqs, Hq=Hkv * G, Hkv=Hkv, D=128, num_blocks=64,
                              base_seed=90 + G)
        check_workload(w)


def test_prefill_short_contexts_single_split():
    """Contexts of at most 4 key tiles run without key splits."""
    seqs = [S.SeqSpec(0, 100, True), S.SeqSpec(150, 106, True), S.SeqSpec(7, 1, False)]
    w = S.custom_workload("short_prefill", seqs, Hq=16, Hkv=8, D=128, num_blocks=48,
                          base_seed=97)
    assert bd.pkv_prefill_workspace_bytes(2, 106, 16, 8, 128, 256) == 0
    check_workload(w)


def test_prefill_many_key_splits():
    """A long context with few row tiles is cut into many key splits."""
    seqs = [S.SeqSpec(6000, 64, True)]
    w = S.custom_workload("long_prefill", seqs, Hq=32, Hkv=8, D=128, num_blocks=400,
                          base_seed=98)
    assert bd.pkv_prefill_workspace_bytes(1, 64, 32, 8, 128, 6064) > 0
    check_workload(w)


def test_ctx1_is_exact_value_row():
    w = S.custom_workload("ctx1", _seqs_decode([1, 1, 1]), Hq=16, Hkv=8, D=128, num_blocks=8,
                          base_seed=95)
    plan, dev, out_dec, _ = check_workload(w)
    t = S.make_tables(w)
    d = S.make_layer(w, t, 0)
    want = d.v_new.repeat_interleave(2, dim=1)          # head h reads KV head h // 2
    assert torch.equal(out_dec.cpu().view(torch.int16), want.view(torch.int16))


def test_context_zero_gives_zeros():
    B, Hq, Hkv, D = 3, 16, 8, 128
    k = S.randn_bf16((8, 16, Hkv, D), 1).cuda()
    v = S.randn_bf16((8, 16, Hkv, D), 2).cuda()
    q = S.randn_bf16((B, Hq, D), 3).cuda()
    bt = torch.tensor([[0, 1], [2, 3], [4, 5]], dtype=torch.int32, device="cuda")
    ctx = torch.tensor([0, 5, 0], dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 7.0)
    bd.pkv_attn_decode(out, q, k, v, bt, ctx, 32, 128 ** -0.5)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0) and torch.all(out[2] == 0)
    want = O.decode_ref(u16(q[1:2]), u16(k), u16(v), [[2, 3]], [5], 128 ** -0.5)
    assert_close(out[1:2], want, "ctx0 neighbour")


def test_bulk_append_bit_exact():
    slots, k_new, v_new, pk, pv = S.bulk_append_inputs(65536, 4096, 8, 128, seed=123)
    dk, dv = pk.cuda(), pv.cuda()
    bd.pkv_append(k_new.cuda(), v_new.cuda(), slots.cuda(), dk, dv)
    torch.cuda.synchronize()
    kc, vc = O.append_ref(u16(pk), u16(pv), u16(k_new), u16(v_new),
                          slots.numpy().tolist())
    assert np.array_equal(u16(dk), kc) and np.array_equal(u16(dv), vc)


def test_slot_mapping_entries_without_a_slot():
    """Slots are int32: the largest block id with a slot (2^27 - 1) maps to
    2^31 - 16 + offset; a negative entry, an id of 2^27 or more, or a page
    past the table gives -1."""
    big = (1 << 27) - 1
    bt = torch.tensor([[big, 0], [0, 1 << 27], [0, -1], [0, 0], [0, 0]], dtype=torch.int32)
    ctx = torch.tensor([1, 17, 18, 5, 40], dtype=torch.int32)
    cu = torch.arange(6, dtype=torch.int32)
    sm = torch.full((5,), 7, dtype=torch.int32, device="cuda")
    bd.pkv_slot_mapping(sm, bt.cuda(), cu.cuda(), ctx.cuda())
    torch.cuda.synchronize()
    assert sm.cpu().tolist() == [(1 << 31) - 16, -1, -1, 4, -1]


def test_append_skips_negative_slots_and_keeps_bits():
    Hkv, D = 8, 128
    pk = S.randn_bf16((4, 16, Hkv, D), 5)
    pv = S.randn_bf16((4, 16, Hkv, D), 6)
    k_new = torch.full((3, Hkv, D), 0x7FC1, dtype=torch.int16).view(torch.bfloat16)  # NaN payload
    k_new.view(torch.int16)[1] = -32768                                              # -0.0
    v_new = S.randn_bf16((3, Hkv, D), 7)
    slots = torch.tensor([5, -1, 63], dtype=torch.int32)
    dk, dv = pk.cuda(), pv.cuda()
    bd.pkv_append(k_new.cuda(), v_new.cuda(), slots.cuda(), dk, dv)
    torch.cuda.synchronize()
    kc, vc = O.append_ref(u16(pk), u16(pv), u16(k_new), u16(v_new), [5, -1, 63])
    assert np.array_equal(u16(dk), kc) and np.array_equal(u16(dv), vc)


def test_determinism_and_placement_invariance():
    """Repeated runs are bit-identical, and relabelling the physical pages (the
    tables mapped through the same permutation) gives bit-identical outputs:
    the kernels walk logical positions in the same order whatever the
    placement."""
    w = S.workload("c2")
    t = S.make_tables(w)
    d = S.make_layer(w, t, 0)
    _, _, o1, _ = gpu_step(w, t, d)
    _, _, o2, _ = gpu_step(w, t, d)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    perm = torch.randperm(w.num_blocks, generator=torch.Generator().manual_seed(9))
    t2 = S.Tables(torch.where(t.block_tables >= 0, perm[t.block_tables.long().clamp(min=0)].int(),
                              t.block_tables), t.context_lens, t.cu_new, t.pre_lens)
    kc = torch.empty_like(d.k_cache); vc = torch.empty_like(d.v_cache)
    kc[perm] = d.k_cache; vc[perm] = d.v_cache
    d2 = S.LayerData(kc, vc, d.k_new, d.v_new, d.q_decode, d.q_prefill)
    _, _, o3, _ = gpu_step(w, t2, d2)
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))


def test_invalid_indices_poison_outputs_without_faulting():
    """A context beyond the table or a block id outside the pool makes the
    affected outputs NaN; the kernels clamp the address and never read
    outside the pool.  Other sequences are unaffected."""
    Hq, Hkv, D = 16, 8, 128
    k = S.randn_bf16((8, 16, Hkv, D), 11).cuda()
    v = S.randn_bf16((8, 16, Hkv, D), 12).cuda()
    q = S.randn_bf16((3, Hq, D), 13).cuda()
    bt = torch.tensor([[0, 1], [2, 999], [3, 4]], dtype=torch.int32, device="cuda")
    ctx = torch.tensor([20, 20, 20], dtype=torch.int32, device="cuda")
    out = torch.zeros_like(q)
    bd.pkv_attn_decode(out, q, k, v, bt, ctx, 32, 128 ** -0.5)
    torch.cuda.synchronize()
    assert torch.isnan(out[1].float()).all()
    assert torch.isfinite(out[0].float()).all() and torch.isfinite(out[2].float()).all()
    ctx_bad = torch.tensor([20, 40, 20], dtype=torch.int32, device="cuda")   # 40 > 2 pages
    bt_ok = torch.tensor([[0, 1], [2, 5], [3, 4]], dtype=torch.int32, device="cuda")
    bd.pkv_attn_decode(out, q, k, v, bt_ok, ctx_bad, 32, 128 ** -0.5)
    torch.cuda.synchronize()
    assert torch.isnan(out[1].float()).all() and torch.isfinite(out[0].float()).all()


def test_prefill_context_past_the_plan_poisons_that_sequence():
    """A sequence whose context holds more key tiles than the launch was
    planned for (max_context_len below its real length) gets NaN rows, as
    decode does, instead of silently dropping the keys no split reaches; the
    other sequence of the call is unaffected."""
    seqs = [S.SeqSpec(136, 64, True), S.SeqSpec(2936, 64, True)]
    w = S.custom_workload("past_plan", seqs, Hq=16, Hkv=8, D=128, num_blocks=210, base_seed=83)
    t = S.make_tables(w)
    d = S.make_layer(w, t, 0)
    bt, ctx = t.block_tables.numpy().tolist(), t.context_lens.numpy().tolist()
    slots = O.slot_ref(bt, t.cu_new.numpy().tolist(), ctx)
    kc, vc = O.append_ref(u16(d.k_cache), u16(d.v_cache), u16(d.k_new),
                          u16(d.v_new), slots)
    want0 = O.prefill_ref(u16(d.q_prefill[:64]), [0, 64], kc, vc, bt[:1], ctx[:1],
                          O.default_scale(128))
    to_dev = lambda bits: torch.from_numpy(bits.view(np.int16).copy()).view(
        torch.bfloat16).cuda()
    q = d.q_prefill.cuda()
    out = torch.zeros_like(q)
    cu = torch.tensor([0, 64, 128], dtype=torch.int32, device="cuda")
    nbytes = bd.pkv_prefill_workspace_bytes(2, 64, 16, 8, 128, 200)
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda") if nbytes else None
    bd.pkv_attn_prefill_chunk(out, q, cu, to_dev(kc), to_dev(vc), t.block_tables.cuda(),
                              t.context_lens.cuda(), 64, 200, O.default_scale(128),
                              workspace=ws)
    torch.cuda.synchronize()
    assert torch.isnan(out[64:].float()).all(), "rows past the plan must be NaN"
    assert_close(out[:64], want0, "prefill sequence inside the plan")


def test_workspace_too_small_is_rejected():
    w = S.workload("c2")
    need = bd.pkv_decode_workspace_bytes(8, 16, 8, 128, 1024)
    assert need > 0
    q = torch.zeros((8, 16, 128), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((w.num_blocks, 16, 8, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((8, 64), dtype=torch.int32, device="cuda")
    ctx = torch.ones(8, dtype=torch.int32, device="cuda")
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(bd.PkvError) as e:
        bd.pkv_attn_decode(torch.empty_like(q), q, pool, pool.clone(), bt, ctx, 1024,
                           0.088, workspace=ws)
    assert e.value.code == bd.PKV_EWORKSPACE


_FULL_ORACLE = {}


def _full_size_oracle(w, t, k_pre, v_pre, kn, vn, qh):
    """The oracle's slots, append and decode of every (sequence, head) of a
    full-size batch, from the pre-append pools; kept per workload (the inputs
    are seeded, so the fused and unfused calls see the same ones)."""
    if w.name not in _FULL_ORACLE:
        _FULL_ORACLE.clear()
        bt = t.block_tables.numpy().tolist()
        ctx = t.context_lens.numpy().tolist()
        slots = O.slot_ref(bt, t.cu_new.numpy().tolist(), ctx)
        kc, vc = O.append_ref(k_pre, v_pre, kn, vn, slots)
        want = O.decode_ref(qh, kc, vc, bt, ctx, O.default_scale(w.D))
        _FULL_ORACLE[w.name] = (slots, want)
    return _FULL_ORACLE[w.name]


def _full_size(name, fused):
    """Full-size configuration, one layer, generated on the device; every
    (sequence, head) output against the oracle's decode over its own append
    of the step's rows into the pre-append pools."""
    w = S.workload(name)
    print(f"[parity] {w.name} full size, fused={fused}: {w.description}", flush=True)
    t = S.make_tables(w)
    fill = S.page_fill_counts(w, t)
    d = S.make_layer(w, t, 0, device="cuda", fill=fill)
    k_pre, v_pre = u16(d.k_cache), u16(d.v_cache)
    kn, vn, qh = u16(d.k_new), u16(d.v_new), u16(d.q_decode)
    plan = ST.plan_step(w, t, fused=fused)
    assert plan.fused == fused
    out = torch.full_like(d.q_decode, float("nan"))
    ST.slot_mapping(plan)
    ST.layer(plan, d.k_cache, d.v_cache, d.k_new, d.v_new, d.q_decode, out)
    torch.cuda.synchronize()
    slots, want = _full_size_oracle(w, t, k_pre, v_pre, kn, vn, qh)
    assert plan.slot_mapping.cpu().numpy().tolist() == slots
    assert_close(out, want, f"{name} all {want.shape[0]} x {want.shape[1]} rows")
    # the appended rows landed bit-exactly, and nothing else changed
    dk, dv = u16(d.k_cache), u16(d.v_cache)
    sl = np.array(slots)
    assert np.array_equal(dk[sl // 16, sl % 16], kn) and np.array_equal(dv[sl // 16, sl % 16], vn)
    dk[sl // 16, sl % 16] = k_pre[sl // 16, sl % 16]
    dv[sl // 16, sl % 16] = v_pre[sl // 16, sl % 16]
    assert np.array_equal(dk, k_pre) and np.array_equal(dv, v_pre)


def test_full_size_c4a_all_rows():
    """Batch 64 at context 4096 ([P2] Module 04 section 3.2): all 64 x 32 rows."""
    _full_size("c4a", fused=True)


@pytest.mark.parametrize("fused", [True, False])
def test_full_size_c4b_all_rows(fused):
    """13 sequences at context 32768 ([P2] Module 04 section 2.4), 9 key
    splits: all 13 x 32 rows, through the fused call and through append then
    decode."""
    _full_size("c4b", fused=fused)


def test_graph_replays_match_eager():
    """A whole mixed step (slot mapping, append, prefill with key splits,
    decode with splits) captured in one HIP graph: every replay, with eager
    work and synchronisations between replays, is bit-identical to the eager
    step (the kernels are deterministic and leave their workspaces ready)."""
    seqs = [S.SeqSpec(2000, 300, True), S.SeqSpec(900, 1, False), S.SeqSpec(4000, 1, False)]
    w = S.custom_workload("graph_step", seqs, Hq=16, Hkv=8, D=128, num_blocks=480, base_seed=99)
    t = S.make_tables(w)
    d = S.make_layer(w, t, 0, device="cuda")
    plan = ST.plan_step(w, t)
    assert plan.prefill_workspace is not None and plan.workspace is not None
    k0, v0 = d.k_cache.clone(), d.v_cache.clone()
    out_d, out_p = torch.empty_like(d.q_decode), torch.empty_like(d.q_prefill)

    def step(stream=None):
        ST.slot_mapping(plan, stream=stream)
        ST.layer(plan, d.k_cache, d.v_cache, d.k_new, d.v_new, d.q_decode, out_d,
                 d.q_prefill, out_p, stream=stream)

    step()
    torch.cuda.synchronize()
    want_d, want_p = out_d.clone(), out_p.clone()
    want_k = d.k_cache.clone()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            step(stream=cap)
    torch.cuda.synchronize()
    for rep in range(3):
        out_d.fill_(0); out_p.fill_(0)
        d.k_cache.copy_(k0); d.v_cache.copy_(v0)      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_d.view(torch.int16), want_d.view(torch.int16)), rep
        assert torch.equal(out_p.view(torch.int16), want_p.view(torch.int16)), rep
        assert torch.equal(d.k_cache.view(torch.int16), want_k.view(torch.int16)), rep
        step()                                         # an eager step in between
        torch.cuda.synchronize()
        assert torch.equal(out_d.view(torch.int16), want_d.view(torch.int16)), rep


def test_concurrent_decode_stream_matches_and_replays():
    """The decode launch on a second stream, concurrent with the chunk (the
    two only read the pools after the append): outputs and pools bit-identical
    to the one-stream step, eagerly and in every replay of a graph captured
    with both streams."""
    seqs = [S.SeqSpec(2000, 300, True), S.SeqSpec(900, 1, False), S.SeqSpec(4000, 1, False)]
    w = S.custom_workload("two_streams", seqs, Hq=16, Hkv=8, D=128, num_blocks=480,
                          base_seed=98)
    t = S.make_tables(w)
    d = S.make_layer(w, t, 0, device="cuda")
    plan = ST.plan_step(w, t, mixed=False)      # the two-launch path
    k0, v0 = d.k_cache.clone(), d.v_cache.clone()
    out_d, out_p = torch.empty_like(d.q_decode), torch.empty_like(d.q_prefill)

    def step(stream=None, decode_stream=None):
        ST.slot_mapping(plan, stream=stream)
        ST.layer(plan, d.k_cache, d.v_cache, d.k_new, d.v_new, d.q_decode, out_d,
                 d.q_prefill, out_p, stream=stream, decode_stream=decode_stream)

    def reset():
        out_d.fill_(0); out_p.fill_(0)
        d.k_cache.copy_(k0); d.v_cache.copy_(v0)
        torch.cuda.synchronize()

    step()
    torch.cuda.synchronize()
    want_d, want_p, want_k = out_d.clone(), out_p.clone(), d.k_cache.clone()

    def same(tag):
        assert torch.equal(out_d.view(torch.int16), want_d.view(torch.int16)), tag
        assert torch.equal(out_p.view(torch.int16), want_p.view(torch.int16)), tag
        assert torch.equal(d.k_cache.view(torch.int16), want_k.view(torch.int16)), tag

    side = torch.cuda.Stream()
    reset()
    step(decode_stream=side)
    torch.cuda.synchronize()
    same("eager, two streams")
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            step(stream=cap, decode_stream=side)
    torch.cuda.synchronize()
    for rep in range(3):
        reset()
        g.replay()
        torch.cuda.synchronize()
        same(f"replay {rep}")
