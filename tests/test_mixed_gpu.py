"""pkv_attn_prefill_decode, a mixed step's attention in one call ([P1] "Why
chunked prefill": decode tokens beside prompt chunks in one step), through
the C ABI.  Its outputs must be bit-identical to pkv_attn_prefill_chunk
followed by pkv_attn_decode on the same inputs (the one-grid launch runs the
same per-workgroup arithmetic), and within the usual tolerance of the
oracle: for the six c5 steps, group sizes 1, 2, 4 (one launch) and 8 (two
launches), key splits on both sides, and a HIP graph replayed several
times.  pkv_attn_prefill_decode_append, the same with the layer's append in
the launch: the pools afterwards bit-identical to the append's, the prefill
half bit-identical to append + pkv_attn_prefill_chunk, the decode half within
1e-2 of append + pkv_attn_decode (its new rows are reduced from registers)
and within the oracle's tolerance."""
import numpy as np
import pytest
import torch

from oracle import pkv_oracle as O
from paged_kv_gqa_pkv_amd import binding as bd
from paged_kv_gqa_pkv_amd import step as ST
from paged_kv_gqa_pkv_amd import synth as S

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


def u16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def bits_equal(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def setup(w):
    t = S.make_tables(w)
    d = S.make_layer(w, t, 0, device="cuda")
    k0, v0 = u16(d.k_cache), u16(d.v_cache)
    plan = ST.plan_step(w, t, fused=False)
    assert plan.mixed and not plan.fused
    ST.slot_mapping(plan)
    bd.pkv_append(d.k_new, d.v_new, plan.slot_mapping, d.k_cache, d.v_cache)
    return t, d, plan, k0, v0


def mixed_call(d, plan, stream=None):
    op = torch.full_like(d.q_prefill, float("nan"))
    od = torch.full_like(d.q_decode, float("nan"))
    bd.pkv_attn_prefill_decode(op, d.q_prefill, plan.cu_q, plan.bt_prefill, plan.ctx_prefill,
                               plan.max_q_len, plan.max_ctx_prefill, od, d.q_decode,
                               plan.bt_decode, plan.ctx_decode, plan.max_ctx_decode,
                               d.k_cache, d.v_cache, plan.scale,
                               prefill_workspace=plan.prefill_workspace,
                               decode_workspace=plan.workspace, stream=stream)
    return op, od


def separate_calls(d, plan):
    op = torch.full_like(d.q_prefill, float("nan"))
    od = torch.full_like(d.q_decode, float("nan"))
    bd.pkv_attn_prefill_chunk(op, d.q_prefill, plan.cu_q, d.k_cache, d.v_cache, plan.bt_prefill,
                              plan.ctx_prefill, plan.max_q_len, plan.max_ctx_prefill, plan.scale,
                              workspace=plan.prefill_workspace)
    bd.pkv_attn_decode(od, d.q_decode, d.k_cache, d.v_cache, plan.bt_decode, plan.ctx_decode,
                       plan.max_ctx_decode, plan.scale, workspace=plan.workspace)
    return op, od


def check_oracle(w, t, d, k0, v0, op, od, what):
    bt, ctx = t.block_tables.tolist(), t.context_lens.tolist()
    slots = O.slot_ref(bt, t.cu_new.tolist(), ctx)
    kc, vc = O.append_ref(k0, v0, u16(d.k_new), u16(d.v_new), slots)
    npre = len(w.prefill_seqs)
    scale = O.default_scale(w.D)
    want_p = O.prefill_ref(u16(d.q_prefill), S.prefill_cu(w).tolist(), kc, vc, bt[:npre],
                           ctx[:npre], scale)
    want_d = O.decode_ref(u16(d.q_decode), kc, vc, bt[npre:], ctx[npre:], scale)
    for got, want, half in ((op, want_p, "prefill"), (od, want_d, "decode")):
        g = O.bf16_to_f64(u16(got))
        assert np.all(np.isfinite(g)), f"{what} {half}: non-finite outputs"
        err = np.abs(g - want)
        print(f"{what} {half}: max abs {err.max():.3e} mean abs {err.mean():.3e}", flush=True)
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS


def run(w):
    print(f"[mixed] {w.name}: {w.description}", flush=True)
    t, d, plan, k0, v0 = setup(w)
    op, od = mixed_call(d, plan)
    sp, sd = separate_calls(d, plan)
    torch.cuda.synchronize()
    assert bits_equal(op, sp), "prefill half differs from pkv_attn_prefill_chunk"
    assert bits_equal(od, sd), "decode half differs from pkv_attn_decode"
    check_oracle(w, t, d, k0, v0, op, od, w.name)
    return t, d, plan, op, od


@pytest.mark.parametrize("chunk_step", range(6))
def test_c5_steps(chunk_step):
    run(S.workload("c5", chunk_step))


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_group_sizes_ragged_and_splits(G):
    """Two chunk sequences (one long enough for key splits) beside decode
    sequences of ragged lengths, one long enough for decode splits."""
    Hkv = 2
    seqs = [S.SeqSpec(3000, 200, True), S.SeqSpec(40, 33, True),
            S.SeqSpec(0, 1, False), S.SeqSpec(16, 1, False), S.SeqSpec(300, 1, False),
            S.SeqSpec(5000, 1, False)]
    w = S.custom_workload(f"mixed_G{G}", seqs, Hq=Hkv * G, Hkv=Hkv, D=128, num_blocks=640,
                          base_seed=700 + G)
    _, _, plan, _, _ = run(w)
    assert plan.prefill_workspace is not None and plan.workspace is not None


def test_invalid_pages_poison_their_sequences_in_both_forms():
    """A prefill sequence whose table holds an invalid page id and a decode
    sequence whose table holds one: their outputs are NaN, the others'
    finite, and the one-launch form gives the two calls' outputs bit for
    bit (the poisoned rows included)."""
    w = S.workload("c5", 2)
    t, d, plan, k0, v0 = setup(w)
    npre = len(w.prefill_seqs)
    plan.block_tables[0, 3] = -1                      # a page of the chunk's prefix
    plan.block_tables[npre + 1, 0] = 1 << 30          # past the pool
    op, od = mixed_call(d, plan)
    sp, sd = separate_calls(d, plan)
    torch.cuda.synchronize()
    assert bits_equal(op, sp) and bits_equal(od, sd)
    assert torch.isnan(op.float()).all(), "the chunk's rows are poisoned"
    assert torch.isnan(od[1].float()).all()
    keep = [i for i in range(od.shape[0]) if i != 1]
    assert torch.isfinite(od[keep].float()).all()


def test_graph_replays_are_bit_identical():
    w = S.workload("c5", 3)
    t, d, plan, k0, v0 = setup(w)
    want_p, want_d = mixed_call(d, plan)
    torch.cuda.synchronize()
    op = torch.empty_like(want_p)
    od = torch.empty_like(want_d)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            p_, d_ = mixed_call(d, plan, stream=cap)
            op.copy_(p_)
            od.copy_(d_)
    torch.cuda.synchronize()
    for rep in range(3):
        op.fill_(0)
        od.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert bits_equal(op, want_p) and bits_equal(od, want_d), rep
        e_p, e_d = mixed_call(d, plan)                # eager work between replays
        torch.cuda.synchronize()
        assert bits_equal(e_p, want_p) and bits_equal(e_d, want_d), rep


# --------------------------------------------------------------------------
# pkv_attn_prefill_decode_append: the layer's append in the same launch
# --------------------------------------------------------------------------

def fused_setup(w):
    """Pools before the append (the fused call writes the step's rows)."""
    t = S.make_tables(w)
    d = S.make_layer(w, t, 0, device="cuda")
    k0, v0 = u16(d.k_cache), u16(d.v_cache)
    plan = ST.plan_step(w, t)
    assert plan.mixed and plan.fused and plan.needs_slots
    ST.slot_mapping(plan)
    return t, d, plan, k0, v0


def fused_call(d, plan, kc, vc, stream=None):
    op = torch.full_like(d.q_prefill, float("nan"))
    od = torch.full_like(d.q_decode, float("nan"))
    bd.pkv_attn_prefill_decode_append(op, d.q_prefill, plan.cu_q, plan.bt_prefill,
                                      plan.ctx_prefill, plan.max_q_len, plan.max_ctx_prefill, od,
                                      d.q_decode, plan.bt_decode, plan.ctx_decode,
                                      plan.max_ctx_decode, d.k_new, d.v_new, plan.slot_mapping,
                                      kc, vc, plan.scale,
                                      prefill_workspace=plan.prefill_workspace,
                                      decode_workspace=plan.workspace, stream=stream)
    return op, od


def run_fused(w):
    print(f"[mixed fused] {w.name}: {w.description}", flush=True)
    t, d, plan, k0, v0 = fused_setup(w)
    kc, vc = d.k_cache.clone(), d.v_cache.clone()
    op, od = fused_call(d, plan, kc, vc)
    # the same step as separate calls: append, then the chunk and the decode
    bd.pkv_append(d.k_new, d.v_new, plan.slot_mapping, d.k_cache, d.v_cache)
    sp, sd = separate_calls(d, plan)
    torch.cuda.synchronize()
    assert torch.equal(kc.view(torch.int16), d.k_cache.view(torch.int16)), "K pool"
    assert torch.equal(vc.view(torch.int16), d.v_cache.view(torch.int16)), "V pool"
    assert bits_equal(op, sp), "prefill half differs from append + pkv_attn_prefill_chunk"
    diff = (od.float() - sd.float()).abs().max().item()
    print(f"{w.name}: decode half vs append + pkv_attn_decode: max abs {diff:.3e}", flush=True)
    assert torch.isfinite(od.float()).all() and diff <= 1e-2
    check_oracle(w, t, d, k0, v0, op, od, w.name + " fused")
    return t, d, plan, kc, vc, op, od


@pytest.mark.parametrize("chunk_step", range(6))
def test_fused_c5_steps(chunk_step):
    run_fused(S.workload("c5", chunk_step))


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_fused_group_sizes_chunks_starting_mid_page(G):
    """Chunks that start inside a page (positions 3000 and 40: the page holds
    cached rows before the chunk's first and fresh ones from it on), key
    splits, decode sequences of ragged lengths; G = 8 takes the separate
    launches."""
    Hkv = 2
    seqs = [S.SeqSpec(3000, 200, True), S.SeqSpec(40, 33, True),
            S.SeqSpec(0, 1, False), S.SeqSpec(16, 1, False), S.SeqSpec(300, 1, False),
            S.SeqSpec(5000, 1, False)]
    w = S.custom_workload(f"mixed_fused_G{G}", seqs, Hq=Hkv * G, Hkv=Hkv, D=128,
                          num_blocks=640, base_seed=720 + G)
    run_fused(w)


def test_fused_graph_replays_are_bit_identical():
    """The fused call writes the same rows into the same slots on every call,
    so replays and eager calls in between give the same outputs and pools."""
    w = S.workload("c5", 3)
    t, d, plan, k0, v0 = fused_setup(w)
    want_p, want_d = fused_call(d, plan, d.k_cache, d.v_cache)
    torch.cuda.synchronize()
    kc_want = d.k_cache.clone()
    op = torch.empty_like(want_p)
    od = torch.empty_like(want_d)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            p_, d_ = fused_call(d, plan, d.k_cache, d.v_cache, stream=cap)
            op.copy_(p_)
            od.copy_(d_)
    torch.cuda.synchronize()
    for rep in range(3):
        op.fill_(0)
        od.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert bits_equal(op, want_p) and bits_equal(od, want_d), rep
        e_p, e_d = fused_call(d, plan, d.k_cache, d.v_cache)        # eager work between replays
        torch.cuda.synchronize()
        assert bits_equal(e_p, want_p) and bits_equal(e_d, want_d), rep
    assert torch.equal(d.k_cache.view(torch.int16), kc_want.view(torch.int16))
