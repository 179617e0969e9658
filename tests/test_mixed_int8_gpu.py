"""pkv_attn_prefill_decode_int8, a mixed step's attention over int8 pages in
one call ([P1] "Why chunked prefill"; [P2] KV8Cache.read for the pages),
through the C ABI.  After the int8 append of the step's rows, its outputs
must be bit-identical to pkv_attn_prefill_chunk_int8 followed by
pkv_attn_decode_int8 on the same pools (the one-grid launch runs the same
per-workgroup arithmetic), and within the tolerance of the oracle's int8
prefill and decode: c5 steps, group sizes 1, 2, 4 (one launch) and 8 (two
launches) with key splits on both sides, and a HIP graph replayed several
times."""
import numpy as np
import pytest
import torch

from oracle import pkv_int8_oracle as Q
from oracle import pkv_oracle as O
from paged_kv_gqa_pkv_amd import binding as bd
from paged_kv_gqa_pkv_amd import step as ST
from paged_kv_gqa_pkv_amd import synth as S

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


def u16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def host(t):
    return t.detach().contiguous().cpu().numpy()


def bits_equal(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def setup(w):
    """Layer 0 of w over int8 pools on the GPU, the step's rows appended."""
    t = S.make_tables(w)
    d = S.make_layer_int8(w, t, 0)
    host_pools = tuple(host(x) for x in (d.k_codes, d.v_codes, d.k_scales, d.v_scales))
    dev = {n: getattr(d, n).cuda() for n in ("k_codes", "v_codes", "k_scales", "v_scales",
                                             "k_new", "v_new", "q_decode", "q_prefill")}
    plan = ST.plan_step(w, t, fused=False)
    assert plan.mixed and not plan.fused
    ST.slot_mapping(plan)
    bd.pkv_append_int8(dev["k_new"], dev["v_new"], plan.slot_mapping, dev["k_codes"],
                       dev["v_codes"], dev["k_scales"], dev["v_scales"])
    return t, d, dev, plan, host_pools


def mixed_call(dev, plan, stream=None):
    op = torch.full_like(dev["q_prefill"], float("nan"))
    od = torch.full_like(dev["q_decode"], float("nan"))
    bd.pkv_attn_prefill_decode_int8(op, dev["q_prefill"], plan.cu_q, plan.bt_prefill,
                                    plan.ctx_prefill, plan.max_q_len, plan.max_ctx_prefill, od,
                                    dev["q_decode"], plan.bt_decode, plan.ctx_decode,
                                    plan.max_ctx_decode, dev["k_codes"], dev["v_codes"],
                                    dev["k_scales"], dev["v_scales"], plan.scale,
                                    prefill_workspace=plan.prefill_workspace,
                                    decode_workspace=plan.workspace, stream=stream)
    return op, od


def separate_calls(dev, plan):
    op = torch.full_like(dev["q_prefill"], float("nan"))
    od = torch.full_like(dev["q_decode"], float("nan"))
    bd.pkv_attn_prefill_chunk_int8(op, dev["q_prefill"], plan.cu_q, dev["k_codes"],
                                   dev["v_codes"], dev["k_scales"], dev["v_scales"],
                                   plan.bt_prefill, plan.ctx_prefill, plan.max_q_len,
                                   plan.max_ctx_prefill, plan.scale,
                                   workspace=plan.prefill_workspace)
    bd.pkv_attn_decode_int8(od, dev["q_decode"], dev["k_codes"], dev["v_codes"],
                            dev["k_scales"], dev["v_scales"], plan.bt_decode, plan.ctx_decode,
                            plan.max_ctx_decode, plan.scale, workspace=plan.workspace)
    return op, od


def check_oracle(w, t, d, host_pools, op, od, what):
    bt, ctx = t.block_tables.tolist(), t.context_lens.tolist()
    slots = O.slot_ref(bt, t.cu_new.tolist(), ctx)
    kc, vc, ks, vs = Q.append_int8_ref(*host_pools, u16(d.k_new), u16(d.v_new), slots)
    npre = len(w.prefill_seqs)
    scale = O.default_scale(w.D)
    want_p = Q.prefill_int8_ref(u16(d.q_prefill), S.prefill_cu(w).tolist(), kc, ks, vc, vs,
                                bt[:npre], ctx[:npre], scale)
    want_d = Q.decode_int8_ref(u16(d.q_decode), kc, ks, vc, vs, bt[npre:], ctx[npre:], scale)
    for got, want, half in ((op, want_p, "prefill"), (od, want_d, "decode")):
        g = O.bf16_to_f64(u16(got))
        assert np.all(np.isfinite(g)), f"{what} {half}: non-finite outputs"
        err = np.abs(g - want)
        print(f"{what} {half}: max abs {err.max():.3e} mean abs {err.mean():.3e}", flush=True)
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS


def run(w, oracle=True):
    print(f"[mixed int8] {w.name}: {w.description}", flush=True)
    t, d, dev, plan, host_pools = setup(w)
    op, od = mixed_call(dev, plan)
    sp, sd = separate_calls(dev, plan)
    torch.cuda.synchronize()
    assert bits_equal(op, sp), "prefill half differs from pkv_attn_prefill_chunk_int8"
    assert bits_equal(od, sd), "decode half differs from pkv_attn_decode_int8"
    if oracle:
        check_oracle(w, t, d, host_pools, op, od, w.name)
    return dev, plan, op, od


@pytest.mark.parametrize("chunk_step", [0, 2, 5])
def test_c5_steps_against_the_oracle(chunk_step):
    run(S.workload("c5", chunk_step))


@pytest.mark.parametrize("chunk_step", [1, 3, 4])
def test_c5_steps_match_the_two_calls(chunk_step):
    run(S.workload("c5", chunk_step), oracle=False)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_group_sizes_ragged_and_splits(G):
    """Two chunk sequences (one long enough for key splits) beside decode
    sequences of ragged lengths, one long enough for decode splits."""
    Hkv = 2
    seqs = [S.SeqSpec(3000, 200, True), S.SeqSpec(40, 33, True),
            S.SeqSpec(0, 1, False), S.SeqSpec(16, 1, False), S.SeqSpec(300, 1, False),
            S.SeqSpec(5000, 1, False)]
    w = S.custom_workload(f"mixed8_G{G}", seqs, Hq=Hkv * G, Hkv=Hkv, D=128, num_blocks=640,
                          base_seed=720 + G)
    _, plan, _, _ = run(w)
    assert plan.prefill_workspace is not None and plan.workspace is not None


def test_graph_replays_are_bit_identical():
    w = S.workload("c5", 3)
    _, _, dev, plan, _ = setup(w)
    want_p, want_d = mixed_call(dev, plan)
    torch.cuda.synchronize()
    op = torch.empty_like(want_p)
    od = torch.empty_like(want_d)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            p_, d_ = mixed_call(dev, plan, stream=cap)
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
        e_p, e_d = mixed_call(dev, plan)              # eager work between replays
        torch.cuda.synchronize()
        assert bits_equal(e_p, want_p) and bits_equal(e_d, want_d), rep


def test_invalid_pages_poison_their_sequences_in_both_forms():
    """A prefill sequence whose table holds an invalid page id and a decode
    sequence whose table holds one: their outputs are NaN, the others'
    finite, and the one-launch form gives the two calls' outputs bit for
    bit (the poisoned rows included)."""
    w = S.workload("c5", 2)
    t, d, dev, plan, host_pools = setup(w)
    npre = len(w.prefill_seqs)
    plan.block_tables[0, 3] = -1                      # a page of the chunk's prefix
    plan.block_tables[npre + 1, 0] = 1 << 30          # past the pool
    op, od = mixed_call(dev, plan)
    sp, sd = separate_calls(dev, plan)
    torch.cuda.synchronize()
    assert bits_equal(op, sp) and bits_equal(od, sd)
    assert torch.isnan(op.float()).all(), "the chunk's rows are poisoned"
    assert torch.isnan(od[1].float()).all()
    keep = [i for i in range(od.shape[0]) if i != 1]
    assert torch.isfinite(od[keep].float()).all()
