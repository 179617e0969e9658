"""The fused q/k RMSNorm + RoPE + append kernel on the GPU, through the C ABI,
against the oracle that follows [P1] model.py (rms_norm, _rope_tables,
apply_rope, forward).

Slots and V rows must be bit-exact.  q and the appended k rows may differ
from the oracle only through the order of the float32 sum of squares, so
they are compared in bf16 ulps at the larger of the oracle's value and 0.5
(the scale of normalised values): at most 2 ulp, and differing in at most
1 % of the values.  Attention over the resulting q and pools is then
checked against the oracle's attention over its own q and pools.
"""
import numpy as np
import pytest
import torch

from oracle import pkv_oracle as O
from oracle import pkv_rope_oracle as R
from paged_kv_gqa_pkv_amd import binding as bd
from paged_kv_gqa_pkv_amd import step as ST
from paged_kv_gqa_pkv_amd import synth as S

pytestmark = pytest.mark.gpu

THETA, EPS, MAX_POS = 1_000_000.0, 1e-6, 4096


def u16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def ulps(got_bits, want_f32):
    """|got - want| in bf16 ulps at max(|want|, 0.5): the rotated values are
    sums of two products of normalised (order 1) values, so near a
    cancellation a one-ulp change of an input is measured against the inputs'
    scale, not the small result's (NaN never allowed)."""
    g = R.bits_to_f32(got_bits).astype(np.float64)
    w = want_f32.astype(np.float64)
    assert np.all(np.isfinite(g)), "non-finite output"
    e = np.floor(np.log2(np.maximum(np.abs(w), 0.5)))
    return np.abs(g - w) / 2.0 ** (e - 7)


def tables():
    cos, sin = R.rope_tables_ref(128, MAX_POS, THETA, bf16=True)
    return (torch.from_numpy(R.bf16_bits(cos).view(np.int16)).view(torch.bfloat16),
            torch.from_numpy(R.bf16_bits(sin).view(np.int16)).view(torch.bfloat16))


def run_case(w, seed):
    t = S.make_tables(w)
    d = S.make_layer(w, t, 0)
    T = int(t.cu_new[-1])
    gen = torch.Generator().manual_seed(seed)
    q_in = (torch.randn((T, w.Hq, w.D), generator=gen) * 2).to(torch.bfloat16)
    k_in = (torch.randn((T, w.Hkv, w.D), generator=gen) * 3).to(torch.bfloat16)
    v_in = d.v_new
    qw = (1 + 0.2 * torch.randn(w.D, generator=gen)).to(torch.bfloat16)
    kw = (1 + 0.2 * torch.randn(w.D, generator=gen)).to(torch.bfloat16)
    cos_t, sin_t = tables()
    kc0 = u16(d.k_cache)
    vc0 = u16(d.v_cache)
    dk, dv = d.k_cache.cuda(), d.v_cache.cuda()
    q_out = torch.empty((T, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    sm = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    bd.pkv_qk_norm_rope_append(q_out, q_in.cuda(), k_in.cuda(), v_in.cuda(), qw.cuda(), kw.cuda(),
                               cos_t.cuda(), sin_t.cuda(), t.block_tables.cuda(), t.cu_new.cuda(),
                               t.context_lens.cuda(), dk, dv, EPS, slot_mapping=sm)
    torch.cuda.synchronize()
    bt, ctx, cu = t.block_tables.tolist(), t.context_lens.tolist(), t.cu_new.tolist()
    slots = O.slot_ref(bt, cu, ctx)
    assert sm.cpu().tolist() == slots, "slot mapping differs"
    pos = R.positions_ref(cu, ctx)
    f32 = lambda x: R.bits_to_f32(u16(x))
    q_ref, k_ref = R.qk_norm_rope_ref(f32(q_in), f32(k_in), f32(qw), f32(kw),
                                      R.bits_to_f32(u16(cos_t)), R.bits_to_f32(u16(sin_t)),
                                      pos, EPS, bf16=True)
    uq = ulps(u16(q_out), q_ref)
    kc_ref, vc_ref = O.append_ref(kc0, vc0, R.bf16_bits(k_ref), u16(v_in), slots)
    got_k = u16(dk)
    assert np.array_equal(u16(dv), vc_ref), "V rows differ"
    sl = np.array(slots)
    uk = ulps(got_k[sl // 16, sl % 16], R.bits_to_f32(kc_ref[sl // 16, sl % 16]))
    untouched = np.ones(got_k.shape[:2], bool)
    untouched[sl // 16, sl % 16] = False
    assert np.array_equal(got_k[untouched], kc0[untouched]), "K outside the new slots changed"
    for name, u in (("q", uq), ("k", uk)):
        print(f"{w.name} {name}: max {u.max():.2f} ulp, {100 * np.mean(u > 0):.3f} % differ",
              flush=True)
        assert u.max() <= 2 and np.mean(u > 0) <= 0.01, (name, u.max(), np.mean(u > 0))
    return w, t, q_out, dk, dv, R.bf16_bits(q_ref), kc_ref, vc_ref


@pytest.mark.parametrize("chunk_step", [0, 5])
def test_fused_norm_rope_append_mixed_step(chunk_step):
    w, t, q_out, dk, dv, q_ref, kc_ref, vc_ref = run_case(S.workload("c5", chunk_step),
                                                          900 + chunk_step)
    # attention over the fused path's q and pools, against the oracle's
    # attention over the oracle's own rotated q and appended pools
    plan = ST.plan_step(w, t)
    npre = len(w.prefill_seqs)
    Tp = sum(w.seqs[i].new_len for i in w.prefill_seqs)
    qp, qd = q_out[:Tp].contiguous(), q_out[Tp:].contiguous()
    op, od = torch.empty_like(qp), torch.empty_like(qd)
    bd.pkv_attn_prefill_chunk(op, qp, plan.cu_q, dk, dv, plan.bt_prefill, plan.ctx_prefill,
                              plan.max_q_len, plan.max_ctx_prefill, plan.scale,
                              workspace=plan.prefill_workspace)
    bd.pkv_attn_decode(od, qd, dk, dv, plan.bt_decode, plan.ctx_decode, plan.max_ctx_decode,
                       plan.scale, workspace=plan.workspace)
    torch.cuda.synchronize()
    bt, ctx = t.block_tables.tolist(), t.context_lens.tolist()
    want_p = O.prefill_ref(q_ref[:Tp], S.prefill_cu(w).tolist(), kc_ref, vc_ref, bt[:npre],
                           ctx[:npre], plan.scale)
    want_d = O.decode_ref(q_ref[Tp:], kc_ref, vc_ref, bt[npre:], ctx[npre:], plan.scale)
    for got, want, what in ((op, want_p, "prefill"), (od, want_d, "decode")):
        err = np.abs(O.bf16_to_f64(u16(got)) - want)
        print(f"fused step {what}: max abs {err.max():.3e} mean abs {err.mean():.3e}", flush=True)
        assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_fused_decode_batch_and_missing_page():
    """A decode batch; one sequence's table lacks the page of its new token:
    its slot is -1, no K/V is written for it, its q is still produced."""
    ctxs = [1, 17, 300, 1024, 2049]
    seqs = [S.SeqSpec(c - 1, 1, False) for c in ctxs]
    w = S.custom_workload("fused_decode", seqs, Hq=32, Hkv=8, D=128, num_blocks=300,
                          base_seed=910)
    run_case(w, 911)
    t = S.make_tables(w)
    bt = t.block_tables.clone()
    bt[2, (300 - 1) // 16] = -1
    d = S.make_layer(w, t, 0)
    T = len(ctxs)
    cos_t, sin_t = tables()
    q_in = S.randn_bf16((T, 32, 128), 912)
    q_out = torch.empty((T, 32, 128), dtype=torch.bfloat16, device="cuda")
    dk, dv = d.k_cache.cuda(), d.v_cache.cuda()
    before = u16(dk)
    sm = torch.empty(T, dtype=torch.int32, device="cuda")
    ones = torch.ones(128, dtype=torch.bfloat16)
    bd.pkv_qk_norm_rope_append(q_out, q_in.cuda(), d.k_new.cuda(), d.v_new.cuda(), ones.cuda(),
                               ones.cuda(), cos_t.cuda(), sin_t.cuda(), bt.cuda(), t.cu_new.cuda(),
                               t.context_lens.cuda(), dk, dv, EPS, slot_mapping=sm)
    torch.cuda.synchronize()
    assert sm.cpu().tolist()[2] == -1
    assert torch.isfinite(q_out.float()).all()
    changed = np.any(u16(dk) != before, axis=(2, 3))      # [block, slot] rows that changed
    assert changed.sum() == T - 1


def test_fused_positions_beyond_the_tables():
    """Tables of 64 positions; tokens at positions 63 and 64, 99: the first is
    rotated as usual, the others give NaN q rows and write neither K nor V."""
    ctxs = [10, 64, 65, 100]
    seqs = [S.SeqSpec(c - 1, 1, False) for c in ctxs]
    w = S.custom_workload("fused_beyond", seqs, Hq=16, Hkv=8, D=128, num_blocks=40,
                          base_seed=920)
    t = S.make_tables(w)
    d = S.make_layer(w, t, 0)
    T = len(ctxs)
    cos_full, sin_full = tables()
    cos_t, sin_t = cos_full[:64].contiguous(), sin_full[:64].contiguous()
    q_in = S.randn_bf16((T, 16, 128), 921)
    q_out = torch.empty((T, 16, 128), dtype=torch.bfloat16, device="cuda")
    dk, dv = d.k_cache.cuda(), d.v_cache.cuda()
    k0, v0 = u16(dk), u16(dv)
    sm = torch.empty(T, dtype=torch.int32, device="cuda")
    ones = torch.ones(128, dtype=torch.bfloat16)
    bd.pkv_qk_norm_rope_append(q_out, q_in.cuda(), d.k_new.cuda(), d.v_new.cuda(), ones.cuda(),
                               ones.cuda(), cos_t.cuda(), sin_t.cuda(), t.block_tables.cuda(),
                               t.cu_new.cuda(), t.context_lens.cuda(), dk, dv, EPS,
                               slot_mapping=sm)
    torch.cuda.synchronize()
    slots = O.slot_ref(t.block_tables.tolist(), t.cu_new.tolist(), t.context_lens.tolist())
    assert sm.cpu().tolist() == slots
    q = q_out.float().cpu()
    assert torch.isfinite(q[:2]).all() and torch.isnan(q[2:]).all()
    pos = R.positions_ref(t.cu_new.tolist(), t.context_lens.tolist())
    f32 = lambda x: R.bits_to_f32(u16(x))
    q_ref, _ = R.qk_norm_rope_ref(f32(q_in[:2]), f32(d.k_new[:2]), f32(ones), f32(ones),
                                  R.bits_to_f32(u16(cos_t)), R.bits_to_f32(u16(sin_t)), pos[:2],
                                  EPS, bf16=True)
    assert ulps(u16(q_out[:2]), q_ref).max() <= 2
    gk, gv = u16(dk), u16(dv)
    for i, s_ in enumerate(slots):                     # [block][slot] rows of all heads
        blk, off = divmod(s_, 16)
        changed_k = not np.array_equal(gk[blk, off], k0[blk, off])
        changed_v = not np.array_equal(gv[blk, off], v0[blk, off])
        assert changed_k == (i < 2) and changed_v == (i < 2), (i, changed_k, changed_v)
