"""The largest shapes the kernels accept, through the C ABI, against the
oracle on sampled outputs (each recomputed one by one over its full key
range): chunked prefill at the longest supported context (131 072 keys:
64 key tiles of 64 keys in each of 32 splits), in bf16 and int8 pages, and
decode at the same context."""
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
MAX_CTX = 131072


def u16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def workload(kind):
    if kind == "prefill":
        seqs = [S.SeqSpec(MAX_CTX - 64, 64, True)]
    else:
        seqs = [S.SeqSpec(MAX_CTX - 1, 1, False), S.SeqSpec(0, 1, False)]
    return S.custom_workload(f"max_{kind}", seqs, Hq=32, Hkv=8, D=128,
                             num_blocks=MAX_CTX // 16 + 8, base_seed=1300)


def check(got, want_rows, what):
    err = np.concatenate([np.abs(g - w) for g, w in zip(got, want_rows)])
    print(f"{what}: max abs {err.max():.3e} mean abs {err.mean():.3e}", flush=True)
    assert all(np.all(np.isfinite(g)) for g in got)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS


def test_prefill_at_the_longest_context_bf16():
    w = workload("prefill")
    t = S.make_tables(w)
    d = S.make_layer(w, t, 0, device="cuda")
    k0, v0 = u16(d.k_cache), u16(d.v_cache)
    plan = ST.plan_step(w, t)
    assert bd.pkv_prefill_workspace_bytes(1, 64, 32, 8, 128, MAX_CTX) > 0
    out = torch.empty_like(d.q_prefill)
    ST.slot_mapping(plan)
    ST.layer(plan, d.k_cache, d.v_cache, d.k_new, d.v_new, q_prefill=d.q_prefill,
             out_prefill=out)
    torch.cuda.synchronize()
    bt, ctx = t.block_tables.tolist(), t.context_lens.tolist()
    slots = O.slot_ref(bt, t.cu_new.tolist(), ctx)
    kc, vc = O.append_ref(k0, v0, u16(d.k_new), u16(d.v_new), slots)
    K = O.bf16_to_f64(O.gather_ref(kc, bt[0], MAX_CTX))
    V = O.bf16_to_f64(O.gather_ref(vc, bt[0], MAX_CTX))
    q, got = u16(d.q_prefill), O.bf16_to_f64(u16(out))
    rows, want = [], []
    for tq, h in ((0, 0), (21, 13), (63, 31)):
        g = O.kv_head_of(h, 32, 8)
        npos = MAX_CTX - 64 + tq + 1
        want.append(O.attend_one(O.bf16_to_f64(q[tq, h]), K[:npos, g], V[:npos, g],
                                 O.default_scale(128)))
        rows.append(got[tq, h])
    check(rows, want, "prefill 131072 keys")


def test_prefill_at_the_longest_context_int8():
    w = workload("prefill")
    t = S.make_tables(w)
    d = S.make_layer_int8(w, t, 0, device="cuda")
    # the oracle starts from the pre-append pools and appends on its own
    kc0, vc0 = d.k_codes.cpu().numpy(), d.v_codes.cpu().numpy()
    ks0, vs0 = d.k_scales.cpu().numpy(), d.v_scales.cpu().numpy()
    plan = ST.plan_step(w, t)
    ST.slot_mapping(plan)
    bd.pkv_append_int8(d.k_new, d.v_new, plan.slot_mapping, d.k_codes, d.v_codes, d.k_scales,
                       d.v_scales)
    out = torch.empty_like(d.q_prefill)
    bd.pkv_attn_prefill_chunk_int8(out, d.q_prefill, plan.cu_q, d.k_codes, d.v_codes,
                                   d.k_scales, d.v_scales, plan.bt_prefill, plan.ctx_prefill,
                                   plan.max_q_len, plan.max_ctx_prefill, plan.scale,
                                   workspace=plan.prefill_workspace)
    torch.cuda.synchronize()
    bt = t.block_tables.tolist()
    slots = O.slot_ref(bt, t.cu_new.tolist(), t.context_lens.tolist())
    kc, vc, ks, vs = Q.append_int8_ref(kc0, vc0, ks0, vs0, u16(d.k_new), u16(d.v_new), slots)
    K = Q.gather_int8_ref(kc, ks, bt[0], MAX_CTX).astype(np.float64)
    V = Q.gather_int8_ref(vc, vs, bt[0], MAX_CTX).astype(np.float64)
    q, got = u16(d.q_prefill), O.bf16_to_f64(u16(out))
    rows, want = [], []
    for tq, h in ((0, 5), (40, 26), (63, 31)):
        g = O.kv_head_of(h, 32, 8)
        npos = MAX_CTX - 64 + tq + 1
        want.append(O.attend_one(O.bf16_to_f64(q[tq, h]), K[:npos, g], V[:npos, g],
                                 O.default_scale(128)))
        rows.append(got[tq, h])
    check(rows, want, "int8 prefill 131072 keys")


def test_decode_at_the_longest_context():
    w = workload("decode")
    t = S.make_tables(w)
    d = S.make_layer(w, t, 0, device="cuda")
    k0, v0 = u16(d.k_cache), u16(d.v_cache)
    plan = ST.plan_step(w, t)
    assert bd.pkv_decode_num_splits(2, 32, 8, 128, MAX_CTX) > 1
    out = torch.empty_like(d.q_decode)
    ST.slot_mapping(plan)
    ST.layer(plan, d.k_cache, d.v_cache, d.k_new, d.v_new, d.q_decode, out)
    torch.cuda.synchronize()
    bt, ctx = t.block_tables.tolist(), t.context_lens.tolist()
    slots = O.slot_ref(bt, t.cu_new.tolist(), ctx)
    kc, vc = O.append_ref(k0, v0, u16(d.k_new), u16(d.v_new), slots)
    q, got = u16(d.q_decode), O.bf16_to_f64(u16(out))
    rows, want = [], []
    for b in (0, 1):
        K = O.bf16_to_f64(O.gather_ref(kc, bt[b], ctx[b]))
        V = O.bf16_to_f64(O.gather_ref(vc, bt[b], ctx[b]))
        for h in (0, 19, 31):
            g = O.kv_head_of(h, 32, 8)
            want.append(O.attend_one(O.bf16_to_f64(q[b, h]), K[:, g], V[:, g],
                                     O.default_scale(128)))
            rows.append(got[b, h])
    check(rows, want, "decode 131072 and 1 tokens")
