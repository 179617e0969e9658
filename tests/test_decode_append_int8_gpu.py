"""pkv_attn_decode_append_int8, decode over int8 pages with the step's
append fused in ([P1] model.py forward: read the cached prefix, take the
step's own k/v, attend, write it into the cache; [P2] KV8Cache.write for the
quantisation), against the oracle: the code and scale pools after the call
are bit-identical to the oracle's int8 append of the step's rows, and the
outputs are within the tolerance of the oracle's int8 decode over the
appended pools.  Through the C ABI."""
import numpy as np
import pytest
import torch

from oracle import pkv_int8_oracle as Q
from oracle import pkv_oracle as O
from paged_kv_gqa_pkv_amd import binding as bd
from paged_kv_gqa_pkv_amd import synth as S

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy()


def check_close(got, want, what, rows=None):
    g = O.bf16_to_f64(u16(got))
    if rows is not None:
        g, want = g[rows], want[rows]
    assert np.all(np.isfinite(g)), f"{what}: non-finite outputs"
    err = np.abs(g - want)
    print(f"{what}: max abs {err.max():.3e} mean abs {err.mean():.3e}", flush=True)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (what, err.max(), err.mean())


def _ws(w, t, mc):
    n = bd.pkv_decode_workspace_bytes(len(w.seqs), w.Hq, w.Hkv, w.D, mc)
    return torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda") if n else None


def fused(w, t, d, max_ctx=None, bt=None):
    """One fused call on device copies of d's pools; returns (out, kc, vc, ks, vs)."""
    bt = t.block_tables if bt is None else bt
    ctx = t.context_lens
    mc = int(ctx.max()) if max_ctx is None else max_ctx
    kc, vc = d.k_codes.cuda(), d.v_codes.cuda()
    ks, vs = d.k_scales.cuda(), d.v_scales.cuda()
    q = d.q_decode.cuda()
    out = torch.full_like(q, float("nan"))
    bd.pkv_attn_decode_append_int8(out, q, d.k_new.cuda(), d.v_new.cuda(), kc, vc, ks, vs,
                                   bt.cuda(), ctx.cuda(), mc, w.D ** -0.5,
                                   workspace=_ws(w, t, mc))
    torch.cuda.synchronize()
    return out, kc, vc, ks, vs


def oracle(w, t, d, bt=None):
    bt = (t.block_tables if bt is None else bt).tolist()
    ctx = t.context_lens.tolist()
    slots = O.slot_ref(bt, t.cu_new.tolist(), ctx)
    kc, vc, ks, vs = Q.append_int8_ref(host(d.k_codes), host(d.v_codes), host(d.k_scales),
                                       host(d.v_scales), u16(d.k_new), u16(d.v_new), slots)
    want = Q.decode_int8_ref(u16(d.q_decode), kc, ks, vc, vs, bt, ctx, O.default_scale(w.D))
    return kc, vc, ks, vs, want


def check_pools(got, want):
    gkc, gvc, gks, gvs = (host(x) for x in got)
    kc, vc, ks, vs = want
    assert np.array_equal(gkc, kc) and np.array_equal(gvc, vc), "codes after the append"
    assert np.array_equal(gks.view(np.uint32), ks.view(np.uint32)), "K scales after the append"
    assert np.array_equal(gvs.view(np.uint32), vs.view(np.uint32)), "V scales after the append"


def run(w):
    print(f"[fused int8] {w.name}: {len(w.seqs)} sequences, Hq {w.Hq}, Hkv {w.Hkv}", flush=True)
    t = S.make_tables(w)
    d = S.make_layer_int8(w, t, 0)
    out, *pools = fused(w, t, d)
    *want_pools, want = oracle(w, t, d)
    check_pools(pools, want_pools)
    check_close(out, want, f"{w.name} fused int8")
    return t, d, out


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_fused_int8_decode_configs(name):
    run(S.workload(name))


def _seqs(ctxs):
    return [S.SeqSpec(c - 1, 1, False) for c in ctxs]


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_fused_int8_group_sizes_and_page_boundaries(G):
    """Contexts of 1 (only the new token), a new token opening a page (17,
    33) or closing one (16, 32), and ragged ones."""
    Hkv = 2
    ctxs = [1, 15, 16, 17, 31, 32, 33, 200, 515]
    w = S.custom_workload(f"fused8_G{G}", _seqs(ctxs), Hq=Hkv * G, Hkv=Hkv, D=128,
                          num_blocks=110, base_seed=470 + G)
    run(w)


def test_fused_int8_long_context_many_splits_and_repeat():
    """Several splits, the new token on the first page of a split, on the last
    page of one, in the middle, beside a 3-token context; a repeat of the call
    on the same inputs is bit-identical."""
    B, Hq, Hkv, mc = 5, 32, 8, 4608
    S_ = bd.pkv_decode_num_splits(B, Hq, Hkv, 128, mc)
    assert S_ > 2
    pps = -(-(-(-mc // 16)) // S_)                  # pages per split
    ctxs = [mc, 16 * pps + 1, 16 * pps, 16 * pps + 16 * pps // 2 + 7, 3]
    w = S.custom_workload("fused8_splits", _seqs(ctxs), Hq=Hq, Hkv=Hkv, D=128, num_blocks=640,
                          base_seed=480)
    t, d, out = run(w)
    out2, *_ = fused(w, t, d)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_fused_int8_matches_append_then_decode():
    """The same step as pkv_append_int8 then pkv_attn_decode_int8: the same
    pools bit for bit, and outputs equal up to the order of float32 sums (the
    new token is reduced as a page of its own), on c4a-shaped heads."""
    ctxs = [1, 16, 17, 100, 257, 1024, 2048, 4096]
    w = S.custom_workload("fused8_vs_two", _seqs(ctxs), Hq=32, Hkv=8, D=128, num_blocks=800,
                          base_seed=490)
    t = S.make_tables(w)
    d = S.make_layer_int8(w, t, 0)
    out, *pools = fused(w, t, d)
    slots = torch.tensor(O.slot_ref(t.block_tables.tolist(), t.cu_new.tolist(),
                                    t.context_lens.tolist()), dtype=torch.int32, device="cuda")
    kc, vc = d.k_codes.cuda(), d.v_codes.cuda()
    ks, vs = d.k_scales.cuda(), d.v_scales.cuda()
    bd.pkv_append_int8(d.k_new.cuda(), d.v_new.cuda(), slots, kc, vc, ks, vs)
    out2 = torch.full_like(out, float("nan"))
    mc = int(t.context_lens.max())
    bd.pkv_attn_decode_int8(out2, d.q_decode.cuda(), kc, vc, ks, vs, t.block_tables.cuda(),
                            t.context_lens.cuda(), mc, w.D ** -0.5, workspace=_ws(w, t, mc))
    torch.cuda.synchronize()
    check_pools(pools, (host(kc), host(vc), host(ks), host(vs)))
    diff = (out.float() - out2.float()).abs()
    print(f"fused vs append + decode: max abs {diff.max().item():.3e}", flush=True)
    assert torch.isfinite(out).all() and diff.max().item() <= 1e-2
    *_, want = oracle(w, t, d)
    check_close(out, want, "fused int8 (c4a heads)")


def test_fused_int8_missing_page_and_context_past_the_plan():
    """Sequence 1's table has no page for its new token: nothing is written
    for it and its output is NaN, as append + decode give.  A call planned for
    fewer tokens than sequence 2 holds poisons that sequence only, and its row
    is still appended."""
    ctxs = [40, 33, 300, 90]
    w = S.custom_workload("fused8_bad", _seqs(ctxs), Hq=16, Hkv=8, D=128, num_blocks=40,
                          base_seed=495)
    t = S.make_tables(w)
    d = S.make_layer_int8(w, t, 0)
    bt = t.block_tables.clone()
    bt[1, 2] = -1                                   # position 32's page
    out, *pools = fused(w, t, d, bt=bt)
    *want_pools, want = oracle(w, t, d, bt=bt)
    check_pools(pools, want_pools)
    assert torch.isnan(out[1].float()).all()
    check_close(out, want, "fused int8 beside a missing page", rows=[0, 2, 3])
    out, *pools = fused(w, t, d, max_ctx=128)
    *want_pools, want = oracle(w, t, d)
    check_pools(pools, want_pools)
    assert torch.isnan(out[2].float()).all()
    check_close(out, want, "fused int8 beside a context past the plan", rows=[0, 1, 3])
