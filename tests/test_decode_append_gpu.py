"""pkv_attn_decode_append, the decode call with the step's append fused in
([P1] model.py forward: read the cached prefix, take the step's own k/v,
attend, write the step's k/v into the cache), against the oracle: the pools
after the call are bit-identical to the oracle's append of the step's rows,
and the outputs are within the tolerance of the oracle's decode over the
appended pools.  Through the C ABI."""
import numpy as np
import pytest
import torch

from oracle import pkv_oracle as O
from paged_kv_gqa_pkv_amd import binding as bd
from paged_kv_gqa_pkv_amd import synth as S

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def check_close(got, want, what, rows=None):
    g = O.bf16_to_f64(u16(got))
    if rows is not None:
        g, want = g[rows], want[rows]
    assert np.all(np.isfinite(g)), f"{what}: non-finite outputs"
    err = np.abs(g - want)
    print(f"{what}: max abs {err.max():.3e} mean abs {err.mean():.3e}", flush=True)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (what, err.max(), err.mean())


def fused(w, t, d, max_ctx=None, bt=None):
    """One fused call on the device copies of d's pools; returns (out, k, v)."""
    bt = t.block_tables if bt is None else bt
    ctx = t.context_lens
    B = len(w.seqs)
    mc = int(ctx.max()) if max_ctx is None else max_ctx
    nbytes = bd.pkv_decode_workspace_bytes(B, w.Hq, w.Hkv, w.D, mc)
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda") if nbytes else None
    dk, dv = d.k_cache.cuda(), d.v_cache.cuda()
    q = d.q_decode.cuda()
    out = torch.full_like(q, float("nan"))
    bd.pkv_attn_decode_append(out, q, d.k_new.cuda(), d.v_new.cuda(), dk, dv, bt.cuda(),
                              ctx.cuda(), mc, w.D ** -0.5, workspace=ws)
    torch.cuda.synchronize()
    return out, dk, dv


def oracle(w, t, d, bt=None):
    bt = (t.block_tables if bt is None else bt).tolist()
    ctx = t.context_lens.tolist()
    slots = O.slot_ref(bt, t.cu_new.tolist(), ctx)
    kc, vc = O.append_ref(u16(d.k_cache), u16(d.v_cache), u16(d.k_new), u16(d.v_new), slots)
    return kc, vc, O.decode_ref(u16(d.q_decode), kc, vc, bt, ctx, O.default_scale(w.D))


def run(w):
    print(f"[fused] {w.name}: {len(w.seqs)} sequences, Hq {w.Hq}, Hkv {w.Hkv}", flush=True)
    t = S.make_tables(w)
    d = S.make_layer(w, t, 0)
    out, dk, dv = fused(w, t, d)
    kc, vc, want = oracle(w, t, d)
    assert np.array_equal(u16(dk), kc) and np.array_equal(u16(dv), vc), "pools after append"
    check_close(out, want, f"{w.name} fused")
    return t, d, out


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_fused_decode_configs(name):
    run(S.workload(name))


def _seqs(ctxs):
    return [S.SeqSpec(c - 1, 1, False) for c in ctxs]


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_fused_group_sizes_and_page_boundaries(G):
    """Contexts of 1 (only the new token), a new token opening a page (17,
    33) or closing one (16, 32), and ragged ones."""
    Hkv = 2
    ctxs = [1, 15, 16, 17, 31, 32, 33, 200, 515]
    w = S.custom_workload(f"fused_G{G}", _seqs(ctxs), Hq=Hkv * G, Hkv=Hkv, D=128,
                          num_blocks=110, base_seed=270 + G)
    run(w)


def test_fused_long_context_many_splits_and_split_boundaries():
    """Several splits: a new token on the first page of a split, on the last
    page of one, in the middle, and a single-page context beside them."""
    B, Hq, Hkv, mc = 5, 32, 8, 4608
    S_ = bd.pkv_decode_num_splits(B, Hq, Hkv, 128, mc)
    assert S_ > 2
    pps = -(-(-(-mc // 16)) // S_)                  # pages per split
    ctxs = [mc, 16 * pps + 1, 16 * pps, 16 * pps + 16 * pps // 2 + 7, 3]
    assert max(ctxs) == mc
    w = S.custom_workload("fused_splits", _seqs(ctxs), Hq=Hq, Hkv=Hkv, D=128, num_blocks=640,
                          base_seed=280)
    t, d, out = run(w)
    out2, _, _ = fused(w, t, d)                   # a repeat is bit-identical
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_fused_missing_page_and_context_past_the_plan():
    """Sequence 1's table has no page for its new token: nothing is written
    for it and its output is NaN, as append + decode give.  A call planned for
    fewer tokens than sequence 2 holds poisons that sequence only, and its row
    is still appended."""
    ctxs = [40, 33, 300, 90]
    w = S.custom_workload("fused_bad", _seqs(ctxs), Hq=16, Hkv=8, D=128, num_blocks=40,
                          base_seed=290)
    t = S.make_tables(w)
    d = S.make_layer(w, t, 0)
    bt = t.block_tables.clone()
    bt[1, 2] = -1                                   # position 32's page
    out, dk, dv = fused(w, t, d, bt=bt)
    kc, vc, want = oracle(w, t, d, bt=bt)
    assert np.array_equal(u16(dk), kc) and np.array_equal(u16(dv), vc)
    g = out.float().cpu()
    assert torch.isnan(g[1]).all()
    check_close(out, want, "fused beside a missing page", rows=[0, 2, 3])
    # planned for 128 tokens: sequence 2 (300) is past the plan
    out, dk, dv = fused(w, t, d, max_ctx=128)
    kc, vc, want = oracle(w, t, d)
    assert np.array_equal(u16(dk), kc) and np.array_equal(u16(dv), vc)
    g = out.float().cpu()
    assert torch.isnan(g[2]).all()
    check_close(out, want, "fused beside a context past the plan", rows=[0, 1, 3])
