"""Host checks of the seeded input generator (structure only; no GPU)."""
import numpy as np
import torch

from paged_kv_gqa_pkv_amd import synth as S


def test_workloads_shapes_and_budget():
    w = S.workload("c1")
    assert [s.ctx for s in w.seqs] == [64] and w.num_blocks == 32 and w.max_blocks == 4
    w = S.workload("c2")
    assert len(w.seqs) == 8 and all(1 <= s.ctx <= 1024 for s in w.seqs)
    w = S.workload("c3")
    assert w.n_layers == 28 and w.shared_pages == 13 and all(s.ctx == 1024 for s in w.seqs)
    w = S.workload("c4a")
    assert (w.Hq, w.Hkv, len(w.seqs), w.max_ctx) == (32, 8, 64, 4096)
    w = S.workload("c4b")
    assert (len(w.seqs), w.max_ctx, w.num_blocks) == (13, 32768, 13 * 2048 + 32)
    offs, ts = [], []
    for s in range(6):
        w = S.workload("c5", s)
        p = w.seqs[w.prefill_seqs[0]]
        offs.append(p.pre_len); ts.append(p.new_len)
        assert p.new_len + len(w.decode_seqs) <= S.STEP_BUDGET
        assert all(256 <= w.seqs[i].ctx <= 2048 for i in w.decode_seqs)
    assert offs == [0, 512, 1024, 1536, 2048, 2560] and ts == [512] * 5 + [440]
    assert sum(ts) == S.PROMPT_LEN


def test_tables_are_disjoint_except_shared_prefix():
    w = S.workload("c3")
    t = S.make_tables(w)
    bt = t.block_tables.numpy()
    assert np.all(bt[:, :13] == bt[0, :13])
    own = bt[:, 13:64].ravel()
    assert len(set(own.tolist())) == own.size
    assert not set(own.tolist()) & set(bt[0, :13].tolist())
    assert bt.min() >= 0 and bt.max() < w.num_blocks
    assert (t.context_lens.numpy() == 1024).all() and int(t.cu_new[-1]) == 8


def test_canaries_mark_unwritten_slots_and_data_is_seeded():
    w = S.workload("c2")
    t = S.make_tables(w)
    d1 = S.make_layer(w, t, 0)
    d2 = S.make_layer(w, t, 0)
    assert torch.equal(d1.k_cache.view(torch.int16), d2.k_cache.view(torch.int16))
    kb = d1.k_cache.view(torch.int16).numpy()
    fill = S.page_fill_counts(w, t).numpy()
    used = set(t.block_tables.numpy().ravel().tolist()) - {-1}
    for page in range(w.num_blocks):
        if page not in used:
            assert fill[page] == 0 and np.all(kb[page] == S.BF16_CANARY_BITS)
        else:
            assert np.all(kb[page, fill[page]:] == S.BF16_CANARY_BITS)
            assert not np.any(kb[page, :fill[page]] == S.BF16_CANARY_BITS)
    assert kb.shape == (w.num_blocks, S.PAGE, w.Hkv, w.D)   # token-major pages
    assert d1.q_decode.shape == (8, 16, 128) and d1.k_new.shape == (8, 8, 128)
    d3 = S.make_layer(w, t, 1)
    assert not torch.equal(d1.q_decode, d3.q_decode)


def test_int8_pools_hold_head_major_scales_with_canaries():
    """int8 pools: codes token-major, scales [num_blocks, Hkv, 16] (a page's
    scales head-major) with the NaN canary on exactly the unwritten slots."""
    w = S.workload("c2")
    t = S.make_tables(w)
    d = S.make_layer_int8(w, t, 0)
    assert d.k_codes.shape == (w.num_blocks, S.PAGE, w.Hkv, w.D)
    assert d.k_scales.shape == (w.num_blocks, w.Hkv, S.PAGE) == d.v_scales.shape
    assert d.k_scales.is_contiguous() and d.v_scales.is_contiguous()
    fill = S.page_fill_counts(w, t).numpy()
    bits = d.k_scales.view(torch.int32).numpy()
    for page in range(w.num_blocks):
        dead = bits[page, :, fill[page]:]
        assert np.all(dead == np.int32(S.F32_CANARY_BITS))
        live = d.k_scales[page, :, :fill[page]].numpy()
        assert np.all((live >= S.SCALE_LO) & (live <= S.SCALE_HI))


def test_binding_rejects_slot_major_scales(monkeypatch):
    import pytest
    from paged_kv_gqa_pkv_amd import binding as bd
    monkeypatch.setattr(bd, "_need", lambda *a, **k: None)     # host tensors here
    codes = torch.zeros((4, S.PAGE, 2, 128), dtype=torch.int8)
    good = torch.zeros((4, 2, S.PAGE), dtype=torch.float32)
    bd._need_scales(good, good.clone(), codes)
    bad = torch.zeros((4, S.PAGE, 2), dtype=torch.float32)
    with pytest.raises(ValueError, match="head-major"):
        bd._need_scales(bad, bad.clone(), codes)
