"""Host logic of the mixed step (no device): the scheduler's limits that the
step planner enforces before anything is launched (Module 12 page, "Why
chunked prefill": chunks of at most 512 tokens, at most 2048 token slots per
step, one new token per decoding sequence), and the index data it hands to
the kernels."""
import pytest
import torch

from paged_kv_gqa_pkv_amd import binding as bd
from paged_kv_gqa_pkv_amd import step as ST
from paged_kv_gqa_pkv_amd import synth as S


@pytest.fixture(scope="module")
def lib():
    return bd.load()


def _plan(seqs, Hq=16, Hkv=8, D=128):
    need = sum(S.n_pages(s.ctx) for s in seqs)
    w = S.custom_workload("plan", seqs, Hq, Hkv, D, num_blocks=need + 8, base_seed=90)
    return w, ST.plan_step(w, S.make_tables(w), device="cpu")


def test_c5_steps_plan_the_chunk_and_the_decode_batch(lib):
    for s in range(6):
        w = S.workload("c5", s)
        t = S.make_tables(w)
        p = ST.plan_step(w, t, device="cpu")
        o, T = 512 * s, min(512, 3000 - 512 * s)
        assert (p.n_prefill, p.n_decode, p.max_q_len, p.max_ctx_prefill) == (1, 7, T, o + T)
        assert p.cu_q.tolist() == [0, T]
        assert p.mixed and p.fused and p.needs_slots   # one append + attention call per layer
        assert p.slot_mapping.numel() == T + 7
        assert p.ctx_prefill.tolist() == [o + T]
        assert p.bt_prefill.shape[0] == 1 and p.bt_decode.shape[0] == 7
        assert p.max_ctx_decode == max(w.seqs[i].ctx for i in w.decode_seqs)
        assert p.scale == 128 ** -0.5
        nb = bd.pkv_prefill_workspace_bytes(1, T, 16, 8, 128, o + T)
        assert (p.prefill_workspace is None) == (nb == 0)
        if nb:
            assert p.prefill_workspace.numel() == nb
        nd = bd.pkv_decode_workspace_bytes(7, 16, 8, 128, p.max_ctx_decode)
        assert (p.workspace is None) == (nd == 0)


def test_decode_only_steps(lib):
    p = ST.plan_step(S.workload("c4a"), S.make_tables(S.workload("c4a")), device="cpu")
    assert (p.n_prefill, p.n_decode, p.cu_q, p.prefill_workspace) == (0, 64, None, None)
    assert p.fused                              # one append + decode call per layer
    assert p.workspace is None                  # one pass: 64 x 8 (sequence, KV head) units
    p = ST.plan_step(S.workload("c4b"), S.make_tables(S.workload("c4b")), device="cpu")
    assert p.workspace is not None              # split context
    assert p.workspace.numel() == bd.pkv_decode_workspace_bytes(13, 32, 8, 128, 32768)
    p = ST.plan_step(S.workload("c3"), S.make_tables(S.workload("c3")), device="cpu",
                     fused=False)
    assert not p.fused and p.needs_slots


def test_fused_and_mixed_flags(lib):
    w = S.workload("c5", 2)
    t = S.make_tables(w)
    p = ST.plan_step(w, t, device="cpu", fused=False)
    assert p.mixed and not p.fused and p.needs_slots       # append, then one attention call
    p = ST.plan_step(w, t, device="cpu", mixed=False)
    assert not p.mixed and not p.fused and p.needs_slots   # append, chunk call, decode call
    w = S.workload("c4a")
    p = ST.plan_step(w, S.make_tables(w), device="cpu")
    assert p.fused and not p.mixed and not p.needs_slots


def test_step_at_the_budget_is_accepted(lib):
    # three full chunks and one of 511 tokens, plus one decoding sequence: 2048 slots
    seqs = [S.SeqSpec(0, 512, True)] * 3 + [S.SeqSpec(0, 511, True), S.SeqSpec(99, 1, False)]
    _, p = _plan(seqs)
    assert p.slot_mapping.numel() == 2048 and p.cu_q.tolist() == [0, 512, 1024, 1536, 2047]


@pytest.mark.parametrize("seqs, what", [
    ([S.SeqSpec(0, 513, True)], "exceeds 512"),
    ([S.SeqSpec(0, 512, True)] * 4 + [S.SeqSpec(99, 1, False)], "2048 token slots"),
    ([S.SeqSpec(0, 64, True), S.SeqSpec(99, 2, False)], "exactly one token"),
    ([S.SeqSpec(99, 1, False), S.SeqSpec(0, 64, True)], "come first"),
])
def test_steps_outside_the_scheduler_limits_are_refused(lib, seqs, what):
    with pytest.raises(ValueError, match=what):
        _plan(seqs)


def test_index_data_of_a_small_mixed_step(lib):
    seqs = [S.SeqSpec(40, 24, True), S.SeqSpec(7, 1, False), S.SeqSpec(300, 1, False)]
    w, p = _plan(seqs)
    assert p.slot_mapping.dtype == torch.int32 and p.slot_mapping.numel() == 26
    assert p.cu_new.tolist() == [0, 24, 25, 26]
    assert p.context_lens.tolist() == [64, 8, 301]
