"""The 2048-query causal chunk at positions 6144..8191 with Qwen3-8B-shaped
heads (Hq 32, Hkv 8, D 128), bf16 and int8 pages, on the very inputs and
plan the kernel benchmark times, through pkv_attn_prefill_chunk(_int8)
directly (the mixed step caps its chunks at 512 queries).

Row R of KV head g is token R / 4 and query head 4 g + R % 4, so row tile x
(128 rows) holds tokens 32 x .. 32 x + 31.  The sample takes one token of
every row tile, at a different offset within the tile each time (all 32
offsets occur), plus the first and last token, with all 32 heads: every
(row tile, KV head) group.  The planner cuts the 128 key tiles into two
splits of 64 (keys 0..4095 and 4096..8191); every query sits at position
6144 or later, so every row merges partials of both splits.  The oracle
recomputes each sampled row over its causal key range ([P1] Module 12 forward; [P2]
section 1's softmax(q K^T / sqrt(d)) V), from the pools as given.  A graph
replay of the call is bit-identical to the eager call.
"""
import numpy as np
import pytest
import torch

from oracle import pkv_int8_oracle as Q
from oracle import pkv_oracle as O
from paged_kv_gqa_pkv_amd import binding as bd
from paged_kv_gqa_pkv_amd import synth as S

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


def u16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def sample_tokens(T, G):
    rows_per_tile = 128 // G
    toks = {0, T - 1}
    for x in range(T // rows_per_tile):
        toks.add(x * rows_per_tile + (7 * x) % rows_per_tile)
    return sorted(toks)


def run(kind):
    c = S.large_chunk_inputs("cuda")
    T, n, Hq, Hkv, D = c["T"], c["n"], c["Hq"], c["Hkv"], c["D"]
    print(f"[large chunk] {kind}: {T} queries at {c['offset']}..{n - 1}, Hq {Hq} Hkv {Hkv}",
          flush=True)
    nws = bd.pkv_prefill_workspace_bytes(1, T, Hq, Hkv, D, n)
    groups = (T * (Hq // Hkv) // 128) * Hkv
    assert nws >= groups * 2 * 128 * (D + 2) * 4, "the plan cuts the keys into splits"
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda")
    out = torch.full_like(c["q"], float("nan"))
    scale = D ** -0.5

    def call(o):
        if kind == "bf16":
            bd.pkv_attn_prefill_chunk(o, c["q"], c["cu_q"], c["k_cache"], c["v_cache"],
                                      c["block_tables"], c["context_lens"], T, n, scale,
                                      workspace=ws)
        else:
            bd.pkv_attn_prefill_chunk_int8(o, c["q"], c["cu_q"], c["k_codes"], c["v_codes"],
                                           c["k_scales"], c["v_scales"], c["block_tables"],
                                           c["context_lens"], T, n, scale, workspace=ws)

    call(out)
    torch.cuda.synchronize()
    # a graph replay (the benchmark's launch) gives the same bits
    rep = torch.full_like(out, float("nan"))
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            call(rep)
    torch.cuda.synchronize()
    for _ in range(2):
        rep.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(rep.view(torch.int16), out.view(torch.int16))
    bt = c["block_tables"].cpu().tolist()[0]
    if kind == "bf16":
        K = O.bf16_to_f64(O.gather_ref(u16(c["k_cache"]), bt, n))
        V = O.bf16_to_f64(O.gather_ref(u16(c["v_cache"]), bt, n))
    else:
        K = Q.gather_int8_ref(c["k_codes"].cpu().numpy(), c["k_scales"].cpu().numpy(), bt,
                              n).astype(np.float64)
        V = Q.gather_int8_ref(c["v_codes"].cpu().numpy(), c["v_scales"].cpu().numpy(), bt,
                              n).astype(np.float64)
    q, got = u16(c["q"]), O.bf16_to_f64(u16(out))
    assert np.all(np.isfinite(got))
    errs = []
    toks = sample_tokens(T, Hq // Hkv)
    for t in toks:
        npos = n - T + t + 1                   # causal: keys 0 .. position of token t
        for h in range(Hq):
            kv = O.kv_head_of(h, Hq, Hkv)
            want = O.attend_one(O.bf16_to_f64(q[t, h]), K[:npos, kv], V[:npos, kv], scale)
            errs.append(np.abs(got[t, h] - want))
    err = np.concatenate(errs)
    print(f"large chunk {kind}: {len(toks)} tokens x {Hq} heads, max abs {err.max():.3e} "
          f"mean abs {err.mean():.3e}", flush=True)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS


def test_sample_covers_every_row_tile():
    toks = sample_tokens(2048, 4)
    assert {t // 32 for t in toks} == set(range(64))
    assert {t % 32 for t in toks} == set(range(32))


@pytest.mark.gpu
@pytest.mark.parametrize("kind", ["bf16", "int8"])
def test_large_chunk_2048x8192_sampled(kind):
    run(kind)
