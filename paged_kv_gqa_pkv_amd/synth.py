"""Seeded synthetic inputs for paged GQA attention steps.

This module draws random numbers and lays them out in the paged-pool format;
it holds none of the method's arithmetic (no slot mapping, no scatter, no
attention).  Both the HIP path and the CPU oracle consume what it produces.

Shapes and structure follow the workloads the pages describe:

* Page "Module 12: Final project - mini inference engine" (hermes-agent.ru
  LLM Inference Systems course), section "Memory": Qwen3-0.6B geometry
  (28 layers, 16 query heads, 8 KV heads, head_dim 128), pages of 16 tokens,
  a 512-page pool holding 8 sessions of about 1k tokens; section "Prefix
  caching": a system prompt of about 200 tokens = 13 shared pages; section
  "Why chunked prefill": a 3000-token prompt cut into 512-token chunks under
  a 2048-slot step budget.
* Page "Module 04: KV cache and memory arithmetic", section 2.2 and the
  ``MODELS`` table of its listing: Qwen3-8B geometry (36 layers, 32 query
  heads, 8 KV heads, head_dim 128); section 3.2: batch 64 at 4k context;
  section 2.4: 13 requests at 32k context.

Values: fp32 N(0,1) samples rounded to bf16 by round-to-nearest-even (the
torch ``.to(torch.bfloat16)`` cast).  Unused pages and the unwritten tail
slots of each sequence's pages hold the bf16 quiet-NaN canary 0x7FC0, so any
read of a slot the method must not read poisons the result.  Pools are
generated in the pages' token-major order [num_blocks][16][Hkv][D] (the
per-layer slice of the Module 12 listing's [n_layers, capacity, 16,
n_kv_heads, head_dim]).

Seeds: stream ``k`` of layer ``l`` of a workload with base seed ``s`` uses
``s * 1_000_000 + l * 100 + k``.  Streams: 0 context lengths, 1 placement,
2 decode q, 3 K pool, 4 V pool, 5 new K, 6 new V, 7 prefill q.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import torch

PAGE = 16
BF16_CANARY_BITS = 0x7FC0

S_CTX, S_PLACE, S_QDEC, S_KPOOL, S_VPOOL, S_KNEW, S_VNEW, S_QPRE = range(8)
S_KSCALE = 8                     # int8 pools: per-(slot, head) K and V scales

# int8 pools: codes are rounded N(0, CODE_SD^2) clipped to +-127 (the spread of
# quantised N(0,1) rows of 128 values, whose largest magnitude is ~3.3 sd), and
# scales are U[SCALE_LO, SCALE_HI] (that largest magnitude over 127).  Slots a
# sequence has not filled hold scale NaN (float32 0x7FC00000), so any read of
# them poisons the result.
CODE_SD = 38.5
SCALE_LO, SCALE_HI = 0.018, 0.030
F32_CANARY_BITS = 0x7FC00000


def stream_seed(base: int, layer: int, stream: int) -> int:
    return base * 1_000_000 + layer * 100 + stream


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn_bf16(shape: Sequence[int], seed: int, device="cpu") -> torch.Tensor:
    """fp32 N(0,1) -> bf16 (round to nearest even), seeded."""
    x = torch.randn(tuple(shape), generator=_gen(seed, device), device=device,
                    dtype=torch.float32)
    return x.to(torch.bfloat16)


def canary_bf16(shape: Sequence[int], device="cpu") -> torch.Tensor:
    return torch.full(tuple(shape), BF16_CANARY_BITS, dtype=torch.int16,
                      device=device).view(torch.bfloat16)


def n_pages(tokens: int) -> int:
    return (tokens + PAGE - 1) // PAGE


@dataclasses.dataclass(frozen=True)
class SeqSpec:
    """One sequence of a step.

    pre_len: tokens whose K/V already sit in the pages before the step.
    new_len: tokens whose K/V the step appends (1 for a decode sequence).
    prefill: True if all new tokens are queries of a causal chunk; False for
             a decode sequence (one query, the appended token).
    """
    pre_len: int
    new_len: int
    prefill: bool

    @property
    def ctx(self) -> int:
        return self.pre_len + self.new_len


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    description: str
    n_layers: int
    Hq: int
    Hkv: int
    D: int
    num_blocks: int
    base_seed: int
    seqs: Tuple[SeqSpec, ...]
    shared_pages: int = 0

    @property
    def prefill_seqs(self) -> List[int]:
        return [i for i, s in enumerate(self.seqs) if s.prefill]

    @property
    def decode_seqs(self) -> List[int]:
        return [i for i, s in enumerate(self.seqs) if not s.prefill]

    @property
    def max_blocks(self) -> int:
        return max(n_pages(s.ctx) for s in self.seqs)

    @property
    def max_ctx(self) -> int:
        return max(s.ctx for s in self.seqs)


def _uniform_ints(n: int, lo: int, hi: int, seed: int) -> List[int]:
    g = _gen(seed, "cpu")
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g)]


def _decode_seqs(ctxs: Sequence[int]) -> List[SeqSpec]:
    return [SeqSpec(pre_len=c - 1, new_len=1, prefill=False) for c in ctxs]


QWEN3_06B = dict(Hq=16, Hkv=8, D=128)
QWEN3_8B = dict(Hq=32, Hkv=8, D=128)

PROMPT_LEN = 3000
CHUNK = 512
STEP_BUDGET = 2048


def workload(name: str, chunk_step: int = 5) -> Workload:
    """The five measured configurations (c4 split in its two batches).

    c1  1 layer, B=1, ctx 64 (4 pages), pool 32 pages.
    c2  1 layer, B=8, ctx ~ U[1,1024], pool 512 pages.
    c3  28 layers, B=8, ctx 1024, first 13 pages shared by all 8 tables.
    c4a 36 layers (8B-shaped), B=64, ctx 4096.
    c4b 36 layers (8B-shaped), B=13, ctx 32768 (long-context split path).
    c5  28 layers, one 512-query chunk of a 3000-token prompt (sub-step
        ``chunk_step`` in 0..5, offset 512*chunk_step) plus 7 decode
        sequences with ctx ~ U[256,2048].
    Context lengths count the appended token(s).
    """
    if name == "c1":
        return Workload(name, "decode B=1 ctx 64, 1 layer, Qwen3-0.6B attention",
                        1, num_blocks=32, base_seed=1, seqs=tuple(_decode_seqs([64])),
                        **QWEN3_06B)
    if name == "c2":
        ctxs = _uniform_ints(8, 1, 1024, stream_seed(2, 0, S_CTX))
        return Workload(name, "decode B=8 ctx U[1,1024], 1 layer, Qwen3-0.6B attention",
                        1, num_blocks=512, base_seed=2, seqs=tuple(_decode_seqs(ctxs)),
                        **QWEN3_06B)
    if name == "c3":
        return Workload(name, "decode B=8 ctx 1024, 28 layers, 13 shared prefix pages, "
                        "Qwen3-0.6B attention",
                        28, num_blocks=512, base_seed=3,
                        seqs=tuple(_decode_seqs([1024] * 8)), shared_pages=13,
                        **QWEN3_06B)
    if name == "c4a":
        return Workload(name, "decode B=64 ctx 4096, 36 layers, Qwen3-8B attention",
                        36, num_blocks=64 * 256 + 32, base_seed=41,
                        seqs=tuple(_decode_seqs([4096] * 64)), **QWEN3_8B)
    if name == "c4b":
        return Workload(name, "decode B=13 ctx 32768, 36 layers, Qwen3-8B attention",
                        36, num_blocks=13 * 2048 + 32, base_seed=42,
                        seqs=tuple(_decode_seqs([32768] * 13)), **QWEN3_8B)
    if name == "c5":
        if not 0 <= chunk_step <= 5:
            raise ValueError("chunk_step must be in 0..5")
        off = CHUNK * chunk_step
        t = min(CHUNK, PROMPT_LEN - off)
        ctxs = _uniform_ints(7, 256, 2048, stream_seed(5, 0, S_CTX))
        seqs = [SeqSpec(pre_len=off, new_len=t, prefill=True)] + _decode_seqs(ctxs)
        assert t + 7 <= STEP_BUDGET
        return Workload(f"c5.{chunk_step}",
                        f"mixed step: prefill chunk o={off} T={t} of a {PROMPT_LEN}-token "
                        "prompt + 7 decode seqs ctx U[256,2048], 28 layers, Qwen3-0.6B attention",
                        28, num_blocks=2048, base_seed=5, seqs=tuple(seqs), **QWEN3_06B)
    raise KeyError(name)


def custom_workload(name: str, seqs: Sequence[SeqSpec], Hq: int, Hkv: int, D: int,
                    num_blocks: int, base_seed: int, n_layers: int = 1,
                    shared_pages: int = 0) -> Workload:
    return Workload(name, name, n_layers, Hq, Hkv, D, num_blocks, base_seed,
                    tuple(seqs), shared_pages)


@dataclasses.dataclass
class Tables:
    """Layer-independent structure of a step: page placement and lengths."""
    block_tables: torch.Tensor   # int32 [n_seqs, max_blocks]; -1 past each sequence's pages
    context_lens: torch.Tensor   # int32 [n_seqs], post-append
    cu_new: torch.Tensor         # int32 [n_seqs + 1], prefix counts of appended tokens
    pre_lens: torch.Tensor       # int32 [n_seqs]


def make_tables(w: Workload) -> Tables:
    """Random non-contiguous placement: one randperm of the pool, consumed in
    order (shared prefix pages first, then each sequence's own pages)."""
    perm = torch.randperm(w.num_blocks, generator=_gen(stream_seed(w.base_seed, 0, S_PLACE), "cpu"))
    need = w.shared_pages + sum(n_pages(s.ctx) - w.shared_pages for s in w.seqs)
    if need > w.num_blocks:
        raise ValueError(f"{w.name}: pool of {w.num_blocks} pages cannot hold {need}")
    mb = w.max_blocks
    bt = torch.full((len(w.seqs), mb), -1, dtype=torch.int32)
    nxt = 0
    shared = perm[:w.shared_pages].to(torch.int32)
    nxt = w.shared_pages
    for i, s in enumerate(w.seqs):
        npg = n_pages(s.ctx)
        if w.shared_pages:
            if s.pre_len < w.shared_pages * PAGE:
                raise ValueError("shared prefix pages must be full before the step")
            bt[i, :w.shared_pages] = shared
        own = npg - w.shared_pages
        bt[i, w.shared_pages:npg] = perm[nxt:nxt + own].to(torch.int32)
        nxt += own
    ctx = torch.tensor([s.ctx for s in w.seqs], dtype=torch.int32)
    new = torch.tensor([0] + [s.new_len for s in w.seqs], dtype=torch.int64)
    cu = torch.cumsum(new, 0).to(torch.int32)
    pre = torch.tensor([s.pre_len for s in w.seqs], dtype=torch.int32)
    return Tables(bt, ctx, cu, pre)


def page_fill_counts(w: Workload, t: Tables) -> torch.Tensor:
    """int32 [num_blocks]: how many leading slots of each physical page hold
    tokens that are already in the cache before the step (0 for unused pages).
    Page j of a sequence holds its tokens 16j..16j+15 in slot order."""
    cnt = torch.zeros(w.num_blocks, dtype=torch.int32)
    for i, s in enumerate(w.seqs):
        for j in range(n_pages(s.ctx)):
            c = max(0, min(PAGE, s.pre_len - PAGE * j))
            page = int(t.block_tables[i, j])
            cnt[page] = max(int(cnt[page]), c)
    return cnt


@dataclasses.dataclass
class LayerData:
    """One layer's tensors for a step (all on ``device``)."""
    k_cache: torch.Tensor        # bf16 [num_blocks, 16, Hkv, D], pre-append
    v_cache: torch.Tensor
    k_new: torch.Tensor          # bf16 [T_total, Hkv, D]
    v_new: torch.Tensor
    q_decode: Optional[torch.Tensor]   # bf16 [B_dec, Hq, D]
    q_prefill: Optional[torch.Tensor]  # bf16 [T_prefill_total, Hq, D]


def _pool(w: Workload, fill: torch.Tensor, seed: int, device) -> torch.Tensor:
    shape = (w.num_blocks, PAGE, w.Hkv, w.D)
    pool = randn_bf16(shape, seed, device)
    bits = pool.view(torch.int16)
    bits.masked_fill_(_dead_slots(w, fill, device).view(w.num_blocks, PAGE, 1, 1),
                      BF16_CANARY_BITS)
    return pool


def _dead_slots(w: Workload, fill: torch.Tensor, device) -> torch.Tensor:
    """bool [num_blocks, 16]: slots no sequence has filled before the step."""
    slot = torch.arange(PAGE, device=device).view(1, PAGE)
    return slot >= fill.to(device).view(-1, 1)


def make_layer(w: Workload, t: Tables, layer: int, device="cpu",
               fill: Optional[torch.Tensor] = None) -> LayerData:
    if fill is None:
        fill = page_fill_counts(w, t)
    s = lambda k: stream_seed(w.base_seed, layer, k)
    T = int(t.cu_new[-1])
    n_dec = len(w.decode_seqs)
    n_pre_q = sum(w.seqs[i].new_len for i in w.prefill_seqs)
    return LayerData(
        k_cache=_pool(w, fill, s(S_KPOOL), device),
        v_cache=_pool(w, fill, s(S_VPOOL), device),
        k_new=randn_bf16((T, w.Hkv, w.D), s(S_KNEW), device),
        v_new=randn_bf16((T, w.Hkv, w.D), s(S_VNEW), device),
        q_decode=randn_bf16((n_dec, w.Hq, w.D), s(S_QDEC), device) if n_dec else None,
        q_prefill=randn_bf16((n_pre_q, w.Hq, w.D), s(S_QPRE), device) if n_pre_q else None,
    )


@dataclasses.dataclass
class LayerDataInt8:
    """One layer's tensors for a step over int8 pages (all on ``device``)."""
    k_codes: torch.Tensor        # int8 [num_blocks, 16, Hkv, D], pre-append
    v_codes: torch.Tensor
    k_scales: torch.Tensor       # float32 [num_blocks, Hkv, 16] (head-major pages)
    v_scales: torch.Tensor
    k_new: torch.Tensor          # bf16 [T_total, Hkv, D]
    v_new: torch.Tensor
    q_decode: Optional[torch.Tensor]
    q_prefill: Optional[torch.Tensor]


def _codes(shape, seed, device) -> torch.Tensor:
    x = torch.randn(tuple(shape), generator=_gen(seed, device), device=device,
                    dtype=torch.float32)
    return torch.clamp(torch.round(x * CODE_SD), -127, 127).to(torch.int8)


def _kv_scales(w: Workload, fill: torch.Tensor, seed: int, device):
    """(k_scales, v_scales), float32 [num_blocks, Hkv, 16] each (a page's
    scales head-major), drawn as one [2, num_blocks, 16, Hkv] array (slot-major,
    so a (page, slot, head) gets the same value in either layout)."""
    g = _gen(seed, device)
    sc = torch.empty((2, w.num_blocks, PAGE, w.Hkv), device=device, dtype=torch.float32)
    sc.uniform_(SCALE_LO, SCALE_HI, generator=g)
    dead = _dead_slots(w, fill, device).view(1, w.num_blocks, PAGE, 1)
    sc.view(torch.int32).masked_fill_(dead, F32_CANARY_BITS)
    sc = sc.transpose(2, 3)
    return sc[0].contiguous(), sc[1].contiguous()


def make_layer_int8(w: Workload, t: Tables, layer: int, device="cpu",
                    fill: Optional[torch.Tensor] = None) -> LayerDataInt8:
    """The same step as make_layer (same new K/V and queries) over int8 pools."""
    if fill is None:
        fill = page_fill_counts(w, t)
    s = lambda k: stream_seed(w.base_seed, layer, k)
    T = int(t.cu_new[-1])
    n_dec = len(w.decode_seqs)
    n_pre_q = sum(w.seqs[i].new_len for i in w.prefill_seqs)
    shape = (w.num_blocks, PAGE, w.Hkv, w.D)
    k_scales, v_scales = _kv_scales(w, fill, s(S_KSCALE), device)
    return LayerDataInt8(
        k_codes=_codes(shape, s(S_KPOOL), device),
        v_codes=_codes(shape, s(S_VPOOL), device),
        k_scales=k_scales, v_scales=v_scales,
        k_new=randn_bf16((T, w.Hkv, w.D), s(S_KNEW), device),
        v_new=randn_bf16((T, w.Hkv, w.D), s(S_VNEW), device),
        q_decode=randn_bf16((n_dec, w.Hq, w.D), s(S_QDEC), device) if n_dec else None,
        q_prefill=randn_bf16((n_pre_q, w.Hq, w.D), s(S_QPRE), device) if n_pre_q else None,
    )


def prefill_cu(w: Workload) -> torch.Tensor:
    """int32 [n_prefill + 1]: prefix counts of query rows of the prefill sequences."""
    lens = [0] + [w.seqs[i].new_len for i in w.prefill_seqs]
    return torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)


def bulk_append_inputs(n_tokens: int, num_blocks: int, Hkv: int, D: int, seed: int,
                       device="cpu"):
    """Bulk append: ``n_tokens`` new rows to distinct random slots of a pool
    (a random permutation of the pool's slots, cut to length)."""
    if n_tokens > num_blocks * PAGE:
        raise ValueError("more tokens than slots")
    g = _gen(seed, "cpu")
    slots = torch.randperm(num_blocks * PAGE, generator=g)[:n_tokens].to(torch.int32)
    k_new = randn_bf16((n_tokens, Hkv, D), seed + 1, device)
    v_new = randn_bf16((n_tokens, Hkv, D), seed + 2, device)
    pool_k = randn_bf16((num_blocks, PAGE, Hkv, D), seed + 3, device)
    pool_v = randn_bf16((num_blocks, PAGE, Hkv, D), seed + 4, device)
    return slots, k_new, v_new, pool_k, pool_v


def int8_pools(num_blocks: int, Hkv: int, D: int, seed: int, device="cpu"):
    """(k_codes, v_codes, k_scales, v_scales) of a fully written int8 pool:
    codes N(0, CODE_SD) rounded and clamped to +-127, [num_blocks, 16, Hkv, D];
    scales U[SCALE_LO, SCALE_HI], [num_blocks, Hkv, 16] (head-major pages)."""
    kc = _codes((num_blocks, PAGE, Hkv, D), seed, "cpu").to(device)
    vc = _codes((num_blocks, PAGE, Hkv, D), seed + 1, "cpu").to(device)
    sc = torch.empty((2, num_blocks, Hkv, PAGE), dtype=torch.float32)
    sc.uniform_(SCALE_LO, SCALE_HI, generator=_gen(seed + 2, "cpu"))
    return kc, vc, sc[0].contiguous().to(device), sc[1].contiguous().to(device)


def large_chunk_inputs(device="cpu", T: int = 2048, offset: int = 6144, Hq: int = 32,
                       Hkv: int = 8, D: int = 128, seed: int = 430) -> dict:
    """One causal chunk of T queries at positions offset..offset+T-1 of a
    single sequence (Qwen3-8B-shaped heads by default), its pages scattered
    over a pool 8 pages larger than the sequence needs: bf16 q and pools, and
    int8 code pools (N(0, CODE_SD) rounded, clamped to +-127) with float32
    scales uniform in [SCALE_LO, SCALE_HI], all seeded."""
    n = offset + T
    if n % PAGE:
        raise ValueError("the chunk must end on a page boundary")
    nbp = n // PAGE + 8
    perm = torch.randperm(nbp, generator=_gen(seed - 422, "cpu"))[:n // PAGE]
    scales = torch.empty((2, nbp, PAGE, Hkv), dtype=torch.float32)
    scales.uniform_(SCALE_LO, SCALE_HI, generator=_gen(seed + 5, "cpu"))
    return {
        "T": T, "offset": offset, "n": n, "Hq": Hq, "Hkv": Hkv, "D": D, "num_blocks": nbp,
        "block_tables": perm.view(1, -1).to(torch.int32).to(device),
        "context_lens": torch.tensor([n], dtype=torch.int32, device=device),
        "cu_q": torch.tensor([0, T], dtype=torch.int32, device=device),
        "q": randn_bf16((T, Hq, D), seed, device),
        "k_cache": randn_bf16((nbp, PAGE, Hkv, D), seed + 1, device),
        "v_cache": randn_bf16((nbp, PAGE, Hkv, D), seed + 2, device),
        "k_codes": _codes((nbp, PAGE, Hkv, D), seed + 3, "cpu").to(device),
        "v_codes": _codes((nbp, PAGE, Hkv, D), seed + 4, "cpu").to(device),
        "k_scales": scales[0].transpose(1, 2).contiguous().to(device),   # [nb, Hkv, 16]
        "v_scales": scales[1].transpose(1, 2).contiguous().to(device),
    }
