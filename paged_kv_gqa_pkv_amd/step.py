"""One step of the attention hot path: slot mapping, then per layer the KV
append followed by the prefill-chunk and decode attention launches.

Follows the Module 12 page: a scheduler step mixes one decode token per
decoding sequence with prefill chunks of at most 512 tokens under a budget of
2048 token slots (section "Why chunked prefill"; scheduler budget), and per
layer the step's K/V are written into the pages of every sequence and
attention reads each sequence's context through its block table (model.py
forward).  Here the append runs first and attention reads the post-append
context, which gives the same numbers as the page's read-then-write order
since the append is a bit copy.  A step with no prefill chunk (every
sequence appends its one decode token) runs each layer as one fused call,
pkv_attn_decode_append, which takes the step's own K/V from the new rows and
writes them into their slots, as the page's forward does.  A step with both
runs each layer as one pkv_attn_prefill_decode_append call, whose single
launch holds the chunk's and the decode's workgroups and the copy of the
chunk rows into their slots (the chunk reads its own rows from the new rows,
so nothing in the launch reads a slot it writes); unfused, the append and
one pkv_attn_prefill_decode call.

Host code only marshals arguments: every operation is a library kernel.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import binding as bd
from .synth import Tables, Workload, prefill_cu

CHUNK_LIMIT = 512
STEP_BUDGET = 2048


@dataclasses.dataclass
class StepPlan:
    """Device-resident, layer-independent index data of one step."""
    n_prefill: int
    n_decode: int
    Hq: int
    Hkv: int
    D: int
    block_tables: torch.Tensor     # int32 [n_seqs, max_blocks], prefill sequences first
    context_lens: torch.Tensor     # int32 [n_seqs]
    cu_new: torch.Tensor           # int32 [n_seqs + 1]
    slot_mapping: torch.Tensor     # int32 [total_new]
    cu_q: Optional[torch.Tensor]   # int32 [n_prefill + 1]
    max_q_len: int
    max_ctx_prefill: int
    max_ctx_decode: int
    workspace: Optional[torch.Tensor]
    prefill_workspace: Optional[torch.Tensor]
    scale: float
    fused: bool = False            # the layer's append runs inside its attention call
    mixed: bool = False            # chunk and decode: one call for both halves' attention

    @property
    def needs_slots(self) -> bool:
        """Whether the step's slot mapping is used (a fused decode-only step
        finds its slots inside the decode calls)."""
        return not self.fused or self.mixed

    @property
    def bt_prefill(self):
        return self.block_tables[:self.n_prefill]

    @property
    def ctx_prefill(self):
        return self.context_lens[:self.n_prefill]

    @property
    def bt_decode(self):
        return self.block_tables[self.n_prefill:]

    @property
    def ctx_decode(self):
        return self.context_lens[self.n_prefill:]


def plan_step(w: Workload, t: Tables, device="cuda", scale: Optional[float] = None,
              fused: bool = True, mixed: bool = True) -> StepPlan:
    """Index data and workspaces of a step.  mixed: run the attention of a
    step with both chunks and decode tokens as one call for both halves (else
    pkv_attn_prefill_chunk, then pkv_attn_decode).  fused: fold the layer's
    append into that call: pkv_attn_decode_append for a decode-only step,
    pkv_attn_prefill_decode_append for a mixed one (else pkv_append first)."""
    pre, dec = w.prefill_seqs, w.decode_seqs
    if pre != list(range(len(pre))):
        raise ValueError("prefill sequences must come first")
    chunk_tokens = sum(w.seqs[i].new_len for i in pre)
    if any(w.seqs[i].new_len > CHUNK_LIMIT for i in pre):
        raise ValueError(f"a prefill chunk exceeds {CHUNK_LIMIT} tokens")
    if chunk_tokens + len(dec) > STEP_BUDGET:
        raise ValueError(f"step uses more than {STEP_BUDGET} token slots")
    if any(w.seqs[i].new_len != 1 for i in dec):
        raise ValueError("a decode sequence appends exactly one token")
    total_new = int(t.cu_new[-1])
    ws = None
    max_ctx_dec = max((w.seqs[i].ctx for i in dec), default=0)
    if dec:
        nbytes = bd.pkv_decode_workspace_bytes(len(dec), w.Hq, w.Hkv, w.D, max_ctx_dec)
        if nbytes:
            ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    pws = None
    max_q = max((w.seqs[i].new_len for i in pre), default=0)
    max_ctx_pre = max((w.seqs[i].ctx for i in pre), default=0)
    if pre:
        nbytes = bd.pkv_prefill_workspace_bytes(len(pre), max_q, w.Hq, w.Hkv, w.D, max_ctx_pre)
        if nbytes:
            pws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    return StepPlan(
        n_prefill=len(pre), n_decode=len(dec), Hq=w.Hq, Hkv=w.Hkv, D=w.D,
        block_tables=t.block_tables.to(device), context_lens=t.context_lens.to(device),
        cu_new=t.cu_new.to(device),
        slot_mapping=torch.empty(total_new, dtype=torch.int32, device=device),
        cu_q=prefill_cu(w).to(device) if pre else None,
        max_q_len=max_q, max_ctx_prefill=max_ctx_pre,
        max_ctx_decode=max_ctx_dec, workspace=ws, prefill_workspace=pws,
        scale=scale if scale is not None else w.D ** -0.5,
        fused=bool(fused and dec and (not pre or mixed)), mixed=bool(mixed and dec and pre))


def slot_mapping(plan: StepPlan, stream=None) -> None:
    """Slots of the step's new tokens; shared by every layer's append (a
    fused decode-only step finds them inside its decode calls and needs
    none: plan.needs_slots)."""
    bd.pkv_slot_mapping(plan.slot_mapping, plan.block_tables, plan.cu_new, plan.context_lens,
                        stream=stream)


def layer(plan: StepPlan, k_cache, v_cache, k_new, v_new, q_decode=None, out_decode=None,
          q_prefill=None, out_prefill=None, stream=None, decode_stream=None) -> None:
    """Append the layer's new K/V, then run the chunk and decode attention.

    A plan made with mixed=False and a ``decode_stream`` (a stream of default
    priority) runs a step that has both with its decode launch there,
    concurrently with the chunk: both only read the pools once the append is
    done, so the decode stream waits for the append and ``stream`` waits for
    the decode before anything after.
    """
    s = stream if stream is not None else torch.cuda.current_stream()
    if plan.fused and plan.mixed:
        bd.pkv_attn_prefill_decode_append(out_prefill, q_prefill, plan.cu_q, plan.bt_prefill,
                                          plan.ctx_prefill, plan.max_q_len, plan.max_ctx_prefill,
                                          out_decode, q_decode, plan.bt_decode, plan.ctx_decode,
                                          plan.max_ctx_decode, k_new, v_new, plan.slot_mapping,
                                          k_cache, v_cache, plan.scale,
                                          prefill_workspace=plan.prefill_workspace,
                                          decode_workspace=plan.workspace, stream=s)
        return
    if plan.fused:
        bd.pkv_attn_decode_append(out_decode, q_decode, k_new, v_new, k_cache, v_cache,
                                  plan.bt_decode, plan.ctx_decode, plan.max_ctx_decode,
                                  plan.scale, workspace=plan.workspace, stream=s)
        return
    bd.pkv_append(k_new, v_new, plan.slot_mapping, k_cache, v_cache, stream=s)
    if plan.mixed:
        bd.pkv_attn_prefill_decode(out_prefill, q_prefill, plan.cu_q, plan.bt_prefill,
                                   plan.ctx_prefill, plan.max_q_len, plan.max_ctx_prefill,
                                   out_decode, q_decode, plan.bt_decode, plan.ctx_decode,
                                   plan.max_ctx_decode, k_cache, v_cache, plan.scale,
                                   prefill_workspace=plan.prefill_workspace,
                                   decode_workspace=plan.workspace, stream=s)
        return
    both = bool(plan.n_prefill and plan.n_decode and decode_stream is not None)
    if both:
        appended = torch.cuda.Event()
        appended.record(s)
        decode_stream.wait_event(appended)
    if plan.n_prefill:
        bd.pkv_attn_prefill_chunk(out_prefill, q_prefill, plan.cu_q, k_cache, v_cache,
                                  plan.bt_prefill, plan.ctx_prefill, plan.max_q_len,
                                  plan.max_ctx_prefill, plan.scale,
                                  workspace=plan.prefill_workspace, stream=s)
    if plan.n_decode:
        bd.pkv_attn_decode(out_decode, q_decode, k_cache, v_cache, plan.bt_decode,
                           plan.ctx_decode, plan.max_ctx_decode, plan.scale,
                           workspace=plan.workspace, stream=decode_stream if both else s)
    if both:
        decoded = torch.cuda.Event()
        decoded.record(decode_stream)
        s.wait_event(decoded)
