"""CPU reference ("oracle") for paged grouped-query attention -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import or run this module.  The library path never calls it, and it imports
nothing from the library: it shares no code, table or helper with the HIP
kernels.  Everything here is plain, slow and written to be checked by eye
against the pages:

[P1] "Module 12: Final project - mini inference engine" (LLM Inference
     Systems course, hermes-agent.ru/courses/llm-inference/12-final/);
     listings qwen_serve/paged.py and qwen_serve/model.py.
[P2] "Module 04: KV cache and memory arithmetic" (same course,
     .../04-kv-cache/); sections 1, 2.1 and the kv_cache.py listing.
[P3] "Inference Optimization" (AI Engineering from Scratch, phase 10
     lesson 12); section "Paged Attention" and "Step 2: attention with KV
     cache".

Arithmetic is float64 on the bf16 inputs converted exactly (a bf16 value is
the upper half of a float32).  Index arrays are plain Python ints.  All page
memory is handled as uint16 bit patterns so that copies are bit-exact (NaN
payloads, signed zeros).

Every function here is pinned by tests in tests/test_oracle.py against what the
pages and mathematics fix (brute force on tiny inputs, closed forms,
invariants, the pages' printed byte counts).  Nothing is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

BLOCK_SIZE = 16


# --------------------------------------------------------------------------
# bf16 bit patterns <-> float64 (exact widening; no rounding involved)
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns -> float64.  A bf16 number is the high 16 bits of
    the float32 with the same value, so the widening is exact."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Slot mapping and KV append  ([P1] paged.py, PagedKVCache.write; model.py
# forward writes slots start_pos .. start_pos+T-1 of each sequence)
# --------------------------------------------------------------------------

def slot_ref(block_tables: Sequence[Sequence[int]], cu_new: Sequence[int],
             context_lens: Sequence[int], block_size: int = BLOCK_SIZE) -> List[int]:
    """Physical slot of every appended token.

    Sequence b appends ``cu_new[b+1]-cu_new[b]`` tokens that end its context,
    so its first new token sits at logical position
    ``start = context_lens[b] - n_new`` ([P1] forward: the step's tokens take
    positions start_pos .. start_pos+T-1 and start_pos is the committed
    length).  Logical position p lives in logical page ``p // block_size`` at
    offset ``p % block_size`` ([P1] PagedKVCache.write: ``bi, si =
    divmod(s, block_size)``); the flat physical slot is
    ``block_tables[b][page] * block_size + offset``.
    """
    out: List[int] = []
    for b in range(len(context_lens)):
        n_new = int(cu_new[b + 1]) - int(cu_new[b])
        start = int(context_lens[b]) - n_new
        if n_new < 0 or start < 0:
            raise ValueError("inconsistent lengths")
        for p in range(start, start + n_new):
            page, offset = divmod(p, block_size)
            out.append(int(block_tables[b][page]) * block_size + offset)
    return out


def append_ref(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray,
               v_new: np.ndarray, slots: Sequence[int],
               block_size: int = BLOCK_SIZE) -> Tuple[np.ndarray, np.ndarray]:
    """Scatter new K/V rows into the pool ([P1] PagedKVCache.write).

    k_cache/v_cache: uint16 [num_blocks][block_size][Hkv][D]; k_new/v_new:
    uint16 [T][Hkv][D]; slots: T flat slots, a negative slot means "skip".
    Returns updated copies; tokens are written in order (a repeated slot
    keeps the last write, as the page's loop does).
    """
    kc = np.array(k_cache, dtype=np.uint16, copy=True)
    vc = np.array(v_cache, dtype=np.uint16, copy=True)
    num_blocks = kc.shape[0]
    for t, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        blk, off = divmod(s, block_size)
        if not 0 <= blk < num_blocks:
            raise IndexError(f"slot {s} outside a pool of {num_blocks} pages")
        kc[blk, off] = k_new[t]
        vc[blk, off] = v_new[t]
    return kc, vc


def copy_blocks_ref(pool: np.ndarray, src: Sequence[int], dst: Sequence[int]) -> np.ndarray:
    """Copy-on-write / fork page copy ([P1] paged.py, SequenceCache._cow_copy
    and fork_from: ``k[:, nb] = k[:, src]``, the same for v): for each pair,
    in order, every layer's block dst becomes a bit copy of block src.

    pool: [n_layers][num_blocks][...] of any dtype (bits are copied).
    Returns an updated copy; raises IndexError for a block outside the pool.
    """
    out = np.array(pool, copy=True)
    nb = out.shape[1]
    for s, d in zip(src, dst):
        s, d = int(s), int(d)
        if not (0 <= s < nb and 0 <= d < nb):
            raise IndexError(f"block pair ({s}, {d}) outside a pool of {nb} blocks")
        out[:, d] = out[:, s]
    return out


def gather_ref(cache: np.ndarray, table_row: Sequence[int], n: int,
               block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Logical positions 0..n-1 of one sequence -> contiguous [n][Hkv][D]
    ([P1] PagedKVCache.read: one divmod per position)."""
    rows = []
    for p in range(n):
        page, offset = divmod(p, block_size)
        rows.append(cache[int(table_row[page]), offset])
    if not rows:
        return np.zeros((0,) + tuple(cache.shape[2:]), dtype=cache.dtype)
    return np.stack(rows)


# --------------------------------------------------------------------------
# Attention  ([P2] section 1: o_n = softmax(q_n K_{0:n}^T / sqrt(d_head)) V_{0:n};
# [P1] forward: q viewed [T, n_kv, group, D], scores scaled by 1/sqrt(D),
# causal mask kpos <= qpos, fp32 softmax)
# --------------------------------------------------------------------------

def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """Query head h reads KV head h // (Hq/Hkv): [P1] views q as
    [T, n_kv, group, D] (contiguous groups); [P2] attend repeats each KV head
    n_rep times along the head axis (np.repeat), which is the same map."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def softmax_weights(scores: np.ndarray) -> np.ndarray:
    """exp(s - max s) / sum: the softmax of a 1-D score vector in float64."""
    m = np.max(scores)
    w = np.exp(scores - m)
    return w / np.sum(w)


def attend_one(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """One query row over its visible keys: softmax(scale * K q) @ V.
    q: [D]; K, V: [n][D] float64, n >= 1."""
    s = (K @ q) * scale
    return softmax_weights(s) @ V


def decode_ref(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
               block_tables: Sequence[Sequence[int]], context_lens: Sequence[int],
               scale: float, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """One decode query per sequence over its whole (post-append) context.

    q: uint16 bf16 [B][Hq][D]; caches: uint16 [num_blocks][bs][Hkv][D].
    Returns float64 [B][Hq][D].  A sequence with context 0 has no keys; its
    output is defined as zeros.
    """
    B, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = int(context_lens[b])
        if n == 0:
            continue
        K = bf16_to_f64(gather_ref(k_cache, block_tables[b], n, block_size))
        V = bf16_to_f64(gather_ref(v_cache, block_tables[b], n, block_size))
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            out[b, h] = attend_one(bf16_to_f64(q[b, h]), K[:, g, :], V[:, g, :], scale)
    return out


def prefill_ref(q: np.ndarray, cu_q: Sequence[int], k_cache: np.ndarray,
                v_cache: np.ndarray, block_tables: Sequence[Sequence[int]],
                context_lens: Sequence[int], scale: float,
                block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Causal chunk: sequence b owns query rows cu_q[b] .. cu_q[b+1]-1, which
    are the last T_b positions of its (post-append) context n_b, so row t sits
    at position n_b - T_b + t and sees keys 0 .. that position ([P1] forward:
    mask kpos <= qpos on absolute positions).

    q: uint16 [total_q][Hq][D].  Returns float64 [total_q][Hq][D].
    """
    total_q, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    out = np.zeros((total_q, Hq, D), dtype=np.float64)
    for b in range(len(context_lens)):
        lo, hi = int(cu_q[b]), int(cu_q[b + 1])
        T, n = hi - lo, int(context_lens[b])
        if T == 0:
            continue
        if T > n:
            raise ValueError("more query rows than context")
        K = bf16_to_f64(gather_ref(k_cache, block_tables[b], n, block_size))
        V = bf16_to_f64(gather_ref(v_cache, block_tables[b], n, block_size))
        for t in range(T):
            qpos = n - T + t
            for h in range(Hq):
                g = kv_head_of(h, Hq, Hkv)
                out[lo + t, h] = attend_one(bf16_to_f64(q[lo + t, h]),
                                            K[:qpos + 1, g, :], V[:qpos + 1, g, :], scale)
    return out


# --------------------------------------------------------------------------
# Ring (sliding-window) paging  ([P2] section 4, "Capacity-cache": past
# capacity the cache becomes a ring, position p written at p % capacity,
# the oldest token overwritten; reads return the last min(end, capacity)
# positions with their absolute positions; the mask compares absolute
# positions.  [P2] kv_cache.py listing, KVCache.write/read and ring_demo.)
# A ring of W tokens is the first W/block_size pages of a sequence's table.
# --------------------------------------------------------------------------

def ring_slot_ref(block_tables: Sequence[Sequence[int]], cu_new: Sequence[int],
                  context_lens: Sequence[int], window: int,
                  block_size: int = BLOCK_SIZE) -> List[int]:
    """Slots of the appended tokens when each sequence's pages form a ring of
    ``window`` tokens: position p is written at ring index p % window."""
    if window <= 0 or window % block_size:
        raise ValueError("window must be a positive multiple of the block size")
    out: List[int] = []
    for b in range(len(context_lens)):
        n_new = int(cu_new[b + 1]) - int(cu_new[b])
        start = int(context_lens[b]) - n_new
        if n_new < 0 or start < 0:
            raise ValueError("inconsistent lengths")
        for p in range(start, start + n_new):
            page, offset = divmod(p % window, block_size)
            out.append(int(block_tables[b][page]) * block_size + offset)
    return out


def ring_read_ref(cache: np.ndarray, table_row: Sequence[int], end: int, window: int,
                  block_size: int = BLOCK_SIZE) -> Tuple[np.ndarray, np.ndarray]:
    """The ring's contents after ``end`` tokens were written: the rows of the
    last min(end, window) positions in increasing position order, and those
    absolute positions."""
    n = min(end, window)
    pos = np.arange(end - n, end)
    rows = []
    for p in pos:
        page, offset = divmod(int(p) % window, block_size)
        rows.append(cache[int(table_row[page]), offset])
    if not rows:
        return np.zeros((0,) + tuple(cache.shape[2:]), dtype=cache.dtype), pos
    return np.stack(rows), pos


def ring_decode_ref(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                    block_tables: Sequence[Sequence[int]], context_lens: Sequence[int],
                    window: int, scale: float, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Decode over rings: the query at position n-1 attends to the ring's
    keys (positions n - min(n, window) .. n-1, all at or before it)."""
    B, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = int(context_lens[b])
        if n == 0:
            continue
        Kb, _ = ring_read_ref(k_cache, block_tables[b], n, window, block_size)
        Vb, _ = ring_read_ref(v_cache, block_tables[b], n, window, block_size)
        K, V = bf16_to_f64(Kb), bf16_to_f64(Vb)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            out[b, h] = attend_one(bf16_to_f64(q[b, h]), K[:, g, :], V[:, g, :], scale)
    return out


def ring_prefill_ref(q: np.ndarray, cu_q: Sequence[int], k_cache: np.ndarray,
                     v_cache: np.ndarray, block_tables: Sequence[Sequence[int]],
                     context_lens: Sequence[int], window: int, scale: float,
                     block_size: int = BLOCK_SIZE) -> np.ndarray:
    """A chunk over rings, after the chunk was written: row t (absolute
    position n - T + t) attends to the ring's keys whose absolute position is
    at most its own ([P2]: mask k_pos <= q_pos on the positions read returns)."""
    total_q, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    out = np.zeros((total_q, Hq, D), dtype=np.float64)
    for b in range(len(context_lens)):
        lo, hi = int(cu_q[b]), int(cu_q[b + 1])
        T, n = hi - lo, int(context_lens[b])
        if T == 0:
            continue
        if T > n:
            raise ValueError("more query rows than context")
        Kb, pos = ring_read_ref(k_cache, block_tables[b], n, window, block_size)
        Vb, _ = ring_read_ref(v_cache, block_tables[b], n, window, block_size)
        K, V = bf16_to_f64(Kb), bf16_to_f64(Vb)
        for t in range(T):
            qpos = n - T + t
            vis = pos <= qpos
            if not np.any(vis):
                raise ValueError("a query row sees no key (chunk longer than the ring)")
            for h in range(Hq):
                g = kv_head_of(h, Hq, Hkv)
                out[lo + t, h] = attend_one(bf16_to_f64(q[lo + t, h]), K[vis, g, :],
                                            V[vis, g, :], scale)
    return out


def decode_weights_ref(q_row: np.ndarray, k_cache: np.ndarray, table_row: Sequence[int],
                       n: int, g: int, scale: float,
                       block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Softmax weights of one decode query over its n keys (for checks)."""
    K = bf16_to_f64(gather_ref(k_cache, table_row, n, block_size))[:, g, :]
    return softmax_weights((K @ bf16_to_f64(q_row)) * scale)


# --------------------------------------------------------------------------
# KV memory arithmetic  ([P2] section 2.1: KV bytes = 2 * L * H_kv * d_head *
# n_ctx * b * f_full; [P1] "Memory": 112 KiB per token for Qwen3-0.6B)
# --------------------------------------------------------------------------

def kv_bytes(n_layers: int, n_kv_heads: int, head_dim: int, n_ctx: int,
             bytes_per_elem: int, f_full: float = 1.0) -> float:
    v = 2 * n_layers * n_kv_heads * head_dim * n_ctx * bytes_per_elem
    return v if f_full == 1.0 else v * f_full


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int,
                       bytes_per_elem: int) -> int:
    return 2 * n_layers * n_kv_heads * head_dim * bytes_per_elem


def default_scale(head_dim: int) -> float:
    """1/sqrt(head_dim) in float64 ([P1] forward; [P2] attend)."""
    return 1.0 / math.sqrt(head_dim)
