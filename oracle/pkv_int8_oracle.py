"""CPU reference ("oracle") for int8 KV pages -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import or run this module; the library path never calls it and it imports
nothing from the library.

What it follows: [P2] "Module 04: KV cache and memory arithmetic", the
kv_cache.py listing, section 5 (class KV8Cache, "int8 cache: half the bytes
per element plus one scale per (token, head)") and the closing notes on the
int8 cache (1.94x rather than 2x: 2112 B instead of 4096 B per token-layer,
about 0.4 % error per element).

The quantiser is the page's, step by step and in the page's precision
(float32 arrays, as in its listing):
  * per (token, KV head) row x[0..D-1]: scale = max_i |x_i| / 127 + 1e-8;
  * code_i = clip(rint(x_i / scale), -127, 127), stored as int8;
  * reading returns code_i * scale (float32).
Here x is the bf16 K or V row widened exactly to float32.

Pages hold codes in the pages' token-major order, int8
[num_blocks][16][Hkv][D] (the per-layer slice of KV8Cache's k [L, cap,
H_kv, D], with cap cut into 16-slot pages as [P1] paged.py does), and the
per-layer slice of ks [L, cap, H_kv] cut the same way with each page's
block stored head-major: float32 [num_blocks][Hkv][16], the scale of (page
b, slot s, KV head g) at [b][g][s].  Attention on the dequantised rows is
the pinned float64 definition of pkv_oracle.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from oracle.pkv_oracle import BLOCK_SIZE, attend_one, gather_ref, kv_head_of

INT8_MAX = np.float32(127.0)
SCALE_EPS = np.float32(1e-8)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns -> float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def quantize_ref(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """[P2] KV8Cache.write for rows along the last axis: float32 in,
    (int8 codes [..., D], float32 scales [...]) out."""
    x = np.asarray(x, dtype=np.float32)
    scale = np.abs(x).max(axis=-1) / INT8_MAX + SCALE_EPS
    q = np.clip(np.rint(x / scale[..., None]), -127.0, 127.0)
    return q.astype(np.int8), scale.astype(np.float32)


def dequantize_ref(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[P2] KV8Cache.read: codes as float32 times the row's scale."""
    return np.asarray(codes).astype(np.float32) * np.asarray(scales, np.float32)[..., None]


def append_int8_ref(k_codes: np.ndarray, v_codes: np.ndarray, k_scales: np.ndarray,
                    v_scales: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                    slots: Sequence[int], block_size: int = BLOCK_SIZE):
    """Quantise every new (token, KV head) row and write codes and scale into
    its slot ([P2] KV8Cache.write; slots as [P1] PagedKVCache.write).

    k_new/v_new: uint16 bf16 [T][Hkv][D]; codes int8 [num_blocks][bs][Hkv][D];
    scales float32 [num_blocks][Hkv][bs].  Negative slots are skipped; a
    repeated slot keeps the last write.  Returns updated copies.
    """
    kc, vc = np.array(k_codes, np.int8, copy=True), np.array(v_codes, np.int8, copy=True)
    ks, vs = np.array(k_scales, np.float32, copy=True), np.array(v_scales, np.float32, copy=True)
    num_blocks = kc.shape[0]
    for t, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        blk, off = divmod(s, block_size)
        if not 0 <= blk < num_blocks:
            raise IndexError(f"slot {s} outside a pool of {num_blocks} pages")
        kc[blk, off], ks[blk, :, off] = quantize_ref(bf16_to_f32(k_new[t]))
        vc[blk, off], vs[blk, :, off] = quantize_ref(bf16_to_f32(v_new[t]))
    return kc, vc, ks, vs


def gather_int8_ref(codes: np.ndarray, scales: np.ndarray, table_row: Sequence[int], n: int,
                    block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Logical positions 0..n-1 -> dequantised float32 [n][Hkv][D] (scales
    [num_blocks][Hkv][bs], read slot-major here)."""
    c = gather_ref(codes, table_row, n, block_size)
    s = gather_ref(np.swapaxes(np.asarray(scales), 1, 2), table_row, n, block_size)
    return dequantize_ref(c, s)


def decode_int8_ref(q: np.ndarray, k_codes: np.ndarray, k_scales: np.ndarray,
                    v_codes: np.ndarray, v_scales: np.ndarray,
                    block_tables: Sequence[Sequence[int]], context_lens: Sequence[int],
                    scale: float, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Decode attention over int8 pages: the float64 definition applied to the
    dequantised rows.  q: uint16 bf16 [B][Hq][D].  Returns float64 [B][Hq][D];
    context 0 gives zeros."""
    from oracle.pkv_oracle import bf16_to_f64
    B, Hq, D = q.shape
    Hkv = k_codes.shape[2]
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = int(context_lens[b])
        if n == 0:
            continue
        K = gather_int8_ref(k_codes, k_scales, block_tables[b], n, block_size).astype(np.float64)
        V = gather_int8_ref(v_codes, v_scales, block_tables[b], n, block_size).astype(np.float64)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            out[b, h] = attend_one(bf16_to_f64(q[b, h]), K[:, g, :], V[:, g, :], scale)
    return out


def prefill_int8_ref(q: np.ndarray, cu_q: Sequence[int], k_codes: np.ndarray,
                     k_scales: np.ndarray, v_codes: np.ndarray, v_scales: np.ndarray,
                     block_tables: Sequence[Sequence[int]], context_lens: Sequence[int],
                     scale: float, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Causal chunk over int8 pages (rows are the last T_b positions of each
    context, key p visible to the row at position t iff p <= t)."""
    from oracle.pkv_oracle import bf16_to_f64
    total_q, Hq, D = q.shape
    Hkv = k_codes.shape[2]
    out = np.zeros((total_q, Hq, D), dtype=np.float64)
    for b in range(len(context_lens)):
        lo, hi = int(cu_q[b]), int(cu_q[b + 1])
        T, n = hi - lo, int(context_lens[b])
        if T == 0:
            continue
        if T > n:
            raise ValueError("more query rows than context")
        K = gather_int8_ref(k_codes, k_scales, block_tables[b], n, block_size).astype(np.float64)
        V = gather_int8_ref(v_codes, v_scales, block_tables[b], n, block_size).astype(np.float64)
        for t in range(T):
            qpos = n - T + t
            for h in range(Hq):
                g = kv_head_of(h, Hq, Hkv)
                out[lo + t, h] = attend_one(bf16_to_f64(q[lo + t, h]),
                                            K[:qpos + 1, g, :], V[:qpos + 1, g, :], scale)
    return out


def kv_bytes_per_token_layer_int8(n_kv_heads: int, head_dim: int) -> int:
    """K and V codes (1 byte per element) plus one float32 scale each per
    (token, KV head): [P2]'s 2112 B per token-layer at H_kv = 8, d_head = 128."""
    return 2 * n_kv_heads * head_dim * 1 + 2 * n_kv_heads * 4
