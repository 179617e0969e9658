"""CPU reference ("oracle") for the step before attention: q/k RMSNorm, RoPE,
and the append of the rotated k -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import or run this module; the library path never calls it and it imports
nothing from the library.

What it follows: [P1] "Module 12: Final project - mini inference engine",
listing qwen_serve/model.py:
  * rms_norm(x, w, eps): mean of x^2 and rsqrt in float32, (x * inv) cast
    back to the activation dtype, then times the weight;
  * _rope_tables(head_dim, max_seq, theta): inv_freq = 1 / theta^(2i / D) in
    float32, freqs = outer(pos, inv_freq), cos and sin with both halves
    duplicated (rotate-half / NeoX layout), cast to the activation dtype;
  * apply_rope: q * cos[pos] + rotate_half(q) * sin[pos] with
    rotate_half(x) = cat(-x[D/2:], x[:D/2]);
  * forward: q = rms_norm(q, q_norm); k = rms_norm(k, k_norm); RoPE on both
    at the token's absolute position; k and v then go to the cache.
[P2] "Module 04", kv_cache.py listing: rope_tables/apply_rope in the
split-half form x1*c - x2*s, x1*s + x2*c (the same rotation) and rmsnorm.

Precision: with bf16=True every tensor operation of the listing rounds its
result to bf16 (round to nearest even), as torch does for bf16 tensors, and
the reductions and rsqrt run in float32; with bf16=False everything is
float64 (the plain definition, used by the pins).
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from oracle.pkv_oracle import BLOCK_SIZE


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float -> nearest bf16 (ties to even), returned as float32; NaN stays NaN."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    out = r.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(f), f, out)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16-exact float32 values -> uint16 patterns."""
    return (bf16_round(x).view(np.uint32) >> 16).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def rope_tables_ref(head_dim: int, max_seq: int, theta: float,
                    bf16: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """[P1] _rope_tables: cos, sin [max_seq][head_dim] (halves duplicated)."""
    dt = np.float32 if bf16 else np.float64
    expo = np.arange(0, head_dim, 2, dtype=dt) / dt(head_dim)
    inv_freq = dt(1.0) / (dt(theta) ** expo)
    pos = np.arange(max_seq, dtype=dt)
    freqs = np.outer(pos, inv_freq).astype(dt)
    cos, sin = np.cos(freqs), np.sin(freqs)
    cos = np.concatenate([cos, cos], axis=-1)
    sin = np.concatenate([sin, sin], axis=-1)
    if bf16:
        return bf16_round(cos), bf16_round(sin)
    return cos, sin


def rms_norm_ref(x: np.ndarray, w: np.ndarray, eps: float, bf16: bool = True) -> np.ndarray:
    """[P1] rms_norm over the last axis."""
    if bf16:
        xf = np.asarray(x, np.float32)
        var = np.mean(xf * xf, axis=-1, keepdims=True, dtype=np.float32)
        inv = np.float32(1.0) / np.sqrt(var + np.float32(eps))
        return bf16_round(bf16_round(xf * inv) * np.asarray(w, np.float32))
    xd = np.asarray(x, np.float64)
    var = np.mean(xd * xd, axis=-1, keepdims=True)
    return xd / np.sqrt(var + eps) * np.asarray(w, np.float64)


def rotate_half(x: np.ndarray) -> np.ndarray:
    h = x.shape[-1] // 2
    return np.concatenate([-x[..., h:], x[..., :h]], axis=-1)


def apply_rope_ref(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, pos: Sequence[int],
                   bf16: bool = True) -> np.ndarray:
    """[P1] apply_rope for x [T][heads][D] at absolute positions pos [T]."""
    c = cos[np.asarray(pos)][:, None, :]
    s = sin[np.asarray(pos)][:, None, :]
    if bf16:
        x = np.asarray(x, np.float32)
        return bf16_round(bf16_round(x * c) + bf16_round(rotate_half(x) * s))
    x = np.asarray(x, np.float64)
    return x * c + rotate_half(x) * s


def positions_ref(cu_new: Sequence[int], context_lens: Sequence[int]) -> list:
    """Absolute positions of the appended tokens ([P1] forward: the step's
    tokens of a sequence take positions start_pos .. start_pos+T-1)."""
    out = []
    for b in range(len(context_lens)):
        n_new = int(cu_new[b + 1]) - int(cu_new[b])
        start = int(context_lens[b]) - n_new
        out.extend(range(start, start + n_new))
    return out


def qk_norm_rope_ref(q: np.ndarray, k: np.ndarray, q_norm: np.ndarray, k_norm: np.ndarray,
                     cos: np.ndarray, sin: np.ndarray, pos: Sequence[int], eps: float,
                     bf16: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """[P1] forward: q, k normalised per head, then rotated at their positions.
    q [T][Hq][D], k [T][Hkv][D] (float values); returns (q_rot, k_rot)."""
    qn = rms_norm_ref(q, q_norm, eps, bf16)
    kn = rms_norm_ref(k, k_norm, eps, bf16)
    return apply_rope_ref(qn, cos, sin, pos, bf16), apply_rope_ref(kn, cos, sin, pos, bf16)


def split_half_rope_ref(x: np.ndarray, cos_half: np.ndarray, sin_half: np.ndarray,
                        pos: Sequence[int]) -> np.ndarray:
    """[P2] apply_rope (split-half form) in float64, for the equivalence pin."""
    c = cos_half[np.asarray(pos)][:, None, :]
    s = sin_half[np.asarray(pos)][:, None, :]
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


__all__ = ["BLOCK_SIZE", "bf16_round", "bf16_bits", "bits_to_f32", "rope_tables_ref",
           "rms_norm_ref", "rotate_half", "apply_rope_ref", "positions_ref", "qk_norm_rope_ref",
           "split_half_rope_ref"]
