"""Pins for the q/k RMSNorm + RoPE oracle (CPU only).

Sources: [P1] model.py (rms_norm, _rope_tables, apply_rope, forward) and
config (rope_theta 1e6); [P2] kv_cache.py listing (split-half RoPE).  Each
check ties the oracle to something other than its own code: torch's bf16
cast, closed forms, identities of rotations, and the second page's
formulation of the same rotation.
"""
import math

import numpy as np
import pytest
import torch

from oracle import pkv_oracle as O
from oracle import pkv_rope_oracle as R

THETA = 1_000_000.0          # [P1] config: rope_theta


def check_bf16_round_matches_torch_cast():
    """Round-to-nearest-even to bf16 agrees with torch's float32 -> bfloat16
    cast (ties, subnormals, large values, signed zero)."""
    rng = np.random.default_rng(80)
    x = np.concatenate([rng.standard_normal(4000).astype(np.float32) * 10 ** rng.uniform(-40, 38, 4000).astype(np.float32),
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -0.0, 1e-40, 3.4e38], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = R.bf16_round(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert R.bf16_round(np.float32(1 + 2 ** -8)) == 1.0              # tie to even
    assert R.bf16_round(np.float32(1 + 3 * 2 ** -8)) == 1 + 2 ** -6   # tie to even (up)


def check_tables_structure_and_frequencies():
    """Halves duplicated; position 0 gives cos 1, sin 0; the frequencies read
    back from position 1 start at 1 and fall geometrically by theta^(-2/D)
    down to theta^(-(D-2)/D)."""
    D = 128
    cos, sin = R.rope_tables_ref(D, 64, THETA, bf16=False)
    assert np.array_equal(cos[:, :D // 2], cos[:, D // 2:]) and np.array_equal(sin[:, :D // 2], sin[:, D // 2:])
    assert np.all(cos[0] == 1.0) and np.all(sin[0] == 0.0)
    f = np.arctan2(sin[1, :D // 2], cos[1, :D // 2])
    assert abs(f[0] - 1.0) < 1e-12
    assert np.allclose(f[1:] / f[:-1], THETA ** (-2.0 / D), rtol=1e-9)
    assert abs(f[-1] - THETA ** (-(D - 2) / D)) < 1e-15
    cb, sb = R.rope_tables_ref(D, 64, THETA, bf16=True)
    assert np.all(np.abs(cb * cb + sb * sb - 1) < 2 ** -6)
    assert np.all(R.bf16_round(cb) == cb)


def check_rope_identities():
    """fp64: position 0 is the identity; the rotation composes additively;
    q.k after rotation depends only on the position difference; the rotate-half
    form ([P1]) equals the split-half form ([P2])."""
    D, T = 16, 5
    rng = np.random.default_rng(81)
    cos, sin = R.rope_tables_ref(D, 400, THETA ** 0.01, bf16=False)   # faster angles
    q = rng.standard_normal((T, 2, D))
    k = rng.standard_normal((T, 2, D))
    assert np.array_equal(R.apply_rope_ref(q, cos, sin, [0] * T, bf16=False), q)
    p = [3, 17, 40, 101, 250]
    rq = R.apply_rope_ref(q, cos, sin, p, bf16=False)
    twice = R.apply_rope_ref(R.apply_rope_ref(q, cos, sin, [2] * T, bf16=False), cos, sin,
                             [x - 2 for x in p], bf16=False)
    assert np.allclose(twice, rq, atol=1e-12)
    d1 = np.einsum("thd,thd->th", rq, R.apply_rope_ref(k, cos, sin, [x + 7 for x in p], bf16=False))
    d2 = np.einsum("thd,thd->th", R.apply_rope_ref(q, cos, sin, [x + 50 for x in p], bf16=False),
                   R.apply_rope_ref(k, cos, sin, [x + 57 for x in p], bf16=False))
    assert np.allclose(d1, d2, atol=1e-10)
    half_c, half_s = cos[:, :D // 2], sin[:, :D // 2]
    assert np.allclose(R.split_half_rope_ref(q, half_c, half_s, p), rq, atol=1e-14)
    norms = lambda x: x[..., :D // 2] ** 2 + x[..., D // 2:] ** 2
    assert np.allclose(norms(rq), norms(q), atol=1e-12)


def check_rms_norm():
    """fp64: a constant row c gives c / sqrt(c^2 + eps) * w; a zero row gives
    zeros; with unit weight
    the output's RMS is 1 (for var >> eps); scaling the input leaves the
    output unchanged; the bf16 path is within 2 ulp of the fp64 one."""
    D, eps = 128, 1e-6
    w = np.linspace(0.5, 1.5, D)
    y = R.rms_norm_ref(np.full((1, D), -3.0), w, eps, bf16=False)
    assert np.allclose(y, -3.0 / math.sqrt(9.0 + eps) * w, rtol=0, atol=1e-15)
    z = R.rms_norm_ref(np.zeros((2, D), np.float32), np.ones(D, np.float32), eps, bf16=True)
    assert np.all(z == 0)                       # eps keeps an all-zero row finite
    rng = np.random.default_rng(82)
    x = rng.standard_normal((6, 4, D)) * 5
    y1 = R.rms_norm_ref(x, np.ones(D), eps, bf16=False)
    assert np.allclose(np.sqrt(np.mean(y1 * y1, -1)), 1.0, atol=1e-7)
    assert np.allclose(R.rms_norm_ref(x * 1000, w, eps, bf16=False),
                       R.rms_norm_ref(x, w, eps, bf16=False), atol=1e-6)
    xb = R.bf16_round(x.astype(np.float32))
    wb = R.bf16_round(w.astype(np.float32))
    yb = R.rms_norm_ref(xb, wb, eps, bf16=True)
    y64 = R.rms_norm_ref(xb.astype(np.float64), wb.astype(np.float64), eps, bf16=False)
    assert np.all(np.abs(yb - y64) <= 2 * 2 ** -8 * np.abs(y64) + 1e-30)


def check_positions_follow_slots():
    """The appended tokens' positions are the ones slot mapping writes: with
    an identity block table the slot of a token is its position."""
    ctx, cu = [5, 37, 1], [0, 2, 7, 8]
    ident = [list(range(4))] * 3
    assert R.positions_ref(cu, ctx) == O.slot_ref(ident, cu, ctx)


PINS = [check_bf16_round_matches_torch_cast, check_tables_structure_and_frequencies,
        check_rope_identities, check_rms_norm, check_positions_follow_slots]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def _mutants():
    orig_tables = R.rope_tables_ref
    orig_rms = R.rms_norm_ref

    def rotate_half_wrong_sign(x):
        h = x.shape[-1] // 2
        return np.concatenate([x[..., h:], -x[..., :h]], axis=-1)

    def tables_wrong_exponent(head_dim, max_seq, theta, bf16=True):
        dt = np.float32 if bf16 else np.float64
        inv = dt(1.0) / (dt(theta) ** (np.arange(head_dim // 2, dtype=dt) / dt(head_dim)))
        freqs = np.outer(np.arange(max_seq, dtype=dt), inv).astype(dt)
        c, s = np.cos(freqs), np.sin(freqs)
        c, s = np.concatenate([c, c], -1), np.concatenate([s, s], -1)
        return (R.bf16_round(c), R.bf16_round(s)) if bf16 else (c, s)

    def rms_without_eps(x, w, eps, bf16=True):
        return orig_rms(x, w, 0.0, bf16)

    def rms_over_heads(x, w, eps, bf16=True):
        xd = np.asarray(x, np.float64)
        var = np.mean(xd * xd, axis=0, keepdims=True)
        return xd / np.sqrt(var + eps) * np.asarray(w, np.float64)

    def round_half_up(x):
        f = np.asarray(x, dtype=np.float32)
        u = f.view(np.uint32).astype(np.uint64)
        return ((u + 0x8000) & 0xFFFF0000).astype(np.uint32).view(np.float32)

    return {
        "rotate_half sign": ("rotate_half", rotate_half_wrong_sign),
        "frequency exponent i/D": ("rope_tables_ref", tables_wrong_exponent),
        "rms_norm without eps": ("rms_norm_ref", rms_without_eps),
        "rms_norm over the wrong axis": ("rms_norm_ref", rms_over_heads),
        "bf16 ties away from zero": ("bf16_round", round_half_up),
    }


@pytest.mark.parametrize("name", sorted(_mutants()))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = _mutants()[name]
    monkeypatch.setattr(R, attr, fn)
    failed = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception:
            failed += 1
    assert failed, f"mutant '{name}' passes every pin"
