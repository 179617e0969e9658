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


def check_rope_rounds_each_operation():
    """[P1] apply_rope is bf16 tensor arithmetic: q * cos and rotate_half(q) *
    sin are each rounded to bf16, then their sum is.  Hand case (D = 2, one
    head, position 0 of a one-row table with cos = 1 + 2^-7, sin = 1):
    x = (1 + 2^-7, -2^-8), rotate_half(x) = (2^-8, 1 + 2^-7).
      out[0]: (1 + 2^-7)^2 = 1 + 2^-6 + 2^-14 rounds to 1 + 2^-6; adding 2^-8
              gives 1 + 2.5 * 2^-7, a tie that rounds to even: 1 + 2^-6.
              (Rounding only the exact sum 1 + 2.5 * 2^-7 + 2^-14 would give
              1 + 3 * 2^-7.)
      out[1]: -2^-8 (1 + 2^-7) + (1 + 2^-7) = 1.00387573..., which rounds to 1."""
    x = np.array([[[1 + 2 ** -7, -2 ** -8]]], np.float32)
    cos = np.full((1, 2), 1 + 2 ** -7, np.float32)
    sin = np.ones((1, 2), np.float32)
    got = R.apply_rope_ref(x, cos, sin, [0], bf16=True)
    assert got.reshape(-1).tolist() == [1 + 2 ** -6, 1.0]


def check_rms_norm_rounds_each_operation():
    """[P1] rms_norm: mean of squares and rsqrt in float32, x * inv rounded to
    bf16, then the product with the bf16 weight rounded again.  Hand case
    x = (1, 7), eps = 0, w = 1.125: mean(x^2) = 25, inv = 0.2 (float32), x * inv
    = (0.2, 1.4) rounds to (0.2001953125, 1.3984375); times 1.125 that is
    (0.22521972..., 1.5732421875), which round to (0.2255859375, 1.5703125).
    (One rounding of x * inv * w = (0.225, 1.575) would give (0.224609375,
    1.578125).)"""
    got = R.rms_norm_ref(np.array([[1.0, 7.0]], np.float32), np.array([1.125, 1.125], np.float32),
                         0.0, bf16=True)
    assert got.reshape(-1).tolist() == [0.2255859375, 1.5703125]


def _torch_bf16_rope(x, c, s):
    """The rotation in torch bf16 tensor arithmetic (each operation rounds)."""
    h = x.shape[-1] // 2
    return x * c + torch.cat((-x[..., h:], x[..., :h]), dim=-1) * s


def check_against_torch_bf16_arithmetic():
    """The oracle's per-operation rounding against torch's own bf16 tensor
    arithmetic (each elementwise bf16 operation computes in float32 and rounds
    to bf16), on random rows: RoPE bit for bit; RMSNorm (float32 mean of
    squares and rsqrt, then two bf16 roundings) differs in at most 0.01 % of
    the values (the float32 sum order of the mean and rsqrt's last bit may
    differ, which can move the first rounding by one ulp; the weight, up to
    about 1.6 here, can stretch that to two after the second).  The tables from the same formula computed in torch
    float32 agree with the oracle's numpy float32 tables in all but about 0.1 %
    of the bf16 entries, and those by at most 2^-8 (float32 cos/sin of the two
    libraries differ in their last bits, which moves a rounding now and then);
    the tables are caller inputs."""
    rng = np.random.default_rng(83)
    T, H, D, eps = 64, 8, 128, 1e-6
    xb = R.bf16_round((rng.standard_normal((T, H, D)) * 2).astype(np.float32))
    wb = R.bf16_round((1 + 0.2 * rng.standard_normal(D)).astype(np.float32))
    cos, sin = R.rope_tables_ref(D, 4096, THETA, bf16=True)
    pos = rng.integers(0, 4096, T)
    tx = torch.from_numpy(xb).to(torch.bfloat16)
    tc = torch.from_numpy(cos[pos]).to(torch.bfloat16).unsqueeze(1)
    ts = torch.from_numpy(sin[pos]).to(torch.bfloat16).unsqueeze(1)
    want = _torch_bf16_rope(tx, tc, ts).float().numpy()
    got = R.apply_rope_ref(xb, cos, sin, pos, bf16=True)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    var = tx.float().pow(2).mean(dim=-1, keepdim=True)
    want_n = ((tx.float() * torch.rsqrt(var + eps)).to(torch.bfloat16) *
              torch.from_numpy(wb).to(torch.bfloat16)).float().numpy()
    got_n = R.rms_norm_ref(xb, wb, eps, bf16=True)
    ulp = np.abs(got_n.view(np.int32).astype(np.int64) - want_n.view(np.int32).astype(np.int64)) >> 16
    assert ulp.max() <= 2 and np.count_nonzero(ulp) <= 1e-4 * ulp.size, (ulp.max(), np.count_nonzero(ulp))
    expo = torch.arange(0, D, 2, dtype=torch.float32) / D
    freqs = torch.outer(torch.arange(4096, dtype=torch.float32), 1.0 / (THETA ** expo))
    for mine, theirs in ((cos, torch.cos(freqs)), (sin, torch.sin(freqs))):
        theirs = torch.cat([theirs, theirs], -1).to(torch.bfloat16).float().numpy()
        d = np.abs(mine - theirs)               # one bf16 ulp of [0.5, 1) is 2^-8
        assert d.max() <= 2 ** -8 and np.count_nonzero(d) <= 2e-3 * d.size, (d.max(), np.count_nonzero(d))


PINS = [check_bf16_round_matches_torch_cast, check_tables_structure_and_frequencies,
        check_rope_identities, check_rms_norm, check_positions_follow_slots,
        check_rope_rounds_each_operation, check_rms_norm_rounds_each_operation,
        check_against_torch_bf16_arithmetic]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def _mutants():
    orig_tables = R.rope_tables_ref
    orig_rms = R.rms_norm_ref
    orig_rope = R.apply_rope_ref

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

    def rope_one_rounding(x, cos, sin, pos, bf16=True):
        c = cos[np.asarray(pos)][:, None, :]
        sn = sin[np.asarray(pos)][:, None, :]
        if not bf16:
            return orig_rope(x, cos, sin, pos, bf16)
        x = np.asarray(x, np.float32)
        return R.bf16_round(x * c + R.rotate_half(x) * sn)

    def rms_one_rounding(x, w, eps, bf16=True):
        if not bf16:
            return orig_rms(x, w, eps, bf16)
        xf = np.asarray(x, np.float32)
        var = np.mean(xf * xf, axis=-1, keepdims=True, dtype=np.float32)
        inv = np.float32(1.0) / np.sqrt(var + np.float32(eps))
        return R.bf16_round(xf * inv * np.asarray(w, np.float32))

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
        "apply_rope rounds once": ("apply_rope_ref", rope_one_rounding),
        "rms_norm rounds once": ("rms_norm_ref", rms_one_rounding),
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
