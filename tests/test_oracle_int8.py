"""Pins for the int8-page oracle (CPU only).

Sources: [P2] "Module 04: KV cache and memory arithmetic", kv_cache.py listing
section 5 (KV8Cache) and the closing notes on the int8 cache.  Each check
ties the oracle to something other than its own code: the page's printed
figures, hand-derived closed forms, a rounding bound, and a reduction to the
(pinned) bf16 oracle.  Planted mistakes in the oracle must each fail a pin.
"""
import numpy as np
import pytest

from oracle import pkv_int8_oracle as Q
from oracle import pkv_oracle as O

BS = 16


def f32_bits_to_bf16(x):
    """float32 values that are exact in bf16 -> uint16 patterns."""
    b = np.asarray(x, np.float32).view(np.uint32)
    assert np.all(b & 0xFFFF == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


# ---------------------------------------------------------------- pins ---

def check_bytes_printed():
    """[P2] closing notes: 2112 B instead of 4096 B per token-layer (H_kv 8,
    d_head 128), i.e. 1.94x rather than 2x."""
    assert Q.kv_bytes_per_token_layer_int8(8, 128) == 2112
    assert O.kv_bytes_per_token(1, 8, 128, 2) == 4096
    assert f"{4096 / Q.kv_bytes_per_token_layer_int8(8, 128):.2f}" == "1.94"


def check_integer_rows_exact():
    """Integer rows with max |x| = 127: 127/127 = 1 and 1 + 1e-8 rounds to 1 in
    float32 (1e-8 is below half an ulp of 1, 2^-24), so the scale is exactly 1
    and every code is the value itself."""
    rng = np.random.default_rng(1)
    x = rng.integers(-127, 128, size=(5, 32)).astype(np.float32)
    x[:, 3] = 127.0
    x[1, 3] = -127.0
    codes, scale = Q.quantize_ref(x)
    assert np.all(scale == np.float32(1.0))
    assert np.array_equal(codes.astype(np.float32), x)


def check_round_half_even():
    """np.rint rounds halves to even (hand values at scale 1)."""
    x = np.array([127, 0.5, 1.5, 2.5, -0.5, -1.5, 3.5, -2.5], np.float32)
    codes, scale = Q.quantize_ref(x)
    assert scale == np.float32(1.0)
    assert codes.tolist() == [127, 0, 2, 2, 0, -2, 4, -2]


def check_zero_row():
    """The 1e-8 term keeps an all-zero row finite: scale 1e-8, codes 0, and it
    reads back as zeros."""
    codes, scale = Q.quantize_ref(np.zeros((2, 16), np.float32))
    assert np.all(scale == np.float32(1e-8)) and not np.any(codes)
    assert np.all(Q.dequantize_ref(codes, scale) == 0)


def check_extremes_and_signs():
    """The largest |x| of every row maps to +-127 with its sign; negating a row
    negates its codes and keeps its scale; codes stay in [-127, 127]."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((200, 128)).astype(np.float32) * rng.uniform(0.01, 50, (200, 1)).astype(np.float32)
    codes, scale = Q.quantize_ref(x)
    i = np.abs(x).argmax(axis=1)
    r = np.arange(200)
    assert np.array_equal(codes[r, i].astype(np.int64), np.where(x[r, i] > 0, 127, -127))
    assert codes.min() >= -127 and codes.max() <= 127
    c2, s2 = Q.quantize_ref(-x)
    assert np.array_equal(c2, -codes) and np.array_equal(s2, scale)


def check_error_bound_and_page_figure():
    """Rounding to the nearest code errs by at most half a step (scale / 2),
    which is max|x| / 254 = 0.39 % of the row's largest magnitude: the page's
    "about 0.4 % per element".  On N(0,1) rows the bound is nearly reached and
    the mean error is a quarter step (uniform rounding error)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2000, 128)).astype(np.float32)
    codes, scale = Q.quantize_ref(x)
    err = np.abs(Q.dequantize_ref(codes, scale).astype(np.float64) - x)
    assert np.all(err <= scale[:, None] * (0.5 + 1e-5))
    rel = err / np.abs(x).max(axis=1, keepdims=True)
    assert rel.max() <= 1 / 254 * (1 + 1e-4)
    assert rel.max() > 0.0038                    # "about 0.4 %"
    assert 0.0017 < rel.mean() < 0.0022           # a quarter step, max/508


def check_scale_per_row():
    """One scale per (token, head) row along d_head (the page warns that a
    scale over the whole tensor is the usual mistake): rows of very different
    magnitude each reach +-127."""
    x = np.stack([np.linspace(-1e-3, 1e-3, 64), np.linspace(-100, 90, 64)]).astype(np.float32)
    codes, scale = Q.quantize_ref(x.reshape(1, 2, 64))
    assert scale.shape == (1, 2)
    assert np.abs(codes).max(axis=-1).tolist() == [[127, 127]]


def check_append_semantics():
    """Append writes quantised rows of the bf16 input into the slot's page and
    offset (all heads), skips negative slots, keeps the last write, and leaves
    everything else untouched."""
    rng = np.random.default_rng(4)
    nb, Hkv, D = 3, 2, 8
    kc = rng.integers(-127, 128, (nb, BS, Hkv, D)).astype(np.int8)
    vc = rng.integers(-127, 128, (nb, BS, Hkv, D)).astype(np.int8)
    ks = rng.uniform(0.1, 1, (nb, Hkv, BS)).astype(np.float32)    # head-major pages
    vs = rng.uniform(0.1, 1, (nb, Hkv, BS)).astype(np.float32)
    vals = (rng.integers(-64, 64, (4, Hkv, D)) / 8.0).astype(np.float32)   # exact in bf16
    k_new = f32_bits_to_bf16(vals)
    v_new = f32_bits_to_bf16(-vals)
    slots = [5, -1, 40, 5]
    okc, ovc, oks, ovs = Q.append_int8_ref(kc, vc, ks, vs, k_new, v_new, slots)
    want_k, want_ks = kc.copy(), ks.copy()
    for t in (2, 3):                           # slot 5 keeps token 3, slot 40 token 2
        s = slots[t]
        for g in range(Hkv):
            m = np.abs(vals[t, g]).max()
            sc = np.float32(np.float32(m) / np.float32(127)) + np.float32(1e-8)
            want_ks[s // BS, g, s % BS] = sc
            want_k[s // BS, s % BS, g] = np.clip(np.rint(vals[t, g] / sc), -127, 127)
    assert np.array_equal(okc, want_k) and np.array_equal(oks, want_ks)
    assert np.array_equal(ovc[0, 5], -okc[0, 5]) and np.array_equal(ovs[0, :, 5], oks[0, :, 5])
    assert np.array_equal(ovs[2, :, 8], oks[2, :, 8])
    untouched = np.ones((nb, BS), bool); untouched[0, 5] = untouched[2, 8] = False
    assert np.array_equal(okc[untouched], kc[untouched])
    assert np.array_equal(oks.transpose(0, 2, 1)[untouched], ks.transpose(0, 2, 1)[untouched])
    with pytest.raises(IndexError):
        Q.append_int8_ref(kc, vc, ks, vs, k_new[:1], v_new[:1], [nb * BS])


def check_gather_brute_force():
    """Gather walks the table: position p reads page table[p // 16], offset
    p % 16, and multiplies the codes by that row's scale (brute force)."""
    rng = np.random.default_rng(5)
    nb, Hkv, D = 6, 2, 4
    codes = rng.integers(-127, 128, (nb, BS, Hkv, D)).astype(np.int8)
    scales = rng.uniform(0.01, 0.05, (nb, Hkv, BS)).astype(np.float32)   # head-major pages
    row, n = [4, 0, 3], 37
    got = Q.gather_int8_ref(codes, scales, row, n)
    for p in range(n):
        for g in range(Hkv):
            for d in range(D):
                want = np.float32(codes[row[p // 16], p % 16, g, d]) * scales[row[p // 16], g, p % 16]
                assert got[p, g, d] == want


def _integer_pools(rng, nb, Hkv, D):
    """Pools whose rows are integers with max |x| = 127: int8 codes with scale
    1 hold exactly the values a bf16 pool holds."""
    vals = rng.integers(-127, 128, (nb, BS, Hkv, D)).astype(np.float32)
    vals[..., 0] = 127.0
    codes = vals.astype(np.int8)
    scales = np.ones((nb, Hkv, BS), np.float32)
    return vals, codes, scales


def check_attention_reduces_to_bf16_oracle():
    """With exactly representable rows, int8 decode and prefill equal the
    pinned bf16 oracle on the same values."""
    rng = np.random.default_rng(6)
    nb, Hq, Hkv, D = 12, 4, 2, 16
    kv, kcod, ksc = _integer_pools(rng, nb, Hkv, D)
    vv, vcod, vsc = _integer_pools(rng, nb, Hkv, D)
    kb, vb = f32_bits_to_bf16(kv), f32_bits_to_bf16(vv)
    tables = [[3, 7, 1, -1], [0, 11, 5, 2]]
    ctx = [40, 57]
    q = f32_bits_to_bf16((rng.integers(-16, 16, (2, Hq, D)) / 64.0).astype(np.float32))
    scale = 0.25 / 127
    want = O.decode_ref(q, kb, vb, tables, ctx, scale)
    got = Q.decode_int8_ref(q, kcod, ksc, vcod, vsc, tables, ctx, scale)
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    qp = f32_bits_to_bf16((rng.integers(-16, 16, (9, Hq, D)) / 64.0).astype(np.float32))
    cu = [0, 4, 9]
    want = O.prefill_ref(qp, cu, kb, vb, tables, ctx, scale)
    got = Q.prefill_int8_ref(qp, cu, kcod, ksc, vcod, vsc, tables, ctx, scale)
    assert np.allclose(got, want, rtol=0, atol=1e-12)


PINS = [check_bytes_printed, check_integer_rows_exact, check_round_half_even, check_zero_row,
        check_extremes_and_signs, check_error_bound_and_page_figure, check_scale_per_row,
        check_append_semantics, check_gather_brute_force, check_attention_reduces_to_bf16_oracle]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ------------------------------------------------------------- mutants ---

def _mutants():
    orig_q, orig_dq = Q.quantize_ref, Q.dequantize_ref

    def whole_tensor_scale(x):
        x = np.asarray(x, np.float32)
        scale = np.full(x.shape[:-1], np.abs(x).max() / Q.INT8_MAX + Q.SCALE_EPS, np.float32)
        return np.clip(np.rint(x / scale[..., None]), -127, 127).astype(np.int8), scale

    def round_half_up(x):
        x = np.asarray(x, np.float32)
        scale = np.abs(x).max(axis=-1) / Q.INT8_MAX + Q.SCALE_EPS
        return np.clip(np.floor(x / scale[..., None] + 0.5), -127, 127).astype(np.int8), scale

    def range_128(x):
        x = np.asarray(x, np.float32)
        scale = np.abs(x).max(axis=-1) / np.float32(128.0) + Q.SCALE_EPS
        return np.clip(np.rint(x / scale[..., None]), -128, 127).astype(np.int8), scale

    def no_eps(x):
        x = np.asarray(x, np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            scale = np.abs(x).max(axis=-1) / Q.INT8_MAX
            return np.clip(np.rint(x / scale[..., None]), -127, 127).astype(np.int8), scale

    def truncate(x):
        x = np.asarray(x, np.float32)
        scale = np.abs(x).max(axis=-1) / Q.INT8_MAX + Q.SCALE_EPS
        return np.clip(np.trunc(x / scale[..., None]), -127, 127).astype(np.int8), scale

    def dequant_divides(codes, scales):
        return np.asarray(codes).astype(np.float32) / np.asarray(scales, np.float32)[..., None]

    def dequant_head0_scale(codes, scales):
        s = np.asarray(scales, np.float32)
        return orig_dq(codes, np.broadcast_to(s[..., :1], s.shape)) if s.ndim >= 2 else orig_dq(codes, s)

    return {
        "scale over the whole tensor": ("quantize_ref", whole_tensor_scale),
        "round half up": ("quantize_ref", round_half_up),
        "range 128": ("quantize_ref", range_128),
        "no epsilon": ("quantize_ref", no_eps),
        "truncation": ("quantize_ref", truncate),
        "dequantise divides": ("dequantize_ref", dequant_divides),
        "scale of head 0 for all heads": ("dequantize_ref", dequant_head0_scale),
    }


@pytest.mark.parametrize("name", list(_mutants()))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = _mutants()[name]
    monkeypatch.setattr(Q, attr, fn)
    failed = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception:
            failed += 1
    assert failed > 0, f"mutant '{name}' passes every pin"
