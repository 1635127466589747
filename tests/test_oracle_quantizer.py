"""Pins for the oracle's 8-bit page quantizer (CPU only).

Each test checks the oracle against something other than itself: a
hand-worked example, closed forms, invariants the format fixes, and exact
rational rounding.  Format: "Model quantization" page, section "An 8-bit page
format shaped for its kernel".
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def f32(x):
    return float(np.float32(x))


def rne(fr: Fraction) -> int:
    """Round a rational half-to-even (exact)."""
    fl = math.floor(fr)
    rem = fr - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def random_page(seed, P=64, D=256, outliers=True):
    r = np.random.default_rng(seed)
    sk = np.exp(r.uniform(np.log(0.1), np.log(10), D))
    sv = np.exp(r.uniform(np.log(0.5), np.log(2), D))
    K = r.standard_normal((P, D)) * sk
    V = r.standard_normal((P, D)) * sv
    if outliers:
        K[3] *= 8
        V[3] *= 8
    # BF16-representable values, as the pools hold
    K = K.astype(np.float32).astype(np.float64)
    V = V.astype(np.float32).astype(np.float64)
    return K, V


def test_worked_example_page():
    fx = json.load(open(os.path.join(HERE, "golden", "worked_example_page.json")))
    P, D = fx["P"], fx["D"]
    mag = np.array(fx["k_magnitude"])
    sign = np.array([[-1.0 if (t + d) % 3 == 0 else 1.0 for d in range(D)] for t in range(P)])
    K = sign * mag
    wc = fx["v_weight_cycle"]
    V = np.array([[wc[t % len(wc)] * 4.0 ** d for d in range(D)] for t in range(P)])

    c64, c32, s32, vs32 = O.page_scales(K, V)
    c_exp = np.array([2.0 ** e for e in fx["c_log2"]])
    np.testing.assert_allclose(c64, c_exp, rtol=1e-14)
    assert abs(np.prod(c64) - 1.0) < 1e-14
    for d in range(D):
        assert c32[d] == np.float32(c_exp[d])
    s_exp = 2.0 ** fx["s_log2_numerator"] / fx["s_denominator"]
    # s is computed from the FP32 channel factors, so it may sit an ulp or two off
    np.testing.assert_allclose(s32.astype(np.float64), s_exp, rtol=3e-7)
    vs_exp = np.array([2.0 ** e / fx["vs_denominator"] for e in fx["vs_log2_numerator"]])
    np.testing.assert_array_equal(vs32, vs_exp.astype(np.float32))

    kc, vc, kt, vt, ties = O.page_codes(K, V, c32, s32, vs32)
    for t in range(P):
        for d in range(D):
            m = fx["k_code_magnitude"][d]
            if m is None:
                exact = Fraction(float(K[t, d])) / (Fraction(float(c32[d])) * Fraction(float(s32[t])))
                m_signed = rne(exact)
            else:
                m_signed = int(sign[t, d]) * m
            assert kc[t, d] == m_signed, (t, d, kc[t, d], m_signed)
    vexp = np.array([[fx["v_code_cycle"][t % 5] for d in range(D)] for t in range(P)])
    np.testing.assert_array_equal(vc, vexp)
    assert ties == 0


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_invariants_random_page(seed):
    K, V = random_page(seed)
    c64, c32, s32, vs32 = O.page_scales(K, V)
    # factors multiply to one (no clamp binds for these draws)
    assert abs(np.sum(np.log2(c64))) < 1e-9
    assert abs(np.sum(np.log2(c32.astype(np.float64)))) <= 256 * 2.0 ** -24 / math.log(2) + 1e-12
    assert np.all(c32 >= 2.0 ** -14) and np.all(c32 <= 2.0 ** 14)
    kc, vc, _, _, _ = O.page_codes(K, V, c32, s32, vs32)
    assert np.all(np.abs(kc.astype(int)) <= 127) and np.all(np.abs(vc.astype(int)) <= 127)
    assert np.all(kc != -128) and np.all(vc != -128)
    # every nonzero token row and every nonzero V channel reaches +-127
    assert np.all(np.abs(kc.astype(int)).max(axis=1) == 127)
    assert np.all(np.abs(vc.astype(int)).max(axis=0) == 127)
    # reconstruction error at most half a step
    step = c32.astype(np.float64)[None, :] * s32.astype(np.float64)[:, None]
    assert np.all(np.abs(K - kc * step) <= 0.5 * step * (1 + 1e-12))
    vstep = vs32.astype(np.float64)[None, :]
    assert np.all(np.abs(V - vc * vstep) <= 0.5 * vstep * (1 + 1e-12))


def test_channel_power_law():
    """Scaling one channel by 4^k moves its factor by 2^(k(1-1/D)) and every
    other factor by 2^(-k/D): the factor absorbs half the channel's range and
    the normalisation is geometric."""
    K, V = random_page(7, D=64)
    D = K.shape[1]
    c0, _, _, _ = O.page_scales(K, V)
    for k in (1, 2, -3):
        K2 = K.copy()
        K2[:, 5] *= 4.0 ** k
        c1, _, _, _ = O.page_scales(K2, V)
        ratio = c1 / c0
        np.testing.assert_allclose(ratio[5], 2.0 ** (k * (1 - 1 / D)), rtol=1e-12)
        others = np.delete(ratio, 5)
        np.testing.assert_allclose(others, 2.0 ** (-k / D), rtol=1e-12)


def test_scale_equivariance():
    """Scaling a page by 16 leaves channel factors and codes unchanged and
    multiplies token factors by 16."""
    K, V = random_page(11)
    c64, c32, s32, vs32 = O.page_scales(K, V)
    c64b, c32b, s32b, vs32b = O.page_scales(16 * K, 16 * V)
    np.testing.assert_allclose(c64b, c64, rtol=1e-14)
    np.testing.assert_allclose(s32b.astype(np.float64), 16 * s32.astype(np.float64), rtol=2.4e-7)
    np.testing.assert_allclose(vs32b.astype(np.float64), 16 * vs32.astype(np.float64), rtol=2.4e-7)
    kc, vc, kt, vt, _ = O.page_codes(K, V, c32, s32, vs32)
    kcb, vcb, _, _, _ = O.page_codes(16 * K, 16 * V, c32b, s32b, vs32b)
    np.testing.assert_array_equal(kc, kcb)
    np.testing.assert_array_equal(vc, vcb)


def test_clamp_binds_after_normalisation():
    """Clamp is applied after the geometric normalisation: a channel far below
    the rest pins at 2^-14 and the product is then no longer one."""
    P, D = 64, 4
    mag = np.array([1e-30, 1.0, 1.0, 1.0])
    K = np.tile(mag, (P, 1))
    V = np.ones((P, D))
    c64, c32, s32, vs32 = O.page_scales(K, V)
    u = np.sqrt(mag)  # sqrt(RMS) for a constant channel
    g = np.exp(np.mean(np.log(u)))
    assert c64[0] == 2.0 ** -14
    np.testing.assert_allclose(c64[1:], u[1:] / g, rtol=1e-13)
    assert np.prod(c64) > 1.0 + 1e-3


def test_clamp_high():
    P, D = 64, 4
    mag = np.array([1e30, 1.0, 1.0, 1.0])
    K = np.tile(mag, (P, 1))
    c64, _, _, _ = O.page_scales(K, np.ones((P, D)))
    assert c64[0] == 2.0 ** 14


def test_zero_page_channel_token():
    P, D = 64, 16
    Z = np.zeros((P, D))
    c64, c32, s32, vs32 = O.page_scales(Z, Z)
    assert np.all(c64 == 1.0) and np.all(s32 == 0) and np.all(vs32 == 0)
    kc, vc, _, _, _ = O.page_codes(Z, Z, c32, s32, vs32)
    assert np.all(kc == 0) and np.all(vc == 0)

    # a zero channel gets factor 1 and is left out of the geometric mean:
    # the other factors equal those of the page without that channel
    K, V = random_page(3, D=D)
    Kz = K.copy()
    Kz[:, 6] = 0.0
    cz, _, _, _ = O.page_scales(Kz, V)
    cr, _, _, _ = O.page_scales(np.delete(K, 6, axis=1), np.delete(V, 6, axis=1))
    assert cz[6] == 1.0
    np.testing.assert_allclose(np.delete(cz, 6), cr, rtol=1e-14)

    # a zero token gets factor 0 and codes 0
    Kt = K.copy()
    Kt[9] = 0.0
    _, c32t, s32t, vs32t = O.page_scales(Kt, V)
    assert s32t[9] == 0.0
    kc, _, _, _, _ = O.page_codes(Kt, V, c32t, s32t, vs32t)
    assert np.all(kc[9] == 0)


def test_ties_round_half_even():
    """A page built so every channel factor is exactly 1 and every token
    factor exactly 1: codes are the round-half-even of the values, ties are
    counted."""
    base = np.array([127.0, 62.5, -62.5, 63.5, 0.5, 1.5, 2.5, -0.5])
    P, D = 64, 8
    K = np.array([np.roll(base, t % D) for t in range(P)])
    c64, c32, s32, vs32 = O.page_scales(K, K)
    assert np.all(c32 == 1.0) and np.all(s32 == 1.0) and np.all(vs32 == 1.0)
    kc, vc, kt, vt, ties = O.page_codes(K, K, c32, s32, vs32)
    expect = {127.0: 127, 62.5: 62, -62.5: -62, 63.5: 64, 0.5: 0, 1.5: 2, 2.5: 2, -0.5: 0}
    for t in range(P):
        for d in range(D):
            assert kc[t, d] == expect[K[t, d]]
            assert kt[t, d] == (K[t, d] != 127.0)
    np.testing.assert_array_equal(kc, vc)
    assert ties == 2 * 7 * P


def test_pool_quantizer_matches_page_form():
    """The pool entry point gathers, quantizes and scatters pages (V codes
    channel-major) exactly as the per-page form does."""
    from quantized_paged_kv_akv_amd import configs, inputs
    w = configs.tiny()
    d = inputs.make_layer_np(w, 0)
    src, dst = d["plan"].quant_src_dst()
    out = O.quantize_pages(d["k_pool"], d["v_pool"], src, dst, len(dst), w.num_kv_heads)
    for i in range(len(src)):
        K = O.bf16_bits_to_f64(d["k_pool"][src[i], 0])
        V = O.bf16_bits_to_f64(d["v_pool"][src[i], 0]).T
        _, c32, s32, vs32 = O.page_scales(K, V)
        kc, vc, _, _, _ = O.page_codes(K, V, c32, s32, vs32)
        np.testing.assert_array_equal(out["k_chan"][dst[i], 0], c32)
        np.testing.assert_array_equal(out["k_tok"][dst[i], 0], s32)
        np.testing.assert_array_equal(out["v_chan"][dst[i], 0], vs32)
        np.testing.assert_array_equal(out["k_codes"][dst[i], 0], kc)
        np.testing.assert_array_equal(out["v_codes"][dst[i], 0], vc.T)
    again = O.quantize_pages(d["k_pool"], d["v_pool"], src, dst, len(dst), w.num_kv_heads,
                             given=(out["k_chan"], out["k_tok"], out["v_chan"]))
    np.testing.assert_array_equal(again["k_codes"], out["k_codes"])
    np.testing.assert_array_equal(again["v_codes"], out["v_codes"])
