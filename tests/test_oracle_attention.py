"""Pins for the oracle's attention, int8-path formula, decode and merge (CPU).

Checked against closed forms (q = 0, one and two tokens), a library routine
(torch float64 scaled-dot-product attention and logsumexp), and identities
the pages fix: the tiers combine without approximation ("ActiveKV" page,
"The idea"), an unwritten -inf row is an empty partial ("SYCL" page, "A merge
that joins the tiers"), and the int8-path formula equals dequantize-then-attend
("SYCL" page, "Attention that reads 8-bit history").
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as O
from quantized_paged_kv_akv_amd import configs, inputs

SIG = 1.0 / 16.0


def rand_qkv(seed, n, D=256):
    r = np.random.default_rng(seed)
    q = r.standard_normal(D)
    K = r.standard_normal((n, D)) * np.exp(r.uniform(-2, 2, D))
    V = r.standard_normal((n, D))
    return q, K, V


def test_q_zero_gives_mean_and_log_n():
    q, K, V = rand_qkv(0, 137)
    o, lse = O.attend(np.zeros_like(q), K, V, SIG)
    np.testing.assert_allclose(o, V.mean(axis=0), rtol=1e-13, atol=1e-14)
    assert abs(lse - math.log(137)) < 1e-13


def test_one_and_two_tokens():
    q, K, V = rand_qkv(1, 2)
    o, lse = O.attend(q, K[:1], V[:1], SIG)
    np.testing.assert_allclose(o, V[0], rtol=1e-15)
    assert abs(lse - SIG * float(q @ K[0])) < 1e-12
    z = SIG * (K @ q)
    a = 1.0 / (1.0 + math.exp(z[1] - z[0]))  # logistic weight of token 0
    o, lse = O.attend(q, K, V, SIG)
    np.testing.assert_allclose(o, a * V[0] + (1 - a) * V[1], rtol=1e-12, atol=1e-13)
    assert abs(lse - (max(z) + math.log1p(math.exp(-abs(z[0] - z[1]))))) < 1e-12


@pytest.mark.parametrize("n", [1, 64, 300])
def test_matches_torch_float64_attention(n):
    q, K, V = rand_qkv(2 + n, n)
    o, lse = O.attend(q, K, V, SIG)
    tq = torch.from_numpy(q)[None, None, None]
    tk = torch.from_numpy(K)[None, None]
    tv = torch.from_numpy(V)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=SIG)[0, 0, 0].numpy()
    ref_lse = torch.logsumexp(SIG * (torch.from_numpy(K) @ torch.from_numpy(q)), 0).item()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    assert abs(lse - ref_lse) < 1e-12


def test_empty_is_zero_minus_inf():
    o, lse = O.attend(np.ones(8), np.zeros((0, 8)), np.zeros((0, 8)), SIG)
    assert lse == -math.inf and np.all(o == 0)


def test_merge_split_invariance_and_identities():
    q, K, V = rand_qkv(5, 400)
    full_o, full_l = O.attend(q, K, V, SIG)
    r = np.random.default_rng(9)
    for cuts in ([64, 128, 192, 256, 320], sorted(r.choice(np.arange(1, 400), 7, replace=False))):
        bounds = [0] + list(cuts) + [400]
        parts = [O.attend(q, K[a:b], V[a:b], SIG) for a, b in zip(bounds[:-1], bounds[1:])]
        po = np.stack([p[0] for p in parts])[:, None]
        pl = np.array([[p[1]] for p in parts])
        mo, ml = O.merge(po, pl)
        np.testing.assert_allclose(mo[0], full_o, rtol=1e-12, atol=1e-13)
        assert abs(ml[0] - full_l) < 1e-12
        # commutative
        perm = r.permutation(len(parts))
        mo2, ml2 = O.merge(po[perm], pl[perm])
        np.testing.assert_allclose(mo2, mo, rtol=1e-14, atol=1e-15)
    # merging with an empty (-inf) partial is the identity, exactly
    po = np.stack([full_o, np.full_like(full_o, 123.0)])[:, None]
    pl = np.array([[full_l], [-math.inf]])
    mo, ml = O.merge(po, pl)
    np.testing.assert_array_equal(mo[0], full_o)
    assert ml[0] == full_l
    # all empty
    mo, ml = O.merge(np.zeros((3, 2, 8)), np.full((3, 2), -math.inf))
    assert np.all(mo == 0) and np.all(ml == -math.inf)


def _small_int8_setup(seed=0, Hkv=2, G=3, B=3, pages=(5, 0, 3), permute=True):
    """A small pool quantized by the oracle, with a permuted page table."""
    r = np.random.default_rng(seed)
    D, P = 256, 64
    total = sum(pages)
    slots = r.permutation(total) if permute else np.arange(total)
    K = (r.standard_normal((total, Hkv, P, D)) * np.exp(r.uniform(-2, 2, (1, Hkv, 1, D))))
    V = r.standard_normal((total, Hkv, D, P))
    kpool = inputs.f32_to_bf16_bits(K.astype(np.float32))
    vpool = inputs.f32_to_bf16_bits(V.astype(np.float32))
    src = np.arange(total, dtype=np.int32)
    dst = slots.astype(np.int32)
    qz = O.quantize_pages(kpool, vpool, src, dst, total, Hkv)
    table = np.zeros((B, max(pages)), np.int32)
    off = 0
    for b, n in enumerate(pages):
        table[b, :n] = dst[off: off + n]
        off += n
    q = inputs.f32_to_bf16_bits(r.standard_normal((B, Hkv * G, D)).astype(np.float32))
    return q, qz, table, np.array(pages, np.int32), Hkv, G


def test_int8_formula_equals_dequantize_then_attend():
    q, qz, table, npg, Hkv, G = _small_int8_setup()
    args = (q, qz["k_codes"], qz["v_codes"], qz["k_chan"], qz["k_tok"], qz["v_chan"], table, npg,
            Hkv, G, SIG)
    o0, l0 = O.decode_int8(*args, mode=0)
    o1, l1 = O.decode_int8(*args, mode=1)
    np.testing.assert_allclose(o1, o0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1, l0, rtol=0, atol=1e-12)
    assert np.all(l0[1] == -math.inf) and np.all(o0[1] == 0)


def test_int8_decode_matches_gathered_dense():
    """Page-table gather + GQA head map: decode_int8 equals dense attention
    over tokens gathered here with numpy indexing and dequantized by hand."""
    q, qz, table, npg, Hkv, G = _small_int8_setup(seed=4)
    o, l = O.decode_int8(q, qz["k_codes"], qz["v_codes"], qz["k_chan"], qz["k_tok"],
                         qz["v_chan"], table, npg, Hkv, G, SIG)
    for b in range(len(npg)):
        if npg[b] == 0:
            continue
        sl = table[b, : npg[b]]
        for j in range(Hkv * G):
            h = j // G
            kc = qz["k_codes"][sl, h].astype(np.float64)          # [n][P][D]
            vc = qz["v_codes"][sl, h].astype(np.float64)          # [n][D][P]
            Kd = kc * qz["k_chan"][sl, h][:, None, :] * qz["k_tok"][sl, h][:, :, None]
            Vd = (vc * qz["v_chan"][sl, h][:, :, None]).transpose(0, 2, 1)
            qq = O.bf16_bits_to_f64(q[b, j])
            tq = torch.from_numpy(qq)[None, None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(
                tq, torch.from_numpy(Kd.reshape(-1, 256))[None, None],
                torch.from_numpy(Vd.reshape(-1, 256))[None, None], scale=SIG)[0, 0, 0].numpy()
            np.testing.assert_allclose(o[b, j], ref, rtol=1e-11, atol=1e-11)


def test_exact_decode_partial_page_and_permutation():
    w = configs.tiny()
    d = inputs.make_layer_np(w, 0)
    plan = d["plan"]
    for n_tok in (1, 63, 64, 65, 200, 512):
        table = plan.full_table()
        o, l = O.decode_exact(d["q"], d["k_pool"], d["v_pool"], table, np.array([n_tok]),
                              w.num_kv_heads, w.group, SIG)
        # gather by hand
        K = O.bf16_bits_to_f64(d["k_pool"][table[0], 0]).reshape(-1, 256)[:n_tok]
        V = O.bf16_bits_to_f64(d["v_pool"][table[0], 0]).transpose(0, 2, 1).reshape(-1, 256)[:n_tok]
        for j in range(w.num_q_heads):
            qq = O.bf16_bits_to_f64(d["q"][0, j])
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qq)[None, None, None], torch.from_numpy(K)[None, None],
                torch.from_numpy(V)[None, None], scale=SIG)[0, 0, 0].numpy()
            np.testing.assert_allclose(o[0, j], ref, rtol=1e-11, atol=1e-12)
    # relocating pages in the pool (and the table with them) changes nothing
    r = np.random.default_rng(1)
    perm = r.permutation(plan.bf16_slots_total)
    kp = np.empty_like(d["k_pool"]); kp[perm] = d["k_pool"]
    vp = np.empty_like(d["v_pool"]); vp[perm] = d["v_pool"]
    t2 = perm[plan.full_table()].astype(np.int32)
    o1, l1 = O.decode_exact(d["q"], d["k_pool"], d["v_pool"], plan.full_table(), np.array([500]), 1, 2, SIG)
    o2, l2 = O.decode_exact(d["q"], kp, vp, t2, np.array([500]), 1, 2, SIG)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_tiers_merge_to_full_attention():
    """merge(int8 tier, BF16 window) equals dense attention over the whole
    history (int8 pages dequantized, window exact)."""
    w = configs.tiny()
    d = inputs.make_layer_np(w, 0)
    plan = d["plan"]
    src, dst = plan.quant_src_dst()
    qz = O.quantize_pages(d["k_pool"], d["v_pool"], src, dst, plan.int8_slots_total, 1)
    o8, l8 = O.decode_int8(d["q"], qz["k_codes"], qz["v_codes"], qz["k_chan"], qz["k_tok"],
                           qz["v_chan"], plan.int8_table(), np.array(plan.n8), 1, 2, SIG)
    ow, lw = O.decode_exact(d["q"], d["k_pool"], d["v_pool"], plan.window_table(),
                            np.array(plan.win_tokens), 1, 2, SIG)
    mo, ml = O.merge(np.stack([o8[0], ow[0]]), np.stack([l8[0], lw[0]]))
    # dense over the concatenated history
    kc = qz["k_codes"][plan.int8_table()[0], 0].astype(np.float64)
    K8 = (kc * qz["k_chan"][plan.int8_table()[0], 0][:, None, :]
          * qz["k_tok"][plan.int8_table()[0], 0][:, :, None]).reshape(-1, 256)
    vc = qz["v_codes"][plan.int8_table()[0], 0].astype(np.float64)
    V8 = (vc * qz["v_chan"][plan.int8_table()[0], 0][:, :, None]).transpose(0, 2, 1).reshape(-1, 256)
    Kw = O.bf16_bits_to_f64(d["k_pool"][plan.window_table()[0], 0]).reshape(-1, 256)
    Vw = O.bf16_bits_to_f64(d["v_pool"][plan.window_table()[0], 0]).transpose(0, 2, 1).reshape(-1, 256)
    K = np.concatenate([K8, Kw])
    V = np.concatenate([V8, Vw])
    for j in range(2):
        o, l = O.attend(O.bf16_bits_to_f64(d["q"][0, j]), K, V, SIG)
        np.testing.assert_allclose(mo[j], o, rtol=1e-12, atol=1e-12)
        assert abs(ml[j] - l) < 1e-12
