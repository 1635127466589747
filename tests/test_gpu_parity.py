"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Acceptance: codes bit-exact given identical FP32 scales (exact ties listed and
excluded), scales within 1e-6 relative, attention O max-abs <= 2e-3 and
rel-L2 <= 1e-3 against the oracle run on the same codes, LSE within 1e-4.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as O
from quantized_paged_kv_akv_amd import configs, inputs
from tests.gpu_util import (check_attn, check_quantize, dev, gpu_quantize, host, oracle_hybrid, oracle_int8,
                            run_exact, run_int8, say, workspace)

pytestmark = pytest.mark.gpu
SIG = 1.0 / 16.0


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from quantized_paged_kv_akv_amd import binding
    return binding


# ----------------------------------------------------------------------------- quantizer
def test_quantize_tiny(B):
    w = configs.tiny()
    d = inputs.make_layer_np(w, 0)
    plan = d["plan"]
    src = np.arange(plan.bf16_slots_total, dtype=np.int32)  # every page of the tiny history
    dst = src[::-1].copy()
    say("case quantize tiny", len(src))
    g = gpu_quantize(B, d["k_pool"], d["v_pool"], src, dst, len(src), 1)
    check_quantize(O, d["k_pool"], d["v_pool"], src, dst, len(src), 1, g, "tiny")


def test_quantize_random_pages_outliers(B):
    kp, vp = inputs.random_pools(11, 96, 4)
    src = np.arange(96, dtype=np.int32)
    dst = np.random.default_rng(3).permutation(96).astype(np.int32)
    say("case quantize random 96 pages x 4 heads")
    g = gpu_quantize(B, kp, vp, src, dst, 96, 4)
    check_quantize(O, kp, vp, src, dst, 96, 4, g, "random96")


def _edge_pages():
    """Pages that stress the format: all-zero page, zero channel, zero token,
    constant page, a channel far below the rest (clamp binds), exact ties,
    huge and tiny magnitudes, scales beyond 2^+-100 and a token whose |K| / c
    exceeds the FP32 range."""
    r = np.random.default_rng(5)
    pages_k, pages_v = [], []

    def add(K, V):
        pages_k.append(inputs.f32_to_bf16_bits(np.asarray(K, np.float32)))
        pages_v.append(inputs.f32_to_bf16_bits(np.asarray(V, np.float32).T))

    base_k = r.standard_normal((64, 256)) * np.exp(r.uniform(-2, 2, 256))
    base_v = r.standard_normal((64, 256))
    add(np.zeros((64, 256)), np.zeros((64, 256)))
    K = base_k.copy(); K[:, 17] = 0; V = base_v.copy(); V[:, 200] = 0
    add(K, V)
    K = base_k.copy(); K[5] = 0; V = base_v.copy(); V[9] = 0
    add(K, V)
    add(np.full((64, 256), 3.0), np.full((64, 256), -0.5))
    K = base_k.copy(); K[:, 3] *= 1e-30
    add(K, base_v)
    K = base_k.copy(); K[:, 100] *= 1e25
    add(K, base_v * 1e20)
    row = np.array([127.0, 62.5, -62.5, 63.5, 0.5, 1.5, 2.5, -0.5] * 32)
    T = np.array([np.roll(row, t % 8) for t in range(64)])
    add(T, T)
    add(base_k * 1e-20, base_v * 1e-30)
    # scales outside the kernel's FP32 estimate range [2^-100, 2^100]: every
    # code of such a token or channel goes through the float64 divide
    add(base_k * 1e-33, base_v * 1e-33)
    add(base_k * 1e33, base_v * 1e33)
    # |K| / c beyond the FP32 range although s_t is finite: channel 0 holds
    # one huge value (so c_0 < 1) while every other channel is huge throughout
    K = np.full((64, 256), 3.0e38); K[:, 0] = 0.0; K[7, 0] = 3.0e38
    add(K, base_v)
    kp = np.stack(pages_k)[:, None]
    vp = np.stack(pages_v)[:, None]
    return kp, vp


def test_quantize_edge_pages(B):
    kp, vp = _edge_pages()
    n = kp.shape[0]
    src = np.arange(n, dtype=np.int32)
    say("case quantize edge pages", n)
    g = gpu_quantize(B, kp, vp, src, src, n, 1)
    ties = check_quantize(O, kp, vp, src, src, n, 1, g, "edge")
    assert ties > 0  # the tie page must produce listed ties
    kc = host(g["k_codes"])
    assert np.all(kc[0] == 0) and np.all(host(g["k_tok"])[0] == 0) and np.all(host(g["k_chan"])[0] == 1)
    assert host(g["k_chan"])[4, 0, 3] == np.float32(2.0 ** -14)


# ----------------------------------------------------------------------------- merge
def test_merge_lse(B):
    r = np.random.default_rng(2)
    rows = 37
    ao = r.standard_normal((rows, 256)).astype(np.float32)
    po = r.standard_normal((rows, 256)).astype(np.float32)
    al = r.uniform(-5, 50, rows).astype(np.float32)
    pl = r.uniform(-5, 50, rows).astype(np.float32)
    al[[0, 5]] = -np.inf
    pl[[0, 7]] = -np.inf
    ao[[0, 5]] = 0.0
    po[[0, 7]] = 0.0
    acc_o, acc_l = dev(ao), dev(al)
    say("case merge_lse rows", rows)
    B.akv_merge_lse(rows, 256, acc_o, acc_l, dev(po), dev(pl))
    torch.cuda.synchronize()
    ref_o, ref_l = O.merge(np.stack([ao, po]).astype(np.float64), np.stack([al, pl]).astype(np.float64))
    check_attn(acc_o, acc_l, ref_o, ref_l, "merge_lse")
    # empty-side rows are exactly the other side
    assert np.array_equal(host(acc_o)[5], po[5]) and np.array_equal(host(acc_o)[7], ao[7])
    # fill_empty then merge = identity
    fo = torch.full((rows, 256), 7.0, device="cuda")
    fl = torch.zeros(rows, device="cuda")
    B.akv_fill_empty(rows, 256, fo, fl)
    B.akv_merge_lse(rows, 256, fo, fl, dev(po), dev(pl))
    torch.cuda.synchronize()
    assert np.array_equal(host(fo), po) and np.array_equal(host(fl), pl)


# ----------------------------------------------------------------------------- int8 decode
def _int8_case(B, seed, Hkv, G, n_pages, outliers=0.02):
    total = int(sum(n_pages))
    kp, vp = inputs.random_pools(seed, max(total, 1), Hkv, outlier_frac=outliers)
    src = np.arange(max(total, 1), dtype=np.int32)
    dst = np.random.default_rng(seed + 1).permutation(max(total, 1)).astype(np.int32)
    g = gpu_quantize(B, kp, vp, src, dst, max(total, 1), Hkv)
    table = np.zeros((len(n_pages), max(1, max(n_pages))), np.int32)
    off = 0
    for b, n in enumerate(n_pages):
        table[b, :n] = dst[off: off + n]
        off += n
    q = inputs.random_queries(seed + 2, len(n_pages), Hkv * G)
    return g, table, q


@pytest.mark.parametrize("Hkv,G,n_pages", [
    (1, 2, [4]),
    (4, 6, [37]),
    (2, 6, [0, 1, 5, 64, 9]),
    (1, 8, [13, 3]),
    (3, 1, [2, 70]),
])
def test_int8_decode_parity(B, Hkv, G, n_pages):
    say(f"case int8 decode Hkv={Hkv} G={G} pages={n_pages}")
    g, table, q = _int8_case(B, 100 + Hkv * 10 + G, Hkv, G, n_pages)
    o, lse = run_int8(B, Hkv, G, q, g, table, n_pages)
    ro, rl = oracle_int8(O, Hkv, G, q, g, table, n_pages)
    check_attn(o, lse, ro, rl, f"int8 Hkv{Hkv} G{G}")


@pytest.mark.parametrize("pages_per_wave", [0, 64])
def test_int8_long_context(B, pages_per_wave):
    """A 512K-token history (8192 int8 pages) of one KV head: with the default
    plan, 512 splits (the looping second pass); with 64 pages per wave (the
    launch-shape override), every wave at the 64 page slots it can stage."""
    say(f"case int8 long context 8192 pages, pages per wave {pages_per_wave or 'planned'}")
    g, table, q = _int8_case(B, 808, 1, 4, [8192])
    B.akv_set_launch_shape(pages_per_wave=pages_per_wave)
    try:
        o, lse = run_int8(B, 1, 4, q, g, table, [8192])
    finally:
        B.akv_set_launch_shape(reset=True)
    ro, rl = oracle_int8(O, 1, 4, q, g, table, [8192])
    check_attn(o, lse, ro, rl, "int8 8192 pages")


@pytest.mark.parametrize("pv_fp16", [0, 1])
def test_int8_pv_operands_agree(B, pv_fp16):
    """The int8 tier's PV product on the int8 MFMA (weights as three 7-bit
    fixed-point limbs, the default) and on FP16 operands (weights hi + lo,
    codes turned into FP16): each within the tolerances of the oracle, and
    the two within 1e-4 of each other."""
    say(f"case int8 PV operand, pv_fp16={pv_fp16}")
    g, table, q = _int8_case(B, 515, 4, 6, [300, 41])
    B.akv_set_launch_shape(pv_fp16=pv_fp16)
    try:
        o, lse = run_int8(B, 4, 6, q, g, table, [300, 41])
    finally:
        B.akv_set_launch_shape(reset=True)
    ro, rl = oracle_int8(O, 4, 6, q, g, table, [300, 41])
    check_attn(o, lse, ro, rl, f"int8 PV operand fp16={pv_fp16}")
    o_other, l_other = run_int8(B, 4, 6, q, g, table, [300, 41]) if pv_fp16 else (o, lse)
    assert float((o - o_other).abs().max()) <= 1e-4 and float((lse - l_other).abs().max()) <= 1e-5


@pytest.mark.parametrize("weights", ["uniform", "sharp"])
def test_int8_pv_limbs_degenerate_weights(B, weights):
    """The softmax weights' fixed-point limbs at their ends: q = 0 makes every
    weight exactly 1 (every limb 127; O is the mean of the dequantized values,
    LSE = ln(tokens)), and a query 4x the usual scale makes the attention so
    sharp that most weights round to 0 against the largest."""
    say(f"case int8 PV limbs, {weights} weights")
    g, table, q = _int8_case(B, 616, 2, 6, [90, 7])
    if weights == "uniform":
        q = np.zeros_like(q)
    else:
        q = inputs.random_queries(617, 2, 12, scale=4.0)
    o, lse = run_int8(B, 2, 6, q, g, table, [90, 7])
    ro, rl = oracle_int8(O, 2, 6, q, g, table, [90, 7])
    check_attn(o, lse, ro, rl, f"int8 PV limbs {weights}")
    if weights == "uniform":
        assert np.allclose(host(lse), np.log(np.array([90, 7]) * 64.0)[:, None], atol=1e-5)


def test_int8_decode_deterministic(B):
    g, table, q = _int8_case(B, 7, 4, 6, [150])
    say("case int8 determinism")
    o1, l1 = run_int8(B, 4, 6, q, g, table, [150])
    o2, l2 = run_int8(B, 4, 6, q, g, table, [150])
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_int8_wide_channel_range(B):
    """Channel factors far from 1 (key channel stds spanning 1e-3..1e3) keep
    the query's precision: per-column power-of-two scaling before the FP16
    split.  Queries are scaled so the logits stay in the workloads' range
    (|LSE| below ~100): an FP32 LSE near 500 has a spacing of 3e-5, which
    leaves no room for a 1e-4 absolute bound."""
    say("case int8 wide channel range")
    kp, vp = inputs.random_pools(21, 6, 2, outlier_frac=0.0, k_std=(1e-3, 1e3))
    src = np.arange(6, dtype=np.int32)
    g = gpu_quantize(B, kp, vp, src, src, 6, 2)
    table = np.array([[0, 1, 2], [3, 4, 5]], np.int32)
    q = inputs.random_queries(22, 2, 2 * 4, scale=0.1)
    o, lse = run_int8(B, 2, 4, q, g, table, [3, 3])
    ro, rl = oracle_int8(O, 2, 4, q, g, table, [3, 3])
    check_attn(o, lse, ro, rl, "int8 wide-range")


# ----------------------------------------------------------------------------- exact decode
@pytest.mark.parametrize("Hkv,G,seq_len", [
    (1, 2, [256]),
    (4, 6, [1087]),
    (2, 6, [0, 1, 63, 64, 65, 700]),
    (1, 8, [1024, 1]),
])
def test_exact_decode_parity(B, Hkv, G, seq_len):
    say(f"case exact decode Hkv={Hkv} G={G} seq_len={seq_len}")
    pages = [(s + 63) // 64 for s in seq_len]
    total = max(1, sum(pages))
    kp, vp = inputs.random_pools(300 + G, total, Hkv)
    slots = np.random.default_rng(9).permutation(total).astype(np.int32)
    table = np.zeros((len(seq_len), max(1, max(pages))), np.int32)
    off = 0
    for b, n in enumerate(pages):
        table[b, :n] = slots[off: off + n]
        off += n
    q = inputs.random_queries(301, len(seq_len), Hkv * G)
    o, lse = run_exact(B, Hkv, G, q, dev(kp), dev(vp), table, seq_len)
    ro, rl = O.decode_exact(q, kp, vp, table, np.asarray(seq_len, np.int32), Hkv, G, SIG)
    check_attn(o, lse, ro, rl, f"exact Hkv{Hkv} G{G}")


@pytest.mark.parametrize("n_pages", [4, 5, 8, 9, 16, 17, 64, 65, 100, 128, 129, 200, 300])
def test_split_combine_paths(B, n_pages):
    """One page per split (a launch-shape override) so the split-K second pass
    folds that many partials per row, on each side of every boundary between
    its kernels: one thread per 4 channels folding every column (up to 4, 8
    and 16 columns), the in-wave reductions (up to 64 and up to 128), the
    register path (up to 256) and the looping path; the last page is partial
    and one request is empty."""
    seq_len = [64 * n_pages - 17, 0]
    say(f"case split combine n_pages={n_pages}")
    kp, vp = inputs.random_pools(500 + n_pages, n_pages, 1)
    table = np.zeros((2, n_pages), np.int32)
    table[0] = np.random.default_rng(n_pages).permutation(n_pages)
    q = inputs.random_queries(501, 2, 4)
    B.akv_set_launch_shape(pages_per_split=1)
    try:
        o, lse = run_exact(B, 1, 4, q, dev(kp), dev(vp), table, seq_len)
    finally:
        B.akv_set_launch_shape(reset=True)
    ro, rl = O.decode_exact(q, kp, vp, table, np.asarray(seq_len, np.int32), 1, 4, SIG)
    check_attn(o, lse, ro, rl, f"combine {n_pages} splits")


def test_exact_partial_page_ignores_garbage(B):
    """Tokens past seq_len in the last page may hold anything (here NaN and
    Inf bit patterns); they must not reach the result."""
    say("case exact partial page with non-finite padding")
    kp, vp = inputs.random_pools(41, 2, 1)
    kp[1, 0, 10:] = 0x7FC0  # NaN
    vp[1, 0, :, 10:] = 0x7F80  # +Inf
    table = np.array([[0, 1]], np.int32)
    q = inputs.random_queries(42, 1, 2)
    o, lse = run_exact(B, 1, 2, q, dev(kp), dev(vp), table, [74])
    ro, rl = O.decode_exact(q, kp, vp, table, np.array([74], np.int32), 1, 2, SIG)
    check_attn(o, lse, ro, rl, "exact garbage-pad")


# ----------------------------------------------------------------------------- whole hybrid layer
def _hybrid_layer(B, w, d, layer_tag, heads_check=None):
    plan = d["plan"]
    Hkv, G = w.num_kv_heads, w.group
    src, dst = plan.quant_src_dst()
    g = gpu_quantize(B, d["k_pool"], d["v_pool"], src, dst, max(1, plan.int8_slots_total), Hkv)
    kpt, vpt = dev(d["k_pool"]), dev(d["v_pool"])
    t8, tw = plan.int8_table(), plan.window_table()
    o8, l8 = run_int8(B, Hkv, G, d["q"], g, t8, plan.n8)
    ow, lw = run_exact(B, Hkv, G, d["q"], kpt, vpt, tw, plan.win_tokens)
    rows = w.batch * w.num_q_heads
    acc_o = torch.empty((w.batch, w.num_q_heads, 256), device="cuda")
    acc_l = torch.empty((w.batch, w.num_q_heads), device="cuda")
    B.akv_fill_empty(rows, 256, acc_o, acc_l)
    B.akv_merge_lse(rows, 256, acc_o, acc_l, o8, l8)
    B.akv_merge_lse(rows, 256, acc_o, acc_l, ow, lw)
    torch.cuda.synchronize()
    # oracle on the GPU's codes: int8 tier, window tier, merged
    ro8, rl8 = oracle_int8(O, Hkv, G, d["q"], g, t8, plan.n8)
    row, rlw = O.decode_exact(d["q"], d["k_pool"], d["v_pool"], tw, np.asarray(plan.win_tokens, np.int32),
                              Hkv, G, SIG)
    rm, rlm = O.merge(np.stack([ro8.reshape(rows, 256), row.reshape(rows, 256)]),
                      np.stack([rl8.reshape(rows), rlw.reshape(rows)]))
    check_attn(o8, l8, ro8, rl8, f"{layer_tag} int8 tier")
    check_attn(ow, lw, row, rlw, f"{layer_tag} window tier")
    check_attn(acc_o.view(rows, 256), acc_l.view(rows), rm, rlm, f"{layer_tag} merged")
    # the fused hybrid entry point (both tiers in one launch, one exact fold)
    d8 = B.dims(Hkv, G)
    ws = torch.empty(max(16, B.akv_decode_hybrid_workspace_bytes(d8, w.batch, t8.shape[1], tw.shape[1])),
                     dtype=torch.uint8, device="cuda")
    ho = torch.full((w.batch, w.num_q_heads, 256), float("nan"), device="cuda")
    hl = torch.full((w.batch, w.num_q_heads), float("nan"), device="cuda")
    B.akv_decode_hybrid(d8, w.batch, dev(d["q"]), g["k_codes"], g["v_codes"], g["k_chan"], g["k_tok"],
                        g["v_chan"], dev(t8), dev(np.asarray(plan.n8, np.int32)), t8.shape[1], kpt, vpt, dev(tw),
                        dev(np.asarray(plan.win_tokens, np.int32)), tw.shape[1], SIG, ho, hl, ws)
    torch.cuda.synchronize()
    check_attn(ho.view(rows, 256), hl.view(rows), rm, rlm, f"{layer_tag} fused hybrid")
    return g


def test_hybrid_tiny(B):
    w = configs.tiny()
    d = inputs.make_layer_np(w, 0)
    say("case hybrid tiny")
    _hybrid_layer(B, w, d, "tiny")


def test_hybrid_batched_subset(B):
    """Four requests of the batched workload (two equal-length pairs),
    permuted pools, 512-token windows."""
    full = configs.batched()
    w = inputs.Workload("batched4", full.cfg_id, batch=4, layers=1, num_kv_heads=4, group=6,
                        lengths=full.lengths[:4], window=512, outlier_frac=0.02, permute=True)
    d = inputs.make_layer_np(w, 0)
    say("case hybrid batched subset", w.lengths)
    _hybrid_layer(B, w, d, "batched4")


def test_two_owner_equals_one_row_calls(B):
    """One launch of two requests with equal page counts (each with its own
    table row and output rows) equals two single-request launches."""
    say("case two-owner")
    g, table, q = _int8_case(B, 55, 4, 6, [40, 40])
    o2, l2 = run_int8(B, 4, 6, q, g, table, [40, 40])
    for b in range(2):
        o1, l1 = run_int8(B, 4, 6, q[b:b + 1], g, table[b:b + 1], [40])
        np.testing.assert_allclose(host(o1)[0], host(o2)[b], rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(host(l1)[0], host(l2)[b], rtol=0, atol=1e-6)
    ro, rl = oracle_int8(O, 4, 6, q, g, table, [40, 40])
    check_attn(o2, l2, ro, rl, "two-owner")


def test_ctx32k_layer_full_size(B):
    """One full 32K layer (496 int8 pages + 1024-token window per KV head):
    the entire output checked against the oracle."""
    w = configs.ctx32k()
    d = inputs.make_layer_np(w, 3)
    say("case ctx32k layer 3")
    g = _hybrid_layer(B, w, d, "ctx32k")
    plan = d["plan"]
    src, dst = plan.quant_src_dst()
    sel = np.random.default_rng(0).choice(len(src), 48, replace=False)
    check_quantize(O, d["k_pool"], d["v_pool"], src[sel], dst[sel], plan.int8_slots_total, 4, g, "ctx32k sample")


def test_ctx128k_layer_full_size(B):
    """One full 128K layer (2032 int8 pages + 16 window pages per KV head) in
    the launch shape the benchmark times: every output row of the int8 tier,
    the window tier, their merge and the fused hybrid call against the oracle;
    a sample of pages through the quantizer check."""
    w = configs.ctx128k()
    d = inputs.make_layer_np(w, 5)
    say("case ctx128k layer 5")
    g = _hybrid_layer(B, w, d, "ctx128k")
    plan = d["plan"]
    src, dst = plan.quant_src_dst()
    sel = np.random.default_rng(1).choice(len(src), 32, replace=False)
    check_quantize(O, d["k_pool"], d["v_pool"], src[sel], dst[sel], plan.int8_slots_total, 4, g, "ctx128k sample")


def test_batched_full_size(B):
    """All 32 requests of the batched workload (lengths 4K-16K in equal-length
    pairs, permuted pools, 512-token windows) in one launch per tier."""
    w = configs.batched()
    d = inputs.make_layer_np(w, 1)
    say("case batched 32 requests, layer 1")
    _hybrid_layer(B, w, d, "batched32")


@pytest.mark.parametrize("case", ["ctx32k", "batched4"])
def test_issue_priority_probe_keeps_outputs(B, case):
    """The issue-priority probe (akv_set_launch_shape issue_priority 1: by
    pages left, 2: by wave index) changes only how the waves of a compute unit
    interleave, so the fused hybrid layer, the int8 tier alone and the exact
    tier alone must give bit-identical outputs under it.  (A hand-written
    conversion whose half-register writes were read by the very next
    instruction passed every parity test at the default priorities and went
    wrong under this probe.)"""
    if case == "ctx32k":
        w = configs.ctx32k()
    else:
        full = configs.batched()
        w = inputs.Workload("batched4", full.cfg_id, batch=4, layers=1, num_kv_heads=4, group=6,
                            lengths=full.lengths[:4], window=512, outlier_frac=0.02, permute=True)
    d = inputs.make_layer_np(w, 7)
    say("case issue-priority probe", case)
    plan = d["plan"]
    Hkv, G = w.num_kv_heads, w.group
    src, dst = plan.quant_src_dst()
    g = gpu_quantize(B, d["k_pool"], d["v_pool"], src, dst, max(1, plan.int8_slots_total), Hkv)
    kpt, vpt = dev(d["k_pool"]), dev(d["v_pool"])
    t8, tw = plan.int8_table(), plan.window_table()
    n8, nw = dev(np.asarray(plan.n8, np.int32)), dev(np.asarray(plan.win_tokens, np.int32))
    q, t8d, twd = dev(d["q"]), dev(t8), dev(tw)
    d8 = B.dims(Hkv, G)
    ws = torch.empty(max(16, B.akv_decode_hybrid_workspace_bytes(d8, w.batch, t8.shape[1], tw.shape[1])),
                     dtype=torch.uint8, device="cuda")

    def run_all():
        ho = torch.full((w.batch, w.num_q_heads, 256), float("nan"), device="cuda")
        hl = torch.full((w.batch, w.num_q_heads), float("nan"), device="cuda")
        B.akv_decode_hybrid(d8, w.batch, q, g["k_codes"], g["v_codes"], g["k_chan"], g["k_tok"], g["v_chan"],
                            t8d, n8, t8.shape[1], kpt, vpt, twd, nw, tw.shape[1], SIG, ho, hl, ws)
        o8, l8 = run_int8(B, Hkv, G, d["q"], g, t8, plan.n8)
        ow, lw = run_exact(B, Hkv, G, d["q"], kpt, vpt, tw, plan.win_tokens)
        torch.cuda.synchronize()
        return [x.clone() for x in (ho, hl, o8, l8, ow, lw)]

    ref = run_all()
    try:
        for prio in (1, 2):
            B.akv_set_launch_shape(issue_priority=prio)
            got = run_all()
            for name, a, b in zip(("hybrid O", "hybrid LSE", "int8 O", "int8 LSE", "exact O", "exact LSE"),
                                  ref, got):
                assert torch.equal(a, b), f"{case}: {name} changed under issue_priority={prio}"
    finally:
        B.akv_set_launch_shape(reset=True)
    rows = w.batch * w.num_q_heads
    rm, rlm = oracle_hybrid(O, Hkv, G, d["q"], g, t8, plan.n8, d["k_pool"], d["v_pool"], tw, plan.win_tokens)
    check_attn(ref[0].view(rows, 256), ref[1].view(rows), rm, rlm, f"{case} hybrid (probe reference)")


def test_hybrid_step_replays_from_a_graph(B):
    """A two-layer hybrid step captured in a HIP graph replays to the eager
    result, several times, with eager work and synchronisations between the
    replays (decode loops capture their step)."""
    w = configs.ctx32k()
    say("case hybrid step in a graph")
    d8 = B.dims(4, 6)
    layers = []
    for li in (0, 1):
        d = inputs.make_layer_np(w, li)
        plan = d["plan"]
        src, dst = plan.quant_src_dst()
        g = gpu_quantize(B, d["k_pool"], d["v_pool"], src, dst, plan.int8_slots_total, 4)
        layers.append((dev(d["q"]), g, dev(d["k_pool"]), dev(d["v_pool"])))
    t8, tw = plan.int8_table(), plan.window_table()
    tabs = (dev(t8), dev(np.asarray(plan.n8, np.int32)), dev(tw), dev(np.asarray(plan.win_tokens, np.int32)))
    ws = torch.empty(B.akv_decode_hybrid_workspace_bytes(d8, 1, t8.shape[1], tw.shape[1]), dtype=torch.uint8,
                     device="cuda")
    outs = [(torch.zeros((1, 24, 256), device="cuda"), torch.zeros((1, 24), device="cuda")) for _ in layers]

    def step():
        for (q, g, kp, vp), (o, l) in zip(layers, outs):
            B.akv_decode_hybrid(d8, 1, q, g["k_codes"], g["v_codes"], g["k_chan"], g["k_tok"], g["v_chan"],
                                tabs[0], tabs[1], t8.shape[1], kp, vp, tabs[2], tabs[3], tw.shape[1], SIG, o, l, ws)
    step()
    torch.cuda.synchronize()
    ref = [(o.clone(), l.clone()) for o, l in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for o, l in outs:
            o.fill_(float("nan"))
            l.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (o, l), (ro, rl) in zip(outs, ref):
            assert torch.equal(o, ro) and torch.equal(l, rl), f"replay {rep} differs"
        step()  # eager work between replays
        torch.cuda.synchronize()
    # the same calls marshalled once (binding.prepare) give the same bits
    prepared = [B.prepare("akv_decode_hybrid", d8, 1, q, g["k_codes"], g["v_codes"], g["k_chan"], g["k_tok"],
                          g["v_chan"], tabs[0], tabs[1], t8.shape[1], kp, vp, tabs[2], tabs[3], tw.shape[1], SIG, o,
                          l, ws)
                for (q, g, kp, vp), (o, l) in zip(layers, outs)]
    for rep in range(2):
        for o, l in outs:
            o.fill_(float("nan"))
            l.fill_(float("nan"))
        for c in prepared:
            c()
        torch.cuda.synchronize()
        for (o, l), (ro, rl) in zip(outs, ref):
            assert torch.equal(o, ro) and torch.equal(l, rl), f"prepared call {rep} differs"


# ----------------------------------------------------------------------------- fused call edge cases
def _hybrid_custom(B, seed, Hkv, G, n8, win, null_empty_tier=False):
    """akv_decode_hybrid on hand-made tier splits (n8[b] int8 pages and
    win[b] window tokens per request, pools permuted) against the oracle on
    the GPU's codes.  With null_empty_tier, a tier with no pages in any
    request gets zero page-table columns and NULL pointers."""
    batch = len(n8)
    n8_tot, wp = int(sum(n8)), [(t + 63) // 64 for t in win]
    wp_tot = int(sum(wp))
    kp8, vp8 = inputs.random_pools(seed, max(1, n8_tot), Hkv)
    src = np.arange(max(1, n8_tot), dtype=np.int32)
    dst = np.random.default_rng(seed + 1).permutation(max(1, n8_tot)).astype(np.int32)
    g = gpu_quantize(B, kp8, vp8, src, dst, max(1, n8_tot), Hkv)
    kpw, vpw = inputs.random_pools(seed + 2, max(1, wp_tot), Hkv)
    wslots = np.random.default_rng(seed + 3).permutation(max(1, wp_tot)).astype(np.int32)
    m8 = 0 if (null_empty_tier and n8_tot == 0) else max(1, max(n8))
    mw = 0 if (null_empty_tier and wp_tot == 0) else max(1, max(wp))
    t8 = np.zeros((batch, max(1, m8)), np.int32)
    tw = np.zeros((batch, max(1, mw)), np.int32)
    o8 = ow = 0
    for b in range(batch):
        t8[b, :n8[b]] = dst[o8:o8 + n8[b]]
        tw[b, :wp[b]] = wslots[ow:ow + wp[b]]
        o8 += n8[b]
        ow += wp[b]
    q = inputs.random_queries(seed + 4, batch, Hkv * G)
    d8 = B.dims(Hkv, G)
    ws = torch.empty(max(16, B.akv_decode_hybrid_workspace_bytes(d8, batch, m8, mw)), dtype=torch.uint8,
                     device="cuda")
    ho = torch.full((batch, Hkv * G, 256), float("nan"), device="cuda")
    hl = torch.full((batch, Hkv * G), float("nan"), device="cuda")
    i8 = (g["k_codes"], g["v_codes"], g["k_chan"], g["k_tok"], g["v_chan"], dev(t8),
          dev(np.asarray(n8, np.int32)))
    wt = (dev(kpw), dev(vpw), dev(tw), dev(np.asarray(win, np.int32)))
    if m8 == 0:
        i8 = (None,) * 7
    if mw == 0:
        wt = (None,) * 4
    B.akv_decode_hybrid(d8, batch, dev(q), *i8[:7], m8, *wt, mw, SIG, ho, hl, ws)
    torch.cuda.synchronize()
    rm, rl = oracle_hybrid(O, Hkv, G, q, g, t8, n8, kpw, vpw, tw, win)
    rows = batch * Hkv * G
    check_attn(ho.view(rows, 256), hl.view(rows), rm, rl, f"hybrid n8={n8} win={win}")


@pytest.mark.parametrize("n8,win", [
    ([0], [300]),                          # context shorter than the window: no int8 page
    ([0, 61, 0, 1], [300, 1096, 0, 1024]),  # mixed batch with an empty request
    ([40, 3], [0, 0]),                     # empty windows (window tier launched, every split empty)
    ([0, 0], [0, 0]),                      # every request empty
    ([5, 0, 70], [64, 1, 0]),
])
def test_hybrid_edge_cases(B, n8, win):
    say(f"case hybrid edge n8={n8} win={win}")
    _hybrid_custom(B, 1700 + sum(n8) + sum(win), 4, 6, n8, win)


@pytest.mark.parametrize("n8,win", [([0, 0], [700, 65]), ([33, 12], [0, 0])])
def test_hybrid_one_tier_null_pointers(B, n8, win):
    """A tier with no page-table columns at all (max_pages = 0) and NULL
    pointers: the other tier alone, still through the fused call."""
    say(f"case hybrid single tier n8={n8} win={win}")
    _hybrid_custom(B, 1800 + sum(n8) + sum(win), 2, 6, n8, win, null_empty_tier=True)
