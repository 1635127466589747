"""Decode-step benchmark for hybrid-tier decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ctx128k]

A step is one decode step of the whole hot path over one request: for each of
the 16 attention layers, int8 decode over the old pages, exact BF16 decode
over the recent window, and the LSE merge of the two tiers.  Inputs (seeded
synthetic history, drawn on the device; pages quantized with the library's
own quantizer) are resident in HBM before timing starts.  Alongside the
hybrid step the same history is decoded all-BF16 (exact tier over every
page), and the quantizer's throughput is measured separately (it runs off
the decode path).

The default run (ctx128k) also measures, in the same process and outside the
headline's timed region: the 32K config and the batched config (one launch
of 32 requests, 16 two-request launches, 32 one-request launches, all-BF16)
at their real shapes; the host-staged mode from 8K to 128K next to the tier
gate's transfer-model prediction; and, in the cpu_baseline leg, the float64
oracle on the timed step's own inputs, whose outputs check every timed layer.

Prints ONE JSON line (rank 0).  `value` is KV bytes read per second by the
hybrid step; µs per step is in `ms_per_step` and `extra`.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
PAGE_INT8_BYTES = 64 * 256 * 2 + 64 * 4 + 256 * 4 * 2  # codes K+V, k_tok, k_chan, v_chan = 35,072
PAGE_BF16_BYTES = 64 * 256 * 2 * 2  # K+V = 65,536
RING_SLOTS = (2, 4)  # ring slot counts the host-staged sweep measures (the first is the reported one)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the sources and compiler flags that decide the decode
    kernel's code and launch shape, with comments and blank lines removed (a
    comment edit does not change the kernel)."""
    import re
    from quantized_paged_kv_akv_amd import build as akv_build
    h = hashlib.sha256()
    for f in ("decode.hip", "akv_device.h", "akv_host.cpp"):
        text = open(os.path.join(ROOT, "quantized_paged_kv_akv_amd", "csrc", f)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(line.rstrip() for line in text.splitlines() if line.strip()).encode())
    h.update(" ".join(f for f in akv_build.FLAGS if not f.startswith("/")).encode())
    return h.hexdigest()[:16]


def step_kv_bytes(plan, Hkv) -> dict:
    """Algorithmic KV bytes one decode step reads per layer (codes + FP32
    scales of the int8 pages, BF16 K and V of the window pages)."""
    n8 = sum(plan.n8)
    win_pages = sum((t + 63) // 64 for t in plan.win_tokens)
    return dict(int8=n8 * Hkv * PAGE_INT8_BYTES, window=win_pages * Hkv * PAGE_BF16_BYTES,
                bf16_all=sum(plan.n_pages) * Hkv * PAGE_BF16_BYTES)


def build_layers(w, device):
    """Per layer: BF16 pool (whole history), int8 pool of the old pages,
    tables.  The int8 pool is produced by akv_quantize_pages."""
    import numpy as np
    import torch

    from quantized_paged_kv_akv_amd import binding as B
    from quantized_paged_kv_akv_amd import inputs

    plan = inputs.plan_pools(w)
    Hkv = w.num_kv_heads
    dims = B.dims(Hkv, w.group)
    src, dst = plan.quant_src_dst()
    src_t = torch.as_tensor(src, device=device)
    dst_t = torch.as_tensor(dst, device=device)
    layers = []
    qt_ms = []
    for layer in range(w.layers):
        d = inputs.make_layer_torch(w, layer, device, plan)
        n8 = plan.int8_slots_total
        L = dict(q=d["q"], k_pool=d["k_pool"], v_pool=d["v_pool"],
                 k_codes=torch.empty((n8, Hkv, 64, 256), dtype=torch.int8, device=device),
                 v_codes=torch.empty((n8, Hkv, 256, 64), dtype=torch.int8, device=device),
                 k_chan=torch.empty((n8, Hkv, 256), device=device),
                 k_tok=torch.empty((n8, Hkv, 64), device=device),
                 v_chan=torch.empty((n8, Hkv, 256), device=device))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        B.akv_quantize_pages(dims, len(src), L["k_pool"], L["v_pool"], src_t, dst_t, L["k_codes"], L["v_codes"],
                             L["k_chan"], L["k_tok"], L["v_chan"])
        e1.record()
        torch.cuda.synchronize()
        qt_ms.append(e0.elapsed_time(e1))
        layers.append(L)
    tables = dict(t8=torch.as_tensor(plan.int8_table(), device=device),
                  tw=torch.as_tensor(plan.window_table(), device=device),
                  tf=torch.as_tensor(plan.full_table(), device=device),
                  n8=torch.as_tensor(np.asarray(plan.n8, np.int32), device=device),
                  nw=torch.as_tensor(np.asarray(plan.win_tokens, np.int32), device=device),
                  nf=torch.as_tensor(np.asarray([int(x) for x in w.lengths], np.int32), device=device))
    return plan, layers, tables, qt_ms, len(src)


def timed_steps(fn, steps, warmup, stream, min_warm_s=0.3):
    """Average ms of `steps` calls of fn after `warmup` untimed ones (and more
    untimed calls until they have run for min_warm_s: the first ~20 steps
    after the GPU idles run up to 2% slow while its clocks ramp), bracketed
    by device synchronisation and HIP events on `stream`."""
    import torch

    t0 = time.time()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    while time.time() - t0 < min_warm_s:
        fn()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def split_kernel_us(B, fn, steps, calls_per_step, name, stream):
    """Average duration of the split-K kernel of each decode call made through
    entry point `name`, from HIP events the library records around that
    kernel on `stream` (akv_set_profile_events)."""
    import torch

    evs = []
    for _ in range(steps * calls_per_step):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    it = iter(evs)
    orig = getattr(B, name)

    def hooked(*a, **kw):
        e0, e1 = next(it)
        B.akv_set_profile_events(e0, e1)
        try:
            orig(*a, **kw)
        finally:
            B.akv_set_profile_events(None, None)
    setattr(B, name, hooked)
    try:
        for _ in range(steps):
            fn()
    finally:
        setattr(B, name, orig)
    torch.cuda.synchronize()
    d = [a.elapsed_time(b) * 1e3 for a, b in evs]
    return sum(d) / len(d)


class Resident:
    """One workload's 16 layers resident in HBM, with the decode calls of one
    step as closures (all on the current stream)."""

    def __init__(self, w, device):
        import torch

        from quantized_paged_kv_akv_amd import binding as B
        from quantized_paged_kv_akv_amd import configs

        self.B, self.w, self.device = B, w, device
        t0 = time.time()
        self.plan, self.layers, self.T, self.qt_ms, self.n_quant = build_layers(w, device)
        log(f"[bench] {w.name}: inputs resident in HBM after {time.time() - t0:.1f}s")
        self.Hkv, self.G, self.D = w.num_kv_heads, w.group, w.head_dim
        self.dims = B.dims(self.Hkv, self.G)
        self.sigma = configs.SIGMA
        T = self.T
        self.m8, self.mw, self.mf = T["t8"].shape[1], T["tw"].shape[1], T["tf"].shape[1]
        self.stream = torch.cuda.current_stream()
        shape = (w.batch, w.num_q_heads)
        self.out = [torch.empty(shape + (self.D,), device=device) for _ in range(w.layers)]
        self.outl = [torch.empty(shape, device=device) for _ in range(w.layers)]
        self.ws = torch.empty(max(16, max(B.akv_decode_workspace_bytes(self.dims, w.batch, m)
                                          for m in (self.m8, self.mw, self.mf))), dtype=torch.uint8, device=device)
        # sized for launches of the whole batch, of two requests and of one
        self.wsh = torch.empty(max(16, max(B.akv_decode_hybrid_workspace_bytes(self.dims, k, self.m8, self.mw)
                                           for k in {w.batch, min(2, w.batch), 1})),
                               dtype=torch.uint8, device=device)
        by = step_kv_bytes(self.plan, self.Hkv)
        self.layer_bytes = by["int8"] + by["window"]
        self.bf16_layer_bytes = by["bf16_all"]
        self._prepared = {}

    def _hybrid_args(self, k):
        """Arguments of one step's akv_decode_hybrid calls (one layer each,
        or launches of k requests each)."""
        T, w = self.T, self.w
        for i, L in enumerate(self.layers):
            for b0 in range(0, w.batch, k):
                s = slice(b0, b0 + k)
                yield (self.dims, k, L["q"][s], L["k_codes"], L["v_codes"], L["k_chan"], L["k_tok"], L["v_chan"],
                       T["t8"][s], T["n8"][s], self.m8, L["k_pool"], L["v_pool"], T["tw"][s], T["nw"][s], self.mw,
                       self.sigma, self.out[i][s], self.outl[i][s], self.wsh, self.stream)

    def _bf16_args(self):
        T = self.T
        for i, L in enumerate(self.layers):
            yield (self.dims, self.w.batch, L["q"], L["k_pool"], L["v_pool"], T["tf"], T["nf"], self.mf, self.sigma,
                   self.out[i], self.outl[i], self.ws, self.stream)

    def _run_prepared(self, key, name, arg_iter):
        calls = self._prepared.get(key)
        if calls is None:
            calls = self._prepared[key] = [self.B.prepare(name, *a) for a in arg_iter()]
        for c in calls:
            c()

    def hybrid_step(self, k=None):
        """One layer = akv_decode_hybrid (split-K kernel over int8 + window
        pages, then the exact fold); with k, launches of k requests each.
        The calls are marshalled once (binding.prepare), so a step of short
        launches measures the device rather than the host's call overhead."""
        k = k or self.w.batch
        self._run_prepared(("hybrid", k), "akv_decode_hybrid", lambda: self._hybrid_args(k))

    def hybrid_step_plain(self, k=None):
        """The same step through the plain wrappers (what split_kernel_us hooks)."""
        for a in self._hybrid_args(k or self.w.batch):
            self.B.akv_decode_hybrid(*a)

    def bf16_step(self):
        self._run_prepared(("bf16",), "akv_decode_attn_exact", self._bf16_args)

    def bf16_step_plain(self):
        for a in self._bf16_args():
            self.B.akv_decode_attn_exact(*a)

    def time_hybrid(self, steps, warmup):
        ms = timed_steps(self.hybrid_step, steps, warmup, self.stream)
        us = split_kernel_us(self.B, self.hybrid_step_plain, max(2, steps // 2), self.w.layers * 1,
                             "akv_decode_hybrid", self.stream)
        return ms, us

    def free(self):
        import torch

        self._prepared.clear()
        self.layers.clear()
        self.T.clear()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def run_gpu(args, w, res):
    """The headline workload: hybrid step (fused entry), the same layer as four
    separate calls, all-BF16 exact decode, the 13-bit tier, single-step
    spread and the streaming-read ceiling."""
    import torch

    from quantized_paged_kv_akv_amd import binding as B

    device, stream = res.device, res.stream
    layers, T, dims, sigma = res.layers, res.T, res.dims, res.sigma
    Hkv, D, batch = res.Hkv, res.D, w.batch
    rows = batch * w.num_q_heads
    m8, mw, mf = res.m8, res.mw, res.mf
    out, outl, ws = res.out, res.outl, res.ws
    o_w = torch.empty_like(out[0])
    l_w = torch.empty_like(outl[0])

    log("[bench] hybrid step (fused entry) warmup + timed")
    ms_hybrid = timed_steps(res.hybrid_step, args.steps, args.warmup, stream)
    # the timed step's outputs, kept for the oracle check
    hyb_out = [(o.clone(), l.clone()) for o, l in zip(out, outl)]
    hyb_us = split_kernel_us(B, res.hybrid_step_plain, max(2, args.steps // 2), w.layers, "akv_decode_hybrid",
                             stream)

    # the same layer as the separate entry points (int8, exact, merge)
    four_calls = []
    for i, L in enumerate(layers):
        four_calls += [B.prepare("akv_decode_attn_int8", dims, batch, L["q"], L["k_codes"], L["v_codes"], L["k_chan"],
                                 L["k_tok"], L["v_chan"], T["t8"], T["n8"], m8, sigma, out[i], outl[i], ws, stream),
                       B.prepare("akv_decode_attn_exact", dims, batch, L["q"], L["k_pool"], L["v_pool"], T["tw"],
                                 T["nw"], mw, sigma, o_w, l_w, ws, stream),
                       B.prepare("akv_merge_lse", rows, D, out[i], outl[i], o_w, l_w, stream)]

    def four_call_step():
        for c in four_calls:
            c()

    log("[bench] four-call step")
    ms_four = timed_steps(four_call_step, max(2, args.steps // 2), 1, stream)
    log("[bench] all-BF16 step")
    ms_bf16 = timed_steps(res.bf16_step, max(2, args.steps // 2), 1, stream)
    bf16_us = split_kernel_us(B, res.bf16_step_plain, 2, w.layers, "akv_decode_attn_exact", stream)

    # lossless 13-bit tier, HBM-resident: each layer's whole history encoded
    # (akv_l13_encode_pages), then decoded directly by akv_decode_attn_l13
    log("[bench] lossless 13-bit tier: encode every layer, then the all-13-bit step")
    l13_enc_ms = []
    for L in layers:
        n = L["k_pool"].shape[0]
        sz = B.l13_sizes(dims, n)
        rec = dict(arena=torch.empty(sz["arena_bytes"], dtype=torch.uint8, device=device),
                   desc=torch.empty(sz["desc"], dtype=torch.int32, device=device),
                   table=torch.empty(sz["table"], dtype=torch.uint8, device=device),
                   end=torch.empty(1, dtype=torch.int64, device=device))
        sl = torch.arange(n, dtype=torch.int32, device=device)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        B.akv_l13_encode_pages(dims, n, L["k_pool"], L["v_pool"], sl, sl, rec["arena"], 0, rec["desc"],
                               rec["table"], rec["end"], stream)
        e1.record(stream)
        torch.cuda.synchronize()
        l13_enc_ms.append(e0.elapsed_time(e1))
        L["l13"] = rec
    l13_arena = [int(L["l13"]["end"][0]) for L in layers]
    n_planes = layers[0]["k_pool"].shape[0] * Hkv * 2
    # bytes one launch reads: the used planes, plus a descriptor and a table per plane
    l13_layer_bytes = l13_arena[0] + n_planes * (4 + 32)
    l13_raw = sum(int((L["l13"]["desc"] & 1).sum()) for L in layers)

    def l13_args():
        for i, L in enumerate(layers):
            yield (dims, batch, L["q"], L["l13"]["arena"], L["l13"]["desc"], L["l13"]["table"], T["tf"], T["nf"], mf,
                   sigma, out[i], outl[i], ws, stream)

    l13_calls = [B.prepare("akv_decode_attn_l13", *a) for a in l13_args()]

    def l13_step():
        for c in l13_calls:
            c()

    def l13_step_plain():
        for a in l13_args():
            B.akv_decode_attn_l13(*a)

    ms_l13 = timed_steps(l13_step, max(2, args.steps // 2), 1, stream)
    l13_us = split_kernel_us(B, l13_step_plain, 2, w.layers, "akv_decode_attn_l13", stream)
    del l13_calls
    l13_enc = sorted(l13_enc_ms)[len(l13_enc_ms) // 2]
    lossless = dict(ms_step=ms_l13, launch_us=l13_us, bytes_per_launch=l13_layer_bytes,
                    arena_bytes_per_layer=l13_arena[0], arena_frac_of_bf16=l13_arena[0] / res.bf16_layer_bytes,
                    raw_planes=l13_raw, planes=n_planes * w.layers, encode_ms_per_layer=l13_enc,
                    encode_GBps_in=res.bf16_layer_bytes / (l13_enc * 1e-3) / 1e9)
    for L in layers:
        del L["l13"]
    torch.cuda.empty_cache()

    # spread of single steps (events around each of a few more steps)
    step_us = []
    for _ in range(max(10, args.steps)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        res.hybrid_step()
        e1.record(stream)
        e1.synchronize()
        step_us.append(e0.elapsed_time(e1) * 1e3)
    step_us.sort()

    def pct(q):
        return step_us[min(len(step_us) - 1, int(q * (len(step_us) - 1) + 0.5))]

    # streaming-read ceiling of this GPU: a non-temporal 16-byte-load read of 4 GiB
    log("[bench] streaming-read ceiling")
    big = torch.ones(4 << 30, dtype=torch.uint8, device=device)
    sink = torch.zeros(1, dtype=torch.int32, device=device)
    B.akv_stream_read(big, sink, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        B.akv_stream_read(big, sink, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    read_gbps = 5 * (big.numel() // 32768 * 32768) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del big

    quant_ms = sum(res.qt_ms[1:]) / max(1, len(res.qt_ms) - 1) if len(res.qt_ms) > 1 else res.qt_ms[0]
    quant_bytes = res.n_quant * Hkv * (PAGE_BF16_BYTES + PAGE_INT8_BYTES)
    return dict(step_p=(pct(0.1), pct(0.5), pct(0.9)), read_gbps=read_gbps, ms_hybrid=ms_hybrid,
                ms_four=ms_four, ms_bf16=ms_bf16, hybrid_bytes=res.layer_bytes * w.layers,
                bf16_bytes=res.bf16_layer_bytes * w.layers, hyb_launch_us=hyb_us,
                hyb_bytes_per_launch=res.layer_bytes, hyb_achieved_gbps=res.layer_bytes / (hyb_us * 1e-6) / 1e9,
                bf16_launch_us=bf16_us, bf16_achieved_gbps=res.bf16_layer_bytes / (bf16_us * 1e-6) / 1e9,
                quant_ms_per_layer=quant_ms, quant_gbps=quant_bytes / (quant_ms * 1e-3) / 1e9, lossless=lossless,
                hyb_out=hyb_out)


def run_config(args, w, owner_modes=False, res=None):
    """A further workload at its real shape: the hybrid step (one launch per
    layer), its split kernel, and for batched workloads the same step as
    two-request (two-owner) launches and as one launch per request, plus the
    all-BF16 step.  res: the workload's inputs, if already resident."""
    import torch

    device = torch.device("cuda", 0)
    if res is None:
        res = Resident(w, device)
    steps = max(4, args.steps)
    # a second of untimed steps first: right after the previous workload's
    # memory is released, the first timed window of a short step reads up to
    # 4% slow (334 against 322 us per 32K step), the next ones do not
    timed_steps(res.hybrid_step, 1, 1, res.stream, min_warm_s=1.0)
    ms, us = res.time_hybrid(steps, max(1, args.warmup))
    out = dict(us_per_step=round(ms * 1e3, 2), us_per_layer=round(ms * 1e3 / w.layers, 2),
               kv_bytes_per_step=res.layer_bytes * w.layers,
               GBps_step=round(res.layer_bytes * w.layers / (ms * 1e-3) / 1e9, 1),
               frac_of_hbm_peak_step=round(res.layer_bytes * w.layers / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
               split_kernel_us=round(us, 2), split_kernel_GBps=round(res.layer_bytes / (us * 1e-6) / 1e9, 1),
               requests=w.batch, context_tokens=[int(x) for x in w.lengths])
    if owner_modes:
        log(f"[bench] {w.name}: two-owner and one-row launches, all-BF16 step")
        ms2 = timed_steps(lambda: res.hybrid_step(2), max(2, steps // 2), 1, res.stream)
        ms1 = timed_steps(lambda: res.hybrid_step(1), max(2, steps // 2), 1, res.stream)
        msb = timed_steps(res.bf16_step, max(2, steps // 2), 1, res.stream)
        out.update(us_per_step_two_owner_launches=round(ms2 * 1e3, 2),
                   us_per_step_one_row_launches=round(ms1 * 1e3, 2),
                   us_per_step_bf16_all=round(msb * 1e3, 2),
                   bf16_kv_bytes_per_step=res.bf16_layer_bytes * w.layers,
                   hybrid_speedup_vs_bf16=round(msb / ms, 3),
                   two_owner_vs_one_row_time=round(ms2 / ms1, 3))
    res.free()
    return out


def by_layer_bf16(plan, Hkv) -> int:
    """BF16 bytes of one layer's whole history (keys and values)."""
    return step_kv_bytes(plan, Hkv)["bf16_all"]


def run_staged(args, w, with_l13=True, ring_slots=(2,)):
    """Host-staged step: each layer's history sits in pinned host memory and
    is staged into a two-slot device ring on a side stream (events guard slot
    reuse), overlapped with the previous layer's attention.  The hybrid step
    stages the int8 pool (codes + scales) and the BF16 window pages; the
    all-BF16 step stages the whole BF16 pool; the lossless step stages the
    whole history in the 13-bit format (packed planes, descriptors, tables)
    and decodes it with akv_decode_attn_l13.  Before the history leaves HBM,
    the same hybrid and all-BF16 steps are timed HBM-resident (the per-layer
    decode times the tier gate's transfer model needs)."""
    import torch

    from quantized_paged_kv_akv_amd import binding as B
    from quantized_paged_kv_akv_amd import configs

    device = torch.device("cuda", 0)
    torch.cuda.set_device(device)
    log(f"[bench] building {w.name}: {w.layers} layers, lengths {w.lengths[:4]}...")
    res = Resident(w, device)
    plan, layers, T = res.plan, res.layers, res.T
    Hkv, G = w.num_kv_heads, w.group
    dims = B.dims(Hkv, G)
    sigma = configs.SIGMA
    m8, mw, mf = T["t8"].shape[1], T["tw"].shape[1], T["tf"].shape[1]
    comp = torch.cuda.current_stream()
    # HBM-resident decode time per layer of each tier
    res_h = timed_steps(res.hybrid_step, 4, 2, comp) / w.layers
    res_b = timed_steps(res.bf16_step, 4, 2, comp) / w.layers
    tw_c = torch.arange(T["tw"].numel(), dtype=torch.int32, device=device).view(T["tw"].shape)
    widx = T["tw"].reshape(-1).long()

    def pinned(t):
        h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
        h.copy_(t)
        return h

    def packed(ts):
        """One pinned block per layer holding the tensors back to back at
        256-byte aligned offsets (one large copy instead of several small
        ones), plus each tensor's (offset, dtype, shape)."""
        offs, off = [], 0
        for t in ts:
            offs.append(off)
            off += (t.numel() * t.element_size() + 255) // 256 * 256
        blk = torch.empty(off, dtype=torch.uint8, pin_memory=True)
        for t, o in zip(ts, offs):
            n = t.numel() * t.element_size()
            blk[o:o + n].copy_(t.contiguous().view(-1).view(torch.uint8))
        return blk, [(o, t.dtype, tuple(t.shape)) for t, o in zip(ts, offs)]

    log("[bench] copying the history to pinned host memory" + (" (and encoding it 13-bit)" if with_l13 else ""))
    host_h, host_b, host_l, lay_h, lay_l = [], [], [], None, []
    n_slots = layers[0]["k_pool"].shape[0]
    if with_l13:
        sz = B.l13_sizes(dims, n_slots)
        l13_arena = torch.empty(sz["arena_bytes"], dtype=torch.uint8, device=device)
        l13_desc = torch.empty(sz["desc"], dtype=torch.int32, device=device)
        l13_table = torch.empty(sz["table"], dtype=torch.uint8, device=device)
        l13_end = torch.empty(1, dtype=torch.int64, device=device)
        all_slots = torch.arange(n_slots, dtype=torch.int32, device=device)
    for L in layers:
        blk, lay_h = packed([L[k] for k in ("k_codes", "v_codes", "k_chan", "k_tok", "v_chan")]
                            + [L["k_pool"][widx], L["v_pool"][widx]])
        host_h.append([blk])
        host_b.append([pinned(L["k_pool"]), pinned(L["v_pool"])])
        if with_l13:
            B.akv_l13_encode_pages(dims, n_slots, L["k_pool"], L["v_pool"], all_slots, all_slots, l13_arena, 0,
                                   l13_desc, l13_table, l13_end)
            end = int(l13_end[0])
            blk, lay = packed([l13_arena[:end], l13_desc, l13_table])
            host_l.append([blk])
            lay_l.append(lay)
        for k in ("k_codes", "v_codes", "k_chan", "k_tok", "v_chan", "k_pool", "v_pool"):
            del L[k]
    if with_l13:
        del l13_arena
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    def nbytes(srcs):
        return sum((t.numel() * t.element_size() + 255) // 256 * 256 for t in srcs)

    def tbytes(lay):
        return sum(torch.Size(shp).numel() * torch.empty((), dtype=dt).element_size() for _, dt, shp in lay)

    bytes_h = tbytes(lay_h) * w.layers
    bytes_b = sum(t.numel() * t.element_size() for t in host_b[0]) * w.layers
    bytes_l = sum(tbytes(lay) for lay in lay_l)
    n_ring = max(ring_slots)
    ring_h = B.Ring([torch.empty(nbytes(host_h[0]), dtype=torch.uint8, device=device) for _ in range(n_ring)])
    ring_b = B.Ring([torch.empty(nbytes(host_b[0]), dtype=torch.uint8, device=device) for _ in range(n_ring)])
    ring_l = (B.Ring([torch.empty(max(nbytes(h) for h in host_l), dtype=torch.uint8, device=device)
                      for _ in range(2)]) if with_l13 else None)
    # rings of fewer slots reuse the first slots' memory (only one ring is in use at a time)
    rings_h = {k: (ring_h if k == n_ring else B.Ring(ring_h.slots[:k])) for k in ring_slots}
    rings_b = {k: (ring_b if k == n_ring else B.Ring(ring_b.slots[:k])) for k in ring_slots}
    copy_s = torch.cuda.Stream()
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), device=device)
    outl = torch.empty((w.batch, w.num_q_heads), device=device)
    wsh, wsb = res.wsh, torch.empty(max(16, B.akv_decode_workspace_bytes(dims, w.batch, mf)), dtype=torch.uint8,
                                    device=device)

    def views(slot, lay):
        return [slot[o:o + torch.Size(shp).numel() * torch.empty((), dtype=dt).element_size()].view(dt).view(shp)
                for o, dt, shp in lay]

    # device views of each ring slot, made once (the per-layer host work is
    # then the staging call, the decode call and the release call)
    views_h = {t.data_ptr(): views(t, lay_h) for t in ring_h.slots}
    views_b = {}
    for t in ring_b.slots:
        off, vs = 0, []
        for h in host_b[0]:
            n = h.numel() * h.element_size()
            vs.append(t[off:off + n].view(h.dtype).view(h.shape))
            off += (n + 255) // 256 * 256
        views_b[t.data_ptr()] = vs
    q_l = [L["q"] for L in layers]

    cur = dict(h=ring_h, b=ring_b)

    def hybrid_step():
        rh = cur["h"]._h
        for i in range(w.layers):
            v = views_h[B.akv_ring_stage(rh, i, host_h[i], copy_s, comp)[0]]
            B.akv_decode_hybrid(dims, w.batch, q_l[i], v[0], v[1], v[2], v[3], v[4], T["t8"], T["n8"], m8, v[5],
                                v[6], tw_c, T["nw"], mw, sigma, out, outl, wsh, comp)
            B.akv_ring_release(rh, i, comp)

    def bf16_step():
        rb = cur["b"]._h
        for i in range(w.layers):
            v = views_b[B.akv_ring_stage(rb, i, host_b[i], copy_s, comp)[0]]
            B.akv_decode_attn_exact(dims, w.batch, q_l[i], v[0], v[1], T["tf"], T["nf"], mf, sigma, out, outl,
                                    wsb, comp)
            B.akv_ring_release(rb, i, comp)

    def l13_step():
        for i in range(w.layers):
            slot = ring_l.stage_views(i, host_l[i], copy_s, comp)[0]
            v = views(slot, lay_l[i])
            B.akv_decode_attn_l13(dims, w.batch, q_l[i], v[0], v[1], v[2], T["tf"], T["nf"], mf, sigma, out, outl,
                                  wsb, comp)
            ring_l.release(i, comp)

    # plain host-to-device copy rate of one layer's BF16 pool, for reference
    big = host_b[0][0]
    dst = torch.empty(big.shape, dtype=big.dtype, device=device)
    for _ in range(2):
        dst.copy_(big, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(comp)
    for _ in range(5):
        dst.copy_(big, non_blocking=True)
    e1.record(comp)
    torch.cuda.synchronize()
    h2d_gbps = 5 * big.numel() * big.element_size() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del dst

    # untimed passes of every mode first, at least half a second of sustained
    # copies: the first staged mode timed otherwise runs up to 15% slower
    # (host-to-device copy rates ramp up over the first few hundred
    # milliseconds of traffic)
    modes = (hybrid_step, bf16_step, l13_step) if with_l13 else (hybrid_step, bf16_step)
    t_warm = time.time()
    while True:
        for fn in modes:
            fn()
        torch.cuda.synchronize()
        if time.time() - t_warm > 0.5:
            break
    # host time to enqueue one step (16 x stage, decode, release), GPU idle
    enq = {}
    for name, fn in (("hybrid", hybrid_step), ("exact", bf16_step)):
        torch.cuda.synchronize()
        t_h = time.perf_counter()
        fn()
        enq[name] = (time.perf_counter() - t_h) * 1e3
        torch.cuda.synchronize()
    steps = max(2, args.steps // 4)

    def best_of_two(fn):
        # the faster of two timed runs (a single run can catch other traffic on the bus)
        return min(timed_steps(fn, steps, 1, comp), timed_steps(fn, steps, 0, comp, min_warm_s=0.0))

    by_slots = {}
    for k in ring_slots:
        cur["h"], cur["b"] = rings_h[k], rings_b[k]
        log(f"[bench] {w.name}: staged hybrid and all-BF16 steps, {k}-slot ring")
        by_slots[k] = dict(ms_h=best_of_two(hybrid_step), ms_b=best_of_two(bf16_step))
    ms_h, ms_b = by_slots[ring_slots[0]]["ms_h"], by_slots[ring_slots[0]]["ms_b"]
    for k in ring_slots:
        if k != n_ring:
            rings_h[k].destroy()
            rings_b[k].destroy()
    ms_l = None
    if with_l13:
        log(f"[bench] {w.name}: staged lossless 13-bit step")
        ms_l = best_of_two(l13_step)
        ring_l.destroy()
    ring_h.destroy()
    ring_b.destroy()
    res.free()
    return dict(ms_h=ms_h, ms_b=ms_b, ms_l=ms_l, bytes_h=bytes_h, bytes_b=bytes_b, bytes_l=bytes_l,
                h2d_gbps=h2d_gbps, steps=steps, resident_ms_per_layer=dict(hybrid=res_h, exact=res_b),
                host_enqueue_ms=enq, by_slots=by_slots,
                copies_per_layer=dict(hybrid=[nbytes(host_h[0])],
                                      exact=[t.numel() * t.element_size() for t in host_b[0]]))


def pcie_curve(sizes_mib=(0.0625, 0.25, 1, 4, 16, 64, 256, 512)):
    """Pinned host-to-device copy rate against transfer size (the transfer
    model of the exact-vs-hybrid gate)."""
    import torch

    device = torch.device("cuda", 0)
    out = []
    big = torch.empty(int(max(sizes_mib) * (1 << 20)), dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(big.numel(), dtype=torch.uint8, device=device)
    for _ in range(4):  # sustained traffic first: copy rates ramp up over the first few hundred ms
        dst.copy_(big, non_blocking=True)
    torch.cuda.synchronize()
    for mib in sizes_mib:
        n = int(mib * (1 << 20))
        reps = max(3, min(200, int(256 / max(mib, 1e-3))))
        dst[:n].copy_(big[:n], non_blocking=True)
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):  # the fastest of three runs
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                dst[:n].copy_(big[:n], non_blocking=True)
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        out.append((mib, reps * n / (best * 1e-3) / 1e9))
    return out


def staged_copy_curve(sizes_mib=(1, 4, 8, 16, 32, 64, 128, 256), n_slots=2):
    """Host-to-device copy time against size in the staging pattern itself:
    one copy per "layer" through an n_slots akv ring (each copy waits for the
    compute stream to release the slot it overwrites, the compute stream
    waits for each copy), with no kernel in between.  This is the bus
    behaviour the staged step sees, dependencies included; plain
    back-to-back copies (pcie_curve) overlap consecutive transfers and read
    faster for sizes around 10-30 MB."""
    import torch

    from quantized_paged_kv_akv_amd import binding as B

    device = torch.device("cuda", 0)
    big = torch.empty(int(max(sizes_mib) * (1 << 20)), dtype=torch.uint8, pin_memory=True)
    copy_s, comp = torch.cuda.Stream(), torch.cuda.current_stream()
    out = []
    for mib in sizes_mib:
        n = int(mib * (1 << 20))
        src = [big[:n]]
        ring = B.Ring([torch.empty(n, dtype=torch.uint8, device=device) for _ in range(n_slots)])
        reps = max(8, min(128, int(2048 / mib)))

        def run(k):
            for i in range(k):
                B.akv_ring_stage(ring._h, i, src, copy_s, comp)
                B.akv_ring_release(ring._h, i, comp)

        t_warm = time.time()
        while time.time() - t_warm < 0.2:
            run(8)
            torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):  # the fastest of three runs: single runs catch other traffic on the bus
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(comp)
            run(reps)
            e1.record(comp)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        out.append((mib, reps * n / (best * 1e-3) / 1e9))
        ring.destroy()
    return out


def staged_sweep(args, contexts=(8192, 16384, 32768, 65536, 131072), with_l13=False):
    """Host-staged per-token time against context length, hybrid against
    exact (all-BF16) (and the 13-bit tier if asked), next to the tier gate's
    prediction: a copy-time model t(n) = latency + n / bandwidth fitted to
    the measured host-to-device curve, fed each tier's per-layer copy sizes
    and its HBM-resident decode time, through the two-slot staging
    schedule.  The gate picks the tier with the smallest predicted time."""
    import gc

    import torch

    from quantized_paged_kv_akv_amd import inputs
    from quantized_paged_kv_akv_amd import tier_gate as TG

    curve = pcie_curve()
    copy = TG.fit_copy_model([m * (1 << 20) for m, _ in curve], [g * 1e9 for _, g in curve])
    scurve = {ns: staged_copy_curve(n_slots=ns) for ns in RING_SLOTS}
    model = TG.fit_staging_model(copy, {ns: ([m * (1 << 20) for m, _ in c], [g * 1e9 for _, g in c])
                                        for ns, c in scurve.items()})
    log(f"[bench] copy model: latency {copy.latency_s * 1e6:.1f} us, bandwidth {copy.bandwidth_Bps / 1e9:.1f} GB/s; "
        f"through the ring: {model.stage_overhead_s * 1e6:.1f} us per layer, round trip "
        f"{model.round_trip_s * 1e6:.0f} us")
    rows, last = [], None
    for L in contexts:
        w = inputs.Workload(f"staged{L // 1024}k", 4, batch=1, layers=16, num_kv_heads=4, group=6, lengths=(L,),
                            window=1024, outlier_frac=0.02, permute=False)
        r = run_staged(args, w, with_l13=with_l13, ring_slots=RING_SLOTS)
        kern = {k: v * 1e-3 for k, v in r["resident_ms_per_layer"].items()}
        row = dict(context=L)
        for ns in RING_SLOTS:
            meas = {"hybrid": r["by_slots"][ns]["ms_h"], "exact": r["by_slots"][ns]["ms_b"]}
            pred = {k: v * 1e3 for k, v in TG.predict(model, r["copies_per_layer"], kern, layers=w.layers,
                                                      n_slots=ns).items()}
            row[f"slots{ns}"] = dict(
                ms_hybrid=round(meas["hybrid"], 3), ms_bf16=round(meas["exact"], 3),
                predicted_ms_hybrid=round(pred["hybrid"], 3), predicted_ms_bf16=round(pred["exact"], 3),
                prediction_error_hybrid=round(pred["hybrid"] / meas["hybrid"] - 1, 4),
                prediction_error_bf16=round(pred["exact"] / meas["exact"] - 1, 4),
                chosen_by_model=TG.choose(pred), chosen_by_measurement=min(meas, key=meas.get))
        row.update(ms_hybrid=round(r["ms_h"], 3), ms_bf16=round(r["ms_b"], 3),
                   resident_us_per_layer_hybrid=round(r["resident_ms_per_layer"]["hybrid"] * 1e3, 2),
                   resident_us_per_layer_bf16=round(r["resident_ms_per_layer"]["exact"] * 1e3, 2),
                   bytes_hybrid=r["bytes_h"], bytes_bf16=r["bytes_b"],
                   pcie_GBps_hybrid=round(r["bytes_h"] / (r["ms_h"] * 1e-3) / 1e9, 1),
                   pcie_GBps_bf16=round(r["bytes_b"] / (r["ms_b"] * 1e-3) / 1e9, 1),
                   h2d_copy_GBps=round(r["h2d_gbps"], 1),
                   host_enqueue_ms_hybrid=round(r["host_enqueue_ms"]["hybrid"], 3),
                   host_enqueue_ms_bf16=round(r["host_enqueue_ms"]["exact"], 3))
        if with_l13:
            row.update(ms_lossless13=round(r["ms_l"], 3), bytes_lossless13=r["bytes_l"],
                       pcie_GBps_lossless13=round(r["bytes_l"] / (r["ms_l"] * 1e-3) / 1e9, 1))
        rows.append(row)
        for ns in RING_SLOTS:
            x = row[f"slots{ns}"]
            log(f"[bench] {w.name} {ns} slots: hybrid {x['ms_hybrid']:.2f} ms (model {x['predicted_ms_hybrid']:.2f}), "
                f"exact {x['ms_bf16']:.2f} ms (model {x['predicted_ms_bf16']:.2f})")
        last = r
        gc.collect()
        torch.cuda.empty_cache()
    return dict(curve=curve, staged_curve=scurve, model=model, rows=rows, last=last)


def staging_model_json(m) -> dict:
    return {"latency_us": round(m.copy.latency_s * 1e6, 2), "bandwidth_GBps": round(m.copy.bandwidth_Bps / 1e9, 2),
            "fitted_to": "pcie_h2d_curve (plain back-to-back copies)",
            "ring_overhead_us_per_layer": round(m.stage_overhead_s * 1e6, 2),
            "ring_round_trip_us": round(m.round_trip_s * 1e6, 1),
            "ring_terms_fitted_to": "staged_copy_curve (copies through the ring, no kernel, each slot count)"}


def tile_order_to_token_major(a):
    """Key codes in the library's tile order (include/akv.h: K[t][d] of a
    page-head at byte ((4 (d / 64) + (t / 4) % 4) * 64 + 16 ((d / 16) % 4) +
    4 (t / 16) + t % 4) * 16 + d % 16), given as [..., 4, 4, 4, 4, 4, 16]
    (d / 64, (t / 4) % 4, (d / 16) % 4, t / 16, t % 4, d % 16), returned
    token-major [..., t / 16, (t / 4) % 4, t % 4, d / 64, (d / 16) % 4, d % 16]
    = [..., 64, 256] (a transpose)."""
    import numpy as np

    n = a.ndim - 6
    lead = tuple(range(n))
    return np.ascontiguousarray(a.transpose(lead + (n + 3, n + 1, n + 4, n, n + 2, n + 5)))


def cpu_baseline(w, res, hyb_out):
    """The float64 oracle, as it stands, on the timed step's own inputs: all
    64 (layer, KV head) units of one 16-layer decode step, each reading its
    own layer's int8 pages (int8-path formula) and BF16 window pages (exact),
    then the LSE merge -- timed on the host's cores.  Its outputs are the
    oracle check of the timed hybrid step: every layer's O and LSE against
    the GPU's, at the acceptance tolerances."""
    import numpy as np
    import torch

    from oracle import oracle as O

    def bits(t):
        """BF16 device tensor -> uint16 host array of its bit patterns."""
        return t.view(dtype=torch.int16).cpu().numpy().view(np.uint16)

    t0 = time.time()
    plan, T, Hkv, G, D = res.plan, res.T, res.Hkv, res.G, res.D
    nl = w.layers
    t8 = plan.int8_table()
    tw = plan.window_table()
    n8 = int(plan.n8[0])
    wp = tw.shape[1]
    # one pool holding every layer's pages: layer i's int8 pages at slots
    # [i n8, (i + 1) n8), its window pages at [i wp, (i + 1) wp)
    kc = np.empty((nl * n8, Hkv, 64, 256), np.int8)
    vc = np.empty((nl * n8, Hkv, 256, 64), np.int8)
    kch = np.empty((nl * n8, Hkv, 256), np.float32)
    ktk = np.empty((nl * n8, Hkv, 64), np.float32)
    vch = np.empty((nl * n8, Hkv, 256), np.float32)
    kw = np.empty((nl * wp, Hkv, 64, 256), np.uint16)
    vw = np.empty((nl * wp, Hkv, 256, 64), np.uint16)
    q = np.empty((nl, Hkv * G, D), np.uint16)
    sl8 = t8[0, :n8].astype(np.int64)
    slw = tw[0].astype(np.int64)
    ident = bool(np.array_equal(sl8, np.arange(n8)))

    def rows_of(t):
        a = t.cpu().numpy()
        return a[:n8] if ident else a[sl8]

    for i, L in enumerate(res.layers):
        a = rows_of(L["k_codes"]).reshape(n8, Hkv, 4, 4, 4, 4, 4, 16)
        kc[i * n8:(i + 1) * n8] = tile_order_to_token_major(a).reshape(n8, Hkv, 64, 256)
        vc[i * n8:(i + 1) * n8] = rows_of(L["v_codes"])
        kch[i * n8:(i + 1) * n8] = rows_of(L["k_chan"])
        ktk[i * n8:(i + 1) * n8] = rows_of(L["k_tok"])
        vch[i * n8:(i + 1) * n8] = rows_of(L["v_chan"])
        kw[i * wp:(i + 1) * wp] = bits(L["k_pool"][torch.as_tensor(slw, device=L["k_pool"].device)])
        vw[i * wp:(i + 1) * wp] = bits(L["v_pool"][torch.as_tensor(slw, device=L["v_pool"].device)])
        q[i] = bits(L["q"][0])
    t8_all = (np.arange(nl)[:, None] * n8 + np.arange(n8)[None, :]).astype(np.int32)
    tw_all = (np.arange(nl)[:, None] * wp + np.arange(wp)[None, :]).astype(np.int32)
    n8_all = np.full(nl, n8, np.int32)
    nw_all = np.full(nl, int(plan.win_tokens[0]), np.int32)
    log(f"[bench] cpu baseline: the step's {nl * Hkv} units copied to the host in {time.time() - t0:.1f}s")
    t0 = time.time()
    o8, l8 = O.decode_int8(q, kc, vc, kch, ktk, vch, t8_all, n8_all, Hkv, G, res.sigma, mode=1)
    ow, lw = O.decode_exact(q, kw, vw, tw_all, nw_all, Hkv, G, res.sigma)
    rows = nl * Hkv * G
    ro, rl = O.merge(np.stack([o8.reshape(rows, D), ow.reshape(rows, D)]), np.stack([l8.reshape(rows),
                                                                                      lw.reshape(rows)]))
    wall = time.time() - t0
    threads = min(O.num_threads(), nl * Hkv)
    cpu = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    # the oracle check of the timed step's outputs
    go = np.concatenate([o.reshape(-1, D).cpu().numpy() for o, _ in hyb_out]).astype(np.float64)
    gl = np.concatenate([l.reshape(-1).cpu().numpy() for _, l in hyb_out]).astype(np.float64)
    err = float(np.abs(go - ro).max())
    rel = float(np.linalg.norm(go - ro) / np.linalg.norm(ro))
    lerr = float(np.abs(gl - rl).max())
    check = dict(layers_checked=nl, rows=rows, o_max_abs=err, o_rel_l2=rel, lse_max_abs=lerr,
                 tolerances=dict(o_max_abs=2e-3, o_rel_l2=1e-3, lse_max_abs=1e-4),
                 passed=bool(err <= 2e-3 and rel <= 1e-3 and lerr <= 1e-4),
                 reference="float64 oracle (int8-path formula on the GPU's codes and scales, exact window, "
                           "LSE merge) on the same inputs the timed step read")
    step_bytes = res.layer_bytes * nl
    cb = dict(value=round(step_bytes / wall / 1e9, 3), unit="GB/s", cores=threads, kind="oracle",
              sample=f"all {nl * Hkv} (layer, KV head) units of one {w.name} decode step, each reading its own "
                     f"layer's {n8} int8 pages and {plan.win_tokens[0]}-token BF16 window (the timed step's own "
                     f"inputs, copied to the host), float64, {wall:.1f}s wall on {threads} threads of {cpu}; "
                     f"value = the step's {step_bytes} algorithmic KV bytes / that wall time",
              us_per_step=round(wall * 1e6, 1), wall_s=wall)
    return cb, check


def profile_kernels(args, w):
    """Kernel sequence for rocprofv3 counter passes: a plain 1 GiB device copy
    (known bytes, to calibrate FETCH_SIZE / WRITE_SIZE), then `steps` hybrid
    decode steps of the workload, then `steps` steps of the int8 tier alone
    (akv_decode_attn_int8: one wave per int8 page-head, for per-page counts)."""
    import torch

    from quantized_paged_kv_akv_amd import binding as B
    from quantized_paged_kv_akv_amd import configs

    device = torch.device("cuda", 0)
    plan, layers, T, _, _ = build_layers(w, device)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("[profile] 3 x 1 GiB device copy done")
    dims = B.dims(w.num_kv_heads, w.group)
    m8, mw = T["t8"].shape[1], T["tw"].shape[1]
    ws = torch.empty(max(16, B.akv_decode_hybrid_workspace_bytes(dims, w.batch, m8, mw)), dtype=torch.uint8,
                     device=device)
    o = torch.empty((w.batch, w.num_q_heads, w.head_dim), device=device)
    lse = torch.empty((w.batch, w.num_q_heads), device=device)
    for _ in range(args.steps):
        for L in layers:
            B.akv_decode_hybrid(dims, w.batch, L["q"], L["k_codes"], L["v_codes"], L["k_chan"], L["k_tok"],
                                L["v_chan"], T["t8"], T["n8"], m8, L["k_pool"], L["v_pool"], T["tw"], T["nw"], mw,
                                configs.SIGMA, o, lse, ws)
    torch.cuda.synchronize()
    log(f"[profile] {args.steps} hybrid steps done")
    # the int8 tier alone (one wave per page-head): per-page instruction counts
    ws8 = torch.empty(max(16, B.akv_decode_workspace_bytes(dims, w.batch, m8)), dtype=torch.uint8, device=device)
    for _ in range(args.steps):
        for L in layers:
            B.akv_decode_attn_int8(dims, w.batch, L["q"], L["k_codes"], L["v_codes"], L["k_chan"], L["k_tok"],
                                   L["v_chan"], T["t8"], T["n8"], m8, configs.SIGMA, o, lse, ws8)
    torch.cuda.synchronize()
    log(f"[profile] {args.steps} int8-only steps done")


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/<kernel>_<workload>_counters.md, lines `kernel_source_hash: ...`
    and `traffic_bytes_per_launch: ...`), if it was taken on the current
    kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.md")
    if not os.path.exists(p):
        return None
    fields = {}
    for line in open(p):
        if ":" in line and line.split(":", 1)[0].strip() in ("kernel_source_hash", "traffic_bytes_per_launch"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ctx128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="ctx128k only: skip the 32K, batched and host-staged measurements")
    ap.add_argument("--profile-kernels", action="store_true",
                    help="for counter runs: a 1 GiB device copy (calibration), then --steps hybrid steps; no JSON")
    ap.add_argument("--pv-fp16", action="store_true",
                    help="A/B: the int8 tier's PV product on FP16 operands instead of the int8 MFMA")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only (one GPU's share of the path at its real shape; sharding by KV "
              "head, request or page range needs no new kernel and is not run here). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from quantized_paged_kv_akv_amd import binding as B
    from quantized_paged_kv_akv_amd import configs
    if args.pv_fp16:
        B.akv_set_launch_shape(pv_fp16=1)
    w = configs.ALL[args.workload]() if args.workload in configs.ALL else configs.staged128k()
    if args.profile_kernels:
        profile_kernels(args, w)
        return
    if args.workload == "staged-sweep":
        sw = staged_sweep(args, with_l13=True)
        print(json.dumps({"metric": "host-staged ms/token vs context, exact vs lossless 13-bit vs hybrid "
                                    "(the tier gate)",
                          "unit": "ms/token", "n_gpus": 1, "higher_is_better": False,
                          "data": "synthetic (the ctx128k recipe at each context length, pinned host history)",
                          "pcie_h2d_curve_MiB_GBps": [[m, round(g, 2)] for m, g in sw["curve"]],
                          "staged_copy_curve_MiB_GBps": {f"slots{ns}": [[m, round(g, 2)] for m, g in c]
                                                         for ns, c in sw["staged_curve"].items()},
                          "copy_model": staging_model_json(sw["model"]),
                          "contexts": sw["rows"]}), flush=True)
        return
    if w.name == "staged128k":
        r = run_staged(args, w)
        print(json.dumps({
            "metric": "ms/token host-staged at 128K, int8 hybrid vs BF16 (PCIe GB/s)",
            "value": round(r["ms_h"], 3), "unit": "ms/token", "n_gpus": 1, "steps": r["steps"], "warmup": 1,
            "ms_per_step": round(r["ms_h"], 3), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
            "dtype": "int8", "data": "synthetic (the ctx128k recipe, history held in pinned host memory)",
            "config": {"workload": w.name, "context_tokens": int(w.lengths[0]), "layers": w.layers,
                       "kv_heads": w.num_kv_heads, "group": w.group, "ring_slots": 2,
                       "launch": "per layer: akv_ring_stage on a side stream, akv_decode_hybrid, akv_ring_release"},
            "roofline": {"bound": "pcie", "achieved": round(r["bytes_h"] / (r["ms_h"] * 1e-3) / 1e9, 1),
                         "peak": round(r["h2d_gbps"], 1), "unit": "GB/s",
                         "frac": round(r["bytes_h"] / (r["ms_h"] * 1e-3) / 1e9 / r["h2d_gbps"], 4),
                         "traffic": None, "peak_is": "measured plain host-to-device copy of one layer's BF16 pool"},
            "extra": {"hybrid_bytes_staged_per_token": r["bytes_h"], "bf16_bytes_staged_per_token": r["bytes_b"],
                      "bytes_not_moved_per_token": r["bytes_b"] - r["bytes_h"],
                      "ms_per_token_bf16_staged": round(r["ms_b"], 3),
                      "bf16_staged_GBps": round(r["bytes_b"] / (r["ms_b"] * 1e-3) / 1e9, 1),
                      "speedup_vs_bf16_staged": round(r["ms_b"] / r["ms_h"], 3),
                      "lossless13_bytes_staged_per_token": r["bytes_l"],
                      "ms_per_token_lossless13_staged": round(r["ms_l"], 3),
                      "lossless13_staged_GBps": round(r["bytes_l"] / (r["ms_l"] * 1e-3) / 1e9, 1),
                      "lossless13_speedup_vs_bf16_staged": round(r["ms_b"] / r["ms_l"], 3)},
        }), flush=True)
        return
    device = torch.device("cuda", 0)
    torch.cuda.set_device(device)
    res32 = None
    if w.name == "ctx128k" and not args.headline_only:
        # the 32K inputs go into HBM first, while the allocator is fresh: built
        # after the 128K inputs were released, the same 32K step read 3-4%
        # slower (0.297-0.301 against 0.290 ms)
        log("[bench] building ctx32k first")
        res32 = Resident(configs.ctx32k(), device)
    log(f"[bench] building {w.name}: {w.layers} layers, lengths {w.lengths[:4]}...")
    res = Resident(w, device)
    r = run_gpu(args, w, res)
    cb = check = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (float64 oracle on the timed step's inputs) and oracle check")
        cb, check = cpu_baseline(w, res, r["hyb_out"])
    res.free()
    del r["hyb_out"]
    ms = r["ms_hybrid"]
    value = r["hybrid_bytes"] / (ms * 1e-3) / 1e9
    out = {
        "metric": "\u00b5s/decode step + KV bytes/s (% of HBM peak) at 128K, int8 hybrid vs BF16",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded on-device draws: K ~ N(0,1)*logU[0.1,10] per channel, V ~ N(0,1)*logU[0.5,2], "
                "2% outlier tokens x8; pages quantized by akv_quantize_pages)",
        "config": {"workload": w.name, "context_tokens": int(w.lengths[0]), "batch": w.batch,
                   "layers": w.layers, "kv_heads": w.num_kv_heads, "group": w.group, "head_dim": w.head_dim,
                   "page": w.page, "bf16_window_tokens": w.window, "parallelism": "single GPU",
                   "launch": "eager; per layer akv_decode_hybrid = split-K kernel + combine kernel",
                   "pv_operand": "fp16 hi+lo" if args.pv_fp16 else "int8 MFMA, 3 fixed-point limbs"},
        "roofline": {"bound": "hbm", "achieved": round(r["hyb_achieved_gbps"], 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(r["hyb_achieved_gbps"] / HBM_PEAK_GBPS, 4),
                     "traffic": load_traffic("decode_hybrid_kernel", w.name),
                     "kernel": "decode_hybrid_kernel (int8 pages + BF16 window of one layer), split-K pass alone",
                     "bytes_per_launch": r["hyb_bytes_per_launch"],
                     "avg_launch_us": round(r["hyb_launch_us"], 3),
                     "frac_step": round(value / HBM_PEAK_GBPS, 4),
                     "frac_step_is": "whole 16-layer step (split-K kernels, second passes and launch gaps) "
                                     "against the same peak"},
        "extra": {
            "us_per_step_hybrid": round(ms * 1e3, 2),
            "us_per_layer_hybrid": round(ms * 1e3 / w.layers, 2),
            "hybrid_kv_bytes_per_step": r["hybrid_bytes"],
            "hybrid_frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
            "step_us_p10_p50_p90": [round(x, 1) for x in r["step_p"]],
            "stream_read_ceiling_GBps": round(r["read_gbps"], 1),
            "kernel_frac_of_stream_ceiling": round(r["hyb_achieved_gbps"] / r["read_gbps"], 4),
            "step_frac_of_stream_ceiling": round(value / r["read_gbps"], 4),
            "us_per_step_four_call": round(r["ms_four"] * 1e3, 2),
            "us_per_step_bf16_all": round(r["ms_bf16"] * 1e3, 2),
            "bf16_split_kernel_us": round(r["bf16_launch_us"], 2),
            "bf16_split_kernel_GBps": round(r["bf16_achieved_gbps"], 1),
            "bf16_kv_bytes_per_step": r["bf16_bytes"],
            "bf16_GBps": round(r["bf16_bytes"] / (r["ms_bf16"] * 1e-3) / 1e9, 1),
            "hybrid_speedup_vs_bf16": round(r["ms_bf16"] / ms, 3),
            "quantize_ms_per_layer": round(r["quant_ms_per_layer"], 3),
            "quantize_GBps_read_plus_write": round(r["quant_gbps"], 1),
            "lossless13": {
                "us_per_step": round(r["lossless"]["ms_step"] * 1e3, 2),
                "split_kernel_us": round(r["lossless"]["launch_us"], 2),
                "bytes_per_launch": r["lossless"]["bytes_per_launch"],
                "split_kernel_GBps": round(r["lossless"]["bytes_per_launch"] / (r["lossless"]["launch_us"] * 1e-6)
                                           / 1e9, 1),
                "arena_bytes_per_layer": r["lossless"]["arena_bytes_per_layer"],
                "arena_frac_of_bf16": round(r["lossless"]["arena_frac_of_bf16"], 4),
                "raw_planes": r["lossless"]["raw_planes"], "planes": r["lossless"]["planes"],
                "encode_ms_per_layer": round(r["lossless"]["encode_ms_per_layer"], 3),
                "encode_GBps_bf16_in": round(r["lossless"]["encode_GBps_in"], 1),
                "speedup_vs_bf16": round(r["ms_bf16"] / r["lossless"]["ms_step"], 3),
            },
        },
    }
    if check is not None:
        out["extra"]["oracle_check"] = check
    if w.name == "ctx128k" and not args.headline_only:
        log("[bench] ctx32k")
        out["extra"]["ctx32k"] = run_config(args, configs.ctx32k(), res=res32)
        log("[bench] batched")
        out["extra"]["batched"] = run_config(args, configs.batched(), owner_modes=True)
        log("[bench] host-staged sweep 8K..128K with the tier gate's transfer model")
        sw = staged_sweep(args)
        last = sw["last"]
        out["extra"]["staged128k"] = {
            "ms_per_token_hybrid": round(last["ms_h"], 3), "ms_per_token_bf16": round(last["ms_b"], 3),
            "pcie_GBps_hybrid": round(last["bytes_h"] / (last["ms_h"] * 1e-3) / 1e9, 1),
            "pcie_GBps_bf16": round(last["bytes_b"] / (last["ms_b"] * 1e-3) / 1e9, 1),
            "h2d_copy_GBps": round(last["h2d_gbps"], 1), "ring_slots": RING_SLOTS[0],
            "hybrid_frac_of_h2d_copy": round(last["bytes_h"] / (last["ms_h"] * 1e-3) / 1e9 / last["h2d_gbps"], 4),
            "bytes_per_token_hybrid": last["bytes_h"], "bytes_per_token_bf16": last["bytes_b"],
            "bytes_not_moved_per_token": last["bytes_b"] - last["bytes_h"],
            "speedup_vs_bf16_staged": round(last["ms_b"] / last["ms_h"], 3)}
        out["extra"]["tier_gate"] = {
            "pcie_h2d_curve_MiB_GBps": [[m, round(g, 2)] for m, g in sw["curve"]],
            "staged_copy_curve_MiB_GBps": {f"slots{ns}": [[m, round(g, 2)] for m, g in c]
                                           for ns, c in sw["staged_curve"].items()},
            "copy_model": staging_model_json(sw["model"]),
            "ring_slots_measured": list(RING_SLOTS),
            "contexts": sw["rows"],
            "max_abs_prediction_error": round(max(max(abs(x[f"slots{k}"]["prediction_error_hybrid"]),
                                                      abs(x[f"slots{k}"]["prediction_error_bf16"]))
                                                  for x in sw["rows"] for k in RING_SLOTS), 4),
            "model_choice_equals_measured_argmin": all(x[f"slots{k}"]["chosen_by_model"] ==
                                                       x[f"slots{k}"]["chosen_by_measurement"]
                                                       for x in sw["rows"] for k in RING_SLOTS)}
    if cb is not None:
        out["cpu_baseline"] = {k: (round(v, 1) if isinstance(v, float) else v) for k, v in cb.items()}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
