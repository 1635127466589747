"""Host-staged mode through the C ABI: layers staged from pinned host memory
into a ring of device slots decode bit-identically to the same call on
HBM-resident copies, including when the ring is reused many times over, and
every staged layer matches the oracle at the 128K config's head shape (4 KV
heads, 6 query heads each), also when the kernels reading a slot are held
back for tens of milliseconds while later copies are queued (an unguarded
schedule of the same copies is shown to corrupt layers there); an oversize
layer is refused before any copy, and out-of-order use is refused.
"""
import numpy as np
import pytest
import torch

from quantized_paged_kv_akv_amd import configs, inputs
from oracle import oracle as O
from tests.gpu_util import check_attn, dev, gpu_quantize, oracle_hybrid, say

pytestmark = pytest.mark.gpu
SIG = 1.0 / 16.0


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from quantized_paged_kv_akv_amd import binding
    return binding


def _pinned(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.pin_memory()


def _layer(B, w, layer, with_oracle=False):
    """One layer's hybrid inputs: the int8 pool (codes + scales) and a compact
    BF16 pool holding only the window pages, as pinned host tensors, plus the
    query and tables on the device (and, if asked, the oracle's merged
    result on the GPU's codes)."""
    d = inputs.make_layer_np(w, layer)
    plan = d["plan"]
    src, dst = plan.quant_src_dst()
    g = gpu_quantize(B, d["k_pool"], d["v_pool"], src, dst, max(1, plan.int8_slots_total), w.num_kv_heads)
    tw = plan.window_table()
    kw = d["k_pool"][tw.reshape(-1)]
    vw = d["v_pool"][tw.reshape(-1)]
    tw_c = np.arange(tw.size, dtype=np.int32).reshape(tw.shape)
    srcs = [g[k].cpu().pin_memory() for k in ("k_codes", "v_codes", "k_chan", "k_tok", "v_chan")]
    srcs += [_pinned(kw), _pinned(vw)]
    t8 = plan.int8_table()
    meta = dict(q=dev(d["q"]), t8=dev(t8), n8=dev(np.asarray(plan.n8, np.int32)), m8=t8.shape[1],
                tw=dev(tw_c), nw=dev(np.asarray(plan.win_tokens, np.int32)), mw=tw.shape[1])
    if with_oracle:
        meta["ref"] = oracle_hybrid(O, w.num_kv_heads, w.group, d["q"], g, t8, plan.n8, kw, vw, tw_c,
                                    plan.win_tokens)
    return srcs, meta


def _decode(B, w, arrs, meta, o, l, ws, stream=None):
    d8 = B.dims(w.num_kv_heads, w.group)
    B.akv_decode_hybrid(d8, w.batch, meta["q"], arrs[0], arrs[1], arrs[2], arrs[3], arrs[4], meta["t8"],
                        meta["n8"], meta["m8"], arrs[5], arrs[6], meta["tw"], meta["nw"], meta["mw"], SIG, o, l,
                        ws, stream)


def _nbytes(srcs):
    return sum((t.numel() * t.element_size() + 255) // 256 * 256 for t in srcs)


def test_ring_staged_equals_resident(B):
    """Eight layers through a two-slot ring: every slot is reused four times
    while copies of later layers run on a side stream."""
    w = configs.tiny()
    w = inputs.Workload("tiny8", w.cfg_id, batch=w.batch, layers=8, num_kv_heads=w.num_kv_heads, group=w.group,
                        lengths=w.lengths, window=w.window, outlier_frac=w.outlier_frac, permute=w.permute)
    layers = [_layer(B, w, i) for i in range(w.layers)]
    d8 = B.dims(w.num_kv_heads, w.group)
    m8, mw = layers[0][1]["m8"], layers[0][1]["mw"]
    ws = torch.empty(max(16, B.akv_decode_hybrid_workspace_bytes(d8, w.batch, m8, mw)), dtype=torch.uint8,
                     device="cuda")
    rows = (w.batch, w.num_q_heads)
    ref = []
    for srcs, meta in layers:
        o = torch.empty((*rows, 256), device="cuda")
        l = torch.empty(rows, device="cuda")
        _decode(B, w, [t.cuda() for t in srcs], meta, o, l, ws)
        ref.append((o, l))
    torch.cuda.synchronize()

    slot_bytes = _nbytes(layers[0][0])
    say("case ring 8 layers, 2 slots of", slot_bytes, "bytes")
    slots = [torch.empty(slot_bytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    ring = B.Ring(slots)
    copy_s = torch.cuda.Stream()
    comp_s = torch.cuda.current_stream()
    outs = []
    try:
        for i, (srcs, meta) in enumerate(layers):
            views = ring.stage_views(i, srcs, copy_s, comp_s)
            o = torch.full((*rows, 256), float("nan"), device="cuda")
            l = torch.full(rows, float("nan"), device="cuda")
            _decode(B, w, views, meta, o, l, ws, comp_s)
            ring.release(i, comp_s)
            outs.append((o, l))
        torch.cuda.synchronize()
    finally:
        ring.destroy()
    for i, ((o, l), (ro, rl)) in enumerate(zip(outs, ref)):
        assert torch.equal(o, ro) and torch.equal(l, rl), f"layer {i} differs from the resident decode"


def test_ring_refuses_oversize_before_copying(B):
    w = configs.tiny()
    srcs, _ = _layer(B, w, 0)
    need = _nbytes(srcs)
    slots = [torch.full((need - 256,), 7, dtype=torch.uint8, device="cuda") for _ in range(2)]
    ring = B.Ring(slots)
    try:
        with pytest.raises(B.AkvError) as e:
            ring.stage(0, srcs, torch.cuda.Stream(), torch.cuda.current_stream())
        assert e.value.status_name == "AKV_ERR_BUDGET", e.value
        torch.cuda.synchronize()
        assert bool((slots[0] == 7).all()) and bool((slots[1] == 7).all()), "a refused stage wrote to a slot"
    finally:
        ring.destroy()


def test_ring_lifecycle_errors(B):
    w = configs.tiny()
    srcs, _ = _layer(B, w, 0)
    need = _nbytes(srcs)
    slots = [torch.empty(need, dtype=torch.uint8, device="cuda") for _ in range(2)]
    ring = B.Ring(slots)
    cs, ks = torch.cuda.Stream(), torch.cuda.current_stream()
    try:
        with pytest.raises(B.AkvError) as e:
            ring.release(0, ks)  # never staged
        assert e.value.status_name == "AKV_ERR_STATE"
        ring.stage(0, srcs, cs, ks)
        with pytest.raises(B.AkvError) as e:
            ring.stage(2, srcs, cs, ks)  # same slot (2 % 2), not yet released
        assert e.value.status_name == "AKV_ERR_STATE"
        ring.stage(1, srcs, cs, ks)  # the other slot is free
        ring.release(0, ks)
        ring.stage(2, srcs, cs, ks)
        ring.release(1, ks)
        ring.release(2, ks)
        torch.cuda.synchronize()
    finally:
        ring.destroy()


def test_ring_staged_13bit_equals_resident(B):
    """The 13-bit history staged through the ring (packed planes, descriptors
    and tables in one slot per layer) decodes bit-identically to the same
    records resident in HBM."""
    from quantized_paged_kv_akv_amd import inputs as I
    Hkv, G, n, layers = 2, 3, 6, 4
    d = B.dims(Hkv, G)
    seq = [n * 64 - 20, 64 * 3]
    table = torch.tensor([[0, 1, 2, 3, 4, 5], [5, 3, 1, 0, 0, 0]], dtype=torch.int32, device="cuda")
    lens = torch.tensor(seq, dtype=torch.int32, device="cuda")
    recs, qs = [], []
    for layer in range(layers):
        kp, vp = I.random_pools(900 + layer, n, Hkv)
        sz = B.l13_sizes(d, n)
        arena = torch.empty(sz["arena_bytes"], dtype=torch.uint8, device="cuda")
        desc = torch.empty(sz["desc"], dtype=torch.int32, device="cuda")
        tab = torch.empty(sz["table"], dtype=torch.uint8, device="cuda")
        end = torch.empty(1, dtype=torch.int64, device="cuda")
        s = torch.arange(n, dtype=torch.int32, device="cuda")
        B.akv_l13_encode_pages(d, n, dev(kp), dev(vp), s, s, arena, 0, desc, tab, end)
        torch.cuda.synchronize()
        recs.append((arena[:int(end[0])].clone(), desc, tab))
        qs.append(dev(I.random_queries(950 + layer, 2, Hkv * G)))
    ws = torch.empty(max(16, B.akv_decode_workspace_bytes(d, 2, n)), dtype=torch.uint8, device="cuda")
    ref = []
    for (arena, desc, tab), q in zip(recs, qs):
        o = torch.empty((2, Hkv * G, 256), device="cuda")
        l = torch.empty((2, Hkv * G), device="cuda")
        B.akv_decode_attn_l13(d, 2, q, arena, desc, tab, table, lens, n, SIG, o, l, ws)
        ref.append((o, l))
    torch.cuda.synchronize()
    srcs = [[r[0].cpu().pin_memory(), r[1].cpu().pin_memory(), r[2].cpu().pin_memory()] for r in recs]
    slot_bytes = max(_nbytes(x) for x in srcs)
    say("case ring 13-bit, 4 layers, 2 slots of", slot_bytes, "bytes")
    ring = B.Ring([torch.empty(slot_bytes, dtype=torch.uint8, device="cuda") for _ in range(2)])
    copy_s, comp_s = torch.cuda.Stream(), torch.cuda.current_stream()
    outs = []
    try:
        for i, (x, q) in enumerate(zip(srcs, qs)):
            arena, desc, tab = ring.stage_views(i, x, copy_s, comp_s)
            o = torch.full((2, Hkv * G, 256), float("nan"), device="cuda")
            l = torch.full((2, Hkv * G), float("nan"), device="cuda")
            B.akv_decode_attn_l13(d, 2, q, arena, desc, tab, table, lens, n, SIG, o, l, ws, comp_s)
            ring.release(i, comp_s)
            outs.append((o, l))
        torch.cuda.synchronize()
    finally:
        ring.destroy()
    for i, ((o, l), (ro, rl)) in enumerate(zip(outs, ref)):
        assert torch.equal(o, ro) and torch.equal(l, rl), f"layer {i} differs from the resident 13-bit decode"


def _ctx_shape_workload(layers):
    """The 128K config's head shape at a length a test stages quickly: 64
    int8 pages and a 1061-token window (17 pages, the last partial) per
    layer, 2% outlier tokens."""
    return inputs.Workload("staged-test", 4, batch=1, layers=layers, num_kv_heads=4, group=6,
                           lengths=(64 * 64 + 1024 + 37,), window=1024, outlier_frac=0.02, permute=False)


def _ring_decode_all(B, w, layers, slots, delay_cycles=0):
    """Stage every layer through the library ring (two slots), decoding each
    on the compute stream, optionally after a bounded spin of delay_cycles
    on that stream (the reader of a slot is held back while the copy stream
    could already run ahead)."""
    d8 = B.dims(w.num_kv_heads, w.group)
    ws = torch.empty(max(16, B.akv_decode_hybrid_workspace_bytes(d8, w.batch, layers[0][1]["m8"],
                                                                 layers[0][1]["mw"])),
                     dtype=torch.uint8, device="cuda")
    ring = B.Ring(slots)
    copy_s = torch.cuda.Stream()
    comp_s = torch.cuda.current_stream()
    outs = []
    try:
        for i, (srcs, meta) in enumerate(layers):
            views = ring.stage_views(i, srcs, copy_s, comp_s)
            o = torch.full((w.batch, w.num_q_heads, 256), float("nan"), device="cuda")
            l = torch.full((w.batch, w.num_q_heads), float("nan"), device="cuda")
            if delay_cycles:
                torch.cuda._sleep(delay_cycles)
            _decode(B, w, views, meta, o, l, ws, comp_s)
            ring.release(i, comp_s)
            outs.append((o, l))
        torch.cuda.synchronize()
    finally:
        ring.destroy()
    return outs


def test_ring_staged_layers_match_oracle(B):
    """Eight layers at the 128K config's head shape (4 KV heads x 6, 64 int8
    pages + a 1061-token window each) staged through two slots: every staged
    layer's output against the oracle on the GPU's codes."""
    w = _ctx_shape_workload(8)
    layers = [_layer(B, w, i, with_oracle=True) for i in range(w.layers)]
    slot_bytes = _nbytes(layers[0][0])
    say("case ring oracle parity, 8 layers of", slot_bytes, "bytes, 2 slots")
    outs = _ring_decode_all(B, w, layers, [torch.empty(slot_bytes, dtype=torch.uint8, device="cuda")
                                           for _ in range(2)])
    rows = w.batch * w.num_q_heads
    for i, ((o, l), (_, meta)) in enumerate(zip(outs, layers)):
        check_attn(o.view(rows, 256), l.view(rows), *meta["ref"], f"staged layer {i}")


def _cycles_for_ms(ms):
    """Spin cycles of torch.cuda._sleep that take about `ms` milliseconds on
    this GPU (measured)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    e0.record()
    torch.cuda._sleep(1_000_000)
    e1.record()
    torch.cuda.synchronize()
    per_cycle_ms = max(e0.elapsed_time(e1), 1e-3) / 1_000_000
    return int(ms / per_cycle_ms)


def test_ring_fence_holds_under_slow_reader(B):
    """The kernels that read a slot are held back about 20 ms each (a bounded
    spin on the compute stream before every decode), far longer than one
    layer's copy: without the slot-free wait the copy of layer i + 2 would
    overwrite slot i % 2 before layer i is decoded.  With the ring every
    layer still matches the oracle.  The same schedule with the copies
    issued unguarded (only the copy-done wait) is run as a control and must
    corrupt at least one layer, which shows the delay makes this test able
    to catch a missing wait."""
    w = _ctx_shape_workload(6)
    layers = [_layer(B, w, i, with_oracle=True) for i in range(w.layers)]
    slot_bytes = _nbytes(layers[0][0])
    cycles = _cycles_for_ms(20.0)
    say("case ring fence under a slow reader:", w.layers, "layers, spin cycles", cycles)
    rows = w.batch * w.num_q_heads
    slots = [torch.empty(slot_bytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    # the copy of one layer takes far less time than the hold-back
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t, off in zip(layers[0][0], np.cumsum([0] + [(x.numel() * x.element_size() + 255) // 256 * 256
                                                     for x in layers[0][0]])):
        n = t.numel() * t.element_size()
        slots[0][off:off + n].copy_(t.view(-1).view(torch.uint8), non_blocking=True)
    e1.record()
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e2.record()
    torch.cuda._sleep(cycles)
    e3.record()
    torch.cuda.synchronize()
    copy_ms, hold_ms = e0.elapsed_time(e1), e2.elapsed_time(e3)
    say(f"one layer's copy {copy_ms:.3f} ms, hold-back {hold_ms:.1f} ms")
    assert hold_ms > 10 * copy_ms

    outs = _ring_decode_all(B, w, layers, slots, delay_cycles=cycles)
    for i, ((o, l), (_, meta)) in enumerate(zip(outs, layers)):
        check_attn(o.view(rows, 256), l.view(rows), *meta["ref"], f"slow-reader staged layer {i}")

    # control: the same copies into the same two slots with no slot-free wait
    d8 = B.dims(w.num_kv_heads, w.group)
    ws = torch.empty(max(16, B.akv_decode_hybrid_workspace_bytes(d8, w.batch, layers[0][1]["m8"],
                                                                 layers[0][1]["mw"])),
                     dtype=torch.uint8, device="cuda")
    copy_s, comp_s = torch.cuda.Stream(), torch.cuda.current_stream()
    copy_s.wait_stream(comp_s)
    bad = 0
    ctl = []
    for i, (srcs, meta) in enumerate(layers):
        slot = slots[i % 2]
        views, off = [], 0
        with torch.cuda.stream(copy_s):
            for t in srcs:
                n = t.numel() * t.element_size()
                slot[off:off + n].copy_(t.view(-1).view(torch.uint8), non_blocking=True)
                views.append(slot[off:off + n].view(t.dtype).view(t.shape))
                off += (n + 255) // 256 * 256
        done = torch.cuda.Event()
        done.record(copy_s)
        comp_s.wait_event(done)
        o = torch.full((w.batch, w.num_q_heads, 256), float("nan"), device="cuda")
        l = torch.full((w.batch, w.num_q_heads), float("nan"), device="cuda")
        torch.cuda._sleep(cycles)
        _decode(B, w, views, meta, o, l, ws, comp_s)
        ctl.append((o, l))
    torch.cuda.synchronize()
    for (o, l), (_, meta) in zip(ctl, layers):
        err = float(np.abs(o.view(rows, 256).cpu().numpy() - meta["ref"][0]).max())
        bad += err > 2e-3
    say(f"unguarded control: {bad} of {len(layers)} layers corrupted")
    assert bad >= 1
