"""Streaming page publication through the C ABI: decode steps append one
token per layer to the BF16 window; a page that is full and older than the
window is converted on a side stream (akv_publish_pages) while decode keeps
serving it exact, and is moved to the int8 tier by akv_tables_advance only
after its done event has completed.  Every checked step must match the oracle
for the tier assignment in force at that step."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from quantized_paged_kv_akv_amd import inputs
from tests.gpu_util import check_attn, check_quantize, dev, host, k_codes_token_major, say

pytestmark = pytest.mark.gpu
SIG = 1.0 / 16.0


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from quantized_paged_kv_akv_amd import binding
    return binding


def test_streaming_publication(B):
    Hkv, G, D, P = 2, 3, 256, 64
    layers, W, L0, steps, cap = 2, 128, 5 * 64 + 30, 170, 12
    r = np.random.default_rng(77)
    sk = np.exp(r.uniform(np.log(0.1), np.log(10.0), (layers, 1, Hkv, D))).astype(np.float32)
    K = (r.standard_normal((layers, cap * P, Hkv, D), dtype=np.float32) * sk)
    V = r.standard_normal((layers, cap * P, Hkv, D), dtype=np.float32)
    Kb = inputs.f32_to_bf16_bits(K)
    Vb = inputs.f32_to_bf16_bits(V)
    # pools in the library layouts, slot = page index; only the first L0 tokens are written up front
    kp_full = Kb.reshape(layers, cap, P, Hkv, D).transpose(0, 1, 3, 2, 4).copy()     # [l][slot][h][t][d]
    vp_full = Vb.reshape(layers, cap, P, Hkv, D).transpose(0, 1, 3, 4, 2).copy()     # [l][slot][h][d][t]
    kpool = [torch.zeros((cap, Hkv, P, D), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    vpool = [torch.zeros((cap, Hkv, D, P), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    for l in range(layers):
        for t in range(L0):
            kpool[l][t // P, :, t % P, :] = dev(kp_full[l, t // P, :, t % P, :])
            vpool[l][t // P, :, :, t % P] = dev(vp_full[l, t // P, :, :, t % P])
    codes = [dict(k_codes=torch.zeros((cap, Hkv, P, D), dtype=torch.int8, device="cuda"),
                  v_codes=torch.zeros((cap, Hkv, D, P), dtype=torch.int8, device="cuda"),
                  k_chan=torch.zeros((cap, Hkv, D), device="cuda"), k_tok=torch.zeros((cap, Hkv, P), device="cuda"),
                  v_chan=torch.zeros((cap, Hkv, D), device="cuda")) for _ in range(layers)]
    d = B.dims(Hkv, G)
    n8 = (L0 - W) // P
    init = torch.arange(n8, dtype=torch.int32, device="cuda")
    for l in range(layers):
        c = codes[l]
        B.akv_quantize_pages(d, n8, kpool[l], vpool[l], init, init, c["k_codes"], c["v_codes"], c["k_chan"],
                             c["k_tok"], c["v_chan"])
    t8 = torch.zeros((1, cap), dtype=torch.int32, device="cuda")
    t8[0, :n8] = init
    n8_d = torch.tensor([n8], dtype=torch.int32, device="cuda")
    tw = torch.zeros((1, cap), dtype=torch.int32, device="cuda")
    tw[0, :cap - n8] = torch.arange(n8, cap, dtype=torch.int32, device="cuda")
    wl_d = torch.tensor([L0 - n8 * P], dtype=torch.int32, device="cuda")
    q = [torch.from_numpy(inputs.f32_to_bf16_bits(r.standard_normal((1, Hkv * G, D), dtype=np.float32))
                          .view(np.int16)).cuda().view(torch.bfloat16) for _ in range(layers)]
    ws = torch.empty(max(16, B.akv_decode_hybrid_workspace_bytes(d, 1, cap, cap)), dtype=torch.uint8, device="cuda")
    status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    comp = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    state = dict(n8=n8, wlen=L0 - n8 * P)  # host mirror of the tables
    pending = None                          # (page, done event, count, new slot tensors)
    checks, n_published, exact_while_pending = [], 0, 0
    for s in range(steps):
        t = L0 + s
        for l in range(layers):  # append token t
            kpool[l][t // P, :, t % P, :] = dev(kp_full[l, t // P, :, t % P, :])
            vpool[l][t // P, :, :, t % P] = dev(vp_full[l, t // P, :, :, t % P])
        wl_d += 1
        state["wlen"] += 1
        if pending is not None and pending[1].query():
            page, _, cnt, nw = pending
            B.akv_tables_advance(1, cnt, nw, t8, n8_d, tw, wl_d, status, comp)
            state["n8"] += 1
            state["wlen"] -= P
            n_published += 1
            pending = None
        if pending is None and state["wlen"] - P >= W:
            page = state["n8"]  # the oldest window page: full, and W tokens stay exact behind it
            ready = torch.cuda.Event()
            ready.record(comp)
            done = torch.cuda.Event()
            done.record(side)  # creates the HIP event; re-recorded by the library
            sl = torch.tensor([page], dtype=torch.int32, device="cuda")
            for l in range(layers):
                c = codes[l]
                B.akv_publish_pages(d, 1, kpool[l], vpool[l], sl, sl, c["k_codes"], c["v_codes"], c["k_chan"],
                                    c["k_tok"], c["v_chan"], ready, side, done if l == layers - 1 else None)
            pending = (page, done, torch.tensor([1], dtype=torch.int32, device="cuda"), sl.view(1, 1))
        if pending is not None:
            exact_while_pending += 1
        outs = []
        for l in range(layers):
            c = codes[l]
            o = torch.full((1, Hkv * G, D), float("nan"), device="cuda")
            lse = torch.full((1, Hkv * G), float("nan"), device="cuda")
            B.akv_decode_hybrid(d, 1, q[l], c["k_codes"], c["v_codes"], c["k_chan"], c["k_tok"], c["v_chan"], t8,
                                n8_d, cap, kpool[l], vpool[l], tw, wl_d, cap, SIG, o, lse, ws, comp)
            outs.append((o, lse))
        # every step that served a converting page exact is checked, and a sample of the rest
        if s % 17 == 0 or s == steps - 1 or pending is not None:
            checks.append((s, dict(state), outs))
    side.synchronize()
    torch.cuda.synchronize()
    say(f"case streaming publication: {steps} steps, {n_published} pages published, "
        f"{exact_while_pending} steps served a converting page exact, {len(checks)} steps checked")
    assert n_published >= 2 and exact_while_pending >= 1
    assert int(status[0]) == 0
    assert int(n8_d[0]) == state["n8"] and int(wl_d[0]) == state["wlen"]

    for l in range(layers):
        g = codes[l]
        pages = np.arange(state["n8"], dtype=np.int32)
        check_quantize(O, kp_full[l], vp_full[l], pages, pages, cap, Hkv, g, f"published layer {l}")
    for s, st, outs in checks:
        for l in range(layers):
            g = codes[l]
            qn = host(q[l].view(torch.int16)).view(np.uint16)
            n8s, wlen = st["n8"], st["wlen"]
            t8h = np.arange(max(1, n8s), dtype=np.int32).reshape(1, -1)
            ro8, rl8 = O.decode_int8(qn, k_codes_token_major(host(g["k_codes"])), host(g["v_codes"]), host(g["k_chan"]),
                                     host(g["k_tok"]), host(g["v_chan"]), t8h, np.array([n8s], np.int32), Hkv, G,
                                     SIG, mode=0)
            twh = np.arange(n8s, cap, dtype=np.int32).reshape(1, -1)
            row, rlw = O.decode_exact(qn, kp_full[l], vp_full[l], twh, np.array([wlen], np.int32), Hkv, G, SIG)
            rows = Hkv * G
            rm, rlm = O.merge(np.stack([ro8.reshape(rows, D), row.reshape(rows, D)]),
                              np.stack([rl8.reshape(rows), rlw.reshape(rows)]))
            o, lse = outs[l]
            check_attn(o.view(rows, D), lse.view(rows), rm, rlm, f"step {s} layer {l} n8={n8s} window={wlen}")


def test_tables_advance_refuses_rows_that_do_not_fit(B):
    """Rows whose update would not fit are left unchanged and flagged; the
    others are updated (one launch, three requests)."""
    cap = 4
    t8 = torch.tensor([[0, 1, 0, 0], [5, 6, 7, 0], [2, 0, 0, 0]], dtype=torch.int32, device="cuda")
    n8 = torch.tensor([2, 3, 1], dtype=torch.int32, device="cuda")
    tw = torch.tensor([[2, 3, 9, 9], [8, 9, 10, 11], [3, 4, 5, 6]], dtype=torch.int32, device="cuda")
    wl = torch.tensor([100, 150, 40], dtype=torch.int32, device="cuda")
    count = torch.tensor([1, 2, 1], dtype=torch.int32, device="cuda")  # row 1: int8 table full; row 2: < 64 tokens
    new = torch.tensor([[2, 0], [8, 9], [3, 0]], dtype=torch.int32, device="cuda")
    status = torch.full((3,), 7, dtype=torch.int32, device="cuda")
    say("case tables advance with refused rows")
    B.akv_tables_advance(3, count, new, t8, n8, tw, wl, status)
    torch.cuda.synchronize()
    assert status.tolist() == [0, -1, -1]
    assert t8.tolist() == [[0, 1, 2, 0], [5, 6, 7, 0], [2, 0, 0, 0]]
    assert n8.tolist() == [3, 3, 1]
    assert tw.tolist() == [[3, 9, 9, 9], [8, 9, 10, 11], [3, 4, 5, 6]]
    assert wl.tolist() == [36, 150, 40]
    assert cap == t8.shape[1]
