"""akv_decode_hybrid_static (split partials in the library's static
per-device scratch, nothing allocated) through the C ABI: two calls in a row,
the second on a smaller input, each equal to akv_decode_hybrid on the same
inputs with a caller-owned workspace, and both within the acceptance bar of
the oracle; a plan that needs more than the scratch array is refused before
anything is enqueued."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from quantized_paged_kv_akv_amd import configs, inputs
from tests.gpu_util import check_attn, dev, gpu_quantize, oracle_int8, say

pytestmark = pytest.mark.gpu
SIG = 1.0 / 16.0


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from quantized_paged_kv_akv_amd import binding
    return binding


def _layer(B, w, layer):
    d = inputs.make_layer_np(w, layer)
    plan = d["plan"]
    src, dst = plan.quant_src_dst()
    g = gpu_quantize(B, d["k_pool"], d["v_pool"], src, dst, max(1, plan.int8_slots_total), w.num_kv_heads)
    t8, tw = plan.int8_table(), plan.window_table()
    return dict(d=d, g=g, t8=t8, tw=tw, args=(
        dev(d["q"]), g["k_codes"], g["v_codes"], g["k_chan"], g["k_tok"], g["v_chan"], dev(t8),
        dev(np.asarray(plan.n8, np.int32)), t8.shape[1], dev(d["k_pool"]), dev(d["v_pool"]), dev(tw),
        dev(np.asarray(plan.win_tokens, np.int32)), tw.shape[1], SIG))


def _oracle(w, L):
    d, plan = L["d"], L["d"]["plan"]
    rows = w.batch * w.num_q_heads
    ro8, rl8 = oracle_int8(O, w.num_kv_heads, w.group, d["q"], L["g"], L["t8"], plan.n8)
    row, rlw = O.decode_exact(d["q"], d["k_pool"], d["v_pool"], L["tw"], np.asarray(plan.win_tokens, np.int32),
                              w.num_kv_heads, w.group, SIG)
    return O.merge(np.stack([ro8.reshape(rows, 256), row.reshape(rows, 256)]),
                   np.stack([rl8.reshape(rows), rlw.reshape(rows)]))


def test_static_scratch_two_calls_second_smaller(B):
    big = configs.ctx32k()
    full = configs.batched()
    small = inputs.Workload("batched4", full.cfg_id, batch=4, layers=1, num_kv_heads=4, group=6,
                            lengths=full.lengths[:4], window=512, outlier_frac=0.02, permute=True)
    cases = [(big, _layer(B, big, 2)), (small, _layer(B, small, 0))]
    outs = []
    for w, L in cases:  # two calls in a row on the static scratch, the second smaller
        say(f"case static scratch {w.name}")
        d8 = B.dims(w.num_kv_heads, w.group)
        o = torch.full((w.batch, w.num_q_heads, 256), float("nan"), device="cuda")
        lse = torch.full((w.batch, w.num_q_heads), float("nan"), device="cuda")
        B.akv_decode_hybrid_static(d8, w.batch, *L["args"], o, lse)
        outs.append((o, lse))
    torch.cuda.synchronize()
    for (w, L), (o, lse) in zip(cases, outs):
        d8 = B.dims(w.num_kv_heads, w.group)
        ws = torch.empty(max(16, B.akv_decode_hybrid_workspace_bytes(d8, w.batch, L["t8"].shape[1],
                                                                     L["tw"].shape[1])),
                         dtype=torch.uint8, device="cuda")
        ro = torch.full_like(o, float("nan"))
        rl = torch.full_like(lse, float("nan"))
        B.akv_decode_hybrid(d8, w.batch, *L["args"], ro, rl, ws)
        torch.cuda.synchronize()
        rows = w.batch * w.num_q_heads
        # the same kernels and plan: identical to the workspace entry point
        assert torch.equal(o, ro) and torch.equal(lse, rl), w.name
        rm, rlm = _oracle(w, L)
        check_attn(o.view(rows, 256), lse.view(rows), rm, rlm, f"static scratch {w.name}")


def test_static_scratch_refuses_oversize(B):
    """One page per int8 work-group at 128K needs about 51 MB of partials,
    more than the 16 MiB array: refused, nothing written."""
    w = configs.ctx128k()
    plan = inputs.plan_pools(w)
    d8 = B.dims(4, 6)
    m8, mw = max(plan.n8), 16
    B.akv_set_launch_shape(hybrid_int8_pages=1)
    try:
        need = B.akv_decode_hybrid_workspace_bytes(d8, 1, m8, mw)
        assert need > B.STATIC_SCRATCH_BYTES
        o = torch.full((1, 24, 256), 7.0, device="cuda")
        lse = torch.full((1, 24), 7.0, device="cuda")
        kc = torch.zeros((m8, 4, 64, 256), dtype=torch.int8, device="cuda")
        sc = torch.zeros((m8, 4, 256), device="cuda")
        kb = torch.zeros((mw, 4, 64, 256), dtype=torch.bfloat16, device="cuda")
        t8 = torch.zeros((1, m8), dtype=torch.int32, device="cuda")
        n8 = torch.full((1,), m8, dtype=torch.int32, device="cuda")
        tw = torch.zeros((1, mw), dtype=torch.int32, device="cuda")
        nw = torch.full((1,), 64 * mw, dtype=torch.int32, device="cuda")
        q = torch.zeros((1, 24, 256), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(B.AkvError) as e:
            B.akv_decode_hybrid_static(d8, 1, q, kc, kc, sc, sc, sc, t8, n8, m8, kb, kb, tw, nw, mw, SIG, o, lse)
        assert e.value.status_name == "AKV_ERR_WORKSPACE"
        torch.cuda.synchronize()
        assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
    finally:
        B.akv_set_launch_shape(reset=True)
