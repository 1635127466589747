"""Helpers for the GPU parity tests: upload seeded inputs, run the library's
entry points through the binding, and compare with the oracle at the
acceptance tolerances."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

# acceptance bar: attention O max-abs 2e-3 and rel-L2 1e-3, LSE 1e-4 (absolute),
# scales 1e-6 relative, codes bit-exact given identical scales (ties excluded)
TOL_O_ABS = 2e-3
TOL_O_REL = 1e-3
TOL_LSE = 1e-4
TOL_SCALE_REL = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _kcode_order() -> np.ndarray:
    """Byte offset, inside a page-head's 16 KB of key codes, of K[t][d] for
    t*256 + d: the tile order include/akv.h states for k_codes."""
    t = np.arange(64)[:, None]
    d = np.arange(256)[None, :]
    tile = 4 * (d // 64) + (t // 4) % 4
    lane = 16 * ((d // 16) % 4) + 4 * (t // 16) + t % 4
    return ((tile * 64 + lane) * 16 + d % 16).reshape(-1)


KCODE_ORDER = _kcode_order()


def k_codes_token_major(a: np.ndarray) -> np.ndarray:
    """The library's tile-ordered key codes [..., 64, 256] (16 KB per
    page-head) as token-major K[t][d], the oracle's layout."""
    flat = np.ascontiguousarray(a).reshape(a.shape[:-2] + (64 * 256,))
    return flat[..., KCODE_ORDER].reshape(a.shape)


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def workspace(B, d, batch, max_pages):
    n = B.akv_decode_workspace_bytes(d, batch, max_pages)
    return torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")


def gpu_quantize(B, kpool, vpool, src, dst, n_out, Hkv):
    d = B.dims(Hkv, 1)
    kp, vp = dev(kpool), dev(vpool)
    kc = torch.zeros((n_out, Hkv, 64, 256), dtype=torch.int8, device="cuda")
    vc = torch.zeros((n_out, Hkv, 256, 64), dtype=torch.int8, device="cuda")
    kch = torch.zeros((n_out, Hkv, 256), dtype=torch.float32, device="cuda")
    ktk = torch.zeros((n_out, Hkv, 64), dtype=torch.float32, device="cuda")
    vch = torch.zeros((n_out, Hkv, 256), dtype=torch.float32, device="cuda")
    B.akv_quantize_pages(d, len(src), kp, vp, dev(np.asarray(src, np.int32)), dev(np.asarray(dst, np.int32)),
                         kc, vc, kch, ktk, vch)
    torch.cuda.synchronize()
    return dict(k_codes=kc, v_codes=vc, k_chan=kch, k_tok=ktk, v_chan=vch)


def check_quantize(O, kpool, vpool, src, dst, n_out, Hkv, g, tag=""):
    """Scales within 1e-6 relative of the oracle's; codes bit-exact against the
    oracle's stage 2 run on the GPU's own scales, exact ties excluded."""
    ref = O.quantize_pages(kpool, vpool, src, dst, n_out, Hkv)
    gs = {k: host(g[k]) for k in ("k_chan", "k_tok", "v_chan")}
    dst = np.asarray(dst)
    for k in gs:
        a, r = gs[k][dst].astype(np.float64), ref[k][dst].astype(np.float64)
        rel = np.abs(a - r) / np.maximum(np.abs(r), 1e-300)
        rel[(a == 0) & (r == 0)] = 0.0
        assert rel.max() <= TOL_SCALE_REL, (tag, k, rel.max())
    st2 = O.quantize_pages(kpool, vpool, src, dst, n_out, Hkv, given=(gs["k_chan"], gs["k_tok"], gs["v_chan"]))
    n_ties = 0
    for k, t in (("k_codes", "k_ties"), ("v_codes", "v_ties")):
        a = host(g[k])[dst]
        if k == "k_codes":
            a = k_codes_token_major(a)
        r = st2[k][dst]
        tie = st2[t][dst]
        bad = (a != r) & ~tie
        assert not bad.any(), (tag, k, int(bad.sum()), np.argwhere(bad)[:5])
        n_ties += int(tie.sum())
    say(f"[quantize {tag}] pages={len(src)} scales ok, codes bit-exact, exact ties listed={n_ties}")
    return n_ties


def check_attn(o_gpu, lse_gpu, o_ref, lse_ref, tag=""):
    o = host(o_gpu).astype(np.float64)
    lse = host(lse_gpu).astype(np.float64)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), (tag, "empty rows differ")
    assert np.all(o[empty] == 0.0), (tag, "empty rows must have O = 0")
    ne = ~empty
    if not ne.any():
        say(f"[{tag}] all rows empty")
        return
    err = float(np.abs(o[ne] - o_ref[ne]).max())
    rel = float(np.linalg.norm(o[ne] - o_ref[ne]) / max(np.linalg.norm(o_ref[ne]), 1e-300))
    lerr = float(np.abs(lse[ne] - lse_ref[ne]).max())
    say(f"[{tag}] O max-abs {err:.3e}  rel-L2 {rel:.3e}  LSE max-abs {lerr:.3e}")
    assert err <= TOL_O_ABS and rel <= TOL_O_REL and lerr <= TOL_LSE, (tag, err, rel, lerr)


def run_int8(B, Hkv, G, q, g, table, n_pages, sigma=1 / 16):
    d = B.dims(Hkv, G)
    batch = int(len(n_pages))
    max_pages = int(table.shape[1])
    o = torch.full((batch, Hkv * G, 256), float("nan"), device="cuda")
    lse = torch.full((batch, Hkv * G), float("nan"), device="cuda")
    ws = workspace(B, d, batch, max_pages)
    B.akv_decode_attn_int8(d, batch, dev(q), g["k_codes"], g["v_codes"], g["k_chan"], g["k_tok"], g["v_chan"],
                           dev(np.asarray(table, np.int32)), dev(np.asarray(n_pages, np.int32)), max_pages, sigma,
                           o, lse, ws)
    torch.cuda.synchronize()
    return o, lse


def run_exact(B, Hkv, G, q, kpool_t, vpool_t, table, seq_len, sigma=1 / 16):
    d = B.dims(Hkv, G)
    batch = int(len(seq_len))
    max_pages = int(table.shape[1])
    o = torch.full((batch, Hkv * G, 256), float("nan"), device="cuda")
    lse = torch.full((batch, Hkv * G), float("nan"), device="cuda")
    ws = workspace(B, d, batch, max_pages)
    B.akv_decode_attn_exact(d, batch, dev(q), kpool_t, vpool_t, dev(np.asarray(table, np.int32)),
                            dev(np.asarray(seq_len, np.int32)), max_pages, sigma, o, lse, ws)
    torch.cuda.synchronize()
    return o, lse


def oracle_int8(O, Hkv, G, q, g, table, n_pages, sigma=1 / 16):
    return O.decode_int8(q, k_codes_token_major(host(g["k_codes"])), host(g["v_codes"]), host(g["k_chan"]), host(g["k_tok"]),
                         host(g["v_chan"]), np.asarray(table, np.int32), np.asarray(n_pages, np.int32), Hkv, G,
                         sigma, mode=0)


def oracle_hybrid(O, Hkv, G, q, g, t8, n8, kpool, vpool, tw, win, sigma=1 / 16):
    """Oracle of one hybrid layer on the GPU's int8 codes: the int8 tier
    (dequantized pages, dense softmax), the exact window, and their LSE
    merge.  Returns (O [rows][D], LSE [rows]) with rows = batch * Hkv * G."""
    rows = int(len(n8)) * Hkv * G
    ro8, rl8 = oracle_int8(O, Hkv, G, q, g, t8, n8, sigma)
    row, rlw = O.decode_exact(q, kpool, vpool, np.asarray(tw, np.int32), np.asarray(win, np.int32), Hkv, G, sigma)
    return O.merge(np.stack([ro8.reshape(rows, 256), row.reshape(rows, 256)]),
                   np.stack([rl8.reshape(rows), rlw.reshape(rows)]))
