"""Seeded synthetic inputs for hybrid-tier decode attention.

This module is the only code shared by the HIP path's tests/bench and the
float64 oracle.  It draws random numbers and lays them out in the boundary's
pool layouts; it holds none of the method's arithmetic (no scales, no codes,
no attention).

Workload recipe (the pages measure on a 27B model with real prompts; none of
that exists here, so seeded draws of the same shapes stand in for it):

* keys    K = N(0,1) * sigma_K[h, d],  sigma_K ~ log-uniform[0.1, 10]
* values  V = N(0,1) * sigma_V[h, d],  sigma_V ~ log-uniform[0.5, 2]
* queries Q = N(0,1)
* outliers: a fraction of token positions per (request, layer) has its K and
  V rows (all KV heads) multiplied by 8.
* everything is rounded once to BF16 (round to nearest even, through FP32).

Two generators with the same recipe:

* ``numpy`` -- ``Generator(PCG64(SeedSequence(seed, spawn_key=(cfg, req,
  layer, tensor))))``.  Bit-reproducible on any host; the tests and the oracle
  baseline use it.
* ``torch`` -- ``torch.Generator`` on the device (Philox), seeded from the same
  key.  Same distributions, different numbers; used only where host-side
  generation of gigabytes would dominate a timing run.

Pool layouts (as stated in include/akv.h):
  BF16 K  [slot][Hkv][P][D]  token-major
  BF16 V  [slot][Hkv][D][P]  channel-major
  q       [B][Hkv*G][D]
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import List, Optional

import numpy as np

SEED = 1234
T_SIGMA_K, T_SIGMA_V, T_K, T_V, T_Q, T_OUTLIER, T_PERM, T_LEN = range(8)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic decode workload (all requests, all layers)."""
    name: str
    cfg_id: int
    batch: int
    layers: int
    num_kv_heads: int
    group: int
    lengths: tuple          # tokens of history per request
    window: int             # minimum tokens kept BF16 (recent window)
    outlier_frac: float
    permute: bool
    head_dim: int = 256
    page: int = 64

    @property
    def num_q_heads(self) -> int:
        return self.num_kv_heads * self.group

    def split(self, b: int):
        """(n8, window_tokens) for request b: the full pages older than the
        recent window are int8; the window starts on a page boundary."""
        L = int(self.lengths[b])
        n8 = max(0, (L - self.window) // self.page)
        return n8, L - n8 * self.page


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round FP32 to BF16 bits, nearest even (NaN-free inputs): add 0x7FFF
    plus the lowest kept bit, keep the high half (in place, one temporary)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    t = np.right_shift(u, np.uint32(16))
    np.bitwise_and(t, np.uint32(1), out=t)
    np.add(t, np.uint32(0x7FFF), out=t)
    np.add(t, u, out=t)
    np.right_shift(t, np.uint32(16), out=t)
    return t.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def rng(cfg: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(SEED, spawn_key=(cfg,) + tuple(key))))


def torch_seed(cfg: int, *key: int) -> int:
    h = hashlib.sha256(repr((SEED, cfg) + tuple(key)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def draw_lengths(cfg_id: int, n_pairs: int, lo: int, hi: int) -> tuple:
    """Pairs of requests share a length (so each pair has equal page counts)."""
    r = rng(cfg_id, 0, 0, T_LEN)
    L = r.integers(lo, hi + 1, size=n_pairs)
    out = []
    for x in L:
        out += [int(x), int(x)]
    return tuple(out)


# --------------------------------------------------------------------------- pool plan
@dataclasses.dataclass
class PoolPlan:
    """Where every page of every request lives.

    bf16_slot[b][i]: BF16 pool slot of the request's i-th history page (all
    pages, int8-bound and window).  int8_slot[b][i]: int8 pool slot of its
    i-th int8 page (i < n8)."""
    n8: List[int]
    win_tokens: List[int]
    n_pages: List[int]
    bf16_slot: List[np.ndarray]
    int8_slot: List[np.ndarray]
    bf16_slots_total: int
    int8_slots_total: int

    def int8_table(self) -> np.ndarray:
        B = len(self.n8)
        m = max(1, max(self.n8))
        t = np.zeros((B, m), np.int32)
        for b in range(B):
            t[b, : self.n8[b]] = self.int8_slot[b]
        return t

    def window_table(self) -> np.ndarray:
        B = len(self.n8)
        w = [self.n_pages[b] - self.n8[b] for b in range(B)]
        t = np.zeros((B, max(1, max(w))), np.int32)
        for b in range(B):
            t[b, : w[b]] = self.bf16_slot[b][self.n8[b]:]
        return t

    def full_table(self) -> np.ndarray:
        B = len(self.n8)
        t = np.zeros((B, max(1, max(self.n_pages))), np.int32)
        for b in range(B):
            t[b, : self.n_pages[b]] = self.bf16_slot[b]
        return t

    def quant_src_dst(self):
        src, dst = [], []
        for b in range(len(self.n8)):
            src.append(self.bf16_slot[b][: self.n8[b]])
            dst.append(self.int8_slot[b])
        if not src:
            return np.zeros(0, np.int32), np.zeros(0, np.int32)
        return np.concatenate(src).astype(np.int32), np.concatenate(dst).astype(np.int32)


def plan_pools(w: Workload) -> PoolPlan:
    n8, win, npg = [], [], []
    for b in range(w.batch):
        a, wt = w.split(b)
        n8.append(a)
        win.append(wt)
        npg.append(a + (wt + w.page - 1) // w.page)
    tot_bf16 = int(sum(npg))
    tot_i8 = int(sum(n8))
    bf16_order = np.arange(tot_bf16, dtype=np.int64)
    i8_order = np.arange(tot_i8, dtype=np.int64)
    if w.permute:
        r = rng(w.cfg_id, 0, 0, T_PERM)
        bf16_order = r.permutation(tot_bf16)
        i8_order = r.permutation(tot_i8)
    bf16_slot, int8_slot = [], []
    ob = oi = 0
    for b in range(w.batch):
        bf16_slot.append(bf16_order[ob: ob + npg[b]].astype(np.int32))
        int8_slot.append(i8_order[oi: oi + n8[b]].astype(np.int32))
        ob += npg[b]
        oi += n8[b]
    return PoolPlan(n8, win, npg, bf16_slot, int8_slot, tot_bf16, tot_i8)


# --------------------------------------------------------------------------- numpy draws
def _request_tokens_np(w: Workload, b: int, layer: int):
    """K, V float32 [pages*P][Hkv][D] for request b (history padded to whole
    pages with zeros past its length)."""
    Hkv, D, P = w.num_kv_heads, w.head_dim, w.page
    L = int(w.lengths[b])
    npg = (L + P - 1) // P
    sk = np.exp(rng(w.cfg_id, b, layer, T_SIGMA_K).uniform(np.log(0.1), np.log(10.0), size=(Hkv, D)))
    sv = np.exp(rng(w.cfg_id, b, layer, T_SIGMA_V).uniform(np.log(0.5), np.log(2.0), size=(Hkv, D)))
    K = np.zeros((npg * P, Hkv, D), np.float32)
    V = np.zeros((npg * P, Hkv, D), np.float32)
    K[:L] = rng(w.cfg_id, b, layer, T_K).standard_normal((L, Hkv, D), dtype=np.float32)
    V[:L] = rng(w.cfg_id, b, layer, T_V).standard_normal((L, Hkv, D), dtype=np.float32)
    K[:L] *= sk.astype(np.float32)[None]
    V[:L] *= sv.astype(np.float32)[None]
    n_out = int(round(w.outlier_frac * L))
    if n_out > 0:
        pos = rng(w.cfg_id, b, layer, T_OUTLIER).choice(L, size=n_out, replace=False)
        K[pos] *= np.float32(8.0)
        V[pos] *= np.float32(8.0)
    return K, V


def make_layer_np(w: Workload, layer: int, plan: Optional[PoolPlan] = None):
    """All inputs of one layer, numpy generator.

    Returns dict(q [B][Hq][D] u16, k_pool [S][Hkv][P][D] u16,
    v_pool [S][Hkv][D][P] u16, plan)."""
    plan = plan or plan_pools(w)
    Hkv, D, P = w.num_kv_heads, w.head_dim, w.page
    kpool = np.zeros((plan.bf16_slots_total, Hkv, P, D), np.uint16)
    vpool = np.zeros((plan.bf16_slots_total, Hkv, D, P), np.uint16)
    for b in range(w.batch):
        K, V = _request_tokens_np(w, b, layer)
        npg = plan.n_pages[b]
        Kb = f32_to_bf16_bits(K).reshape(npg, P, Hkv, D)
        Vb = f32_to_bf16_bits(V).reshape(npg, P, Hkv, D)
        slots = plan.bf16_slot[b]
        kpool[slots] = Kb.transpose(0, 2, 1, 3)
        vpool[slots] = Vb.transpose(0, 2, 3, 1)
    q = f32_to_bf16_bits(rng(w.cfg_id, 0, layer, T_Q).standard_normal((w.batch, w.num_q_heads, D),
                                                                       dtype=np.float32))
    return dict(q=q, k_pool=kpool, v_pool=vpool, plan=plan)


# --------------------------------------------------------------------------- torch draws
def make_layer_torch(w: Workload, layer: int, device, plan: Optional[PoolPlan] = None):
    """Same recipe drawn on the device with torch's generator (different
    numbers from the numpy path).  Returns device tensors: q, k_pool, v_pool
    as torch.bfloat16 in the pool layouts, plus the plan."""
    import torch

    plan = plan or plan_pools(w)
    Hkv, D, P = w.num_kv_heads, w.head_dim, w.page
    S = plan.bf16_slots_total
    kpool = torch.zeros((S, Hkv, P, D), dtype=torch.bfloat16, device=device)
    vpool = torch.zeros((S, Hkv, D, P), dtype=torch.bfloat16, device=device)

    def gen(*key):
        g = torch.Generator(device=device)
        g.manual_seed(torch_seed(w.cfg_id, *key))
        return g

    for b in range(w.batch):
        L = int(w.lengths[b])
        npg = plan.n_pages[b]
        sk = torch.exp(torch.empty((Hkv, D), device=device).uniform_(np.log(0.1), np.log(10.0), generator=gen(b, layer, T_SIGMA_K)))
        sv = torch.exp(torch.empty((Hkv, D), device=device).uniform_(np.log(0.5), np.log(2.0), generator=gen(b, layer, T_SIGMA_V)))
        K = torch.zeros((npg * P, Hkv, D), device=device)
        V = torch.zeros((npg * P, Hkv, D), device=device)
        K[:L] = torch.randn((L, Hkv, D), device=device, generator=gen(b, layer, T_K)) * sk
        V[:L] = torch.randn((L, Hkv, D), device=device, generator=gen(b, layer, T_V)) * sv
        n_out = int(round(w.outlier_frac * L))
        if n_out > 0:
            pos = torch.randperm(L, device=device, generator=gen(b, layer, T_OUTLIER))[:n_out]
            K[pos] *= 8.0
            V[pos] *= 8.0
        slots = torch.as_tensor(plan.bf16_slot[b], device=device, dtype=torch.long)
        kpool[slots] = K.to(torch.bfloat16).view(npg, P, Hkv, D).permute(0, 2, 1, 3)
        vpool[slots] = V.to(torch.bfloat16).view(npg, P, Hkv, D).permute(0, 2, 3, 1)
        del K, V
    q = torch.randn((w.batch, w.num_q_heads, D), device=device, generator=gen(0, layer, T_Q)).to(torch.bfloat16)
    return dict(q=q, k_pool=kpool, v_pool=vpool, plan=plan)


# --------------------------------------------------------------------------- free-form pools
def random_pools(seed: int, n_slots: int, Hkv: int, outlier_frac: float = 0.02,
                 k_std=(0.1, 10.0), v_std=(0.5, 2.0)):
    """BF16 K [S][Hkv][P][D] and V [S][Hkv][D][P] pools of whole random pages
    with the workload's distributions (per-channel log-uniform std, a fraction
    of token rows x8).  For tests that need arbitrary page counts."""
    import math
    r = np.random.default_rng(seed)
    P, D = 64, 256
    sk = np.exp(r.uniform(math.log(k_std[0]), math.log(k_std[1]), (1, Hkv, 1, D))).astype(np.float32)
    sv = np.exp(r.uniform(math.log(v_std[0]), math.log(v_std[1]), (1, Hkv, D, 1))).astype(np.float32)
    K = r.standard_normal((n_slots, Hkv, P, D), dtype=np.float32) * sk
    V = r.standard_normal((n_slots, Hkv, D, P), dtype=np.float32) * sv
    if outlier_frac > 0:
        s_idx, t_idx = np.nonzero(r.random((n_slots, P)) < outlier_frac)
        K[s_idx, :, t_idx, :] *= np.float32(8.0)
        V[s_idx, :, :, t_idx] *= np.float32(8.0)
    return f32_to_bf16_bits(K), f32_to_bf16_bits(V)


def random_queries(seed: int, batch: int, Hq: int, D: int = 256, scale: float = 1.0) -> np.ndarray:
    r = np.random.default_rng(seed)
    return f32_to_bf16_bits(r.standard_normal((batch, Hq, D), dtype=np.float32) * np.float32(scale))
