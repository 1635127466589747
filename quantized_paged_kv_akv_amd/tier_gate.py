"""Economic gate of the host-staged mode: pick the history tier whose decode
step is fastest once the bytes it moves over the bus are priced with a model
of the bus fitted to measurements on this card.

("Judge a representation by the bytes it stops moving", "My approach" and
"What I built": a representation is worth its loss bound only if the bytes
it no longer moves make the step faster, and candidates are judged with a
transfer model derived from measured bus behaviour, at each target context
length.)

The model has two parts, both plain host arithmetic:

* copy time of one host-to-device copy of n bytes, t(n) = latency + n /
  bandwidth, fitted to a measured curve of copy rate against size (weighted
  least squares on relative error, so 64 KiB and 512 MiB copies count
  alike);
* the staged step itself: layer l's copies run on a copy stream into a ring
  of slots while the compute stream decodes layer l - 1; a copy into a slot
  waits until the kernel that last read the slot has finished, and a kernel
  waits for its own copies.  Those cross-stream waits cost a round-trip
  latency, and a copy issued after a wait pays a fixed overhead of its own;
  both are fitted to copies measured through the ring with no kernel in
  between, at two ring sizes (small copies through a two-slot ring are
  bounded by the round trip, not by the bus).  Simulating that two-stream
  schedule over a few steps gives the steady-state time per generated
  token.

Nothing here touches a GPU; bench.py feeds it measurements.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Sequence


@dataclasses.dataclass(frozen=True)
class CopyModel:
    latency_s: float
    bandwidth_Bps: float

    def copy_s(self, nbytes: float) -> float:
        return self.latency_s + nbytes / self.bandwidth_Bps if nbytes > 0 else 0.0


def fit_copy_model(sizes_bytes: Sequence[float], rates_Bps: Sequence[float]) -> CopyModel:
    """Fit t(n) = a + n / b to measured (size, rate) points.

    Each point's time is t_i = n_i / r_i; minimising sum(((a + n_i x - t_i) /
    t_i)^2) over (a, x = 1 / b) is a 2x2 linear system."""
    if len(sizes_bytes) != len(rates_Bps) or len(sizes_bytes) < 2:
        raise ValueError("need at least two (size, rate) points")
    s00 = s01 = s11 = r0 = r1 = 0.0
    for n, r in zip(sizes_bytes, rates_Bps):
        if n <= 0 or r <= 0:
            raise ValueError("sizes and rates must be positive")
        t = n / r
        w = 1.0 / (t * t)
        s00 += w
        s01 += w * n
        s11 += w * n * n
        r0 += w * t
        r1 += w * n * t
    det = s00 * s11 - s01 * s01
    if det <= 0:
        raise ValueError("degenerate curve (all sizes equal)")
    a = (r0 * s11 - r1 * s01) / det
    x = (s00 * r1 - s01 * r0) / det
    if x <= 0:
        raise ValueError("fitted bandwidth is not positive")
    return CopyModel(max(a, 0.0), 1.0 / x)


def staged_token_s(copy_s: Sequence[float], kernel_s: Sequence[float], n_slots: int = 2, steps: int = 12,
                   dep_s: float = 0.0) -> float:
    """Steady-state time per decode step of the staged schedule.

    copy_s[l]: time of layer l's copies (all of them, back to back on the
    copy stream); kernel_s[l]: time of layer l's decode on the compute
    stream.  Layer l uses slot l % n_slots (counted over the whole run, as
    the ring does); its copy starts when the copy stream is free and the
    kernel that last used the slot has ended; its kernel starts when its
    copy and the previous kernel have ended.  dep_s is the latency of one
    round trip of those cross-stream dependencies (copy done -> compute
    stream -> slot released -> copy stream), charged half to each hop.
    Returns the time between the ends of the last two simulated steps."""
    L = len(copy_s)
    if L == 0 or len(kernel_s) != L or n_slots < 1:
        raise ValueError("copy_s and kernel_s must have one entry per layer, n_slots >= 1")
    hop = 0.5 * dep_s
    copy_end = 0.0
    kernel_end_hist = []  # kernel end time of every layer issued so far, in order
    step_ends = []
    for _ in range(steps):
        for l in range(L):
            i = len(kernel_end_hist)
            slot_free = kernel_end_hist[i - n_slots] + hop if i >= n_slots else 0.0
            c_start = max(copy_end, slot_free)
            copy_end = c_start + copy_s[l]
            k_start = max(copy_end + hop, kernel_end_hist[-1] if kernel_end_hist else 0.0)
            kernel_end_hist.append(k_start + kernel_s[l])
        step_ends.append(kernel_end_hist[-1])
    if steps >= 3:
        return (step_ends[-1] - step_ends[1]) / (steps - 2)
    return step_ends[-1] - step_ends[-2] if steps == 2 else step_ends[-1]


@dataclasses.dataclass(frozen=True)
class StagingModel:
    """The bus as the staged step sees it: the copy model of plain
    back-to-back copies, plus what a copy through the ring costs on top --
    stage_overhead_s for the first copy of a layer (it starts after a
    cross-stream wait, so it cannot overlap the previous copy's tail) and
    round_trip_s for the dependency round trip (copy done -> compute stream
    -> slot released -> copy stream)."""
    copy: CopyModel
    stage_overhead_s: float
    round_trip_s: float

    def layer_copy_s(self, copies: Sequence[float]) -> float:
        """Time of one layer's copies, issued back to back after the wait."""
        live = [n for n in copies if n > 0]
        if not live:
            return 0.0
        return (self.stage_overhead_s + sum(n / self.copy.bandwidth_Bps for n in live)
                + (len(live) - 1) * self.copy.latency_s)


def ring_copy_period_s(c: float, round_trip_s: float, n_slots: int) -> float:
    """Per-copy period of identical copies of time c through an n-slot ring
    with no kernel in between: a copy into a slot waits one round trip after
    the copy n_slots back ended, so n_slots periods are at least c plus the
    round trip, and a period is at least c."""
    return max(c, (c + round_trip_s) / n_slots)


def fit_staging_model(copy: CopyModel, staged: Dict[int, Sequence[Sequence[float]]]) -> StagingModel:
    """Fit the per-layer overhead and the round trip to copy rates measured
    through the ring with no kernel: staged[n_slots] = (sizes, rates).  The
    squared relative error of ring_copy_period_s over every point is
    minimised by a grid scan (4 us x 10 us) refined around its best cell
    (0.25 us x 0.5 us)."""
    pts = [(ns, n, n / r) for ns, (sizes, rates) in staged.items() for n, r in zip(sizes, rates)]
    if len(pts) < 2:
        raise ValueError("need at least two staged points")

    def loss(a, d):
        return sum((ring_copy_period_s(a + n / copy.bandwidth_Bps, d, ns) / t - 1.0) ** 2 for ns, n, t in pts)

    a0, d0 = min(((i * 4e-6, j * 10e-6) for i in range(76) for j in range(301)), key=lambda x: loss(*x))
    a1, d1 = min(((max(0.0, a0 - 4e-6 + i * 0.25e-6), max(0.0, d0 - 10e-6 + j * 0.5e-6))
                  for i in range(33) for j in range(41)), key=lambda x: loss(*x))
    return StagingModel(copy, a1, d1)


def hybrid_layer_bytes(context: int, window: int, num_kv_heads: int, page: int = 64,
                       int8_page_head: int = 35_072, bf16_page_head: int = 65_536) -> Dict[str, int]:
    """Bytes one layer of the hybrid tier stages at `context` tokens: the
    int8 pages older than the window (codes + FP32 scales) and the BF16
    window pages (the window starts on a page boundary)."""
    n8 = max(0, (context - window) // page)
    win_pages = -(-(context - n8 * page) // page)
    return dict(int8=n8 * num_kv_heads * int8_page_head, window=win_pages * num_kv_heads * bf16_page_head,
                n8=n8, window_pages=win_pages)


def exact_layer_bytes(context: int, num_kv_heads: int, page: int = 64, bf16_page_head: int = 65_536) -> int:
    """Bytes one layer of the all-BF16 exact tier stages at `context` tokens."""
    return -(-context // page) * num_kv_heads * bf16_page_head


def predict(model: StagingModel, copies_per_layer: Dict[str, Sequence[float]], kernel_s: Dict[str, float],
            layers: int, n_slots: int = 2) -> Dict[str, float]:
    """Predicted per-token staged time of each tier: copies_per_layer[tier]
    lists the byte counts of one layer's copies, kernel_s[tier] its decode
    time with the history resident in HBM."""
    out = {}
    for tier, copies in copies_per_layer.items():
        c = model.layer_copy_s(copies)
        out[tier] = staged_token_s([c] * layers, [kernel_s[tier]] * layers, n_slots, dep_s=model.round_trip_s)
    return out


def choose(predicted: Dict[str, float]) -> str:
    """The tier with the smallest predicted step time (ties: first listed)."""
    best, best_t = None, math.inf
    for tier, t in predicted.items():
        if t < best_t:
            best, best_t = tier, t
    return best
