"""The host-staged tier gate's transfer model (CPU only): the copy-time fit
recovers a known latency and bandwidth exactly, the two-stream staging
schedule reduces to its closed forms (copy-bound, kernel-bound, no overlap
with one slot), and the per-layer byte counts follow the page formats."""
import math

import pytest

from quantized_paged_kv_akv_amd import tier_gate as TG


def test_fit_recovers_latency_and_bandwidth():
    a, b = 9.5e-6, 56.8e9
    sizes = [64 << 10, 256 << 10, 1 << 20, 4 << 20, 16 << 20, 64 << 20, 512 << 20]
    rates = [n / (a + n / b) for n in sizes]
    m = TG.fit_copy_model(sizes, rates)
    assert math.isclose(m.latency_s, a, rel_tol=1e-9)
    assert math.isclose(m.bandwidth_Bps, b, rel_tol=1e-9)
    assert math.isclose(m.copy_s(1 << 30), a + (1 << 30) / b, rel_tol=1e-12)
    assert m.copy_s(0) == 0.0


def test_fit_rejects_degenerate_curves():
    with pytest.raises(ValueError):
        TG.fit_copy_model([1 << 20], [50e9])
    with pytest.raises(ValueError):
        TG.fit_copy_model([1 << 20, 1 << 20], [50e9, 40e9])
    with pytest.raises(ValueError):
        TG.fit_copy_model([1 << 20, -1], [50e9, 40e9])


@pytest.mark.parametrize("layers", [1, 2, 16])
def test_schedule_closed_forms(layers):
    c, k = 5.0e-3, 0.05e-3
    # copy-bound: copies run back to back, every kernel hides under the next copy
    assert math.isclose(TG.staged_token_s([c] * layers, [k] * layers, 2), layers * c, rel_tol=1e-12)
    # kernel-bound: kernels run back to back once the ring is primed
    assert math.isclose(TG.staged_token_s([k] * layers, [c] * layers, 2), layers * c, rel_tol=1e-12)
    # one slot: every copy waits for the previous kernel, nothing overlaps
    assert math.isclose(TG.staged_token_s([c] * layers, [k] * layers, 1), layers * (c + k), rel_tol=1e-12)


def test_schedule_uneven_layers():
    # two layers, copy 3 then 1, kernels 2 then 2, two slots: layer 0 copy [0,3],
    # kernel [3,5]; layer 1 copy [3,4], kernel [5,7]; next step layer 0 copy
    # waits for slot 0 (kernel 0 ended at 5) -> [5,8], kernel [8,10]; layer 1
    # copy waits for slot 1 (kernel ended 7) and the copy stream (8) -> [8,9],
    # kernel [10,12]: period 12 - 7 = 5, and every later step repeats it.
    assert math.isclose(TG.staged_token_s([3.0, 1.0], [2.0, 2.0], 2, steps=2), 5.0)
    assert math.isclose(TG.staged_token_s([3.0, 1.0], [2.0, 2.0], 2), 5.0)


def test_layer_bytes_follow_the_page_formats():
    h = TG.hybrid_layer_bytes(131072, 1024, 4)
    assert h["n8"] == 2032 and h["window_pages"] == 16
    assert h["int8"] + h["window"] == 289_259_520
    assert TG.exact_layer_bytes(131072, 4) == 536_870_912
    # context shorter than the window: all pages exact
    s = TG.hybrid_layer_bytes(700, 1024, 4)
    assert s["n8"] == 0 and s["window_pages"] == 11 and s["int8"] == 0


def test_predict_and_choose():
    m = TG.StagingModel(TG.CopyModel(10e-6, 50e9), 0.0, 0.0)
    h = TG.hybrid_layer_bytes(131072, 1024, 4)
    x = TG.exact_layer_bytes(131072, 4)
    pred = TG.predict(m, {"hybrid": [h["int8"] + h["window"]], "exact": [x / 2, x / 2]},
                      {"hybrid": 55e-6, "exact": 90e-6}, layers=16)
    assert TG.choose(pred) == "hybrid"
    # two copies per layer: the second pays the plain copy latency
    assert math.isclose(pred["exact"], 16 * (10e-6 + x / 50e9), rel_tol=1e-12)
    assert TG.choose({"a": 2.0, "b": 1.0, "c": 1.0}) == "b"


def test_dependency_latency_closed_form():
    # with zero kernel time the per-copy period is max(c, (c + D) / slots):
    # a copy into a slot waits one round trip D after the copy `slots` back
    c, D = 100e-6, 300e-6
    for slots in (2, 4, 8):
        per = TG.staged_token_s([c] * 16, [0.0] * 16, slots, dep_s=D) / 16
        assert math.isclose(per, TG.ring_copy_period_s(c, D, slots), rel_tol=1e-9)
        assert math.isclose(per, max(c, (c + D) / slots), rel_tol=1e-9)
    # 16 layers through 3 slots: the ring's phase drifts from step to step,
    # the average over the simulated steps is within a copy of the long-run rate
    per3 = TG.staged_token_s([c] * 16, [0.0] * 16, 3, dep_s=D, steps=30) / 16
    assert abs(per3 - (c + D) / 3) < 0.01 * (c + D) / 3


def test_staging_model_fit_recovers_parameters():
    copy = TG.CopyModel(10e-6, 57e9)
    a, D = 48e-6, 350e-6
    sizes = [1 << 20, 4 << 20, 8 << 20, 16 << 20, 32 << 20, 64 << 20, 256 << 20]
    staged = {ns: (sizes, [n / TG.ring_copy_period_s(a + n / copy.bandwidth_Bps, D, ns) for n in sizes])
              for ns in (2, 4)}
    m = TG.fit_staging_model(copy, staged)
    assert abs(m.stage_overhead_s - a) < 0.3e-6 and abs(m.round_trip_s - D) < 0.6e-6
    assert math.isclose(m.layer_copy_s([64 << 20]), a + (64 << 20) / 57e9, rel_tol=1e-3)
    assert m.layer_copy_s([]) == 0.0


def test_model_replays_a_recorded_sweep():
    """Refit the model to copy curves recorded on an MI355X and predict the
    staged step of both tiers at every recorded context length and ring size
    from the recorded HBM-resident decode times: every prediction within 10%
    of the recorded step time, and the gate's choice equal to the recorded
    fastest tier."""
    import json
    import os

    rec = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "staged_sweep_mi355x.json")))
    plain = rec["pcie_h2d_curve_MiB_GBps"]
    copy = TG.fit_copy_model([m * (1 << 20) for m, _ in plain], [g * 1e9 for _, g in plain])
    staged = {int(k[5:]): ([m * (1 << 20) for m, _ in c], [g * 1e9 for _, g in c])
              for k, c in rec["staged_copy_curve_MiB_GBps"].items()}
    model = TG.fit_staging_model(copy, staged)
    H = rec["num_kv_heads"]
    for row in rec["contexts"]:
        L = row["context"]
        h = TG.hybrid_layer_bytes(L, rec["window"], H)
        x = TG.exact_layer_bytes(L, H)
        copies = {"hybrid": [h["int8"] + h["window"]], "exact": [x / 2, x / 2]}
        kern = {k: v * 1e-6 for k, v in row["resident_us_per_layer"].items()}
        for key, meas in row["measured_ms"].items():
            pred = TG.predict(model, copies, kern, layers=rec["layers"], n_slots=int(key[5:]))
            for tier in ("hybrid", "exact"):
                err = pred[tier] * 1e3 / meas[tier] - 1
                assert abs(err) <= 0.10, (L, key, tier, err)
            assert TG.choose(pred) == min(meas, key=meas.get), (L, key)
