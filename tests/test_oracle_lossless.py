"""Pins for the oracle of the lossless 13-bit tier (CPU only).

Passage: "Model quantization" page, section "A lossless tier first".  Each
test checks the oracle against something other than itself: the figures the
page prints, a plane worked by hand, the exactness a lossless format must
have, the 32/33-entry boundary of the raw fallback, and numpy's ``unique``.
"""
import json
import math
import os

import numpy as np

from oracle import lossless as L

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "lossless_tier.json")))


def hexes(xs, dtype):
    return np.array([int(x, 16) for x in xs], dtype=dtype)


def test_printed_figures():
    """13 bits per value and a 32-entry table; the saving over BF16 is 3/16 =
    18.75%, which the page prints truncated as 18.7."""
    p = GOLD["printed"]
    assert L.CODED_BITS == p["bits_per_value"]
    assert L.TABLE_ENTRIES == p["table_entries"] == 2 ** L.INDEX_BITS
    n = 64 * 256
    saving = 1.0 - L.plane_bits(n, False) / L.plane_bits(n, True)
    assert saving == 3 / 16
    assert math.floor(saving * 1000) / 10 == p["saving_percent"]
    assert L.plane_bits(n, False) // 8 == 26_624 and L.plane_bits(n, True) // 8 == 32_768


def test_worked_plane():
    w = GOLD["worked_plane"]
    bits = hexes(w["bits_hex"], np.uint16)
    rec = L.encode_plane(bits)
    assert not rec["raw"]
    k = len(w["table_hex"])
    assert rec["table"][:k].tolist() == hexes(w["table_hex"], np.uint8).tolist()
    assert not rec["table"][k:].any()
    assert rec["index"].tolist() == w["index"]
    assert rec["low"].tolist() == hexes(w["low_hex"], np.uint8).tolist()
    assert L.decode_plane(rec).tolist() == bits.tolist()


def test_fallback_boundary():
    """A plane with 32 distinct high bytes is coded; one with 33 is raw."""
    r = np.random.default_rng(3)
    for k, raw in ((1, False), (31, False), (32, False), (33, True), (256, True)):
        his = r.choice(256, size=k, replace=False).astype(np.uint16)
        hi = np.concatenate([his, r.choice(his, size=16384 - k)])
        r.shuffle(hi)
        bits = (hi << 8) | r.integers(0, 256, size=16384).astype(np.uint16)
        rec = L.encode_plane(bits)
        assert rec["raw"] == raw, k
        assert L.decode_plane(rec).tolist() == bits.tolist()
        if not raw:
            assert int(rec["index"].max()) == k - 1


def test_round_trip_random_and_special_patterns():
    r = np.random.default_rng(5)
    planes = []
    # BF16 of scaled normals (the workload's recipe), through an independent FP32 -> BF16 rounding
    for sigma in (0.1, 1.0, 10.0):
        x = (r.standard_normal(16384) * sigma).astype(np.float32)
        planes.append((x.view(np.uint32) >> 16).astype(np.uint16))  # truncation is still a valid BF16 pattern
    # IEEE specials: +-0, +-inf, NaNs with payloads, subnormals, the extreme normals
    sp = [0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0x7F81, 0xFFFF, 0x0001, 0x807F, 0x0080, 0x7F7F, 0xFF7F]
    planes.append(np.array(sp * 16, dtype=np.uint16))
    # uniformly random patterns: almost surely more than 32 high bytes -> raw
    planes.append(r.integers(0, 65536, size=16384).astype(np.uint16))
    kinds = []
    for p in planes:
        rec = L.encode_plane(p)
        kinds.append(rec["raw"])
        assert L.decode_plane(rec).tolist() == p.tolist()
    assert kinds == [False, False, False, False, True]


def test_table_and_positions_match_numpy_unique():
    r = np.random.default_rng(9)
    x = (r.standard_normal(16384) * np.exp(r.uniform(-2, 2, 16384))).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    rec = L.encode_plane(bits)
    u, inv = np.unique(bits >> 8, return_inverse=True)
    assert not rec["raw"] and len(u) <= 32
    assert rec["table"][:len(u)].tolist() == u.tolist()
    assert rec["index"].tolist() == inv.ravel().tolist()
    assert rec["low"].tolist() == (bits % 256).tolist()


def test_pool_records_follow_dst_slots():
    r = np.random.default_rng(11)
    Hkv, slots = 2, 5
    kpool = (r.standard_normal((slots, Hkv, 64, 256)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    vpool = (r.standard_normal((slots, Hkv, 256, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    vpool[3, 1] = r.integers(0, 65536, size=(256, 64)).astype(np.uint16)  # one raw plane
    src, dst = np.array([3, 0, 4]), np.array([1, 2, 0])
    rec = L.encode_pool(kpool, vpool, src, dst, 3, Hkv)
    assert rec["raw"].tolist() == [[[False, False], [False, False]], [[False, False], [False, True]],
                                   [[False, False], [False, False]]]
    for s, d in zip(src, dst):
        for h in range(Hkv):
            for kv, plane in enumerate((kpool[s, h], vpool[s, h])):
                if rec["raw"][d, h, kv]:
                    continue
                got = (rec["table"][d, h, kv][rec["index"][d, h, kv]].astype(np.uint16) << 8) | rec["low"][d, h, kv]
                assert got.tolist() == plane.ravel().tolist()
