"""CPU oracle of the lossless 13-bit page tier.

TEST INFRASTRUCTURE ONLY: only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library.

Passage: "Model quantization" page, section "A lossless tier first": before
the 8-bit format, history was kept at 13 bits per value (an 18.7% saving over
16), with a 32-entry table per plane and a raw fallback for a plane whose
values need more than 32 entries.  The pages give no more than that; the
reading taken here (the plainest one that yields exactly 13 bits):

* a plane is one page of one KV head, keys or values: 64 tokens x 256
  channels of BF16, 16,384 values;
* each BF16 value is its high byte (sign and the upper seven exponent bits)
  and its low byte (lowest exponent bit and the seven mantissa bits);
* the table lists the plane's distinct high bytes in ascending order (unused
  entries zero); a value is stored as the 5-bit position of its high byte in
  the table plus its low byte unchanged: 5 + 8 = 13 bits;
* a plane with more than 32 distinct high bytes is kept raw (16 bits).

Every value decodes to its exact bit pattern, NaN payloads, signed zeros,
infinities and subnormals included.  Arrays here are in the pool's natural
order (keys [t][d], values [d][t]); the device format's storage order is a
layout question the tests settle separately.

Parity pins: ``tests/test_oracle_lossless.py`` checks a hand-worked plane, the
sizes the page prints, the fallback boundary at 32/33 entries, round trips on
random and special bit patterns, and the table and positions against numpy's
``unique``; none of this is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

TABLE_ENTRIES = 32
INDEX_BITS = 5
CODED_BITS = INDEX_BITS + 8  # index + the low byte kept as is
RAW_BITS = 16


def encode_plane(bits: np.ndarray) -> dict:
    """Encode one plane of BF16 bit patterns (any shape; flattened in C order).

    Returns dict(raw, table[32] uint8, index uint8 [n] or None, low uint8 [n]
    or None, bits uint16 [n] (the raw plane, kept for a raw record only))."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).ravel()
    hi = (b >> 8).astype(np.uint8)
    present = np.zeros(256, dtype=bool)
    present[hi] = True
    distinct = np.flatnonzero(present)  # ascending high bytes that occur
    table = np.zeros(TABLE_ENTRIES, dtype=np.uint8)
    if distinct.size > TABLE_ENTRIES:
        return dict(raw=True, table=table, index=None, low=None, bits=b.copy())
    table[:distinct.size] = distinct
    position = np.full(256, 255, dtype=np.uint8)
    position[distinct] = np.arange(distinct.size, dtype=np.uint8)
    return dict(raw=False, table=table, index=position[hi], low=(b & 0xFF).astype(np.uint8), bits=None)


def decode_plane(rec: dict) -> np.ndarray:
    """Bit patterns of an encoded plane (flattened)."""
    if rec["raw"]:
        return rec["bits"].copy()
    hi = rec["table"][rec["index"]].astype(np.uint16)
    return (hi << 8) | rec["low"].astype(np.uint16)


def plane_bits(n_values: int, raw: bool) -> int:
    """Stored bits of a plane of n_values (table and flag not counted)."""
    return n_values * (RAW_BITS if raw else CODED_BITS)


def encode_pool(kpool, vpool, src, dst, n_slots: int, Hkv: int):
    """Encode BF16 pool pages src[i] into record slots dst[i].

    kpool uint16 [slots][Hkv][P][D], vpool uint16 [slots][Hkv][D][P].
    Returns dict of arrays indexed [slot][h][kv] (kv 0 = keys, 1 = values):
    raw bool, table uint8 [.., 32], index uint8 [.., n], low uint8 [.., n]
    (index/low zero for raw planes), in each plane's natural order."""
    kpool = np.asarray(kpool, dtype=np.uint16)
    vpool = np.asarray(vpool, dtype=np.uint16)
    n = kpool.shape[2] * kpool.shape[3]
    raw = np.zeros((n_slots, Hkv, 2), dtype=bool)
    table = np.zeros((n_slots, Hkv, 2, TABLE_ENTRIES), dtype=np.uint8)
    index = np.zeros((n_slots, Hkv, 2, n), dtype=np.uint8)
    low = np.zeros((n_slots, Hkv, 2, n), dtype=np.uint8)
    for s, d in zip(np.asarray(src).tolist(), np.asarray(dst).tolist()):
        for h in range(Hkv):
            for kv, plane in enumerate((kpool[s, h], vpool[s, h])):
                rec = encode_plane(plane)
                raw[d, h, kv] = rec["raw"]
                table[d, h, kv] = rec["table"]
                if not rec["raw"]:
                    index[d, h, kv] = rec["index"]
                    low[d, h, kv] = rec["low"]
    return dict(raw=raw, table=table, index=index, low=low)
