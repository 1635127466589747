"""The lossless 13-bit tier through the C ABI ("Model quantization" page,
"A lossless tier first").

* The GPU encoder's records equal the oracle's, bit for bit: raw flags,
  tables, every value's table position and low byte (read back from the
  arena through the storage order include/akv.h states), raw planes stored
  verbatim, planes packed back to back in call order from the given offset.
* akv_l13_decode_pages returns every page bit-exactly.
* akv_decode_attn_l13 is bit-identical to akv_decode_attn_exact on the same
  pages and within the attention tolerance of the oracle, including raw
  planes, partial pages, empty requests and the full 128K layer.
"""
import numpy as np
import pytest
import torch

from oracle import lossless as L
from oracle import oracle as O
from quantized_paged_kv_akv_amd import configs, inputs
from tests.gpu_util import check_attn, dev, host, run_exact, say, workspace

pytestmark = pytest.mark.gpu
SIG = 1.0 / 16.0
PLANE = 26624
RAW = 32768


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from quantized_paged_kv_akv_amd import binding
    return binding


def _storage_maps():
    """For lane slot (w, l, v): the natural position it stands for and where
    its bytes sit in a coded plane (the formulas of include/akv.h)."""
    w, l, v = np.meshgrid(np.arange(4), np.arange(64), np.arange(64), indexing="ij")
    n, g = l % 16, l // 16
    m = dict(
        k_t=16 * (n // 4) + 4 * (v // 16) + n % 4, k_d=64 * w + 16 * g + 8 * ((v // 8) % 2) + v % 8,
        v_d=64 * w + 16 * ((v // 16) % 4) + n, v_t=16 * g + 8 * ((v // 8) % 2) + v % 8,
        low=((4 * w + v // 16) * 64 + l) * 16 + v % 16,
        nib=16384 + ((2 * w + v // 32) * 64 + l) * 16 + 4 * ((v // 8) % 4) + v % 4, nib_shift=4 * ((v // 4) % 2),
        hib=24576 + (w * 64 + l) * 8 + 4 * (v // 32) + v % 4, hib_bit=(v // 4) % 8)
    return {k: a.reshape(-1) for k, a in m.items()}


MAPS = _storage_maps()


def read_coded_plane(buf: np.ndarray, kv: int):
    """(index, low) of a coded plane's bytes, in the plane's natural order
    (keys [t][d], values [d][t]) flattened."""
    low = buf[MAPS["low"]]
    idx = ((buf[MAPS["nib"]] >> MAPS["nib_shift"]) & 15) | (((buf[MAPS["hib"]] >> MAPS["hib_bit"]) & 1) << 4)
    nat = MAPS["k_t"] * 256 + MAPS["k_d"] if kv == 0 else MAPS["v_d"] * 64 + MAPS["v_t"]
    out_i = np.empty(16384, np.uint8)
    out_l = np.empty(16384, np.uint8)
    out_i[nat] = idx
    out_l[nat] = low
    return out_i, out_l


def special_pools(seed, n_pages, Hkv, finite=False):
    """Seeded pools with hand-made planes mixed in (n_pages >= 4): one raw
    plane (more than 32 distinct high bytes), one with exactly 32, one of IEEE
    specials (unless finite), one all zero.  finite: every value finite and
    at most 8 in magnitude, so attention over the pages stays well-conditioned."""
    kp, vp = inputs.random_pools(seed, n_pages, Hkv)
    r = np.random.default_rng(seed + 1)
    if n_pages < 4:
        return kp, vp
    if finite:
        # magnitudes 2^-40 .. 2^2 with both signs: 42 binades, 42 distinct high bytes
        x = np.where(r.random((256, 64)) < 0.5, -1.0, 1.0) * np.exp2(r.uniform(-40, 2.999, (256, 64)))
        vp[1, 0] = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        pool = np.array([s << 7 | e for s in (0, 1) for e in range(44, 65)], np.uint16)  # |x| in [2^-39, 2^3)
    else:
        vp[1, 0] = r.integers(0, 65536, size=(256, 64)).astype(np.uint16)
        pool = np.arange(256, dtype=np.uint16)
    his = r.choice(pool, size=32, replace=False)
    hi = np.concatenate([his, r.choice(his, size=16384 - 32)])
    r.shuffle(hi)
    kp[2, Hkv - 1] = ((hi << 8) | r.integers(0, 256, size=16384).astype(np.uint16)).reshape(64, 256)
    if not finite:
        sp = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0x7F81, 0xFFFF, 0x0001, 0x807F, 0x0080], np.uint16)
        kp[3, 0] = r.choice(sp, size=(64, 256))
    vp[3, Hkv - 1] = 0
    return kp, vp


def encode(B, kp_t, vp_t, Hkv, src, dst, n_slots, offset=0, extra=0):
    d = B.dims(Hkv, 1)
    sz = B.l13_sizes(d, n_slots)
    arena = torch.full((offset + len(src) * Hkv * 2 * RAW + extra,), 0xA5, dtype=torch.uint8, device="cuda")
    desc = torch.full(sz["desc"], -7, dtype=torch.int32, device="cuda")
    table = torch.full(sz["table"], 0x5A, dtype=torch.uint8, device="cuda")
    end = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    B.akv_l13_encode_pages(d, len(src), kp_t, vp_t, dev(np.asarray(src, np.int32)), dev(np.asarray(dst, np.int32)),
                           arena, offset, desc, table, end)
    torch.cuda.synchronize()
    return dict(arena=arena, desc=desc, table=table, end=int(end[0]))


def check_records(rec, kp, vp, src, dst, Hkv, offset, tag):
    ref = L.encode_pool(kp, vp, src, dst, int(max(dst)) + 1, Hkv)
    arena, desc, table = host(rec["arena"]), host(rec["desc"]), host(rec["table"])
    pos = offset
    n_raw = 0
    for s, d in zip(src, dst):
        for h in range(Hkv):
            for kv in range(2):
                raw = bool(ref["raw"][d, h, kv])
                n_raw += raw
                assert desc[d, h, kv] == ((pos // 256) << 1 | int(raw)), (tag, s, d, h, kv, desc[d, h, kv], pos)
                assert np.array_equal(table[d, h, kv], ref["table"][d, h, kv]), (tag, "table", d, h, kv)
                if raw:
                    plane = (kp if kv == 0 else vp)[s, h]
                    got = arena[pos:pos + RAW].view(np.uint16).reshape(plane.shape)
                    assert np.array_equal(got, plane), (tag, "raw plane", d, h, kv)
                    pos += RAW
                else:
                    gi, gl = read_coded_plane(arena[pos:pos + PLANE], kv)
                    assert np.array_equal(gi, ref["index"][d, h, kv]), (tag, "index", d, h, kv)
                    assert np.array_equal(gl, ref["low"][d, h, kv]), (tag, "low", d, h, kv)
                    pos += PLANE
    assert rec["end"] == pos, (tag, rec["end"], pos)
    assert (arena[:offset] == 0xA5).all() and (arena[pos:] == 0xA5).all(), (tag, "bytes outside the planes written")
    say(f"[l13 {tag}] {len(src)} pages x {Hkv} heads: records bit-exact, {n_raw} raw planes, {pos - offset} bytes")
    return n_raw


def test_encode_matches_oracle_and_decodes_exactly(B):
    Hkv, n = 2, 7
    kp, vp = special_pools(71, n, Hkv)
    src = np.array([4, 1, 6, 3, 0, 2, 5], np.int32)
    dst = np.array([2, 0, 6, 5, 1, 4, 3], np.int32)
    say("case l13 encode 7 pages Hkv 2, offset 768")
    rec = encode(B, dev(kp), dev(vp), Hkv, src, dst, n, offset=768, extra=4096)
    n_raw = check_records(rec, kp, vp, src, dst, Hkv, 768, "special")
    assert n_raw == 1
    # back to BF16 pages: record slot dst[i] -> pool slot src[i]
    d = B.dims(Hkv, 1)
    ko = torch.zeros((n, Hkv, 64, 256), dtype=torch.bfloat16, device="cuda")
    vo = torch.zeros((n, Hkv, 256, 64), dtype=torch.bfloat16, device="cuda")
    B.akv_l13_decode_pages(d, n, rec["arena"], rec["desc"], rec["table"], dev(dst), dev(src), ko, vo)
    torch.cuda.synchronize()
    assert np.array_equal(host(ko.view(torch.int16)).view(np.uint16), kp)
    assert np.array_equal(host(vo.view(torch.int16)).view(np.uint16), vp)
    say("[l13 special] decode_pages bit-exact")


def test_encode_workload_pages(B):
    """Pages of the 32K workload's recipe (per-channel key scales, 8x outlier
    tokens): every plane coded."""
    w = configs.ctx32k()
    d = inputs.make_layer_np(w, 2)
    src = np.arange(0, 512, 37, dtype=np.int32)
    dst = np.arange(len(src), dtype=np.int32)
    say("case l13 encode ctx32k pages", len(src))
    rec = encode(B, dev(d["k_pool"]), dev(d["v_pool"]), w.num_kv_heads, src, dst, len(src))
    assert check_records(rec, d["k_pool"], d["v_pool"], src, dst, w.num_kv_heads, 0, "ctx32k") == 0


def test_encode_refuses_small_arena(B):
    Hkv, n = 1, 3
    kp, vp = inputs.random_pools(5, n, Hkv)
    d = B.dims(Hkv, 1)
    arena = torch.full((n * 2 * RAW - 256,), 7, dtype=torch.uint8, device="cuda")
    desc = torch.full((n, Hkv, 2), -3, dtype=torch.int32, device="cuda")
    table = torch.full((n, Hkv, 2, 32), 9, dtype=torch.uint8, device="cuda")
    end = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    s = dev(np.arange(n, dtype=np.int32))
    say("case l13 refused arena")
    with pytest.raises(B.AkvError) as e:
        B.akv_l13_encode_pages(d, n, dev(kp), dev(vp), s, s, arena, 0, desc, table, end)
    assert e.value.status_name == "AKV_ERR_BUDGET", e.value
    with pytest.raises(B.AkvError) as e:
        B.akv_l13_encode_pages(d, n, dev(kp), dev(vp), s, s, arena, 100, desc, table, end)  # not a multiple of 256
    assert e.value.status_name == "AKV_ERR_ARG", e.value
    torch.cuda.synchronize()
    assert bool((arena == 7).all()) and bool((desc == -3).all()) and bool((table == 9).all()) and int(end[0]) == -1


def run_l13(B, Hkv, G, q, rec, table, seq_len, sigma=SIG):
    d = B.dims(Hkv, G)
    batch = len(seq_len)
    max_pages = int(table.shape[1])
    o = torch.full((batch, Hkv * G, 256), float("nan"), device="cuda")
    lse = torch.full((batch, Hkv * G), float("nan"), device="cuda")
    ws = workspace(B, d, batch, max_pages)
    B.akv_decode_attn_l13(d, batch, dev(q), rec["arena"], rec["desc"], rec["table"], dev(np.asarray(table, np.int32)),
                          dev(np.asarray(seq_len, np.int32)), max_pages, sigma, o, lse, ws)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("Hkv,G,seq_len", [
    (1, 2, [256]),
    (2, 6, [0, 1, 63, 64, 65, 700]),
    (4, 6, [1087, 300]),
    (1, 8, [1024, 1]),
    (2, 1, [500]),
])
def test_decode_l13_parity(B, Hkv, G, seq_len):
    """Records in permuted slots (a raw plane, a 32-entry plane, IEEE
    specials and an all-zero plane among them when there are enough pages):
    bit-identical to the exact decode on the BF16 pages, and within tolerance
    of the oracle."""
    pages = [(s + 63) // 64 for s in seq_len]
    total = max(4, sum(pages))
    kp, vp = special_pools(800 + G, total, Hkv, finite=True)
    slots = np.random.default_rng(9).permutation(total).astype(np.int32)
    table = np.zeros((len(seq_len), max(1, max(pages))), np.int32)
    off = 0
    for b, n in enumerate(pages):
        table[b, :n] = slots[off: off + n]
        off += n
    say(f"case l13 decode Hkv={Hkv} G={G} seq_len={seq_len}")
    all_slots = np.arange(total, dtype=np.int32)
    rec = encode(B, dev(kp), dev(vp), Hkv, all_slots, all_slots, total)
    q = inputs.random_queries(801, len(seq_len), Hkv * G)
    o, lse = run_l13(B, Hkv, G, q, rec, table, seq_len)
    eo, el = run_exact(B, Hkv, G, q, dev(kp), dev(vp), table, seq_len)
    assert torch.equal(o, eo) and torch.equal(lse, el), "l13 decode differs from the exact decode"
    ro, rl = O.decode_exact(q, kp, vp, table, np.asarray(seq_len, np.int32), Hkv, G, SIG)
    check_attn(o, lse, ro, rl, f"l13 Hkv{Hkv} G{G}")


def test_decode_l13_ctx128k_full_size(B):
    """The full 128K layer (2048 pages per KV head, 4 KV heads, G = 6), every
    page coded: bit-identical to the exact decode over the BF16 pages, which
    the oracle then checks on every row."""
    w = configs.ctx128k()
    d = inputs.make_layer_np(w, 7)
    plan = d["plan"]
    Hkv, G = w.num_kv_heads, w.group
    tf = plan.full_table()
    n = d["k_pool"].shape[0]
    say("case l13 ctx128k full layer, pages", n)
    slots = np.arange(n, dtype=np.int32)
    kpt, vpt = dev(d["k_pool"]), dev(d["v_pool"])
    rec = encode(B, kpt, vpt, Hkv, slots, slots, n)
    n_raw = int((host(rec["desc"]) & 1).sum())
    assert rec["end"] == (n * Hkv * 2 - n_raw) * PLANE + n_raw * RAW, (rec["end"], n_raw)
    say(f"[l13 ctx128k] {n * Hkv * 2} planes, {n_raw} raw, {rec['end']} bytes")
    seq = [int(x) for x in w.lengths]
    o, lse = run_l13(B, Hkv, G, d["q"], rec, tf, seq)
    eo, el = run_exact(B, Hkv, G, d["q"], kpt, vpt, tf, seq)
    assert torch.equal(o, eo) and torch.equal(lse, el), "l13 decode differs from the exact decode"
    ro, rl = O.decode_exact(d["q"], d["k_pool"], d["v_pool"], tf, np.asarray(seq, np.int32), Hkv, G, SIG)
    rows = w.batch * w.num_q_heads
    check_attn(o.view(rows, 256), lse.view(rows), ro.reshape(rows, 256), rl.reshape(rows), "l13 ctx128k")
