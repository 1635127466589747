"""The C-ABI library loads and exports every function include/akv.h declares;
host-side argument checks answer without touching a GPU."""
import ctypes
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "quantized_paged_kv_akv_amd", "libakv.so")


@pytest.fixture(scope="module")
def B():
    if not os.path.exists(LIB):
        from quantized_paged_kv_akv_amd import build
        build.build()
    from quantized_paged_kv_akv_amd import binding
    return binding


def test_exports_every_declared_symbol(B):
    names = B.header_functions()
    assert len(names) >= 13
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(LIB)
    for n in names:
        getattr(lib, n)


def test_status_strings_and_version(B):
    for code, name in B.STATUS.items():
        assert B._lib.akv_status_string(code).decode() == name
    assert B.version().startswith("akv ")


def test_prepare_covers_the_decode_calls_only(B):
    """binding.prepare marshals the decode entry points and akv_merge_lse;
    every one of them is a symbol the header declares, and other names are
    refused before anything is called."""
    assert set(B._PREPARABLE) <= set(B.header_functions())
    with pytest.raises(ValueError):
        B.prepare("akv_quantize_pages")


def test_host_side_validation(B):
    lib = B._lib
    d = B.dims(4, 6)
    # unsupported shapes and bad arguments are refused before any GPU work
    assert lib.akv_quantize_pages(None, 1, *([None] * 9), None) == -1
    bad = B.dims(4, 6, head_dim=128)
    assert lib.akv_quantize_pages(ctypes.byref(bad), 1, *([None] * 9), None) == -2
    assert "head_dim" in lib.akv_last_error().decode()
    g9 = B.dims(1, 9)
    assert lib.akv_quantize_pages(ctypes.byref(g9), 1, *([None] * 9), None) == -2
    assert lib.akv_quantize_pages(ctypes.byref(d), -1, *([None] * 9), None) == -1
    assert lib.akv_quantize_pages(ctypes.byref(d), 0, *([None] * 9), None) == 0
    assert lib.akv_merge_lse(-1, 256, None, None, None, None, None) == -1
    assert lib.akv_merge_lse(4, 256, None, None, None, None, None) == -1
    assert lib.akv_fill_empty(0, 256, None, None, None) == 0
    # misaligned pointer
    assert lib.akv_merge_lse(1, 256, 8, 16, 16, 16, None) == -3
    # workspace too small
    ws = B.akv_decode_workspace_bytes(d, 1, 2032)
    assert ws > 0 and B.akv_decode_workspace_bytes(d, 0, 10) == 0
    p = ctypes.c_void_p(16)
    st = lib.akv_decode_attn_int8(ctypes.byref(d), 1, p, p, p, p, p, p, p, p, 2032, 0.0625, p, p, p, 16, None)
    assert st == -4
    st = lib.akv_decode_attn_exact(ctypes.byref(d), 1, p, p, p, p, p, 2032, 0.0625, p, p, p, 16, None)
    assert st == -4
    # int32 tables need only 4-byte alignment (slices of requests); tensors need 16
    t4, t2 = ctypes.c_void_p(20), ctypes.c_void_p(18)
    st = lib.akv_decode_attn_int8(ctypes.byref(d), 1, p, p, p, p, p, p, t4, t4, 2032, 0.0625, p, p, p, 16, None)
    assert st == -4
    st = lib.akv_decode_attn_int8(ctypes.byref(d), 1, p, p, p, p, p, p, t2, t4, 2032, 0.0625, p, p, p, 16, None)
    assert st == -3
    st = lib.akv_decode_attn_int8(ctypes.byref(d), 1, t4, p, p, p, p, p, t4, t4, 2032, 0.0625, p, p, p, 16, None)
    assert st == -3
    # the kernel's page shares are 32-bit: splits x max_pages must stay below 2^32
    try:
        B.akv_set_launch_shape(pages_per_wave=1)  # 4 pages per work-group: 35,000 splits of 140,000 pages
        st = lib.akv_decode_attn_int8(ctypes.byref(d), 1, p, p, p, p, p, p, t4, t4, 140000, 0.0625, p, p, p, 16,
                                      None)
        assert st == -2 and "2^32" in lib.akv_last_error().decode()
        st = lib.akv_decode_attn_int8(ctypes.byref(d), 1, p, p, p, p, p, p, t4, t4, 60000, 0.0625, p, p, p, 16,
                                      None)
        assert st == -4  # 15,000 x 60,000 < 2^32: on to the workspace check
    finally:
        B.akv_set_launch_shape(reset=True)
    # ring refuses fewer than 2 slots and NULL slots
    h = ctypes.c_void_p()
    arr = (ctypes.c_void_p * 1)(ctypes.c_void_p(16))
    assert lib.akv_ring_create(arr, 1024, 1, ctypes.byref(h)) == -1
    arr2 = (ctypes.c_void_p * 2)(ctypes.c_void_p(16), ctypes.c_void_p(0))
    assert lib.akv_ring_create(arr2, 1024, 2, ctypes.byref(h)) == -1


def test_workspace_is_deterministic_and_covers_splits(B):
    d = B.dims(4, 6)
    for batch, mp in [(1, 2032), (1, 496), (32, 256), (2, 17), (1, 1)]:
        a = B.akv_decode_workspace_bytes(d, batch, mp)
        assert a == B.akv_decode_workspace_bytes(d, batch, mp)
        # at least one partial row per (request, query head)
        assert a >= batch * 24 * (256 + 1) * 4


def test_lossless_host_side_validation(B):
    """The 13-bit entry points refuse bad arguments before any GPU work: an
    arena too small for the worst case, an unaligned offset or arena, a
    negative count, a small decode workspace."""
    lib = B._lib
    d = B.dims(2, 3)
    p, a256, end = ctypes.c_void_p(256), ctypes.c_void_p(4096), ctypes.c_void_p(64)
    worst = 5 * 2 * 2 * 32768
    # 5 pages x 2 heads x 2 planes: the arena must hold them all raw
    assert lib.akv_l13_encode_pages(ctypes.byref(d), 5, p, p, p, p, a256, 0, worst - 256, p, p, end, None) == -5
    assert "raw" in lib.akv_last_error().decode()
    assert lib.akv_l13_encode_pages(ctypes.byref(d), 5, p, p, p, p, a256, 256, worst, p, p, end, None) == -5
    assert lib.akv_l13_encode_pages(ctypes.byref(d), 5, p, p, p, p, a256, 100, 10 * worst, p, p, end, None) == -1
    assert lib.akv_l13_encode_pages(ctypes.byref(d), 5, p, p, p, p, ctypes.c_void_p(4112), 0, worst, p, p, end,
                                    None) == -3
    assert lib.akv_l13_encode_pages(ctypes.byref(d), -1, p, p, p, p, a256, 0, worst, p, p, end, None) == -1
    assert lib.akv_l13_encode_pages(ctypes.byref(d), 5, p, p, p, p, a256, 0, worst, p, p, None, None) == -1
    bad = B.dims(2, 3, page_size=32)
    assert lib.akv_l13_encode_pages(ctypes.byref(bad), 5, p, p, p, p, a256, 0, worst, p, p, end, None) == -2
    assert lib.akv_l13_decode_pages(ctypes.byref(d), 0, None, None, None, None, None, None, None, None) == 0
    assert lib.akv_l13_decode_pages(ctypes.byref(d), 3, a256, p, p, p, p, p, None, None) == -1
    # decode: arena alignment and workspace size
    t4 = ctypes.c_void_p(20)
    st = lib.akv_decode_attn_l13(ctypes.byref(d), 1, p, ctypes.c_void_p(4112), t4, p, t4, t4, 64, 0.0625, p, p, p,
                                 1 << 20, None)
    assert st == -3
    st = lib.akv_decode_attn_l13(ctypes.byref(d), 1, p, a256, t4, p, t4, t4, 64, 0.0625, p, p, p, 16, None)
    assert st == -4
    sz = B.l13_sizes(d, 7)
    assert sz["desc"] == (7, 2, 2) and sz["table"] == (7, 2, 2, 32) and sz["arena_bytes"] == 7 * 2 * 2 * 32768


def test_launch_shape_validation(B):
    """The launch-shape override refuses negative fields and shapes beyond
    what a wave can stage, leaves the setting unchanged then, and the
    workspace queries follow the setting that is in force."""
    lib = B._lib
    d = B.dims(4, 6)
    planned = B.akv_decode_workspace_bytes(d, 1, 2032)
    planned_h = B.akv_decode_hybrid_workspace_bytes(d, 1, 2032, 16)
    for bad in (dict(pages_per_split=-1), dict(pages_per_wave=65), dict(hybrid_int8_pages=257),
                dict(hybrid_window_pages=-3), dict(pv_fp16=2), dict(pv_fp16=-1), dict(issue_priority=3),
                dict(issue_priority=-1)):
        with pytest.raises(B.AkvError) as e:
            B.akv_set_launch_shape(**bad)
        assert e.value.status_name == "AKV_ERR_ARG"
        assert B.akv_decode_workspace_bytes(d, 1, 2032) == planned
    try:
        B.akv_set_launch_shape(pages_per_split=1, pages_per_wave=1)
        # one page per exact split: 2032 partial columns per row
        assert B.akv_decode_workspace_bytes(d, 1, 2032) >= 24 * 2032 * 257 * 4
        B.akv_set_launch_shape(hybrid_int8_pages=8, hybrid_window_pages=1)
        need = B.akv_decode_hybrid_workspace_bytes(d, 1, 2032, 16)
        assert need >= 24 * (254 + 16) * 257 * 4
        # the PV operand choice and the issue-priority probe do not change the plan
        B.akv_set_launch_shape(pv_fp16=1)
        assert B.akv_decode_workspace_bytes(d, 1, 2032) == planned
        for prio in (1, 2):
            B.akv_set_launch_shape(issue_priority=prio)
            assert B.akv_decode_workspace_bytes(d, 1, 2032) == planned
            assert B.akv_decode_hybrid_workspace_bytes(d, 1, 2032, 16) == planned_h
    finally:
        B.akv_set_launch_shape(reset=True)
    assert B.akv_decode_workspace_bytes(d, 1, 2032) == planned
    assert lib.akv_set_launch_shape(None) == 0


def test_hybrid_empty_tier_pointers_may_be_null(B):
    """A tier with no page-table columns is never read, so its pointers may be
    NULL; the other tier's pointers are still checked."""
    lib = B._lib
    d = B.dims(4, 6)
    p, t4, z = ctypes.c_void_p(16), ctypes.c_void_p(20), ctypes.c_void_p(0)
    # window-only call (max_pages_int8 = 0) with NULL int8 pointers: passes the
    # pointer checks and stops at the workspace check (16 bytes is too small)
    st = lib.akv_decode_hybrid(ctypes.byref(d), 1, p, z, z, z, z, z, z, z, 0, p, p, t4, t4, 16, 0.0625, p, p, p,
                               16, None)
    assert st == -4, lib.akv_last_error()
    # int8-only call with NULL window pointers
    st = lib.akv_decode_hybrid(ctypes.byref(d), 1, p, p, p, p, p, p, t4, t4, 2032, z, z, z, z, 0, 0.0625, p, p, p,
                               16, None)
    assert st == -4, lib.akv_last_error()
    # a NULL pointer of a non-empty tier is refused
    st = lib.akv_decode_hybrid(ctypes.byref(d), 1, p, p, p, p, p, p, t4, t4, 2032, z, p, t4, t4, 16, 0.0625, p, p,
                               p, 16, None)
    assert st == -1
