"""Python face of the float64 CPU oracle (oracle/akv_oracle.c).

TEST INFRASTRUCTURE ONLY: only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library in ``quantized_paged_kv_akv_amd/``; the only thing the
two sides have in common is the seeded input generator, which holds none of
the method's arithmetic.

What each function computes and the passage it follows:

* ``page_scales`` / ``page_codes`` -- the 8-bit page format ("Model
  quantization" page, section "An 8-bit page format shaped for its kernel").
* ``attend`` -- dense softmax attention for one query row, the plain
  definition the exact tier is held to ("ActiveKV" page, sections "The idea"
  and "What I built").
* ``merge`` -- exact log-sum-exp merge of partials with -inf as the empty
  partial ("SYCL" page, section "A merge that joins the tiers").
* ``decode_int8`` -- mode 0 dequantizes and applies the dense definition;
  mode 1 follows the int8-path formula ("SYCL" page, section "Attention that
  reads 8-bit history").
* ``decode_exact`` -- dense attention over BF16 pages with a token count.

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against closed forms, invariants, a hand-worked example and a library routine
(torch float64 attention); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "akv_oracle.c")
_LIB = os.path.join(_HERE, "libakv_oracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (IEEE float64, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-std=c99", "-D_DEFAULT_SOURCE", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-shared", "-fPIC", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        _lib.akvo_page_scales.argtypes = [I, I, P, P, P, P, P, P]
        _lib.akvo_page_codes.argtypes = [I, I, P, P, P, P, P, P, P, P, P]
        _lib.akvo_quantize_pages.argtypes = [I, I, I, I, P, P, P, P, P, P, P, P, P, I, P, P, P]
        _lib.akvo_attend.argtypes = [I, I, P, P, P, D, P, P]
        _lib.akvo_merge.argtypes = [I, I, I, P, P, P, P]
        _lib.akvo_decode_exact.argtypes = [I, I, I, I, I, P, P, P, P, P, I, D, P, P]
        _lib.akvo_decode_int8.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, I, D, I, P, P]
        _lib.akvo_num_threads.restype = I
        for name in ("akvo_page_scales", "akvo_page_codes", "akvo_quantize_pages", "akvo_attend",
                     "akvo_merge", "akvo_decode_exact", "akvo_decode_int8"):
            getattr(_lib, name).restype = I
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().akvo_num_threads())


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of BF16 bit patterns to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------- quantizer
def page_scales(K: np.ndarray, V: np.ndarray):
    """Scales of one page-head.  K, V float64 token-major [P][D].

    Returns (c64, c32, s32, vs32)."""
    K = _c(K, np.float64)
    V = _c(V, np.float64)
    P, D = K.shape
    c64 = np.empty(D, np.float64)
    c32 = np.empty(D, np.float32)
    s32 = np.empty(P, np.float32)
    vs32 = np.empty(D, np.float32)
    rc = _load().akvo_page_scales(P, D, _p(K), _p(V), _p(c64), _p(c32), _p(s32), _p(vs32))
    assert rc == 0, rc
    return c64, c32, s32, vs32


def page_codes(K, V, c32, s32, vs32):
    """Codes of one page-head given FP32 scales.  Token-major [P][D] in and out.

    Returns (kcode, vcode, ktie, vtie, n_ties)."""
    K = _c(K, np.float64)
    V = _c(V, np.float64)
    P, D = K.shape
    c32 = _c(c32, np.float32)
    s32 = _c(s32, np.float32)
    vs32 = _c(vs32, np.float32)
    kc = np.empty((P, D), np.int8)
    vc = np.empty((P, D), np.int8)
    kt = np.empty((P, D), np.uint8)
    vt = np.empty((P, D), np.uint8)
    n = _load().akvo_page_codes(P, D, _p(K), _p(V), _p(c32), _p(s32), _p(vs32),
                                _p(kc), _p(vc), _p(kt), _p(vt))
    return kc, vc, kt.astype(bool), vt.astype(bool), int(n)


def quantize_pages(kpool, vpool, src, dst, n_slots_out, Hkv, D=256, P=64, given=None):
    """Quantize BF16 pool pages src[i] into int8 pool slots dst[i].

    kpool uint16 [slots][Hkv][P][D], vpool uint16 [slots][Hkv][D][P].
    ``given`` = (k_chan, k_tok, v_chan) to run stage 2 only with those scales.
    Returns dict(k_codes, v_codes, k_chan, k_tok, v_chan, ties, k_ties, v_ties);
    the tie masks mark codes whose float64 quotient was exactly k + 0.5."""
    kpool = _c(kpool, np.uint16)
    vpool = _c(vpool, np.uint16)
    src = _c(src, np.int32)
    dst = _c(dst, np.int32)
    n = int(src.shape[0])
    kc = np.zeros((n_slots_out, Hkv, P, D), np.int8)
    vc = np.zeros((n_slots_out, Hkv, D, P), np.int8)
    if given is None:
        k_chan = np.zeros((n_slots_out, Hkv, D), np.float32)
        k_tok = np.zeros((n_slots_out, Hkv, P), np.float32)
        v_chan = np.zeros((n_slots_out, Hkv, D), np.float32)
        use = 0
    else:
        k_chan, k_tok, v_chan = (_c(a, np.float32).copy() for a in given)
        use = 1
    ties = np.zeros(1, np.int64)
    kt = np.zeros(kc.shape, np.uint8)
    vt = np.zeros(vc.shape, np.uint8)
    rc = _load().akvo_quantize_pages(n, Hkv, D, P, _p(kpool), _p(vpool), _p(src), _p(dst),
                                     _p(kc), _p(vc), _p(k_chan), _p(k_tok), _p(v_chan), use,
                                     _p(ties), _p(kt), _p(vt))
    assert rc == 0, rc
    return dict(k_codes=kc, v_codes=vc, k_chan=k_chan, k_tok=k_tok, v_chan=v_chan,
                ties=int(ties[0]), k_ties=kt.astype(bool), v_ties=vt.astype(bool))


# --------------------------------------------------------------------------- attention
def attend(q, K, V, sigma):
    """Dense softmax attention, one query row.  Returns (O[D], lse)."""
    q = _c(q, np.float64)
    K = _c(K, np.float64).reshape(-1, q.shape[0])
    V = _c(V, np.float64).reshape(-1, q.shape[0])
    n, D = K.shape
    O = np.empty(D, np.float64)
    lse = np.empty(1, np.float64)
    rc = _load().akvo_attend(n, D, _p(q), _p(K), _p(V), float(sigma), _p(O), _p(lse))
    assert rc == 0
    return O, float(lse[0])


def merge(parts_O, parts_lse):
    """Exact LSE merge.  parts_O [n][rows][D], parts_lse [n][rows]."""
    parts_O = _c(parts_O, np.float64)
    parts_lse = _c(parts_lse, np.float64)
    n, rows, D = parts_O.shape
    O = np.empty((rows, D), np.float64)
    lse = np.empty(rows, np.float64)
    rc = _load().akvo_merge(n, rows, D, _p(parts_O), _p(parts_lse), _p(O), _p(lse))
    assert rc == 0
    return O, lse


def decode_exact(q, kpool, vpool, page_table, seq_len, Hkv, G, sigma, D=256, P=64):
    """Dense attention over BF16 pages.  Returns O [B][Hq][D], lse [B][Hq]."""
    q = _c(q, np.uint16)
    kpool = _c(kpool, np.uint16)
    vpool = _c(vpool, np.uint16)
    page_table = _c(page_table, np.int32)
    seq_len = _c(seq_len, np.int32)
    B = int(seq_len.shape[0])
    max_pages = int(page_table.shape[1]) if page_table.ndim == 2 else 0
    O = np.empty((B, Hkv * G, D), np.float64)
    lse = np.empty((B, Hkv * G), np.float64)
    rc = _load().akvo_decode_exact(B, Hkv, G, D, P, _p(q), _p(kpool), _p(vpool), _p(page_table),
                                   _p(seq_len), max_pages, float(sigma), _p(O), _p(lse))
    assert rc == 0
    return O, lse


def decode_int8(q, k_codes, v_codes, k_chan, k_tok, v_chan, page_table, n_pages, Hkv, G, sigma,
                mode=0, D=256, P=64):
    """int8-tier attention.  mode 0: dequantize + dense; mode 1: int8-path formula."""
    q = _c(q, np.uint16)
    args = [_c(k_codes, np.int8), _c(v_codes, np.int8), _c(k_chan, np.float32),
            _c(k_tok, np.float32), _c(v_chan, np.float32)]
    page_table = _c(page_table, np.int32)
    n_pages = _c(n_pages, np.int32)
    B = int(n_pages.shape[0])
    max_pages = int(page_table.shape[1]) if page_table.ndim == 2 else 0
    O = np.empty((B, Hkv * G, D), np.float64)
    lse = np.empty((B, Hkv * G), np.float64)
    rc = _load().akvo_decode_int8(B, Hkv, G, D, P, _p(q), *[_p(a) for a in args], _p(page_table),
                                  _p(n_pages), max_pages, float(sigma), int(mode), _p(O), _p(lse))
    assert rc == 0
    return O, lse
