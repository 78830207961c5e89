"""Oracle: plain fp64 CPU reference for paged Q8_0-K / Q4_0-V attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (``long_context_attention_amd``) and never imports
it; the two meet only through the seeded inputs of ``inputs/``.

The arithmetic lives in ``oracle.c`` (plain loops, fp64, OpenMP threads over
independent (row, head) units).  This module compiles it with gcc and wraps
it with ctypes.  What it computes: exact softmax attention of the query rows
over the complete KV history read through a page table ("Adaptive KV
Streaming for llama.cpp", section "Adaptive KV streaming": residency and
transfer scheduling change, the attended history does not).

Every function here is pinned by ``tests/test_oracle_pins.py`` against
things other than itself: exhaustive fp16 decoding against numpy, exact
rational dequantisation, numpy dense attention on the quantiser's unpaged
arrays, closed-form special cases and brute-force invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

HEAD_DIM = 128
BLOCK = 32
F16, Q4_0, Q8_0 = 1, 2, 8   # element types (K, V pairs: (Q8_0, Q4_0), (Q8_0, Q8_0), (Q4_0, Q4_0), (F16, F16))
HOST_ENTRY = 0xFFFFFFFF
RING_FLAG = 0x80000000


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        Z = ctypes.c_size_t
        D = ctypes.c_double
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = D
        lib.oracle_page_bytes.argtypes = [I, I, I, I]
        lib.oracle_page_bytes.restype = Z
        lib.oracle_pair_supported.argtypes = [I, I]
        lib.oracle_pair_supported.restype = I
        for name in ("oracle_k_code", "oracle_v_code"):
            getattr(lib, name).argtypes = [P, I, I, I, I, I, I, I]
            getattr(lib, name).restype = I
        for name in ("oracle_k_scale", "oracle_v_scale", "oracle_k_value", "oracle_v_value"):
            getattr(lib, name).argtypes = [P, I, I, I, I, I, I, I]
            getattr(lib, name).restype = D
        lib.oracle_attend_paged.argtypes = [P, Z, P, Z, P, P, I, I, I, I, I, I, P, I, D, P, I, P, P, I]
        lib.oracle_attend_paged.restype = I
        lib.oracle_attend_values.argtypes = [P, P, I, I, I, P, I, D, P, I, P, P, I]
        lib.oracle_attend_values.restype = I
        lib.oracle_attend_logical.argtypes = [P, P, P, P, I, I, I, P, I, D, P, I, P, P, I]
        lib.oracle_attend_logical.restype = I
        lib.oracle_split_partials.argtypes = [P, I, I, I, I, I, I, P, I, D, P, I, P, P, P]
        lib.oracle_split_partials.restype = I
        lib.oracle_merge.argtypes = [P, P, P, I, I, P]
        lib.oracle_merge.restype = I
        lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_f16.restype = ctypes.c_uint16
        lib.oracle_quantize_q8_0.argtypes = [P, I, P, P]
        lib.oracle_quantize_q8_0.restype = None
        lib.oracle_quantize_q4_0.argtypes = [P, I, P, P]
        lib.oracle_quantize_q4_0.restype = None
        lib.oracle_unpack_page.argtypes = [P, I, I, I, I, P, P, P, P]
        lib.oracle_unpack_page.restype = None
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _threads(n):
    return n if n else max(1, min(16, os.cpu_count() or 1))


def f16_to_f64(bits: int) -> float:
    """IEEE binary16 bit pattern -> float, decoded from the format definition."""
    return _load().oracle_f16_to_f64(int(bits) & 0xFFFF)


def page_bytes(n_kv_heads: int, page_tokens: int, k_type: int = Q8_0, v_type: int = Q4_0) -> int:
    return int(_load().oracle_page_bytes(k_type, v_type, n_kv_heads, page_tokens))


def pair_supported(k_type: int, v_type: int) -> bool:
    return bool(_load().oracle_pair_supported(k_type, v_type))


def _page_arg(page):
    page = np.ascontiguousarray(page, dtype=np.uint8)
    return page, ctypes.c_void_p(page.ctypes.data)


def k_code(page, H, T, head, j, t, k_type=Q8_0, v_type=Q4_0):
    page, p = _page_arg(page)
    return _load().oracle_k_code(p, k_type, v_type, H, T, head, j, t)


def v_code(page, H, T, head, j, t, k_type=Q8_0, v_type=Q4_0):
    page, p = _page_arg(page)
    return _load().oracle_v_code(p, k_type, v_type, H, T, head, j, t)


def k_scale(page, H, T, head, j, b, k_type=Q8_0, v_type=Q4_0):
    page, p = _page_arg(page)
    return _load().oracle_k_scale(p, k_type, v_type, H, T, head, j, b)


def v_scale(page, H, T, head, j, b, k_type=Q8_0, v_type=Q4_0):
    page, p = _page_arg(page)
    return _load().oracle_v_scale(p, k_type, v_type, H, T, head, j, b)


def decode_page(page, H, T, k_type=Q8_0, v_type=Q4_0):
    """All dequantised K-hat and V-hat of one page: two float64 [T][H][128]."""
    page, p = _page_arg(page)
    lib = _load()
    K = np.empty((T, H, HEAD_DIM))
    V = np.empty((T, H, HEAD_DIM))
    for j in range(T):
        for h in range(H):
            for t in range(HEAD_DIM):
                K[j, h, t] = lib.oracle_k_value(p, k_type, v_type, H, T, h, j, t)
                V[j, h, t] = lib.oracle_v_value(p, k_type, v_type, H, T, h, j, t)
    return K, V


def attend_paged(page_table, n_tokens, page_tokens, n_q_heads, n_kv_heads, q, scale,
                 pool=None, ring=None, history=None, rows=None, n_threads=None, k_type=Q8_0, v_type=Q4_0):
    """Exact attention read through a page table.

    page_table: uint32 [ceil(N/T)] entries (pool id, RING_FLAG|slot, HOST_ENTRY).
    pool / ring: uint8 [n][page_bytes]; history: uint8 [n_pages][page_bytes]
    (the layer's host copy in logical order).  q: float32 [W][Hq][128].
    rows: optional list of row indices in [0, W).
    Returns (out float64 [n_rows][Hq][128], lse float64 [n_rows][Hq]).
    """
    q = np.ascontiguousarray(q, dtype=np.float32)
    W = q.shape[0]
    pt = np.ascontiguousarray(page_table, dtype=np.uint32)
    pool = None if pool is None else np.ascontiguousarray(pool, dtype=np.uint8)
    ring = None if ring is None else np.ascontiguousarray(ring, dtype=np.uint8)
    history = None if history is None else np.ascontiguousarray(history, dtype=np.uint8)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    n_rows = W if rows_a is None else len(rows_a)
    out = np.empty((n_rows, n_q_heads, HEAD_DIM))
    lse = np.empty((n_rows, n_q_heads))
    rc = _load().oracle_attend_paged(
        _ptr(pool), 0 if pool is None else pool.shape[0], _ptr(ring), 0 if ring is None else ring.shape[0],
        _ptr(history), _ptr(pt), n_tokens, page_tokens, k_type, v_type, n_q_heads, n_kv_heads, _ptr(q), W,
        float(scale),
        _ptr(rows_a), n_rows, _ptr(out), _ptr(lse), _threads(n_threads))
    if rc != 0:
        raise ValueError(f"oracle_attend_paged failed ({rc})")
    return out, lse


def attend_logical(kc, kd, vc, vd, n_q_heads, q, scale, rows=None, n_threads=None):
    """Exact attention over unpaged logical arrays.

    kc int8 [N][H][128]; kd uint16 (binary16 bits) [N][H][4];
    vc uint8 [N][H][128] (0..15); vd uint16 [N][H][4]; q float32 [W][Hq][128].
    """
    kc = np.ascontiguousarray(kc, dtype=np.int8)
    kd = np.ascontiguousarray(kd, dtype=np.uint16)
    vc = np.ascontiguousarray(vc, dtype=np.uint8)
    vd = np.ascontiguousarray(vd, dtype=np.uint16)
    q = np.ascontiguousarray(q, dtype=np.float32)
    N, H = kc.shape[0], kc.shape[1]
    W = q.shape[0]
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    n_rows = W if rows_a is None else len(rows_a)
    out = np.empty((n_rows, n_q_heads, HEAD_DIM))
    lse = np.empty((n_rows, n_q_heads))
    rc = _load().oracle_attend_logical(_ptr(kc), _ptr(kd), _ptr(vc), _ptr(vd), N, n_q_heads, H, _ptr(q), W,
                                       float(scale), _ptr(rows_a), n_rows, _ptr(out), _ptr(lse),
                                       _threads(n_threads))
    if rc != 0:
        raise ValueError(f"oracle_attend_logical failed ({rc})")
    return out, lse


def split_partials(pages, page_tokens, n_tokens, n_q_heads, n_kv_heads, q, scale, bounds, k_type=Q8_0,
                   v_type=Q4_0):
    """Per-split un-normalised partials (m, l, acc) over logical pages.

    pages: uint8 [n_pages][page_bytes] in logical order.  bounds: split key
    boundaries, bounds[0] = 0, increasing, bounds[-1] >= n_tokens.
    """
    pages = np.ascontiguousarray(pages, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.float32)
    W = q.shape[0]
    b = np.ascontiguousarray(bounds, dtype=np.int32)
    S = len(b) - 1
    ptrs = (ctypes.c_void_p * pages.shape[0])(*[pages.ctypes.data + i * pages.shape[1]
                                               for i in range(pages.shape[0])])
    m = np.empty((S, W, n_q_heads))
    l = np.empty((S, W, n_q_heads))
    acc = np.empty((S, W, n_q_heads, HEAD_DIM))
    rc = _load().oracle_split_partials(ctypes.cast(ptrs, ctypes.c_void_p), page_tokens, k_type, v_type, n_tokens,
                                       n_q_heads,
                                       n_kv_heads, _ptr(q), W, float(scale), _ptr(b), S, _ptr(m), _ptr(l),
                                       _ptr(acc))
    if rc != 0:
        raise ValueError("oracle_split_partials failed")
    return m, l, acc


def merge(m, l, acc):
    """Log-sum-exp merge of split partials in split order."""
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    acc = np.ascontiguousarray(acc, dtype=np.float64)
    S = m.shape[0]
    units = int(np.prod(m.shape[1:]))
    out = np.empty(m.shape[1:] + (HEAD_DIM,))
    rc = _load().oracle_merge(_ptr(m), _ptr(l), _ptr(acc), S, units, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_merge: a unit has no visible key")
    return out


def f32_to_f16(x: float) -> int:
    """binary32 -> binary16 bits, round to nearest even (the oracle's own
    conversion from the formats' definitions)."""
    return int(_load().oracle_f32_to_f16(ctypes.c_float(x)))


def quantize_q8_0(x):
    """fp32 [..., 32 k] -> (int8 codes [..., 32 k], binary16 bits [..., k]):
    d = amax / 127 rounded to binary16, code = round-half-even(x / d) clamped
    to +-127 (binary32 arithmetic); d = 0 gives codes 0."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    n = x.size // BLOCK
    codes = np.empty(x.shape, dtype=np.int8)
    scales = np.empty(x.shape[:-1] + (x.shape[-1] // BLOCK,), dtype=np.uint16)
    _load().oracle_quantize_q8_0(_ptr(x), n, _ptr(codes), _ptr(scales))
    return codes, scales


def quantize_q4_0(x):
    """fp32 [..., 32 k] -> (codes 0..15 uint8 [..., 32 k], binary16 bits
    [..., k]): m = the element of largest magnitude (first on ties), d = m / -8
    rounded to binary16, code = round-half-even(x / d) + 8 clamped to [0, 15];
    d = 0 gives codes 8."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    n = x.size // BLOCK
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[:-1] + (x.shape[-1] // BLOCK,), dtype=np.uint16)
    _load().oracle_quantize_q4_0(_ptr(x), n, _ptr(codes), _ptr(scales))
    return codes, scales


def unpack_page(page, H, T, k_type=Q8_0, v_type=Q4_0):
    """Codes and scales of one page in logical order: kcode int32 [T][H][128]
    (Q8_0 the signed code, Q4_0 the nibble, F16 the binary16 bits), kd uint16
    [T][H][4], vcode int32 [T][H][128], vd uint16 [T][H][4] (zero for F16)."""
    page, p = _page_arg(page)
    kc = np.empty((T, H, HEAD_DIM), dtype=np.int32)
    vc = np.empty((T, H, HEAD_DIM), dtype=np.int32)
    kd = np.empty((T, H, HEAD_DIM // BLOCK), dtype=np.uint16)
    vd = np.empty((T, H, HEAD_DIM // BLOCK), dtype=np.uint16)
    _load().oracle_unpack_page(p, k_type, v_type, H, T, _ptr(kc), _ptr(kd), _ptr(vc), _ptr(vd))
    return kc, kd, vc, vd


def attend_values(K, V, n_q_heads, q, scale, rows=None, n_threads=None):
    """Exact attention over plain fp64 keys / values [N][Hkv][128]."""
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    q = np.ascontiguousarray(q, dtype=np.float32)
    N, H = K.shape[0], K.shape[1]
    W = q.shape[0]
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    n_rows = W if rows_a is None else len(rows_a)
    out = np.empty((n_rows, n_q_heads, HEAD_DIM))
    lse = np.empty((n_rows, n_q_heads))
    rc = _load().oracle_attend_values(_ptr(K), _ptr(V), N, n_q_heads, H, _ptr(q), W, float(scale), _ptr(rows_a),
                                      n_rows, _ptr(out), _ptr(lse), _threads(n_threads))
    if rc != 0:
        raise ValueError(f"oracle_attend_values failed ({rc})")
    return out, lse
