"""CPU pins of the oracle's KV-writer reference (binary32 -> binary16
conversion, Q8_0 and Q4_0 quantisers), each against something other than the
oracle itself: numpy's binary16 conversion (a library routine), exactly
representable blocks with a closed-form answer, ties, bounds and symmetries.
Planted mistakes in a copy of the oracle source must fail them.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "oracle.c")


class Lib:
    """ctypes view of an oracle build (the real one or a mutated copy)."""

    def __init__(self, path):
        lib = ctypes.CDLL(path)
        P, I = ctypes.c_void_p, ctypes.c_int
        lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_f16.restype = ctypes.c_uint16
        lib.oracle_quantize_q8_0.argtypes = [P, I, P, P]
        lib.oracle_quantize_q4_0.argtypes = [P, I, P, P]
        self.lib = lib

    def f16(self, x):
        return int(self.lib.oracle_f32_to_f16(ctypes.c_float(x)))

    def q8(self, x):
        x = np.ascontiguousarray(x, dtype=np.float32)
        c = np.empty(x.shape, np.int8)
        d = np.empty(x.shape[:-1] + (x.shape[-1] // 32,), np.uint16)
        self.lib.oracle_quantize_q8_0(x.ctypes.data, x.size // 32, c.ctypes.data, d.ctypes.data)
        return c, d

    def q4(self, x):
        x = np.ascontiguousarray(x, dtype=np.float32)
        c = np.empty(x.shape, np.uint8)
        d = np.empty(x.shape[:-1] + (x.shape[-1] // 32,), np.uint16)
        self.lib.oracle_quantize_q4_0(x.ctypes.data, x.size // 32, c.ctypes.data, d.ctypes.data)
        return c, d


@pytest.fixture(scope="module")
def lib(oracle_mod):
    return Lib(oracle_mod.build(force=False))


def f16_bits(x):
    with np.errstate(over="ignore"):
        return int(np.float32(x).astype(np.float16).view(np.uint16))


def f16_value(bits):
    return float(np.uint16(bits).view(np.float16))


# ---------------------------------------------------------------- pins
def pin_f16_boundaries(L):
    """Every finite binary16 value, its binary32 neighbours, the midpoints to
    the next value (exact in binary32: ties) and one binary32 ulp either side
    of each midpoint, both signs; compared bit for bit with numpy."""
    vals = np.arange(0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    nxt = np.arange(1, 0x7C01, dtype=np.uint16).view(np.float16).astype(np.float32)
    nxt[-1] = np.float32(65536.0)  # beyond the largest finite: the overflow threshold midpoint
    mid = ((vals.astype(np.float64) + nxt.astype(np.float64)) / 2).astype(np.float32)
    cand = np.concatenate([vals, np.nextafter(vals, np.float32(np.inf)), np.nextafter(vals, np.float32(0)),
                           mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(0))])
    cand = np.concatenate([cand, -cand, np.float32([np.inf, -np.inf, 65519.996, 65520.0, 2.0**-25, 2.0**-24])])
    bad = 0
    for x in cand[::7]:  # a regular subsample keeps the suite fast; every class of case stays in
        if L.f16(float(x)) != f16_bits(x):
            bad += 1
    return bad == 0


def pin_f16_random(L):
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)
    xs = bits.view(np.float32)
    for x in xs:
        got, want = L.f16(float(x)), f16_bits(x)
        if np.isnan(x):
            if (got & 0x7C00) != 0x7C00 or (got & 0x3FF) == 0:
                return False
        elif got != want:
            return False
    return True


def pin_q8_exact_multiples(L):
    """x = k * d with |k| <= 127, some |k| = 127 and d a binary16 value: the
    scale is d and the codes are k exactly."""
    rng = np.random.default_rng(6)
    for d in (1.0, 0.5, 0.0625, 3.0, 0.013671875, 2.0 ** -10, 48.0):
        k = rng.integers(-127, 128, (8, 32))
        k[:, 3] = np.where(rng.integers(0, 2, 8) == 1, 127, -127)
        x = (k * d).astype(np.float32)
        c, s = L.q8(x)
        if not (np.array_equal(c, k.astype(np.int8)) and np.all(s == f16_bits(d))):
            return False
    return True


def pin_q8_ties_even(L):
    """amax = 127 (d = 1); values k + 1/2 round to the even neighbour."""
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 127.0
    halves = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 100.5, -126.5], np.float32)
    x[0, 1:9] = halves
    c, s = L.q8(x)
    return s[0, 0] == f16_bits(1.0) and list(c[0, 1:9]) == [0, 2, 2, 0, -2, -2, 100, -126]


def pin_q8_bound_and_symmetry(L):
    """|x - d c| <= d / 2 unless clamped (then |x / d| > 127); codes of -x
    are minus the codes of x with the same scale; a zero block gives d = 0
    and codes 0."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 128)).astype(np.float32) * rng.uniform(0.01, 10, (64, 1)).astype(np.float32)
    c, s = L.q8(x)
    d = np.repeat(s.view(np.float16).astype(np.float64), 32, axis=-1)
    err = np.abs(x.astype(np.float64) - d * c)
    clamped = np.abs(c) == 127
    if not np.all(err[~clamped] <= d[~clamped] / 2):
        return False
    if not np.all(np.abs(x[clamped] / d[clamped]) >= 126.5):
        return False
    c2, s2 = L.q8(-x)
    if not (np.array_equal(c2, -c) and np.array_equal(s2, s)):
        return False
    z, zs = L.q8(np.zeros((2, 32), np.float32))
    return np.all(z == 0) and np.all(zs == 0)


def pin_q4_closed_forms(L):
    """d = m / -8 for the first element of largest magnitude: that element
    gets code 0, an equal-magnitude element of the other sign later in the
    block gets 16 clamped to 15; x = (n - 8) d exactly gives code n; a zero
    block gives d = 0 and codes 8."""
    x = np.zeros((2, 32), np.float32)
    x[0, 3] = -2.0   # first of the two largest magnitudes: m = -2, d = 0.25
    x[0, 7] = 2.0
    x[0, 10] = 1.25
    x[1, 8:24] = (np.arange(16) - 8) * 0.25  # unique largest magnitude -2: codes 0..15
    c, s = L.q4(x)
    if not (s[0, 0] == f16_bits(0.25) and c[0, 3] == 0 and c[0, 7] == 15 and c[0, 10] == 13):
        return False
    if not (s[1, 0] == f16_bits(0.25) and list(c[1, 8:24]) == list(range(16))):
        return False
    # sign of the first maximum decides the sign of d
    cy, sy = L.q4(-x)
    if not (sy[0, 0] == f16_bits(-0.25) and cy[0, 3] == 0 and cy[0, 7] == 15):
        return False
    z, zs = L.q4(np.zeros((1, 32), np.float32))
    return np.all(z == 8) and np.all(zs == 0x8000)  # m = +0, so d = +0 / -8 = -0


def pin_q4_bound(L):
    rng = np.random.default_rng(8)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    c, s = L.q4(x)
    d = np.repeat(s.view(np.float16).astype(np.float64), 32, axis=-1)
    err = np.abs(x.astype(np.float64) - d * (c.astype(np.float64) - 8))
    top = c == 15
    return np.all(err[~top] <= np.abs(d[~top]) / 2 * (1 + 1e-12)) and np.all(err[top] <= np.abs(d[top]) * (1 + 1e-12))


PINS = [pin_f16_boundaries, pin_f16_random, pin_q8_exact_multiples, pin_q8_ties_even, pin_q8_bound_and_symmetry,
        pin_q4_closed_forms, pin_q4_bound]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_writer_pin(lib, pin):
    assert pin(lib)


WRITER_MUTATIONS = [
    ("f16 ties away from zero", "if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h++;",
     "if (rest >= 0x1000u) h++;"),
    ("f16 subnormal tie rule", "if (rem > half || (rem == half && (q & 1u))) q++;", "if (rem >= half) q++;"),
    ("Q8_0 scale over 128", "oracle_f32_to_f16(amax / 127.0f)", "oracle_f32_to_f16(amax / 128.0f)"),
    ("Q8_0 truncating codes", "c = rintf(xb[i] / d);", "c = truncf(xb[i] / d);"),
    ("Q4_0 last maximum on ties", "if (fabsf(xb[i]) > amax) {", "if (fabsf(xb[i]) >= amax) {"),
    ("Q4_0 offset 7", "c = rintf(xb[i] / d) + 8.0f;", "c = rintf(xb[i] / d) + 7.0f;"),
    ("Q4_0 scale sign", "oracle_f32_to_f16(xb[imax] / -8.0f)", "oracle_f32_to_f16(xb[imax] / 8.0f)"),
]


@pytest.mark.parametrize("name,old,new", WRITER_MUTATIONS, ids=[m[0] for m in WRITER_MUTATIONS])
def test_planted_writer_mistake_fails_a_pin(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-o", str(so), str(mutated),
                           "-lm"])
    L = Lib(str(so))
    assert not all(p(L) for p in PINS), f"no pin caught: {name}"
