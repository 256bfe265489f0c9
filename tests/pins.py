"""Pins of the CPU oracle to facts fixed by the pages and by mathematics.

Each ``pin_*`` takes an oracle object (``oracle.Oracle``) and raises
AssertionError when the oracle disagrees with a fact that does not come from
the oracle itself:

* hand-derived values of small worked matrices (``tests/golden/*.json``,
  each with its citation and derivation) and of the pages' own worked
  example of 4-bit dequantization;
* closed forms: a one-hot activation reads out one weight column; all-zero
  codes leave only the bias term; all-one / all-zero sign bits give plus /
  minus the scaled activation sums;
* exact integer arithmetic: with power-of-two scales and integer activations
  every result is exactly representable, and is computed here independently
  in int64;
* invariants: linearity in x, permutation of activation rows, duplicate rows;
* a second opinion from numpy's own half-precision decoding and bit
  unpacking on random tiny matrices, including the extreme codes;
* brute-force argmax on tiny vectors with ties;
* embedding rows: float32 -> binary16 rounding against numpy's own
  conversion over every binary16 value, its neighbours and the midpoints
  between them; whole rows against an exact-rational reference (the affine
  value as a fraction, rounded to float32 here in integer arithmetic, then
  numpy's binary16 round trip) and against hand-derived IEEE cases (ties to
  even, signed zeros, the smallest subnormal, overflow).

The same pins run against planted-mistake builds of the oracle
(``test_oracle_mutants.py``) to show that each plausible mistake fails one.
"""
from __future__ import annotations

import glob
import json
import os

import numpy as np

I8, U4, B1, I8G = 1, 2, 3, 4
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# fixture loading
# ---------------------------------------------------------------------------

def load_fixture(name):
    with open(os.path.join(GOLDEN, name)) as f:
        d = json.load(f)
    M, K = d["M"], d["K"]
    codes = np.frombuffer(bytes.fromhex(d["codes_hex"]), dtype=np.uint8).copy()
    if d["fmt"] in (I8, I8G):
        codes = codes.view(np.int8).reshape(M, K)
        scales = np.asarray(d["scales_f32"], np.float32)
        if d["fmt"] == I8G:
            scales = scales.reshape(M, K // 64)
    else:
        codes = codes.reshape(M, -1)
        scales = np.asarray(d["scales_bits"], np.uint16).reshape(M, -1)
    biases = None if d.get("biases_bits") is None else \
        np.asarray(d["biases_bits"], np.uint16).reshape(M, -1)
    return d, codes, scales, biases


def hand_fixtures():
    return sorted(os.path.basename(p) for p in glob.glob(os.path.join(GOLDEN, "hw*.json")))


# ---------------------------------------------------------------------------
# an independent numpy decode (numpy's float16 and unpackbits, not the
# oracle's bit-by-bit decoders)
# ---------------------------------------------------------------------------

def numpy_weights(fmt, codes, scales, biases, M, K):
    if fmt == I8:
        return codes.astype(np.float64) * scales.astype(np.float64)[:, None]
    if fmt == I8G:
        return codes.astype(np.float64) * np.repeat(scales.astype(np.float64), 64, axis=1)
    if fmt == U4:
        q = np.empty((M, K), np.float64)
        q[:, 0::2] = codes & 0x0F
        q[:, 1::2] = codes >> 4
        s = (scales.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        b = (biases.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return q * np.repeat(s, 64, axis=1) + np.repeat(b, 64, axis=1)
    if fmt == B1:
        bits = np.unpackbits(codes, axis=1, bitorder="little").astype(np.float64)
        s = scales.view(np.float16).astype(np.float64)
        return (2.0 * bits - 1.0) * np.repeat(s, 128, axis=1)
    raise ValueError(fmt)


def random_tiny(fmt, M, K, rng, extremes=True):
    """Random codes over the whole code range (extremes forced in), random
    scales and biases of both signs, as raw bit patterns."""
    if fmt == I8:
        codes = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
        if extremes:
            codes.flat[0], codes.flat[-1] = -128, 127
        scales = rng.uniform(-2, 2, size=M).astype(np.float32)
        return codes, scales, None
    if fmt == I8G:
        codes = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
        if extremes:
            codes.flat[0], codes.flat[-1] = -128, 127
        scales = rng.uniform(-2, 2, size=(M, K // 64)).astype(np.float32)
        return codes, scales, None
    if fmt == U4:
        codes = rng.integers(0, 256, size=(M, K // 2)).astype(np.uint8)
        if extremes:
            codes.flat[0], codes.flat[-1] = 0x00, 0xFF
        f = rng.uniform(-1, 1, size=(2, M, K // 64)).astype(np.float32)
        bits = (f.view(np.uint32) >> 16).astype(np.uint16)   # truncation: any bf16
        return codes, bits[0], bits[1]
    if fmt == B1:
        codes = rng.integers(0, 256, size=(M, K // 8)).astype(np.uint8)
        if extremes:
            codes.flat[0], codes.flat[-1] = 0x00, 0xFF
        scales = rng.uniform(-1, 1, size=(M, K // 128)).astype(np.float16).view(np.uint16)
        return codes, scales, None
    raise ValueError(fmt)


def _close(a, b, rel=1e-12, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = np.maximum(np.abs(b), 1e-300)
    assert np.all(np.abs(a - b) <= rel * scale + 1e-300), \
        f"{what}: max diff {np.max(np.abs(a - b))}"


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_hand_fixtures(orc):
    """Hand-worked matrices: exact y, Σ|w·x| and argmax."""
    for name in hand_fixtures():
        d, codes, scales, biases = load_fixture(name)
        x = np.asarray(d["x"], np.float32)
        y, a = orc.qgemv(d["fmt"], codes, scales, biases, x, d["M"], d["K"])
        assert np.array_equal(y, np.asarray(d["y"])), f"{name}: y {y} != {d['y']}"
        assert np.array_equal(a, np.asarray(d["absdot"])), f"{name}: absdot {a}"
        idx, _ = orc.argmax(y)
        assert list(idx[: len(d["idx"])]) == d["idx"][: len(idx)], f"{name}: idx {idx}"


def pin_decode_values(orc):
    """bf16 and fp16 bit patterns decode to their IEEE values."""
    with open(os.path.join(GOLDEN, "decode_values.json")) as f:
        d = json.load(f)
    for bits, v in d["bf16"]:
        got = orc.bf16_value(bits)
        assert got == v and np.signbit(got) == np.signbit(v), f"bf16 {bits:#x}: {got} != {v}"
    for bits, v in d["fp16"]:
        got = orc.fp16_value(bits)
        assert got == v and np.signbit(got) == np.signbit(v), f"fp16 {bits:#x}: {got} != {v}"


def pin_worked_example(orc):
    """The pages' worked 4-bit example: code 9 -> ~0.28, 0 -> min, 15 -> max."""
    d, codes, scales, biases = load_fixture("p3_worked_example.json")
    w = orc.decode(d["fmt"], codes, scales, biases, d["M"], d["K"])
    for k, want, tol in d["expect"]:
        assert abs(w[0, k] - want) <= tol, f"w[{k}] = {w[0, k]}, expected {want}±{tol}"


def pin_one_hot(orc):
    """x = e_j reads out column j: y[m] = w[m][j] for every (m, j), with
    the weights built here from known codes by this test's own packing."""
    rng = np.random.default_rng(11)
    M = 5
    # I8: w = s*q
    K = 32
    q = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    s = (2.0 ** rng.integers(-6, 3, size=M)).astype(np.float32)
    x = np.eye(K, dtype=np.float32)
    y, _ = orc.qgemv(I8, q, s, None, x, M, K)
    assert np.array_equal(y, (q.astype(np.float64) * s[:, None]).T), "i8 one-hot"
    # I8 group-64: w = s[m][k/64]*q
    K = 192
    q = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    sg = (2.0 ** rng.integers(-6, 3, size=(M, K // 64))).astype(np.float32)
    x = np.eye(K, dtype=np.float32)
    y, _ = orc.qgemv(I8G, q, sg, None, x, M, K)
    want = np.zeros((M, K))
    for m in range(M):
        for k in range(K):
            want[m, k] = float(q[m, k]) * float(sg[m, k // 64])
    assert np.array_equal(y, want.T), "i8 group-64 one-hot"
    # U4: w = s*q + b with q packed low nibble = even k
    K = 128
    qu = rng.integers(0, 16, size=(M, K))
    packed = (qu[:, 0::2] | (qu[:, 1::2] << 4)).astype(np.uint8)
    sv = 2.0 ** rng.integers(-6, 2, size=(M, K // 64))
    bv = rng.integers(-8, 8, size=(M, K // 64)) / 16.0
    sb = ((sv.astype(np.float32).view(np.uint32)) >> 16).astype(np.uint16)
    bb = ((bv.astype(np.float32).view(np.uint32)) >> 16).astype(np.uint16)
    x = np.eye(K, dtype=np.float32)
    y, _ = orc.qgemv(U4, packed, sb, bb, x, M, K)
    want = qu * np.repeat(sv, 64, axis=1) + np.repeat(bv, 64, axis=1)
    assert np.array_equal(y, want.T), "u4 one-hot"
    # B1: w = ±s, bit k%8 of byte k/8
    K = 256
    bits = rng.integers(0, 2, size=(M, K))
    packed = np.zeros((M, K // 8), np.uint8)
    for k in range(K):
        packed[:, k // 8] |= (bits[:, k] << (k % 8)).astype(np.uint8)
    sv = 2.0 ** rng.integers(-6, 2, size=(M, K // 128))
    sh = sv.astype(np.float16).view(np.uint16)
    x = np.eye(K, dtype=np.float32)
    y, _ = orc.qgemv(B1, packed, sh, None, x, M, K)
    want = np.where(bits == 1, 1.0, -1.0) * np.repeat(sv, 128, axis=1)
    assert np.array_equal(y, want.T), "b1 one-hot"


def pin_zero_and_sign_codes(orc):
    """Closed forms of constant codes: U4 zeros -> y = Σ_g b_g Σ_{k∈g} x;
    I8 zeros -> 0; B1 all ones -> +Σ_g s_g Σ x_g, all zeros -> the negation."""
    rng = np.random.default_rng(12)
    M, K, N = 3, 192, 2
    x = rng.standard_normal((N, K)).astype(np.float32)
    xg64 = x.astype(np.float64).reshape(N, K // 64, 64).sum(-1)
    b = rng.uniform(-1, 1, size=(M, K // 64)).astype(np.float32)
    bb = (b.view(np.uint32) >> 16).astype(np.uint16)
    bval = (bb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    sb = np.full((M, K // 64), 0x3F80, np.uint16)
    y, _ = orc.qgemv(U4, np.zeros((M, K // 2), np.uint8), sb, bb, x, M, K)
    _close(y, xg64 @ bval.T, 1e-13, "u4 zero codes")
    y, _ = orc.qgemv(I8, np.zeros((M, K), np.int8), np.ones(M, np.float32), None, x, M, K)
    assert np.all(y == 0), "i8 zero codes"
    y, _ = orc.qgemv(I8G, np.zeros((M, K), np.int8), np.ones((M, K // 64), np.float32), None,
                     x, M, K)
    assert np.all(y == 0), "i8 group-64 zero codes"
    # constant code c in every group: y = c * Σ_g s_g Σ_{k∈g} x
    sg = rng.uniform(0.01, 1, size=(M, K // 64)).astype(np.float32)
    y, _ = orc.qgemv(I8G, np.full((M, K), -3, np.int8), sg, None, x, M, K)
    _close(y, -3.0 * (xg64 @ sg.astype(np.float64).T), 1e-13, "i8 group-64 constant codes")
    K = 256
    x = rng.standard_normal((N, K)).astype(np.float32)
    xg128 = x.astype(np.float64).reshape(N, K // 128, 128).sum(-1)
    s = rng.uniform(0.01, 1, size=(M, K // 128)).astype(np.float16)
    ones, _ = orc.qgemv(B1, np.full((M, K // 8), 0xFF, np.uint8), s.view(np.uint16), None, x, M, K)
    zeros, _ = orc.qgemv(B1, np.zeros((M, K // 8), np.uint8), s.view(np.uint16), None, x, M, K)
    want = xg128 @ s.astype(np.float64).T
    _close(ones, want, 1e-13, "b1 all ones")
    _close(zeros, -want, 1e-13, "b1 all zeros")


def pin_exact_integer_arithmetic(orc):
    """Power-of-two scales, biases on a 2^-8 grid and integer x in [-8, 8]:
    the result is an exact dyadic rational, computed here in int64."""
    rng = np.random.default_rng(13)
    M, K, N = 7, 384, 3
    x = rng.integers(-8, 9, size=(N, K))
    xf = x.astype(np.float32)
    # I8
    q = rng.integers(-128, 128, size=(M, K))
    e = rng.integers(4, 8, size=M)                      # scale 2^-e
    y, _ = orc.qgemv(I8, q.astype(np.int8), (2.0 ** -e).astype(np.float32), None, xf, M, K)
    num = x @ q.T                                        # int64
    assert np.array_equal(y * (2.0 ** e)[None, :], num.astype(np.float64)), "i8 exact"
    # I8 group-64: y * 2^7 = Σ_g (q·x)_g * 2^(7-e_g)
    eg = rng.integers(0, 8, size=(M, K // 64))
    y, _ = orc.qgemv(I8G, q.astype(np.int8), (2.0 ** -eg).astype(np.float32), None, xf, M, K)
    want = np.zeros((N, M), np.int64)
    for g in range(K // 64):
        sl = slice(64 * g, 64 * g + 64)
        want += (x[:, sl] @ q[:, sl].T) * (2 ** (7 - eg[:, g]))[None, :]
    assert np.array_equal(y * 2.0 ** 7, want.astype(np.float64)), "i8 group-64 exact"
    # U4: y * 2^8 * 2^7 = Σ_g (q·x)_g * 2^(15-e) + (b*2^8)_g * Σx_g * 2^7
    qu = rng.integers(0, 16, size=(M, K))
    packed = (qu[:, 0::2] | (qu[:, 1::2] << 4)).astype(np.uint8)
    G = K // 64
    e = rng.integers(4, 8, size=(M, G))
    bn = rng.integers(-64, 65, size=(M, G))              # bias = bn / 256
    sb = ((2.0 ** -e).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bb = ((bn / 256.0).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y, _ = orc.qgemv(U4, packed, sb, bb, xf, M, K)
    want = np.zeros((N, M), np.int64)
    for g in range(G):
        sl = slice(64 * g, 64 * g + 64)
        qx = x[:, sl] @ qu[:, sl].T
        want += qx * (2 ** (15 - e[:, g]))[None, :] + (x[:, sl].sum(1)[:, None] * bn[:, g][None, :]) * 2 ** 7
    assert np.array_equal(y * 2.0 ** 15, want.astype(np.float64)), "u4 exact"
    # B1: y * 2^7 = Σ_g s_g*2^7 * Σ ±x
    bits = rng.integers(0, 2, size=(M, K))
    packed = np.zeros((M, K // 8), np.uint8)
    for k in range(K):
        packed[:, k // 8] |= (bits[:, k] << (k % 8)).astype(np.uint8)
    G = K // 128
    e = rng.integers(0, 8, size=(M, G))
    sh = (2.0 ** -e).astype(np.float16).view(np.uint16)
    y, _ = orc.qgemv(B1, packed, sh, None, xf, M, K)
    sgn = 2 * bits - 1
    want = np.zeros((N, M), np.int64)
    for g in range(G):
        sl = slice(128 * g, 128 * g + 128)
        want += (x[:, sl] @ sgn[:, sl].T) * (2 ** (7 - e[:, g]))[None, :]
    assert np.array_equal(y * 2.0 ** 7, want.astype(np.float64)), "b1 exact"


def pin_numpy_second_opinion(orc):
    """Random tiny matrices over the full code range, all four formats,
    K <= 256, against numpy's float16 / bit unpacking and a float64 matmul."""
    rng = np.random.default_rng(14)
    for fmt, K in ((I8, 48), (I8, 256), (I8G, 64), (I8G, 320), (U4, 64), (U4, 256), (B1, 128),
                   (B1, 256)):
        for M in (1, 3, 17):
            codes, scales, biases = random_tiny(fmt, M, K, rng)
            x = rng.standard_normal((4, K)).astype(np.float32)
            y, a = orc.qgemv(fmt, codes, scales, biases, x, M, K)
            w = numpy_weights(fmt, codes, scales, biases, M, K)
            ref = x.astype(np.float64) @ w.T
            refa = np.abs(x.astype(np.float64)) @ np.abs(w).T
            tol = 1e-12 * refa + 1e-300
            assert np.all(np.abs(y - ref) <= tol), f"fmt {fmt} K {K} M {M}: y"
            assert np.all(np.abs(a - refa) <= tol), f"fmt {fmt} K {K} M {M}: absdot"
            wd = orc.decode(fmt, codes, scales, biases, M, K)
            assert np.array_equal(wd, w), f"fmt {fmt} K {K} M {M}: decode"


def pin_invariants(orc):
    """Linearity in x, permuted activation rows, duplicate weight rows, and
    the prefill product row n equal to the matvec of x[n]."""
    rng = np.random.default_rng(15)
    for fmt, K in ((I8, 64), (I8G, 192), (U4, 128), (B1, 256)):
        M = 9
        codes, scales, biases = random_tiny(fmt, M, K, rng)
        # activations on a 1/8 grid, so that 2*x1 - x2 is exact in float32
        x1 = (rng.integers(-64, 64, size=(3, K)) / 8.0).astype(np.float32)
        x2 = (rng.integers(-64, 64, size=(3, K)) / 8.0).astype(np.float32)
        y1, a1 = orc.qgemv(fmt, codes, scales, biases, x1, M, K)
        y2, a2 = orc.qgemv(fmt, codes, scales, biases, x2, M, K)
        # linearity with exactly representable combinations
        y3, _ = orc.qgemv(fmt, codes, scales, biases, 2 * x1 - x2, M, K)
        bound = 1e-12 * (2 * a1 + a2)
        assert np.all(np.abs(y3 - (2 * y1 - y2)) <= bound), f"fmt {fmt}: linearity"
        # permuting activation rows permutes outputs
        p = np.array([2, 0, 1])
        yp, _ = orc.qgemv(fmt, codes, scales, biases, x1[p], M, K)
        assert np.array_equal(yp, y1[p]), f"fmt {fmt}: row permutation"
        # each activation row alone gives the same row of the product
        for n in range(3):
            yn, _ = orc.qgemv(fmt, codes, scales, biases, x1[n:n + 1], M, K)
            assert np.array_equal(yn[0], y1[n]), f"fmt {fmt}: row {n} alone"
        # duplicate weight rows give identical outputs
        c2 = codes.copy()
        s2 = scales.copy()
        b2 = None if biases is None else biases.copy()
        c2[4] = c2[1]
        s2[4] = s2[1]
        if b2 is not None:
            b2[4] = b2[1]
        yd, _ = orc.qgemv(fmt, c2, s2, b2, x1, M, K)
        assert np.array_equal(yd[:, 4], yd[:, 1]), f"fmt {fmt}: duplicate rows"
        # zero activations give zero outputs
        yz, _ = orc.qgemv(fmt, codes, scales, biases, np.zeros((1, K), np.float32), M, K)
        assert np.all(yz == 0), f"fmt {fmt}: x = 0"


def pin_argmax_brute_force(orc):
    """Lowest index of the maximum, checked by brute force over all pairs;
    ties at the ends, all-equal rows, and -0 against +0."""
    rng = np.random.default_rng(16)
    rows = [
        np.array([1.0, 3.0, 3.0, 2.0]),
        np.array([5.0, 1.0, 5.0]),
        np.array([0.0, 0.0, 0.0]),
        np.array([-0.0, 0.0]),
        np.array([-1.0, -0.0, 0.0, -0.0]),
        np.array([-3.0, -2.0, -2.0]),
        np.array([1.0, 2.0, 7.0]),
    ]
    for _ in range(50):
        rows.append(rng.integers(-3, 4, size=rng.integers(1, 12)).astype(np.float64))
    for r in rows:
        idx, gap = orc.argmax(r[None, :])
        want = min(i for i in range(len(r)) if all(r[i] >= r[j] for j in range(len(r))))
        assert idx[0] == want, f"argmax {r}: {idx[0]} != {want}"
        others = [r[j] for j in range(len(r)) if j != want]
        if others:
            assert gap[0] == r[want] - max(others), f"gap {r}"
    # several rows at once
    y = np.array([[0.0, 2.0, 1.0], [4.0, 4.0, -1.0]])
    idx, _ = orc.argmax(y)
    assert list(idx) == [1, 0]


# ---------------------------------------------------------------------------
# embedding rows (4-bit format)
# ---------------------------------------------------------------------------

def pin_f16_rounding(orc):
    """The oracle's float32 -> binary16 rounding equals numpy's on every
    binary16 value, one float32 step either side of it, and the float32
    midpoints between neighbouring binary16 values (ties) with a float32
    step either side."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = h.view(np.float16).astype(np.float32)
    fin = np.isfinite(v)
    v = v[fin]
    nxt = np.nextafter(v, np.float32(np.inf))
    prv = np.nextafter(v, np.float32(-np.inf))
    hf = h[fin].view(np.float16)
    up = np.nextafter(hf, np.float16(np.inf)).astype(np.float32)
    mid = ((v.astype(np.float64) + up.astype(np.float64)) / 2).astype(np.float32)   # exact
    cases = np.concatenate([v, nxt, prv, mid, np.nextafter(mid, np.float32(np.inf)),
                            np.nextafter(mid, np.float32(-np.inf)),
                            np.array([np.inf, -np.inf, 65520.0, -65520.0, 1e-30, -1e-30], np.float32)])
    cases = cases[np.isfinite(cases) | np.isinf(cases)]
    with np.errstate(over="ignore"):
        want = cases.astype(np.float16).view(np.uint16)
    got = np.array([orc.f32_to_f16(float(c)) for c in cases], np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"binary16 rounding differs for {cases[bad[:5]]}: {got[bad[:5]]} vs {want[bad[:5]]}"


def _f32_nearest_even(fr):
    """float32 nearest (ties to even) to the exact rational fr."""
    from fractions import Fraction
    if fr == 0:
        return np.float32(0.0)
    sign = -1.0 if fr < 0 else 1.0
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    qe = max(e - 23, -149)                     # exponent of the float32 quantum
    sc = a / Fraction(2) ** qe
    n = sc.numerator // sc.denominator
    rem = sc - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    if n * 2.0 ** qe >= 2.0 ** 128:
        return np.float32(sign * np.inf)
    return np.float32(sign * n * 2.0 ** qe)


def _embed_reference(scale_bits, bias_bits, q):
    """The embedding value written out: exact scale * code + bias, one
    rounding to float32, one to binary16, widened back (float32 bits)."""
    from fractions import Fraction
    sf = np.array([scale_bits << 16], np.uint32).view(np.float32)[0]
    bf = np.array([bias_bits << 16], np.uint32).view(np.float32)[0]
    exact = Fraction(float(sf)) * q + Fraction(float(bf))
    if exact != 0:
        a = _f32_nearest_even(exact)
    elif Fraction(float(sf)) * q == 0 and bf == 0:
        # both terms are zeros: the product carries the scale's sign (q >= 0),
        # and a sum of zeros is -0 only when both are -0 (round to nearest)
        a = np.float32(-0.0) if (np.signbit(sf) and np.signbit(bf)) else np.float32(0.0)
    else:
        a = np.float32(0.0)                     # x + (-x) = +0 (round to nearest)
    return np.float32(a).astype(np.float16).astype(np.float32).view(np.uint32)


def _bf16(v):
    return int(np.array([v], np.float32).view(np.uint32)[0] >> 16)


def _embed_one(orc, scale_bits, bias_bits, q, K=64):
    """Oracle embedding value of code q (input 0 of a one-row table)."""
    codes = np.full((1, K // 2), q | (q << 4), np.uint8)
    e = orc.embed(codes, np.array([[scale_bits]], np.uint16), np.array([[bias_bits]], np.uint16),
                  np.array([0], np.int32), 1, K)
    return e[0, 0]


def pin_embed_hand_cases(orc):
    """Hand-derived IEEE cases: (scale, bias, code) -> value."""
    cases = [
        (0.5, -1.0, 3, 0.5),                    # 0.5 * 3 - 1, exact everywhere
        (1.0, -2.0 ** -30, 0, -0.0),            # below half the smallest binary16 subnormal: -0
        (1.0, -3 * 2.0 ** -26, 0, -2.0 ** -24), # three quarters of it rounds to the subnormal
        (1.0, -2.0 ** -25, 0, -0.0),            # exactly half: tie to even, the zero
        (8192.0, 0.0, 15, np.inf),              # 122880 overflows binary16
        (1.0, 2.0 ** -11, 1, 1.0),              # 1 + half a binary16 ulp: tie to even, 1
        (1.0, 3 * 2.0 ** -12, 1, 1.0 + 2.0 ** -10),  # above the tie: rounds up
        (-0.5, 0.0, 0, 0.0),                    # -0 + +0 = +0
        (-0.5, -0.0, 0, -0.0),                  # -0 + -0 = -0
        (2.0 ** -10, 2.0 ** -14, 1, 2.0 ** -14 + 2.0 ** -10),   # normal binary16, exact
    ]
    for s, b, q, want in cases:
        got = _embed_one(orc, _bf16(s), _bf16(b), q)
        assert (np.isinf(want) and got == want) or \
            (got == want and np.signbit(got) == np.signbit(want)), \
            f"embed({s}, {b}, {q}) = {got!r}, expected {want!r}"


def pin_embed_exact_reference(orc):
    """Random rows (scales of both signs, biases from tiny to large) against
    the exact-rational reference, bit for bit; ids outside the table give
    NaN rows."""
    rng = np.random.default_rng(77)
    M, K = 5, 256
    codes = rng.integers(0, 256, size=(M, K // 2)).astype(np.uint8)
    sc = rng.uniform(-0.05, 0.05, size=(M, K // 64)).astype(np.float32)
    bi = (rng.choice([-1.0, 1.0], size=(M, K // 64)) *
          2.0 ** rng.integers(-40, 2, size=(M, K // 64))).astype(np.float32)
    sc[1, 1], bi[1, 1] = -0.0, -0.0          # signed zeros in both terms
    sc[2, 0], bi[2, 0] = 0.0, -0.0
    sc[3, 2], bi[3, 2] = -0.0, 0.0
    bi[4, 3] = 0.0
    sb = (sc.view(np.uint32) >> 16).astype(np.uint16)
    bb = (bi.view(np.uint32) >> 16).astype(np.uint16)
    ids = np.array([3, 0, 4, 4, -1, 5, 1], np.int32)
    e = orc.embed(codes, sb, bb, ids, M, K)
    for t, i in enumerate(ids):
        if i < 0 or i >= M:
            assert np.all(np.isnan(e[t])), "rows outside the table must be NaN"
            continue
        for k in range(K):
            byte = int(codes[i, k // 2])
            q = (byte >> 4) if k & 1 else (byte & 15)
            want = _embed_reference(int(sb[i, k // 64]), int(bb[i, k // 64]), q)
            got = e[t, k:k + 1].view(np.uint32)[0]
            assert got == want, f"row {i} k {k}: {got:#x} vs {want:#x}"


def pin_sampled_outputs(orc):
    """The sampled form of the product (chosen (row, output) pairs only, the
    reference of the large prefill cases) against numpy's independent decode
    and a float64 matmul, and against the oracle's full product, for all four
    formats. The activation rows and outputs are equal in number (N == M), so
    a mistake that swaps the two indices, or indexes the activations by the
    output, still reads in bounds and shows up as a wrong value; the pairs
    include the first and last row and output and both orders of each
    off-diagonal pair."""
    rng = np.random.default_rng(23)
    for fmt, K in ((I8, 96), (I8G, 192), (U4, 128), (B1, 256)):
        M = N = 19
        codes, scales, biases = random_tiny(fmt, M, K, rng)
        x = rng.standard_normal((N, K)).astype(np.float32)
        w = numpy_weights(fmt, codes, scales, biases, M, K)
        ref = x.astype(np.float64) @ w.T
        refa = np.abs(x.astype(np.float64)) @ np.abs(w).T
        ends = [0, 1, M - 2, M - 1]
        n = [a for a in ends for b in ends] + list(rng.integers(0, N, 40))
        m = [b for a in ends for b in ends] + list(rng.integers(0, M, 40))
        n, m = np.asarray(n, np.int64), np.asarray(m, np.int64)
        y, a = orc.qgemv_sample(fmt, codes, scales, biases, x, M, K, n, m)
        tol = 1e-12 * refa[n, m] + 1e-300
        assert np.all(np.abs(y - ref[n, m]) <= tol), f"fmt {fmt}: sampled y"
        assert np.all(np.abs(a - refa[n, m]) <= tol), f"fmt {fmt}: sampled absdot"
        yf, af = orc.qgemv(fmt, codes, scales, biases, x, M, K)
        assert np.array_equal(y, yf[n, m]) and np.array_equal(a, af[n, m]), \
            f"fmt {fmt}: sampled and full products differ"


def pin_dense_product(orc):
    """The decode-then-matmul form of the product (the reference of the full
    prefill comparisons) equals numpy's independent decode times the
    activations, and the oracle's per-output loops, on random tiny matrices
    of all four formats with several activation rows."""
    rng = np.random.default_rng(29)
    for fmt, K in ((I8, 80), (I8G, 192), (U4, 192), (B1, 384)):
        for M, N in ((1, 1), (7, 3), (33, 20)):
            codes, scales, biases = random_tiny(fmt, M, K, rng)
            x = rng.standard_normal((N, K)).astype(np.float32)
            w = numpy_weights(fmt, codes, scales, biases, M, K)
            ref = x.astype(np.float64) @ w.T
            refa = np.abs(x.astype(np.float64)) @ np.abs(w).T
            y, a = orc.qgemm_dense(fmt, codes, scales, biases, x, M, K)
            tol = 1e-12 * refa + 1e-300
            assert np.all(np.abs(y - ref) <= tol), f"fmt {fmt} M {M} N {N}: dense y"
            assert np.all(np.abs(a - refa) <= tol), f"fmt {fmt} M {M} N {N}: dense absdot"
            yl, al = orc.qgemv(fmt, codes, scales, biases, x, M, K)
            assert np.all(np.abs(y - yl) <= tol) and np.all(np.abs(a - al) <= tol), \
                f"fmt {fmt} M {M} N {N}: dense and per-output products differ"


PINS = [pin_hand_fixtures, pin_decode_values, pin_worked_example, pin_one_hot,
        pin_zero_and_sign_codes, pin_exact_integer_arithmetic,
        pin_numpy_second_opinion, pin_invariants, pin_argmax_brute_force,
        pin_f16_rounding, pin_embed_hand_cases, pin_embed_exact_reference,
        pin_sampled_outputs, pin_dense_product]
