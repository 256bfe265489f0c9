"""Seeded synthetic inputs for the quantized matvec / prefill / greedy-head
workloads.

This module only draws random numbers and lays them out in the three packed
weight formats; it holds none of the product's arithmetic. Both the GPU path
(tests, benchmark) and the CPU oracle read the arrays it returns.

Formats (W is M x K, M outputs by K inputs, all arrays row-major):

* ``I8_ROW``   codes int8 [M][K] uniform in [-127, 127]; scales fp32 [M]
  uniform in [1e-3, 1e-2].
* ``U4_G64``   codes uint8 [M][K/2], two 4-bit codes per byte (even k in the
  low nibble); scales and biases bf16 bit patterns (uint16) [M][K/64], scale
  uniform in [1e-3, 2e-2], bias uniform in [-0.1, 0.1], each rounded to the
  nearest bf16 so the stored value is exactly a bf16.
* ``B1_G128``  codes uint8 [M][K/8], one sign bit per weight (bit k%8 of byte
  k/8); scales fp16 bit patterns (uint16) [M][K/128] uniform in [5e-3, 5e-2]
  rounded to the nearest fp16.

Uniform random bytes give exactly uniform 4-bit codes in both nibbles and
Bernoulli(0.5) sign bits, so the packed formats are drawn as bytes directly.

Activations are float32 N(0, 1), shape [rows][K].

Draws use ``numpy.random.default_rng(SeedSequence([2026, case, variant]))`` in
the order codes, scales, biases, activations.
"""
from __future__ import annotations

import dataclasses

import numpy as np

I8_ROW, U4_G64, B1_G128, I8_G64 = 1, 2, 3, 4
FORMAT_NAMES = {I8_ROW: "i8_row", U4_G64: "u4_g64", B1_G128: "b1_g128", I8_G64: "i8_g64"}
K_UNIT = {I8_ROW: 16, U4_G64: 64, B1_G128: 128, I8_G64: 64}


def rng_for(case: int, variant: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([2026, case, variant]))


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Nearest bf16 (ties to even) of float32 values, as uint16 bit patterns.
    Inputs must be finite."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def to_fp16_bits(v: np.ndarray) -> np.ndarray:
    """Nearest fp16 (numpy's IEEE conversion, ties to even) as uint16 bits."""
    return np.ascontiguousarray(v, dtype=np.float32).astype(np.float16).view(np.uint16)


@dataclasses.dataclass
class QWeights:
    fmt: int
    M: int
    K: int
    codes: np.ndarray
    scales: np.ndarray
    biases: np.ndarray | None

    @property
    def nbytes(self) -> int:
        """Bytes of codes + scales + biases: what one pass must read."""
        n = self.codes.nbytes + self.scales.nbytes
        return n + (self.biases.nbytes if self.biases is not None else 0)


def weight_bytes(fmt: int, M: int, K: int) -> int:
    """Bytes of codes + scales (+ biases) of an M x K matrix in `fmt`."""
    if fmt == I8_ROW:
        return M * K + 4 * M
    if fmt == I8_G64:
        return M * K + 4 * M * (K // 64)
    if fmt == U4_G64:
        return M * K // 2 + 2 * 2 * M * (K // 64)
    if fmt == B1_G128:
        return M * K // 8 + 2 * M * (K // 128)
    raise ValueError(fmt)


def draw_weights(fmt: int, M: int, K: int, rng: np.random.Generator) -> QWeights:
    if K % K_UNIT[fmt]:
        raise ValueError(f"K={K} is not a multiple of {K_UNIT[fmt]} for {FORMAT_NAMES[fmt]}")
    if fmt == I8_ROW:
        codes = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
        scales = rng.uniform(1e-3, 1e-2, size=M).astype(np.float32)
        return QWeights(fmt, M, K, codes, scales, None)
    if fmt == I8_G64:
        codes = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
        scales = rng.uniform(1e-3, 1e-2, size=(M, K // 64)).astype(np.float32)
        return QWeights(fmt, M, K, codes, scales, None)
    if fmt == U4_G64:
        codes = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
        scales = to_bf16_bits(rng.uniform(1e-3, 2e-2, size=(M, K // 64)).astype(np.float32))
        biases = to_bf16_bits(rng.uniform(-0.1, 0.1, size=(M, K // 64)).astype(np.float32))
        return QWeights(fmt, M, K, codes, scales, biases)
    if fmt == B1_G128:
        codes = rng.integers(0, 256, size=(M, K // 8), dtype=np.uint8)
        scales = to_fp16_bits(rng.uniform(5e-3, 5e-2, size=(M, K // 128)).astype(np.float32))
        return QWeights(fmt, M, K, codes, scales, None)
    raise ValueError(fmt)


def draw_x(rows: int, K: int, rng: np.random.Generator) -> np.ndarray:
    return rng.standard_normal(size=(rows, K), dtype=np.float32)


def draw_ids(n: int, M: int, rng: np.random.Generator) -> np.ndarray:
    """Token ids of a prompt: uniform over the vocabulary (int32)."""
    return rng.integers(0, M, size=n, dtype=np.int32)


# bf16 patterns of signed zeros and of the smallest and largest subnormals
_BF16_EDGES = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x807F], np.uint16)


def draw_embed_stress(M: int, K: int, rng: np.random.Generator) -> QWeights:
    """A 4-bit table whose groups hit the corners of decoding a row: each
    64-input group takes one of four recipes,
      0  scale and bias any bf16 bit pattern (zeros, subnormals, huge values
         whose products overflow, infinities, NaNs);
      1  typical magnitudes of both signs;
      2  a bias close to -scale * q0 and codes within one of q0, so that
         scale * code + bias cancels to tiny values of either sign, zeros
         and binary16 subnormals;
      3  a signed zero or a bf16 subnormal as scale or bias, the other term
         typical."""
    if K % 64:
        raise ValueError("K must be a multiple of 64")
    G = K // 64
    codes = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    mode = rng.integers(0, 4, size=(M, G))
    sb = rng.integers(0, 1 << 16, size=(M, G)).astype(np.uint16)
    bb = rng.integers(0, 1 << 16, size=(M, G)).astype(np.uint16)

    s1 = to_bf16_bits(rng.uniform(-2e-2, 2e-2, size=(M, G)).astype(np.float32))
    b1 = to_bf16_bits(rng.uniform(-0.1, 0.1, size=(M, G)).astype(np.float32))
    sb = np.where(mode == 1, s1, sb)
    bb = np.where(mode == 1, b1, bb)

    sign = rng.choice([-1.0, 1.0], size=(M, G))
    mag = rng.uniform(1.0, 2.0, size=(M, G)) * 2.0 ** rng.integers(-30, 6, size=(M, G))
    s2 = to_bf16_bits((sign * mag).astype(np.float32))
    sval = (s2.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q0 = rng.integers(1, 15, size=(M, G))
    b2 = to_bf16_bits((-(sval * q0)).astype(np.float32))
    sb = np.where(mode == 2, s2, sb)
    bb = np.where(mode == 2, b2, bb)
    near = np.clip(q0[:, :, None] + rng.integers(-1, 2, size=(M, G, 64)), 0, 15)
    near = near.reshape(M, K).astype(np.uint8)
    packed = near[:, 0::2] | (near[:, 1::2] << 4)
    in_mode2 = np.repeat(mode == 2, 32, axis=1)
    codes = np.where(in_mode2, packed, codes).astype(np.uint8)

    edge = _BF16_EDGES[rng.integers(0, len(_BF16_EDGES), size=(M, G))]
    which = rng.integers(0, 2, size=(M, G))
    sb = np.where((mode == 3) & (which == 0), edge, np.where(mode == 3, s1, sb))
    bb = np.where((mode == 3) & (which == 1), edge, np.where(mode == 3, b1, bb))
    return QWeights(U4_G64, M, K, np.ascontiguousarray(codes),
                    np.ascontiguousarray(sb.astype(np.uint16)),
                    np.ascontiguousarray(bb.astype(np.uint16)))


# ---------------------------------------------------------------------------
# The measured workloads: thirteen concrete cases in five families (8-bit
# 1024x1024 matvec, 4-bit 2B-model matvecs, the 151936x2048 greedy head at 1
# and 8 rows, 8-bit prefill, 1-bit matvec and prefill).
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Case:
    name: str
    op: str          # "gemv", "gemv_argmax", "greedy" (argmax, no logits), "gemm"
                     # or "embed" (rows = token ids gathered)
    fmt: int
    M: int
    K: int
    rows: int        # batch (gemv) or tokens N (gemm)
    case: int        # seed component: workload family
    variant: int     # seed component: variant within it
    x_variant: int | None = None  # draw x from another variant's stream

    @property
    def weight_bytes(self) -> int:
        return weight_bytes(self.fmt, self.M, self.K)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.K * self.rows


CASES = [
    Case("c0_i8_gemv_1024x1024", "gemv", I8_ROW, 1024, 1024, 1, 0, 0),
    Case("c1a_u4_gemv_6144x2048", "gemv", U4_G64, 6144, 2048, 1, 1, 0),
    Case("c1b_u4_gemv_2048x6144", "gemv", U4_G64, 2048, 6144, 1, 1, 1),
    Case("c2_u4_head_151936x2048_b1", "gemv_argmax", U4_G64, 151936, 2048, 1, 2, 0),
    Case("c2_u4_head_151936x2048_b8", "gemv_argmax", U4_G64, 151936, 2048, 8, 2, 0, x_variant=1),
    Case("c3a_i8_gemm_3584x1024_n2048", "gemm", I8_ROW, 3584, 1024, 2048, 3, 0),
    Case("c3b_i8_gemm_1024x3584_n2048", "gemm", I8_ROW, 1024, 3584, 2048, 3, 1),
    Case("c3c_i8_gemm_3584x1024_n10240", "gemm", I8_ROW, 3584, 1024, 10240, 3, 2),
    Case("c3d_i8_gemm_1024x3584_n10240", "gemm", I8_ROW, 1024, 3584, 10240, 3, 3),
    Case("c4a_b1_gemv_17408x5120", "gemv", B1_G128, 17408, 5120, 1, 4, 0),
    Case("c4b_b1_gemv_5120x17408", "gemv", B1_G128, 5120, 17408, 1, 4, 1),
    Case("c4c_b1_gemm_17408x5120_n512", "gemm", B1_G128, 17408, 5120, 512, 4, 2),
    Case("c4d_b1_gemm_5120x17408_n512", "gemm", B1_G128, 5120, 17408, 512, 4, 3),
]
# Measurement cases beyond those thirteen: the 4-bit prefill
# at the 4-bit matvec shapes, with a 2048-token prompt; the greedy head at 64
# and 128 rows, with logits and without ("greedy": qgemv_argmax, logits NULL);
# the embedding rows of a 2048-token prompt gathered from the same (tied)
# head matrix; the greedy head at the largest matrix-vector batch (16); the
# 8-bit format with one scale per 64 inputs at the 8-bit projection shapes,
# batch 1 and a 2048-token prompt.
NEXT_CASES = [
    Case("n2a_u4_gemm_6144x2048_n2048", "gemm", U4_G64, 6144, 2048, 2048, 5, 0),
    Case("n2b_u4_gemm_2048x6144_n2048", "gemm", U4_G64, 2048, 6144, 2048, 5, 1),
    Case("n1a_u4_head_151936x2048_b64", "gemv_argmax", U4_G64, 151936, 2048, 64, 2, 0, x_variant=6),
    Case("n1b_u4_head_151936x2048_b64_nologits", "greedy", U4_G64, 151936, 2048, 64, 2, 0, x_variant=6),
    Case("n1c_u4_head_151936x2048_b128", "gemv_argmax", U4_G64, 151936, 2048, 128, 2, 0, x_variant=7),
    Case("n1d_u4_head_151936x2048_b128_nologits", "greedy", U4_G64, 151936, 2048, 128, 2, 0, x_variant=7),
    Case("n3_u4_embed_151936x2048_t2048", "embed", U4_G64, 151936, 2048, 2048, 2, 0, x_variant=8),
    Case("n4_u4_head_151936x2048_b16", "gemv_argmax", U4_G64, 151936, 2048, 16, 2, 0, x_variant=9),
    Case("n2c_i8g_gemv_3584x1024", "gemv", I8_G64, 3584, 1024, 1, 6, 0),
    Case("n2d_i8g_gemv_1024x3584", "gemv", I8_G64, 1024, 3584, 1, 6, 1),
    Case("n2e_i8g_gemm_3584x1024_n2048", "gemm", I8_G64, 3584, 1024, 2048, 6, 2),
    Case("n2f_i8g_gemm_1024x3584_n2048", "gemm", I8_G64, 1024, 3584, 2048, 6, 3),
]
CASES_BY_NAME = {c.name: c for c in CASES + NEXT_CASES}


def case_inputs(c: Case) -> tuple[QWeights, np.ndarray]:
    """Weights and activations (token ids for "embed") of one case. Cases
    that share a (case, variant) weight stream get the same weights;
    `x_variant` draws the activations from a separate stream."""
    rng = rng_for(c.case, c.variant)
    w = draw_weights(c.fmt, c.M, c.K, rng)
    if c.op == "embed":
        return w, draw_ids(c.rows, c.M, rng_for(c.case, c.x_variant))
    if c.x_variant is None:
        x = draw_x(c.rows, c.K, rng)
    else:
        x = draw_x(c.rows, c.K, rng_for(c.case, c.x_variant))
    return w, x
