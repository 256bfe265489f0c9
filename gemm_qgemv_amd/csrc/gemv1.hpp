// gemv1.hpp -- batch-1 matrix-vector kernel for the 8-bit and 4-bit formats.
//
// One wave per workgroup; no LDS and no barrier. Lane l owns the 16-byte
// slices t = l + 64 j (j < NS) of every row, so it keeps exactly the
// activations of those slices in registers for the whole kernel (loaded
// once, straight from global memory) together with their sums. Each wave
// streams a contiguous run of rows in blocks of R rows; the codes (and
// scales) of the next block are requested before the current block is
// reduced, and the very first block is requested before the activations, so
// the two memory round trips overlap. Every wave instruction still reads 64
// consecutive 16-byte pieces of one row (1 KiB, fully coalesced).
#pragma once

#include "gemv.hpp"

namespace qg {

struct Gemv1Params {
    const uint8_t *codes;
    const void *scales;
    const void *biases;
    const float *x;      // [K]
    float *y;            // [M]
    uint64_t *keys;      // [nkeys] argmax keys (one per wave), or nullptr
    int64_t M;
    int64_t K;
    int64_t rows_per_wave;
    int nkeys;
};

template <int FMT, int NS, int R>
struct Gemv1Block {
    uint4 c[R][NS];
    uint32_t s[R][NS];   // U4: bf16 bits of the scale; I8: unused
    uint32_t b[R][NS];   // U4: bf16 bits of the bias
    float rs;            // I8: scale of the row this lane writes
};

template <int FMT, int NS, int R>
__device__ __forceinline__ void gemv1_load(const Gemv1Params &p, int64_t rb, int64_t m_end,
                                           int S, int64_t row_bytes, int lane, int own,
                                           Gemv1Block<FMT, NS, R> &blk)
{
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t m = rb + r;
        const bool mv = m < m_end;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int t = lane + kWave * j;
            const bool v = mv && t < S;
            blk.c[r][j] = v ? *reinterpret_cast<const uint4 *>(p.codes + m * row_bytes + 16 * t)
                            : make_uint4(0, 0, 0, 0);
            if (FMT == FMT_U4_G64) {
                const int64_t gi = m * (p.K / 64) + t / 2;
                blk.s[r][j] = v ? static_cast<const uint16_t *>(p.scales)[gi] : 0u;
                blk.b[r][j] = v ? static_cast<const uint16_t *>(p.biases)[gi] : 0u;
            }
        }
    }
    if (FMT == FMT_I8_ROW) {
        const int64_t m = rb + own;
        blk.rs = m < m_end ? static_cast<const float *>(p.scales)[m] : 0.f;
    }
}

template <int FMT, int NS, int R>
__global__ __launch_bounds__(64) void gemv1_kernel(Gemv1Params p)
{
    constexpr int KPS = Fmt<FMT>::KPS;   // 16 (I8) or 32 (U4)
    constexpr int CPS = KPS / 4;         // float4 chunks per slice
    constexpr int P = R == 1 ? 0 : R == 2 ? 1 : R == 4 ? 2 : 3;
    static_assert(FMT == FMT_I8_ROW || FMT == FMT_U4_G64, "8-bit and 4-bit formats only");

    const int lane = threadIdx.x;
    const int S = static_cast<int>(p.K / KPS);
    const int64_t row_bytes = FMT == FMT_I8_ROW ? p.K : p.K / 2;
    const int64_t m_begin = static_cast<int64_t>(blockIdx.x) * p.rows_per_wave;
    const int64_t m_end = min(p.M, m_begin + p.rows_per_wave);
    const int own = lane >> (6 - P);
    const bool writer = (lane & ((1 << (6 - P)) - 1)) == 0;

    Gemv1Block<FMT, NS, R> cur;
    gemv1_load<FMT, NS, R>(p, m_begin, m_end, S, row_bytes, lane, own, cur);

    // this lane's activations (odd k of the 4-bit format pre-divided by 16)
    float4 xv[NS][CPS];
    float xs[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int t = lane + kWave * j;
        const float4 *src = reinterpret_cast<const float4 *>(p.x + static_cast<int64_t>(t) * KPS);
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < CPS; ++q) {
            float4 v = t < S ? src[q] : make_float4(0.f, 0.f, 0.f, 0.f);
            s += (v.x + v.y) + (v.z + v.w);
            if (FMT == FMT_U4_G64) {
                v.y *= 0.0625f;
                v.w *= 0.0625f;
            }
            xv[j][q] = v;
        }
        xs[j] = s;
    }

    float best_v = 0.f;
    int64_t best_m = -1;
    for (int64_t rb = m_begin; rb < m_end; rb += R) {
        Gemv1Block<FMT, NS, R> nxt;
        const bool more = rb + R < m_end;
        if (more) gemv1_load<FMT, NS, R>(p, rb + R, m_end, S, row_bytes, lane, own, nxt);

        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float a = 0.f;
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                const uint4 c = cur.c[r][j];
                if (FMT == FMT_I8_ROW) {
                    a = dot_i8x4(c.x, xv[j][0], a);
                    a = dot_i8x4(c.y, xv[j][1], a);
                    a = dot_i8x4(c.z, xv[j][2], a);
                    a = dot_i8x4(c.w, xv[j][3], a);
                } else {
                    float d = 0.f;
                    d = dot_u4x8(c.x, xv[j][0], xv[j][1], d);
                    d = dot_u4x8(c.y, xv[j][2], xv[j][3], d);
                    d = dot_u4x8(c.z, xv[j][4], xv[j][5], d);
                    d = dot_u4x8(c.w, xv[j][6], xv[j][7], d);
                    a = fmaf(bf16_bits_to_f32(cur.s[r][j]), d,
                             fmaf(bf16_bits_to_f32(cur.b[r][j]), xs[j], a));
                }
            }
            acc[r] = a;
        }
        wave_transpose_reduce<R>(acc, lane);
        if (writer) {
            const int64_t m = rb + own;
            if (m < m_end) {
                float v = acc[0];
                if (FMT == FMT_I8_ROW) v *= cur.rs;
                p.y[m] = v;
                if (best_m < 0 || v > best_v || (v == best_v && m < best_m)) {
                    best_v = v;
                    best_m = m;
                }
            }
        }
        if (more) cur = nxt;
    }

    if (p.keys != nullptr) {
        uint64_t key = (writer && best_m >= 0) ? argmax_key(best_v, static_cast<uint32_t>(best_m)) : 0ull;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const uint64_t other = shfl_xor_u64(key, o);
            key = other > key ? other : key;
        }
        if (lane == 0) p.keys[blockIdx.x] = key;
    }
}

}  // namespace qg
