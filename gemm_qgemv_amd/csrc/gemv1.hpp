// gemv1.hpp -- batch-1 matrix-vector kernel for the 8-bit (per-row and
// group-64 scales) and 4-bit formats.
//
// Workgroups of 4 (or 8) independent waves; no LDS and no barrier on the
// hot path.
// Lane l owns the 16-byte slices t = l + 64 j (j < NS) of every row, so it
// keeps exactly the activations of those slices in registers for the whole
// kernel (loaded once, straight from global memory) together with their
// sums. Each wave streams a contiguous run of rows in blocks of R rows with
// two register blocks (A, B): the codes and coefficients of the next block
// are requested before the current one is reduced, and the first block is
// requested before the activations, so the two memory round trips overlap.
// Every wave instruction reads 64 consecutive 16-byte pieces of one row
// (1 KiB, fully coalesced); full blocks need no bounds checks, so their
// addresses are running pointers. The per-lane partial sums of the R rows
// are combined with DPP and permlane exchanges (no LDS).
//
// Greedy head: each wave keeps the (value, index) of its best row; the
// workgroup parks one key in its row of the workspace, and the last
// workgroup to finish reduces them and writes the index (greedy_finish_rows).
#pragma once

#include "gemv.hpp"

namespace qg {

struct Gemv1Params {
    const uint8_t *codes;
    const void *scales;
    const void *biases;
    const float *x;      // [K]
    float *y;            // [M]
    GreedyCtl *ctl;      // greedy head control words, or nullptr
    unsigned long long *keys;  // greedy keys, one per workgroup, in the workspace
    int32_t *idx;        // greedy index output
    int64_t M;
    int64_t K;
    int64_t rows_per_wave;
};

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ uint4 load_codes(const uint8_t *p)
{
    if constexpr (NT) {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *reinterpret_cast<const uint4 *>(p);
    }
}

template <int NS, int R>
struct Gemv1Block {
    uint4 c[R][NS];
    uint32_t s[R][NS];   // 4-bit: bf16 bits of the scale; 8-bit group-64: fp32 bits
    uint32_t b[R][NS];   // 4-bit: bf16 bits of the bias
    float rs;            // 8-bit: scale of the row this lane writes
};

// Per-lane cursor over the wave's rows: codes, coefficient and row-scale
// pointers of the next block to load.
struct Gemv1Cursor {
    const uint8_t *c;
    const uint16_t *s;
    const uint16_t *b;
    const float *rs;
    const float *gs;     // 8-bit group-64: this lane's first group scale
};

// Load the next block of R rows and advance the cursor. CHECK: rows at or
// beyond `rows_left` read as zero (only the final, partial block).
template <int FMT, int NS, int R, bool FULL, bool NT, bool CHECK>
__device__ __forceinline__ void gemv1_load(Gemv1Cursor &cur, int64_t row_bytes, int64_t groups,
                                           int lane, int S, int own, int rows_left,
                                           Gemv1Block<NS, R> &blk)
{
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool rv = !CHECK || r < rows_left;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const bool v = rv && (FULL || lane + kWave * j < S);
            blk.c[r][j] = v ? load_codes<NT>(cur.c + r * row_bytes + 16 * kWave * j) : make_uint4(0, 0, 0, 0);
            if constexpr (FMT == FMT_U4_G64) {
                blk.s[r][j] = v ? cur.s[r * groups + 32 * j] : 0u;
                blk.b[r][j] = v ? cur.b[r * groups + 32 * j] : 0u;
            } else if constexpr (FMT == FMT_I8_G64) {
                // slice t = lane + 64 j covers inputs 16 t .. 16 t + 15, in group t / 4
                blk.s[r][j] = v ? __float_as_uint(cur.gs[r * groups + 16 * j]) : 0u;
            }
        }
    }
    if constexpr (FMT == FMT_I8_ROW) blk.rs = (!CHECK || own < rows_left) ? cur.rs[0] : 0.f;
    cur.c += R * row_bytes;
    cur.s += R * groups;
    cur.b += R * groups;
    cur.rs += R;
    cur.gs += R * groups;
}

// WGW: waves per workgroup (4; 8 for greedy-head calls with K of one or two
// slices per lane, which halves the workgroups folding keys at the end)
template <int FMT, int NS, int R, bool FULL, bool NT, int WGW>
__global__ __launch_bounds__(64 * WGW) void gemv1_kernel(Gemv1Params p)
{
    constexpr int KPS = Fmt<FMT>::KPS;   // 16 (8-bit) or 32 (4-bit)
    constexpr int CPS = KPS / 4;         // float4 chunks per slice
    static_assert(FMT == FMT_I8_ROW || FMT == FMT_U4_G64 || FMT == FMT_I8_G64,
                  "8-bit and 4-bit formats only");

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int S = static_cast<int>(p.K / KPS);
    const int64_t row_bytes = FMT == FMT_U4_G64 ? p.K / 2 : p.K;
    const int64_t groups = p.K / 64;
    const int64_t m_begin = (static_cast<int64_t>(blockIdx.x) * WGW + wave) * p.rows_per_wave;
    const int64_t m_end = min(p.M, m_begin + p.rows_per_wave);
    const int64_t rows = m_end > m_begin ? m_end - m_begin : 0;
    const int nfull = static_cast<int>(rows / R);
    const int tail = static_cast<int>(rows % R);
    const int own = dpp_owner<R>(lane);
    const bool writer = dpp_writer<R>(lane);

    Gemv1Cursor cur;
    cur.c = p.codes + m_begin * row_bytes + 16 * lane;
    cur.s = static_cast<const uint16_t *>(p.scales) + (FMT == FMT_U4_G64 ? m_begin * groups + lane / 2 : 0);
    cur.b = static_cast<const uint16_t *>(FMT == FMT_U4_G64 ? p.biases : p.scales) +
            (FMT == FMT_U4_G64 ? m_begin * groups + lane / 2 : 0);
    cur.rs = static_cast<const float *>(p.scales) + (FMT == FMT_I8_ROW ? m_begin + own : 0);
    cur.gs = static_cast<const float *>(p.scales) + (FMT == FMT_I8_G64 ? m_begin * groups + lane / 4 : 0);

    Gemv1Block<NS, R> A, B;
    if (nfull > 0) gemv1_load<FMT, NS, R, FULL, NT, false>(cur, row_bytes, groups, lane, S, own, R, A);

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
            float4 v = (FULL || t < S) ? src[q] : make_float4(0.f, 0.f, 0.f, 0.f);
            s += (v.x + v.y) + (v.z + v.w);
            if (FMT == FMT_U4_G64) {
                v.y *= 0.0625f;
                v.w *= 0.0625f;
            }
            xv[j][q] = v;
        }
        xs[j] = s;
    }

    // greedy head: read the completion word as it stands at the start (after the
    // first block's and the activations' loads, so that the first wait does
    // not include it)
    const uint32_t tag = p.ctl != nullptr ? dispatch_tag() : 0u;
    if (p.ctl != nullptr && blockIdx.x == 0 && threadIdx.x == 0) arrival_preclaim(&p.ctl->arrive, tag);

    float best_v = 0.f;
    int64_t best_m = -1;

    // reduce one block and store its R outputs
    auto finish = [&](const Gemv1Block<NS, R> &blk, int bi) {
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float a = 0.f;
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                const uint4 c = blk.c[r][j];
                if constexpr (FMT == FMT_I8_ROW) {
                    a = dot_i8x4(c.x, xv[j][0], a);
                    a = dot_i8x4(c.y, xv[j][1], a);
                    a = dot_i8x4(c.z, xv[j][2], a);
                    a = dot_i8x4(c.w, xv[j][3], a);
                } else if constexpr (FMT == FMT_I8_G64) {
                    float d = 0.f;
                    d = dot_i8x4(c.x, xv[j][0], d);
                    d = dot_i8x4(c.y, xv[j][1], d);
                    d = dot_i8x4(c.z, xv[j][2], d);
                    d = dot_i8x4(c.w, xv[j][3], d);
                    a = fmaf(__uint_as_float(blk.s[r][j]), d, a);
                } else {
                    float d = 0.f;
                    d = dot_u4x8(c.x, xv[j][0], xv[j][1], d);
                    d = dot_u4x8(c.y, xv[j][2], xv[j][3], d);
                    d = dot_u4x8(c.z, xv[j][4], xv[j][5], d);
                    d = dot_u4x8(c.w, xv[j][6], xv[j][7], d);
                    a = fmaf(bf16_bits_to_f32(blk.s[r][j]), d, fmaf(bf16_bits_to_f32(blk.b[r][j]), xs[j], a));
                }
            }
            acc[r] = a;
        }
        wave_reduce_dpp<R>(acc, lane);
        const int64_t m = m_begin + static_cast<int64_t>(bi) * R + own;
        if (writer && m < m_end) {
            float v = acc[0];
            if constexpr (FMT == FMT_I8_ROW) v *= blk.rs;
            if (p.y) p.y[m] = v;
            if (best_m < 0 || v > best_v) {  // rows arrive in increasing order
                best_v = v;
                best_m = m;
            }
        }
    };

    int i = 0;
    for (; i + 1 < nfull; i += 2) {
        gemv1_load<FMT, NS, R, FULL, NT, false>(cur, row_bytes, groups, lane, S, own, R, B);
        finish(A, i);
        if (i + 2 < nfull) gemv1_load<FMT, NS, R, FULL, NT, false>(cur, row_bytes, groups, lane, S, own, R, A);
        finish(B, i + 1);
    }
    if (i < nfull) finish(A, i);
    if (tail > 0) {
        gemv1_load<FMT, NS, R, FULL, NT, true>(cur, row_bytes, groups, lane, S, own, tail, A);
        finish(A, nfull);
    }

    if (p.ctl != nullptr) {
        __shared__ unsigned long long s_key;
        if (threadIdx.x == 0) s_key = 0ull;
        __syncthreads();
        uint64_t key = (writer && best_m >= 0) ? argmax_key(best_v, static_cast<uint32_t>(best_m)) : 0ull;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const uint64_t other = shfl_xor_u64(key, o);
            key = other > key ? other : key;
        }
        if (lane == 0) atomicMax(&s_key, static_cast<unsigned long long>(key));
        __syncthreads();
        greedy_finish_rows(&s_key, 1, p.ctl, p.keys, p.idx, static_cast<int>(gridDim.x), tag);
    }
}

}  // namespace qg
