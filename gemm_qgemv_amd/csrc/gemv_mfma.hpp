// gemv_mfma.hpp -- small-batch (2..8 activation rows) product for the 4-bit
// group-64 affine format on the gfx950 matrix cores.
//
// With several activation rows every weight takes several multiply-adds,
// which on the vector ALUs costs more time than streaming the weight from
// HBM; the matrix cores take the contraction instead (Pushing the limits of
// legacy hardware, "Build the execution path, then share the weights":
// batching lets many sequences reuse one pass over the weights).
//
// One v_mfma_f32_16x16x32_bf16 computes D[i][m] += sum_k A[i][k] B[k][m] for
// 16 operand rows i and 16 weight rows m. Each float32 activation is split
// by truncation into three bf16 pieces (top, middle and bottom 8 significant
// bits) whose sum is exact. Operand A row i < 8 holds the top piece of
// activation row n = i, row 8 + n its middle piece; a second MFMA gives
// both rows n and 8 + n half the bottom piece (halving is exact). The two
// halves of D (rows n and 8 + n) are added once per tile, which restores
// top + middle + bottom. Codes 0..15 are exact in bf16 and the products
// accumulate in float32.
//
// Codes to bf16: a byte holding one code (0..15) is, read as an OCP e4m3
// number, exactly code * 2^-9; the gfx950 scaled fp8 -> bf16 conversion
// turns two such bytes into two exact bf16 codes in one instruction.
//
// Affine groups: the scale changes every 64 inputs, so each group is
// accumulated on its own and folded in as acc += scale * tmp. The bias term
// sum_g bias[m][g] * X[n][g], X the group sums of the activations, is one
// more contraction over the groups, done with the same MFMA per tile (the
// biases are bf16 already; X is split into three pieces like x).
//
// Operand order. Lane l is operand row r = l % 16, quarter q = l / 16. Each
// lane loads 16 bytes of its weight row per pair of groups (byte 64 p + 16 q):
// quarters 0, 1 hold group 2p, quarters 2, 3 group 2p + 1. One permlane32
// swap per dword pair hands each quarter 8 inputs of both groups, so that at
// k-step s of group g lane (r, q) holds inputs
//     k = 64 g + 32 (q & 1) + 16 (q >> 1) + 8 s + {0, 2, 4, 6, 1, 3, 5, 7}
// (the last term: even-k nibbles first, as the conversion produces them).
// The activation pieces are staged in LDS in exactly this order.
//
// Mapping. One workgroup of 8 waves per compute unit. The workgroup stages
// the activation pieces of all K in LDS (3 KiB per group, 97 KiB for
// K = 2048) and the pieces of the group sums; each wave then streams its
// contiguous run of 16-row tiles in chunks of 8 groups held in a ring of
// register buffers, so two chunks are in flight while one is reduced.
#pragma once

#include "gemm.hpp"
#include "gemv.hpp"

namespace qg {

struct GemvMfmaParams {
    const uint8_t *codes;
    const uint16_t *scales;
    const uint16_t *biases;
    const float *x;        // [nb][K]
    float *y;              // [nb][M]
    GreedyCtl *ctl;        // greedy head control words, or nullptr
    unsigned long long *keys;   // greedy head: [workgroups][8] scratch
    int32_t *idx;          // [nb] greedy indices, or nullptr
    int64_t M, K;
    int nb;                // 1..8 (one-pass kernel: 1..16)
    int stage_out;         // outputs staged in LDS, written at the end
    float *part;           // one-pass kernel with K split over blockIdx.y:
                           // partial outputs [splits][nb][M] (y and the
                           // greedy head unused), else nullptr
};

constexpr int kMfmaWaves = 8;          // waves per workgroup
constexpr int kMfmaThreads = 64 * kMfmaWaves;
constexpr int kStageItems = 8;          // staging items per thread: K <= 4096
constexpr int kMfmaChunk = 8;           // groups per register chunk
constexpr int kMfmaBufs = 3;           // register chunks in the ring
// One operand block in LDS: 1 KiB top/middle pieces [q][row 16] and 512 B
// halved bottom pieces [q][n 8] (read by operand rows n and 8 + n). A group
// has two (one per k-step); each 32 groups of the bias contraction have one.
constexpr int kMfmaBlockBytes = 1024 + 512;
constexpr int kMfmaGroupBytes = 2 * kMfmaBlockBytes;

__host__ __device__ constexpr int gemv_mfma_bias_steps(int64_t K)
{
    return static_cast<int>((K / 64 + 31) / 32);
}

// LDS bytes of one workgroup: the group blocks, then the bias blocks.
__host__ __device__ constexpr size_t gemv_mfma_lds_bytes(int64_t K)
{
    return static_cast<size_t>(K / 64) * kMfmaGroupBytes +
           static_cast<size_t>(gemv_mfma_bias_steps(K)) * kMfmaBlockBytes;
}

// Outputs of one 16-row tile staged in LDS: [8 activation rows][16] floats.
constexpr int kMfmaTileOutBytes = 8 * 16 * 4;

typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t u4_word(const uint4 &v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// bf16 number j (0..7) of 8 packed in a uint4 -> float32
__device__ __forceinline__ float bf16_at(const uint4 &v, int j)
{
    const uint32_t w = u4_word(v, j >> 1);
    return (j & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
}

// Split float32 v exactly into top, middle and half the bottom bf16 piece
// (truncation; v = top + middle + 2 * half), as bf16 bit patterns.
__device__ __forceinline__ void split3h(float v, uint32_t &hi, uint32_t &mid, uint32_t &half)
{
    const uint32_t h = __float_as_uint(v) & 0xFFFF0000u;
    const float r = v - __uint_as_float(h);                 // exact
    const uint32_t m = __float_as_uint(r) & 0xFFFF0000u;
    hi = h >> 16;
    mid = m >> 16;
    half = __float_as_uint((r - __uint_as_float(m)) * 0.5f) >> 16;   // 8 bits, exact
}

// The same for two values, packed as bf16 pairs (a in the low half).
__device__ __forceinline__ void split3h_pair(float a, float b, uint32_t &hi, uint32_t &mid,
                                             uint32_t &half)
{
    uint32_t ha, ma, la, hb, mb, lb;
    split3h(a, ha, ma, la);
    split3h(b, hb, mb, lb);
    hi = ha | (hb << 16);
    mid = ma | (mb << 16);
    half = la | (lb << 16);
}

// One chunk of one lane: 4 pairs of groups of codes (16 bytes each), the 8
// scales of its weight row, and (first chunks of a tile only) 8 biases.
struct MfmaChunk {
    uint4 c[kMfmaChunk / 2];
    uint4 s, b;
};

__global__ __launch_bounds__(kMfmaThreads) void gemv_mfma_u4_kernel(GemvMfmaParams p)
{
    extern __shared__ float4 lds_f4[];
    uint8_t *lds = reinterpret_cast<uint8_t *>(lds_f4);
    const int G = static_cast<int>(p.K / 64);
    const int C = G / kMfmaChunk;
    const int NBS = gemv_mfma_bias_steps(p.K);
    uint8_t *bias_blocks = lds + static_cast<size_t>(G) * kMfmaGroupBytes;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar loop control
    const int r = lane & 15, q = lane >> 4;
    const int64_t row_bytes = p.K / 2;

    // this wave's run of 16-row tiles
    const int64_t ntiles = (p.M + 15) / 16;
    const int64_t W = static_cast<int64_t>(gridDim.x) * kMfmaWaves;
    const int64_t gw = static_cast<int64_t>(blockIdx.x) * kMfmaWaves + wave;
    const int64_t tb = gw * ntiles / W, te = (gw + 1) * ntiles / W;
    const int64_t total = (te - tb) * C;   // chunks to reduce
    // the workgroup's tiles (its waves' runs are adjacent); with stage_out
    // their outputs collect in LDS after the operand blocks, so that no
    // store waits in the same in-order memory counter as the weight loads
    const int64_t tb_wg = static_cast<int64_t>(blockIdx.x) * ntiles / gridDim.x;
    const int64_t te_wg = static_cast<int64_t>(blockIdx.x + 1) * ntiles / gridDim.x;
    float *out_stage = reinterpret_cast<float *>(bias_blocks + static_cast<size_t>(NBS) * kMfmaBlockBytes);

    // load cursor: this lane's weight row in the tile being loaded (rows
    // past M read row M - 1; their outputs are not written)
    const uint8_t *lc_c = nullptr;
    const uint16_t *lc_s = nullptr, *lc_b = nullptr;
    int lc_chunk = 0;
    int64_t lc_tile = tb;
    auto point = [&](int64_t t) {
        const int64_t m = min(t * 16 + r, p.M - 1);
        lc_c = p.codes + m * row_bytes + 16 * q;
        lc_s = p.scales + m * G;
        lc_b = p.biases + m * G + 8 * q;
        lc_chunk = 0;
        lc_tile = t;
    };
    auto load = [&](MfmaChunk &k) {
#pragma unroll
        for (int j = 0; j < kMfmaChunk / 2; ++j) {
            const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(lc_c + 64 * j));
            k.c[j] = make_uint4(v.x, v.y, v.z, v.w);
        }
        k.s = *reinterpret_cast<const uint4 *>(lc_s);
        if (lc_chunk < NBS)   // biases of groups 32 c + 8 q .. + 7
            k.b = 32 * lc_chunk + 8 * q < G ? *reinterpret_cast<const uint4 *>(lc_b + 32 * lc_chunk)
                                            : make_uint4(0u, 0u, 0u, 0u);
        if (++lc_chunk == C) {
            point(lc_tile + 1);
        } else {
            lc_c += 32 * kMfmaChunk;
            lc_s += kMfmaChunk;
        }
    };

    // 1. activation pieces in operand order. Item (n, g, qq, s) covers 8
    //    inputs of activation row n; a thread's items (at most kStageItems)
    //    are requested before the first weight chunks, so that waiting for
    //    them (memory counters count in order) does not wait for the weights.
    const int nitems = 8 * G * 8;
    float4 xa[kStageItems], xb[kStageItems];
#pragma unroll
    for (int u = 0; u < kStageItems; ++u) {
        const int it = tid + u * kMfmaThreads;
        xa[u] = xb[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        const int n = it / (G * 8), rem = it - n * (G * 8);
        if (it < nitems && n < p.nb) {
            const int g = rem >> 3, qq = (rem >> 1) & 3, s = rem & 1;
            const int k0 = 64 * g + 32 * (qq & 1) + 16 * (qq >> 1) + 8 * s;
            const float4 *src = reinterpret_cast<const float4 *>(p.x + static_cast<int64_t>(n) * p.K + k0);
            xa[u] = src[0];
            xb[u] = src[1];
        }
    }

    MfmaChunk buf[kMfmaBufs];
    point(tb);
#pragma unroll
    for (int u = 0; u < kMfmaBufs - 1; ++u)
        if (u < total) load(buf[u]);

    // greedy head: read the completion word as it stands at the start
    const uint32_t tag = p.ctl != nullptr ? dispatch_tag() : 0u;
    if (p.ctl != nullptr && blockIdx.x == 0 && tid == 0) arrival_preclaim(&p.ctl->arrive, tag);

    // split and store the pieces; the 8 items of one group of one row sit
    // in 8 consecutive lanes, which add their sums into the group sum X[n][g]
    // (the bias-contraction operand: group g is input k = g % 32 of bias
    // step g / 32, quarter (g / 8) % 4, element g % 8)
#pragma unroll
    for (int u = 0; u < kStageItems; ++u) {
        const int it = tid + u * kMfmaThreads;
        if (u * kMfmaThreads < nitems) {   // uniform over the workgroup
            const int n = it / (G * 8), rem = it - n * (G * 8);
            const int g = rem >> 3, qq = (rem >> 1) & 3, s = rem & 1;
            const float4 a = xa[u], b = xb[u];
            float sum = ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
            sum += __shfl_xor(sum, 1);
            sum += __shfl_xor(sum, 2);
            sum += __shfl_xor(sum, 4);
            if (it < nitems) {
                // operand order k0 + {0, 2, 4, 6, 1, 3, 5, 7}
                const float v[8] = {a.x, a.z, b.x, b.z, a.y, a.w, b.y, b.w};
                uint32_t h[4], md[4], lo[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) split3h_pair(v[2 * j], v[2 * j + 1], h[j], md[j], lo[j]);
                uint8_t *blk = lds + static_cast<size_t>(g) * kMfmaGroupBytes + s * kMfmaBlockBytes;
                *reinterpret_cast<uint4 *>(blk + (qq * 16 + n) * 16) = make_uint4(h[0], h[1], h[2], h[3]);
                *reinterpret_cast<uint4 *>(blk + (qq * 16 + 8 + n) * 16) = make_uint4(md[0], md[1], md[2], md[3]);
                *reinterpret_cast<uint4 *>(blk + 1024 + (qq * 8 + n) * 16) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
                if ((rem & 7) == 0) {
                    uint32_t sh, sm, sl;
                    split3h(sum, sh, sm, sl);
                    uint8_t *bb = bias_blocks + static_cast<size_t>(g >> 5) * kMfmaBlockBytes;
                    const int bq = (g >> 3) & 3, e = g & 7;
                    *reinterpret_cast<uint16_t *>(bb + (bq * 16 + n) * 16 + 2 * e) = static_cast<uint16_t>(sh);
                    *reinterpret_cast<uint16_t *>(bb + (bq * 16 + 8 + n) * 16 + 2 * e) = static_cast<uint16_t>(sm);
                    *reinterpret_cast<uint16_t *>(bb + 1024 + (bq * 8 + n) * 16 + 2 * e) = static_cast<uint16_t>(sl);
                }
            }
        }
    }
    // the last bias step's groups beyond G contribute zero
    for (int it = tid; it < (NBS * 32 - G) * 8; it += blockDim.x) {
        const int n = it & 7, g = G + (it >> 3);
        uint8_t *bb = bias_blocks + static_cast<size_t>(g >> 5) * kMfmaBlockBytes;
        const int bq = (g >> 3) & 3, e = g & 7;
        *reinterpret_cast<uint16_t *>(bb + (bq * 16 + n) * 16 + 2 * e) = 0;
        *reinterpret_cast<uint16_t *>(bb + (bq * 16 + 8 + n) * 16 + 2 * e) = 0;
        *reinterpret_cast<uint16_t *>(bb + 1024 + (bq * 8 + n) * 16 + 2 * e) = 0;
    }
    __syncthreads();

    // 2. reduce the chunks
    const int hm_off = lane * 16;
    const int lo_off = 1024 + (q * 8 + (r & 7)) * 16;   // rows n and 8 + n: same half piece
    float best_v[4] = {0.f, 0.f, 0.f, 0.f};
    int64_t best_m[4] = {-1, -1, -1, -1};
    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
    int cc = 0;            // chunk within the tile being reduced
    int64_t ct = tb;       // tile being reduced

    auto mfma = [](uint4 a, bf16x8_t b, floatx4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), b, c, 0, 0, 0);
    };
    auto reduce = [&](const MfmaChunk &k) {
        const uint8_t *gb = lds + static_cast<size_t>(cc) * kMfmaChunk * kMfmaGroupBytes;
#pragma unroll
        for (int j = 0; j < kMfmaChunk / 2; ++j) {
            // quarters 0, 1 hold group 2j, quarters 2, 3 group 2j + 1: swap
            // halves between quarters q and q ^ 2
            const auto s0 = __builtin_amdgcn_permlane32_swap(k.c[j].x, k.c[j].z, false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(k.c[j].y, k.c[j].w, false, false);
            const uint32_t dw[2][2] = {{s0[0], s1[0]}, {s0[1], s1[1]}};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int g = 2 * j + h;
                const uint8_t *b = gb + g * kMfmaGroupBytes;
                const bf16x8_t w0 = nibbles_to_bf16(dw[h][0]), w1 = nibbles_to_bf16(dw[h][1]);
                const float sc = bf16_at(k.s, g);
                floatx4_t t = {0.f, 0.f, 0.f, 0.f};
                t = mfma(*reinterpret_cast<const uint4 *>(b + hm_off), w0, t);
                t = mfma(*reinterpret_cast<const uint4 *>(b + lo_off), w0, t);
                t = mfma(*reinterpret_cast<const uint4 *>(b + kMfmaBlockBytes + hm_off), w1, t);
                t = mfma(*reinterpret_cast<const uint4 *>(b + kMfmaBlockBytes + lo_off), w1, t);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = fmaf(sc, t[i], acc[i]);
            }
        }
        if (cc < NBS) {
            // bias contraction, groups 32 cc .. 32 cc + 31
            const uint8_t *b = bias_blocks + static_cast<size_t>(cc) * kMfmaBlockBytes;
            const bf16x8_t wb = __builtin_bit_cast(bf16x8_t, k.b);
            acc = mfma(*reinterpret_cast<const uint4 *>(b + hm_off), wb, acc);
            acc = mfma(*reinterpret_cast<const uint4 *>(b + lo_off), wb, acc);
        }
        if (++cc == C) {
            // tile done: lane (r, q) holds D rows 4q..4q+3 of column r; add
            // the half from operand rows 8..15 (quarters 2, 3) and store
            const int64_t m = ct * 16 + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = pair_sum<5>(acc[i]);
                const int n = 4 * q + i;
                if (q < 2 && n < p.nb && m < p.M) {
                    if (p.stage_out)
                        out_stage[((ct - tb_wg) * 8 + n) * 16 + r] = v;
                    else if (p.y)
                        p.y[static_cast<int64_t>(n) * p.M + m] = v;
                    if (best_m[i] < 0 || v > best_v[i]) {   // rows arrive in increasing order
                        best_v[i] = v;
                        best_m[i] = m;
                    }
                }
                acc[i] = 0.f;
            }
            cc = 0;
            ++ct;
        }
    };

    // steady state: every step requests the chunk kMfmaBufs - 1 ahead, so
    // the wait before each reduction leaves the later chunks in flight
    constexpr int NB = kMfmaBufs;
    int64_t i = 0;
    for (; i + 2 * NB - 1 <= total; i += NB) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            load(buf[(u + NB - 1) % NB]);
            reduce(buf[u]);
        }
    }
    // drain: fewer than 2 * NB - 1 chunks left
#pragma unroll
    for (int u = 0; u < 2 * NB - 2; ++u) {
        if (i + u < total) {
            if (i + u + NB - 1 < total) load(buf[(u + NB - 1) % NB]);
            reduce(buf[u % NB]);
        }
    }

    if (p.stage_out && p.y) {
        __syncthreads();
        const int64_t m0 = tb_wg * 16, rows = min(te_wg * 16, p.M) - m0;
        for (int n = 0; n < p.nb; ++n)
            for (int64_t j = tid; j < rows; j += blockDim.x) {
                const int64_t tl = j >> 4;
                p.y[static_cast<int64_t>(n) * p.M + m0 + j] = out_stage[(tl * 8 + n) * 16 + (j & 15)];
            }
    }

    if (p.ctl != nullptr) {
        __shared__ unsigned long long wg_key[8];
        if (tid < 8) wg_key[tid] = 0ull;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint64_t key = best_m[i] >= 0 ? argmax_key(best_v[i], static_cast<uint32_t>(best_m[i])) : 0ull;
            // the 16 lanes of a quarter share the activation row: reduce over r
#pragma unroll
            for (int o = 8; o >= 1; o >>= 1) {
                const uint64_t other = shfl_xor_u64(key, o);
                key = other > key ? other : key;
            }
            const int n = 4 * q + i;
            if (r == 0 && q < 2 && n < p.nb) atomicMax(&wg_key[n], static_cast<unsigned long long>(key));
        }
        __syncthreads();
        greedy_finish_rows(wg_key, p.nb, p.ctl, p.keys, p.idx, static_cast<int>(gridDim.x), tag);
    }
}

}  // namespace qg
