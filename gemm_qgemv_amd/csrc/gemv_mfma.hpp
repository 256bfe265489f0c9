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
// 16 operand rows i and 16 weight rows m. Operand A row i < 8 holds the top
// bf16 piece of activation row n = i, row 8 + n its middle piece; a second
// MFMA adds the bottom pieces (rows 0..7; rows 8..15 read zeros). Each
// float32 activation is the exact sum of its three pieces (top, middle and
// bottom 8 significant bits, split by truncation), codes 0..15 are exact in
// bf16, and the products accumulate in float32; the two halves of D (rows
// n and 8 + n) are added once per tile.
//
// Affine groups: the scale and bias change every 64 inputs, so each group is
// accumulated on its own and folded in as
//     acc += scale * tmp + bias * sum_{k in group} x[n][k].
// The k order inside a group is permuted so that each MFMA stays inside one
// group: lane l (operand row r = l % 16, quarter q = l / 16) holds, at k-step
// s (0, 1), the inputs k = 64 g + 16 q + 8 s + e (e = 0..7). On the weight
// side that is 4 bytes of row r at byte 32 g + 8 q + 4 s, so a lane reads
// its 8 bytes of a group with one load. Odd k take the high nibble in place
// (16 * code) against activations pre-divided by 16.
//
// Mapping. One workgroup of 8 waves per compute unit. The workgroup stages
// the activation pieces of all K in LDS, already in operand order (3 KiB per
// group, 96 KiB for K = 2048), plus the group sums; each wave then streams
// its contiguous run of 16-row tiles in chunks of 8 groups held in a ring
// of register buffers, so two chunks are in flight while one is reduced.
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
    int32_t *idx;          // [nb] greedy indices, or nullptr
    int64_t M, K;
    int nb;                // 1..8
};

constexpr int kMfmaWaves = 8;           // waves per workgroup
constexpr int kMfmaChunk = 8;           // groups per register chunk
constexpr int kMfmaBufs = 3;            // register chunks in the ring
// LDS per (group, k-step): 1 KiB top/middle pieces, 512 B bottom pieces and
// a 16-byte zero entry (read by operand rows 8..15 in the bottom pass)
constexpr int kMfmaHalfBytes = 1024 + 512 + 16;
constexpr int kMfmaGroupBytes = 2 * kMfmaHalfBytes + 64;   // + 16 group sums

// LDS bytes of one workgroup: per group two k-steps and the sums.
__host__ __device__ constexpr size_t gemv_mfma_lds_bytes(int64_t K)
{
    return static_cast<size_t>(K / 64) * kMfmaGroupBytes;
}

typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// bf16 pair (lo in the low half) of two float32 values that are exact in
// bf16: their top halves, gathered with one byte permute.
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi)
{
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// 8 nibbles of one dword (8 consecutive inputs, even k in the low nibbles)
// -> 8 bf16 operand values: even k as the code, odd k as 16 * code.
__device__ __forceinline__ bf16x8_t nibbles_to_bf16(uint32_t d)
{
    uint32_t lo, hi;
    asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(lo) : "v"(d));
    asm("v_and_b32 %0, 0xf0f0f0f0, %1" : "=v"(hi) : "v"(d));
    uint4 v;
    v.x = bf16_pair(static_cast<float>(lo & 0xff), static_cast<float>(hi & 0xff));
    v.y = bf16_pair(static_cast<float>((lo >> 8) & 0xff), static_cast<float>((hi >> 8) & 0xff));
    v.z = bf16_pair(static_cast<float>((lo >> 16) & 0xff), static_cast<float>((hi >> 16) & 0xff));
    v.w = bf16_pair(static_cast<float>(lo >> 24), static_cast<float>(hi >> 24));
    return __builtin_bit_cast(bf16x8_t, v);
}

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

// One chunk of one lane: 8 groups of codes (8 bytes each), and the 8 scales
// and biases of its weight row.
struct MfmaChunk {
    u32x2_t c[kMfmaChunk];
    uint4 s, b;
};

__global__ __launch_bounds__(64 * kMfmaWaves) void gemv_mfma_u4_kernel(GemvMfmaParams p)
{
    extern __shared__ float4 lds_f4[];
    uint8_t *lds = reinterpret_cast<uint8_t *>(lds_f4);
    const int G = static_cast<int>(p.K / 64);
    const int C = G / kMfmaChunk;
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

    // load cursor: this lane's weight row in the tile being loaded (rows
    // past M read row M - 1; their outputs are not written)
    const uint8_t *lc_c = nullptr;
    const uint16_t *lc_s = nullptr, *lc_b = nullptr;
    int lc_chunk = 0;
    int64_t lc_tile = tb;
    auto point = [&](int64_t t) {
        const int64_t m = min(t * 16 + r, p.M - 1);
        lc_c = p.codes + m * row_bytes + 8 * q;
        lc_s = p.scales + m * G;
        lc_b = p.biases + m * G;
        lc_chunk = 0;
        lc_tile = t;
    };
    auto load = [&](MfmaChunk &k) {
#pragma unroll
        for (int j = 0; j < kMfmaChunk; ++j)
            k.c[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(lc_c + 32 * j));
        k.s = *reinterpret_cast<const uint4 *>(lc_s);
        k.b = *reinterpret_cast<const uint4 *>(lc_b);
        if (++lc_chunk == C) {
            point(lc_tile + 1);
        } else {
            lc_c += 32 * kMfmaChunk;
            lc_s += kMfmaChunk;
            lc_b += kMfmaChunk;
        }
    };

    MfmaChunk buf[kMfmaBufs];
    point(tb);
#pragma unroll
    for (int u = 0; u < kMfmaBufs - 1; ++u)
        if (u < total) load(buf[u]);

    // 1. activation pieces in operand order, zero entries, group sums.
    //    Consecutive threads read consecutive 32-byte pieces of one row.
    for (int it = tid; it < 8 * G * 8; it += blockDim.x) {
        const int n = it / (G * 8), rem = it - n * (G * 8);
        const int g = rem >> 3, qq = (rem >> 1) & 3, s = rem & 1;
        uint32_t h[4] = {0u, 0u, 0u, 0u}, md[4] = {0u, 0u, 0u, 0u}, lo[4] = {0u, 0u, 0u, 0u};
        if (n < p.nb) {
            const float4 *src = reinterpret_cast<const float4 *>(p.x + static_cast<int64_t>(n) * p.K + 8 * rem);
            const float4 a = src[0], b = src[1];
            const float v[8] = {a.x, a.y * 0.0625f, a.z, a.w * 0.0625f, b.x, b.y * 0.0625f, b.z, b.w * 0.0625f};
#pragma unroll
            for (int j = 0; j < 4; ++j) split3_pair(v[2 * j], v[2 * j + 1], h[j], md[j], lo[j]);
        }
        uint8_t *blk = lds + static_cast<size_t>(g) * kMfmaGroupBytes + s * kMfmaHalfBytes;
        *reinterpret_cast<uint4 *>(blk + (qq * 16 + n) * 16) = make_uint4(h[0], h[1], h[2], h[3]);
        *reinterpret_cast<uint4 *>(blk + (qq * 16 + 8 + n) * 16) = make_uint4(md[0], md[1], md[2], md[3]);
        *reinterpret_cast<uint4 *>(blk + 1024 + (qq * 8 + n) * 16) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        if (rem < 2 * G && n == 0)   // one thread per (group, k-step)
            *reinterpret_cast<uint4 *>(lds + static_cast<size_t>(rem >> 1) * kMfmaGroupBytes +
                                       (rem & 1) * kMfmaHalfBytes + 1536) = make_uint4(0u, 0u, 0u, 0u);
    }
    for (int it = tid; it < G * 16; it += blockDim.x) {
        const int n = it & 15, g = it >> 4;
        float sum = 0.f;
        if (n < p.nb) {
            const float4 *src = reinterpret_cast<const float4 *>(p.x + static_cast<int64_t>(n) * p.K + 64 * g);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float4 v = src[j];
                sum += (v.x + v.y) + (v.z + v.w);
            }
        }
        *reinterpret_cast<float *>(lds + static_cast<size_t>(g) * kMfmaGroupBytes + 2 * kMfmaHalfBytes + 4 * n) = sum;
    }
    __syncthreads();

    // 2. reduce the chunks
    const int hm_off = lane * 16;
    const int lo_off = r < 8 ? 1024 + (q * 8 + r) * 16 : 1536;   // rows 8..15: zero entry
    float best_v[4] = {0.f, 0.f, 0.f, 0.f};
    int64_t best_m[4] = {-1, -1, -1, -1};
    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
    int cc = 0;            // chunk within the tile being reduced
    int64_t ct = tb;       // tile being reduced

    auto reduce = [&](const MfmaChunk &k) {
        const uint8_t *gb = lds + static_cast<size_t>(cc) * kMfmaChunk * kMfmaGroupBytes;
#pragma unroll
        for (int j = 0; j < kMfmaChunk; ++j) {
            const uint8_t *b = gb + j * kMfmaGroupBytes;
            const bf16x8_t w0 = nibbles_to_bf16(k.c[j].x), w1 = nibbles_to_bf16(k.c[j].y);
            const uint4 h0 = *reinterpret_cast<const uint4 *>(b + hm_off);
            const uint4 l0 = *reinterpret_cast<const uint4 *>(b + lo_off);
            const uint4 h1 = *reinterpret_cast<const uint4 *>(b + kMfmaHalfBytes + hm_off);
            const uint4 l1 = *reinterpret_cast<const uint4 *>(b + kMfmaHalfBytes + lo_off);
            floatx4_t t = {0.f, 0.f, 0.f, 0.f};
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, h0), w0, t, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, l0), w0, t, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, h1), w1, t, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, l1), w1, t, 0, 0, 0);
            // lane (r, q) holds D rows 4q..4q+3 of column r: quarters 0, 1 the
            // top+bottom sums of activation rows 4q + i, quarters 2, 3 the
            // middle sums of rows 4(q - 2) + i (their group sums read zero)
            const float4 xs = *reinterpret_cast<const float4 *>(b + 2 * kMfmaHalfBytes + 16 * q);
            const float sc = bf16_at(k.s, j), bi = bf16_at(k.b, j);
            acc[0] = fmaf(sc, t[0], fmaf(bi, xs.x, acc[0]));
            acc[1] = fmaf(sc, t[1], fmaf(bi, xs.y, acc[1]));
            acc[2] = fmaf(sc, t[2], fmaf(bi, xs.z, acc[2]));
            acc[3] = fmaf(sc, t[3], fmaf(bi, xs.w, acc[3]));
        }
        if (++cc == C) {
            // tile done: add the middle-piece half (lane ^ 32), store
            const int64_t m = ct * 16 + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = pair_sum<5>(acc[i]);
                const int n = 4 * q + i;
                if (q < 2 && n < p.nb && m < p.M) {
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
        greedy_finish(wg_key, p.nb, p.ctl, p.idx, static_cast<int>(gridDim.x));
    }
}

}  // namespace qg
