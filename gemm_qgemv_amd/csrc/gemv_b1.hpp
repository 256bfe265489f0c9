// gemv_b1.hpp -- batch-1 matrix-vector kernel for the 1-bit sign format,
// by table lookup.
//
// For every 4 consecutive inputs k = 4q .. 4q+3 a 16-entry table holds
//     T_q[n] = sum_{i<4} (bit i of n ? +x[4q+i] : -x[4q+i]),
// so one nibble of sign bits selects the signed sum of its 4 activations in a
// single LDS read, and a row's output is sum_g scale[g] * sum_{q in g}
// T_q[nibble_q] (A 27B model on two 4GB Maxwell GPUs, "A packed Q1 prefill
// kernel with a narrow dispatch window": the weights stay packed and
// LUT-based products over low-bit weights are the related method).
//
// Mapping. A workgroup covers 64 rows (one row per lane) and one chunk of KC
// inputs; its 4 waves split the chunk four ways, so all four run the same
// rows over different quarters of the tables, and their partial sums meet
// in LDS. The chunk's tables (KC/4 positions x 16 floats = 16 KiB for
// KC = 1024) are built once by the workgroup. At any instant the 64 lanes
// of a wave read the same 64-byte table (same position, different rows), so
// every lookup is served without bank conflicts (same-address lanes are
// broadcast, distinct entries sit in distinct banks). The tile's codes are
// read with coalesced 16-byte loads (8 consecutive threads per 128-byte row
// segment), issued before the tables are built, and passed through padded
// LDS rows to the lane that owns the row. Small 64-row tiles give many
// workgroups (several per compute unit at once), which spreads the lookups
// evenly over the SIMDs and lets one workgroup's lookups overlap another's
// loads. Chunks of K go to different workgroups; their partial sums are
// combined in split order by the last workgroup of each row tile
// (splitk_arrive), or by gemv_combine_kernel when there are more row tiles
// than completion words.
#pragma once

#include "gemv.hpp"

namespace qg {

// Rows per workgroup of the lookup kernel (one per lane of each wave).
constexpr int kB1Rows = 64;

struct B1LutParams {
    const uint8_t *codes;
    const uint16_t *scales;
    const float *x;       // [nb][K]
    float *y;             // [nb][M] (one chunk)
    float *part;          // [nsplit][nb][M] (several chunks)
    GreedyCtl *ctl;       // control words (greedy head, split-K tile counters)
    unsigned long long *keys;  // greedy keys [row tiles][nb] in the workspace
    int32_t *idx;         // greedy index output, or nullptr
    int64_t M, K;
    int nb;               // activation rows of this launch (x [nb][K], y [nb][M])
    int nsplit;
    int fused;            // several chunks: combine in this kernel (else partials only)
};

// n-th nibble (0..7) of a dword, times 4: the byte offset of entry n of a
// 16-float table. The masks go through opaque instructions so that the
// byte extraction stays a single byte-select operation per nibble.
__device__ __forceinline__ void nibble_offsets(uint32_t d, uint32_t &lo4, uint32_t &hi4)
{
    uint32_t t;
    asm("v_lshlrev_b32 %0, 2, %1" : "=v"(t) : "v"(d));
    asm("v_and_b32 %0, 0x3c3c3c3c, %1" : "=v"(lo4) : "v"(t));   // low nibble of byte i, x4
    asm("v_lshrrev_b32 %0, 2, %1" : "=v"(t) : "v"(d));
    asm("v_and_b32 %0, 0x3c3c3c3c, %1" : "=v"(hi4) : "v"(t));   // high nibble of byte i, x4
}

// KC inputs per chunk; NB activation rows per launch, each with its own
// tables (the launch's nb <= NB rows; rows nb .. NB-1 repeat row nb - 1 and
// their results are dropped, so every loop has a fixed trip count and no
// load or lookup sits behind a branch). A lane's lookups for the NB rows
// share the nibble offsets.
template <int KC, int NB>
__global__ __launch_bounds__(256) void gemv_b1_lut_kernel(B1LutParams p)
{
    constexpr int NG = KC / 128;          // 16-byte groups per row and chunk
    constexpr int GPW = NG / 4;           // groups per wave
    constexpr int NQ = KC / 4;            // nibble positions per chunk
    constexpr int ROWS = kB1Rows;
    constexpr int CROW = 16 * NG + 16;    // padded LDS row of codes (bytes)
    constexpr int NLD = ROWS * NG / 256;  // 16-byte code loads per thread
    static_assert(NG % 4 == 0 && NLD >= 1 && ROWS * NG % 256 == 0, "chunk shape");
    __shared__ __attribute__((aligned(16))) float lut[NB][NQ * 16];
    __shared__ __attribute__((aligned(16))) uint8_t codes_l[ROWS * CROW];
    __shared__ float red[4][NB][ROWS];

    const int split = blockIdx.y;
    const int64_t k0 = static_cast<int64_t>(split) * KC;
    const int ng = static_cast<int>(min(static_cast<int64_t>(NG), (p.K - k0) / 128));
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nb = NB == 1 ? 1 : p.nb;
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * ROWS;
    const int64_t m = row0 + lane;
    const bool mv = m < p.M;
    const int64_t row_bytes = p.K / 8;
    const int64_t groups = p.K / 128;

    // 1. request the tile's codes, coalesced: 8 consecutive threads read one
    //    row's 128 contiguous bytes; also the scales of this wave's groups
    uint4 st[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int ci = tid + 256 * i, r = ci / NG, g = ci % NG;
        const bool v = row0 + r < p.M && g < ng;
        st[i] = v ? *reinterpret_cast<const uint4 *>(p.codes + (row0 + r) * row_bytes + k0 / 8 + 16 * g)
                  : make_uint4(0, 0, 0, 0);
    }
    uint32_t sc[GPW];
    const uint16_t *sp = p.scales + (mv ? m : 0) * groups + k0 / 128 + wave * GPW;
#pragma unroll
    for (int j = 0; j < GPW; ++j) sc[j] = (mv && wave * GPW + j < ng) ? sp[j] : 0u;

    // tag of this dispatch for the completion words it counts on: the row
    // tile's (in-kernel split-K combine) and the greedy head's
    const bool fused_split = p.nsplit > 1 && p.fused;
    const uint32_t tag = (fused_split || p.idx != nullptr) ? dispatch_tag() : 0u;
    if (tid == 0 && split == 0) {
        if (fused_split) arrival_preclaim(&tile_counters(p.ctl)[blockIdx.x], tag);
        if (p.idx != nullptr && blockIdx.x == 0) arrival_preclaim(&p.ctl->arrive, tag);
    }

    // 2. tables of this chunk: thread q builds position q (16 signed sums)
    //    for every activation row (all rows' activations requested first)
    for (int q = tid; q < NQ; q += blockDim.x) {
        if (q < 32 * ng) {
            float4 xr[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b)
                xr[b] = *reinterpret_cast<const float4 *>(p.x + min(b, nb - 1) * p.K + k0 + 4 * q);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                {
                    const float4 xv = xr[b];
                    float t[16];
                    t[0] = -((xv.x + xv.y) + (xv.z + xv.w));
                    const float d0 = 2.f * xv.x, d1 = 2.f * xv.y, d2 = 2.f * xv.z, d3 = 2.f * xv.w;
#pragma unroll
                    for (int n = 1; n < 16; ++n) {
                        // add 2x_i for the lowest set bit i of n to the entry without it
                        const int i = __builtin_ctz(n);
                        const float di = i == 0 ? d0 : i == 1 ? d1 : i == 2 ? d2 : d3;
                        t[n] = t[n & (n - 1)] + di;
                    }
                    float4 *dst = reinterpret_cast<float4 *>(lut[b] + 16 * q);
                    dst[0] = make_float4(t[0], t[1], t[2], t[3]);
                    dst[1] = make_float4(t[4], t[5], t[6], t[7]);
                    dst[2] = make_float4(t[8], t[9], t[10], t[11]);
                    dst[3] = make_float4(t[12], t[13], t[14], t[15]);
                }
            }
        }
    }
    // 3. codes into LDS rows (padded: one lane per row reads conflict-free)
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int ci = tid + 256 * i, r = ci / NG, g = ci % NG;
        *reinterpret_cast<uint4 *>(codes_l + r * CROW + 16 * g) = st[i];
    }
    __syncthreads();

    // 4. lookups: this lane's row, this wave's groups, every activation row
    float acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.f;
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
        const int g = wave * GPW + j;
        if (g < ng) {
            const uint4 cg = *reinterpret_cast<const uint4 *>(codes_l + lane * CROW + 16 * g);
            const uint32_t dw[4] = {cg.x, cg.y, cg.z, cg.w};
            const float scale = fp16_bits_to_f32(static_cast<uint16_t>(sc[j]));
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                {
                    const char *lb = reinterpret_cast<const char *>(lut[b]);
                    // two batches of 16 independent lookups (the LDS counter
                    // tracks at most 15 in flight), each summed as a tree
                    float half[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        float v[16];
#pragma unroll
                        for (int jj = 0; jj < 2; ++jj) {
                            const int d = 2 * h + jj;
                            uint32_t lo4, hi4;
                            nibble_offsets(dw[d], lo4, hi4);
#pragma unroll
                            for (int bb = 0; bb < 4; ++bb) {
                                const int q = 32 * g + 8 * d + 2 * bb;   // position of the low nibble of byte bb
                                const uint32_t ol = (lo4 >> (8 * bb)) & 0xffu;
                                const uint32_t oh = (hi4 >> (8 * bb)) & 0xffu;
                                v[8 * jj + 2 * bb] = *reinterpret_cast<const float *>(lb + 64 * q + ol);
                                v[8 * jj + 2 * bb + 1] = *reinterpret_cast<const float *>(lb + 64 * (q + 1) + oh);
                            }
                        }
#pragma unroll
                        for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
                            for (int i = 0; i < w; ++i) v[i] += v[i + w];
                        half[h] = v[0];
                    }
                    acc[b] = fmaf(scale, half[0] + half[1], acc[b]);
                }
            }
        }
    }
    // the four quarters of the chunk, summed in wave order
#pragma unroll
    for (int b = 0; b < NB; ++b) red[wave][b][lane] = acc[b];
    __syncthreads();
#pragma unroll
    for (int b = 0; b < NB; ++b)
        acc[b] = wave != 0 ? 0.f
                           : ((red[0][b][lane] + red[1][b][lane]) + red[2][b][lane]) + red[3][b][lane];
    // only wave 0 carries the rows from here; the others still take part in
    // the workgroup-wide steps below
    const bool own = wave == 0 && mv;

    // 5. several chunks: fused combine, finished by the tile's last workgroup
    //    (partials [split][activation row][M])
    if (p.nsplit > 1) {
        float *part = p.part + static_cast<int64_t>(split) * nb * p.M + m;
        if (p.fused) {
            if (own)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    if (b < nb) splitk_put(part + b * p.M, acc[b]);
            if (!splitk_arrive(&tile_counters(p.ctl)[blockIdx.x], p.nsplit, tag)) return;
#pragma unroll
            for (int b = 0; b < NB; ++b)
                acc[b] = own && b < nb ? splitk_sum(p.part + b * p.M + m, nb * p.M, p.nsplit) : 0.f;
        } else {
            if (own)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    if (b < nb) part[b * p.M] = acc[b];
            return;
        }
    }
    if (own && p.y)
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (b < nb) p.y[b * p.M + m] = acc[b];
    if (p.idx != nullptr) {
        __shared__ unsigned long long s_key[NB];
        if (tid < NB) s_key[tid] = 0ull;
        __syncthreads();
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            uint64_t key = own && b < nb ? argmax_key(acc[b], static_cast<uint32_t>(m)) : 0ull;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const uint64_t other = shfl_xor_u64(key, o);
                key = other > key ? other : key;
            }
            if (lane == 0) atomicMax(&s_key[b], static_cast<unsigned long long>(key));
        }
        __syncthreads();
        greedy_finish_rows(s_key, nb, p.ctl, p.keys, p.idx, static_cast<int>(gridDim.x), tag);
    }
}

}  // namespace qg
