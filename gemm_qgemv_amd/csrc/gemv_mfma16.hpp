// gemv_mfma16.hpp -- up to 16 activation rows of the 4-bit group-64 format,
// the two 8-bit formats and the 1-bit format, in one pass over the weights,
// on the gfx950 matrix cores.
//
// The 8-row kernel (gemv_mfma.hpp) stages the activation pieces of all K in
// LDS; 16 rows of them would not fit, so 9..16 rows there take two launches
// that each read the weights, and its waves each take their own tiles, which
// leaves compute units idle when M is small. Here K is cut across the
// workgroup's 8 waves instead: wave w owns groups GW w .. GW (w + 1) - 1
// (K = 512 GW) and keeps the exact bf16 pieces of all 16 activation rows
// for those inputs in registers for the whole kernel; all 8 waves stream the
// same 16-row weight tiles, each reading its part of every row, so the
// weights are read once. Per k-step a tile takes three MFMAs, one per piece
// (top, middle, bottom of the three-way split; 16 operand rows = 16
// activation rows), each group's sum is folded with its scale, and the bias
// term sum_g b[m][g] X[n][g] is added on the vector ALUs (the wave's group
// sums of the activations sit in registers). The 8 partial sums of a tile
// meet in LDS and are added in wave order after a barrier, every k16Tiles
// tiles, so the result does not depend on timing.
//
// Operand order as in gemv_mfma.hpp: lane l is operand row r = l % 16 and
// quarter q = l / 16; its 16-byte code load covers a pair of groups, and one
// permlane32 swap per dword pair gives it, at k-step s of group g, inputs
//     k = 64 g + 32 (q & 1) + 16 (q >> 1) + 8 s + {0, 2, 4, 6, 1, 3, 5, 7}.
// The same lane holds activation row r at those inputs. D: lane (r, q) holds
// weight row r of the tile for activation rows 4 q .. 4 q + 3.
//
// 8-bit codes (exact in bf16) use the same inputs in natural order: lane
// (r, q) loads the 16 bytes 64 g + 32 (q & 1) + 16 (q >> 1) of group g and
// takes its first 8 at k-step 0, the other 8 at k-step 1. The per-row scale
// multiplies the finished sum; the per-group scales (8-bit group-64) fold
// each group's sum as for the 4-bit format; there is no bias term.
//
// 1-bit signs (exactly +-1 in bf16): lane (r, q) holds inputs 32 q .. 32 q
// + 31 of each 128-input group (one 4-byte load), byte b at k-step b; the
// fp16 scale folds the group's sum.
//
// Longer K: the grid's second dimension cuts K into slices of 8 GW groups;
// each slice writes its partial outputs to p.part, and the split-K combine
// kernel adds them in slice order (matrix-vector calls only).
#pragma once

#include "gemv_mfma.hpp"

namespace qg {

constexpr int k16Tiles = 4;   // tiles between two barriers (and code loads in flight per wave)
// LDS: partial sums [2][k16Tiles][8 waves][16 x 16] floats, then staged
// outputs [tiles][16 activation rows][16 weight rows] floats
constexpr int k16RedFloats = 2 * k16Tiles * 8 * 256;
constexpr int k16TileOutBytes = 16 * 16 * 4;

__host__ __device__ constexpr size_t gemv_mfma16_lds_bytes() { return k16RedFloats * 4; }

// GW: groups of 64 inputs per wave (K = 512 GW).
template <int FMT, int GW>
__global__ __launch_bounds__(kMfmaThreads) void gemv_mfma16_kernel(GemvMfmaParams p)
{
    static_assert(kMfmaWaves == 8, "K is cut into 8 slices");
    static_assert(FMT == FMT_U4_G64 || FMT == FMT_I8_ROW || FMT == FMT_I8_G64 || FMT == FMT_B1_G128,
                  "4-bit, 8-bit or 1-bit");
    static_assert(GW % 2 == 0 || FMT == FMT_I8_ROW || FMT == FMT_I8_G64,
                  "whole pairs of groups (4-bit loads, 1-bit 128-input groups)");
    // K may be split over blockIdx.y into slices of 8 GW groups; each slice
    // writes its partial outputs to p.part
    constexpr bool U4 = FMT == FMT_U4_G64;
    constexpr bool B1 = FMT == FMT_B1_G128;
    constexpr int PAIRS = GW / 2;   // 1-bit: groups of 128 inputs per wave
    extern __shared__ float4 lds_f4[];
    float *red = reinterpret_cast<float *>(lds_f4);
    float *out_stage = red + k16RedFloats;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, q = lane >> 4;
    const int64_t row_bytes = U4 ? p.K / 2 : B1 ? p.K / 8 : p.K;
    const int64_t G = p.K / 64;
    const int gw = (static_cast<int>(blockIdx.y) * 8 + wave) * GW;   // this wave's first group
    float *const out = p.part ? p.part + static_cast<int64_t>(blockIdx.y) * p.nb * p.M : p.y;

    // the workgroup's run of 16-row tiles; every wave takes every tile
    const int64_t ntiles = (p.M + 15) / 16;
    const int64_t tb = static_cast<int64_t>(blockIdx.x) * ntiles / gridDim.x;
    const int64_t te = static_cast<int64_t>(blockIdx.x + 1) * ntiles / gridDim.x;
    const int64_t nt = te - tb;

    // 1a. this lane's activations (row r, its inputs of the wave's groups),
    //     requested before the first code loads (the memory counters count
    //     in order)
    float4 xa[GW][2][2];
#pragma unroll
    for (int gi = 0; gi < GW; ++gi)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            // 1-bit: lane q holds 32 consecutive inputs of each 128-input
            // group (one 4-byte code load), k-steps in 8-input blocks
            const int64_t k0 = B1 ? 64 * gw + 128 * (gi >> 1) + 32 * q + 16 * (gi & 1) + 8 * s
                                  : 64 * (gw + gi) + 32 * (q & 1) + 16 * (q >> 1) + 8 * s;
            xa[gi][s][0] = xa[gi][s][1] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (r < p.nb) {
                const float4 *src = reinterpret_cast<const float4 *>(p.x + r * p.K + k0);
                xa[gi][s][0] = src[0];
                xa[gi][s][1] = src[1];
            }
        }

    // code ring: tile t's codes, scales and biases of this lane's weight row
    // for the wave's groups (rows past M read row M - 1; their outputs are
    // not written). 4-bit: one 16-byte load per pair of groups, bf16 scale
    // and bias pairs; 8-bit: one per group, fp32 group scales (group-64);
    // 1-bit: 4 bytes (in .x) and the fp16 scale per 128-input group
    constexpr int NC = U4 || B1 ? PAIRS : GW;
    constexpr int NS = FMT == FMT_I8_ROW ? 1 : U4 || B1 ? PAIRS : GW;
    struct Tile16 {
        uint4 c[NC];
        uint32_t s[NS], b[U4 ? PAIRS : 1];
    };
    auto load = [&](Tile16 &T, int64_t t) {
        const int64_t m = min(t * 16 + r, p.M - 1);
        if constexpr (B1) {
            const uint8_t *c = p.codes + m * row_bytes + 8 * gw + 4 * q;
            const uint16_t *sc = p.scales + m * (p.K / 128) + gw / 2;
#pragma unroll
            for (int j = 0; j < PAIRS; ++j) {
                T.c[j].x = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(c + 16 * j));
                T.s[j] = sc[j];
            }
            return;
        }
        const uint8_t *c = p.codes + m * row_bytes + (U4 ? 32 * gw + 16 * q
                                                          : 64 * gw + 32 * (q & 1) + 16 * (q >> 1));
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(c + 64 * j));
            T.c[j] = make_uint4(v.x, v.y, v.z, v.w);
        }
        if constexpr (U4) {
            const uint32_t *sc = reinterpret_cast<const uint32_t *>(p.scales + m * G + gw);
            const uint32_t *bi = reinterpret_cast<const uint32_t *>(p.biases + m * G + gw);
#pragma unroll
            for (int pp = 0; pp < PAIRS; ++pp) {
                T.s[pp] = sc[pp];
                T.b[pp] = bi[pp];
            }
        } else if constexpr (FMT == FMT_I8_G64) {
            const uint32_t *sc = reinterpret_cast<const uint32_t *>(p.scales) + m * G + gw;
#pragma unroll
            for (int gi = 0; gi < GW; ++gi) T.s[gi] = sc[gi];
        }
    };
    constexpr int NB = k16Tiles;
    Tile16 ring[NB];
#pragma unroll
    for (int u = 0; u < NB - 1; ++u)
        if (u < nt) load(ring[u], tb + u);

    // greedy head: read the completion word as it stands at the start
    const uint32_t tag = p.ctl != nullptr ? dispatch_tag() : 0u;
    if (p.ctl != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) arrival_preclaim(&p.ctl->arrive, tag);

    // 1b. exact three-way split into operand pieces; for the 4-bit bias
    //     term the group sums X[n][g] of the activations, gathered to the
    //     lanes that hold D rows n = 4 q .. 4 q + 3
    bf16x8_t at[GW][2][3];
    float xg[U4 ? GW : 1][4];
#pragma unroll
    for (int gi = 0; gi < GW; ++gi) {
        float sum = 0.f;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const float4 a = xa[gi][s][0], b = xa[gi][s][1];
            // 4-bit operand order k = 0, 2, 4, 6, 1, 3, 5, 7; 8-bit natural
            float v[8];
            if constexpr (U4) {   // (1-bit and 8-bit: natural order)
                v[0] = a.x; v[1] = a.z; v[2] = b.x; v[3] = b.z;
                v[4] = a.y; v[5] = a.w; v[6] = b.y; v[7] = b.w;
            } else {
                v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
                v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
            }
            uint32_t hi[4], md[4], lo[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) split3_pair(v[2 * j], v[2 * j + 1], hi[j], md[j], lo[j]);
            at[gi][s][0] = __builtin_bit_cast(bf16x8_t, make_uint4(hi[0], hi[1], hi[2], hi[3]));
            at[gi][s][1] = __builtin_bit_cast(bf16x8_t, make_uint4(md[0], md[1], md[2], md[3]));
            at[gi][s][2] = __builtin_bit_cast(bf16x8_t, make_uint4(lo[0], lo[1], lo[2], lo[3]));
            if constexpr (U4) sum += ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
        }
        if constexpr (U4) {
            sum += __shfl_xor(sum, 16);
            sum += __shfl_xor(sum, 32);   // X[r][g] in every lane of row r
#pragma unroll
            for (int i = 0; i < 4; ++i) xg[gi][i] = __shfl(sum, 4 * q + i);
        }
    }

    auto mfma = [](bf16x8_t a, bf16x8_t b, floatx4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    };
    // the two k-steps of 64-input unit gi against codes w0, w1 (bf16)
    auto group = [&](int gi, bf16x8_t w0, bf16x8_t w1) {
        floatx4_t t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < 3; ++f) t = mfma(at[gi][0][f], w0, t);
#pragma unroll
        for (int f = 0; f < 3; ++f) t = mfma(at[gi][1][f], w1, t);
        return t;
    };
    // one tile's partial product over the wave's groups, into LDS slot u of
    // buffer buf
    auto reduce = [&](const Tile16 &T, int buf, int u) {
        floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (U4) {
#pragma unroll
            for (int pp = 0; pp < PAIRS; ++pp) {
                const auto s0 = __builtin_amdgcn_permlane32_swap(T.c[pp].x, T.c[pp].z, false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(T.c[pp].y, T.c[pp].w, false, false);
                const uint32_t dw[2][2] = {{s0[0], s1[0]}, {s0[1], s1[1]}};
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const floatx4_t t = group(2 * pp + h, nibbles_to_bf16(dw[h][0]), nibbles_to_bf16(dw[h][1]));
                    const float sc = h ? __uint_as_float(T.s[pp] & 0xFFFF0000u) : __uint_as_float(T.s[pp] << 16);
                    const float bv = h ? __uint_as_float(T.b[pp] & 0xFFFF0000u) : __uint_as_float(T.b[pp] << 16);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = fmaf(bv, xg[2 * pp + h][i], fmaf(sc, t[i], acc[i]));
                }
            }
        } else if constexpr (B1) {
#pragma unroll
            for (int gb = 0; gb < PAIRS; ++gb) {
                // byte b of the lane's 4 is k-step b of the group: 8 signs
                // -> 8 bf16 +-1 (the conversion takes inverted bits)
                const uint32_t nbits = ~T.c[gb].x;
                bf16x8_t w[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t nb8 = nbits >> (8 * b);
                    w[b] = __builtin_bit_cast(
                        bf16x8_t, make_uint4(signpair_to_bf16x2(nb8 & 3u), signpair_to_bf16x2((nb8 >> 2) & 3u),
                                             signpair_to_bf16x2((nb8 >> 4) & 3u),
                                             signpair_to_bf16x2((nb8 >> 6) & 3u)));
                }
                const floatx4_t t0 = group(2 * gb, w[0], w[1]), t1 = group(2 * gb + 1, w[2], w[3]);
                const float sc = fp16_bits_to_f32(static_cast<uint16_t>(T.s[gb]));
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = fmaf(sc, t0[i] + t1[i], acc[i]);
            }
        } else {
#pragma unroll
            for (int gi = 0; gi < GW; ++gi) {
                const uint4 c = T.c[gi];   // bytes 0..7: k-step 0, 8..15: k-step 1
                const bf16x8_t w0 = __builtin_bit_cast(
                    bf16x8_t, make_uint4(i8pair_to_bf16x2(c.x, 0), i8pair_to_bf16x2(c.x, 2),
                                         i8pair_to_bf16x2(c.y, 0), i8pair_to_bf16x2(c.y, 2)));
                const bf16x8_t w1 = __builtin_bit_cast(
                    bf16x8_t, make_uint4(i8pair_to_bf16x2(c.z, 0), i8pair_to_bf16x2(c.z, 2),
                                         i8pair_to_bf16x2(c.w, 0), i8pair_to_bf16x2(c.w, 2)));
                const floatx4_t t = group(gi, w0, w1);
                if constexpr (FMT == FMT_I8_G64) {
                    const float sc = __uint_as_float(T.s[gi]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = fmaf(sc, t[i], acc[i]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] += t[i];
                }
            }
        }
        float *dst = red + ((buf * NB + u) * 8 + wave) * 256;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(4 * q + i) * 16 + r] = acc[i];
    };

    // 2. after each batch of NB tiles: thread t adds the 8 partials of
    //    output (n, tile row rr) of batch slots (t >> 8) and (t >> 8) + 2 in
    //    wave order; n and rr are fixed per thread, so its rows arrive in
    //    increasing order for the greedy head
    const int sn = (tid & 255) >> 4, srr = tid & 15, su0 = tid >> 8;
    const int64_t tb_wg = tb;
    float best_v = 0.f;
    int64_t best_m = -1;
    auto finish = [&](int buf, int64_t t0) {
#pragma unroll
        for (int j = 0; j < NB / 2; ++j) {
            const int u = su0 + 2 * j;
            const int64_t tile = t0 + u;
            if (tile < te) {
                const float *src = red + (buf * NB + u) * 8 * 256 + sn * 16 + srr;
                float v = src[0];
#pragma unroll
                for (int w = 1; w < 8; ++w) v += src[w * 256];
                const int64_t m = tile * 16 + srr;
                if (sn < p.nb && m < p.M) {
                    if constexpr (FMT == FMT_I8_ROW) v *= reinterpret_cast<const float *>(p.scales)[m];
                    if (p.stage_out)
                        out_stage[((tile - tb_wg) * 16 + sn) * 16 + srr] = v;
                    else if (out)
                        out[static_cast<int64_t>(sn) * p.M + m] = v;
                    if (best_m < 0 || v > best_v) {
                        best_v = v;
                        best_m = m;
                    }
                }
            }
        }
    };

    // steady state: batches whose code loads (NB - 1 tiles ahead) all lie
    // in the run, so every load is issued unconditionally
    int buf = 0;
    int64_t t0 = 0;
    for (; t0 + 2 * NB - 1 <= nt; t0 += NB) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            load(ring[(u + NB - 1) % NB], tb + t0 + u + NB - 1);
            reduce(ring[u], buf, u);
        }
        __syncthreads();
        finish(buf, tb + t0);
        buf ^= 1;
    }
    // drain: fewer than 2 NB - 1 tiles left (uniform conditions)
    for (; t0 < nt; t0 += NB) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            if (t0 + u < nt) {
                if (t0 + u + NB - 1 < nt) load(ring[(u + NB - 1) % NB], tb + t0 + u + NB - 1);
                reduce(ring[u], buf, u);
            }
        }
        __syncthreads();
        finish(buf, tb + t0);
        buf ^= 1;
    }

    if (p.stage_out && out) {
        __syncthreads();
        const int64_t m0 = tb * 16, rows = min(te * 16, p.M) - m0;
        for (int n = 0; n < p.nb; ++n)
            for (int64_t j = tid; j < rows; j += blockDim.x)
                out[static_cast<int64_t>(n) * p.M + m0 + j] = out_stage[((j >> 4) * 16 + n) * 16 + (j & 15)];
    }

    if (p.ctl != nullptr) {
        __shared__ unsigned long long wg_key[16];
        if (tid < 16) wg_key[tid] = 0ull;
        __syncthreads();
        uint64_t key = best_m >= 0 ? argmax_key(best_v, static_cast<uint32_t>(best_m)) : 0ull;
        // the 16 lanes srr = 0..15 of a 16-lane group share n
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) {
            const uint64_t other = shfl_xor_u64(key, o);
            key = other > key ? other : key;
        }
        if (srr == 0 && sn < p.nb) atomicMax(&wg_key[sn], static_cast<unsigned long long>(key));
        __syncthreads();
        greedy_finish_rows(wg_key, p.nb, p.ctl, p.keys, p.idx, static_cast<int>(gridDim.x), tag);
    }
}

}  // namespace qg
