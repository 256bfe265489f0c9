// gemv_stream_mfma.hpp -- 2..8 activation rows against large 4-bit group-64
// matrices with K = 2048 (the greedy head of a decode step over a few
// sequences), with the weights streamed through LDS by loader waves and
// reduced on the matrix cores.
//
// Why. Batching several sequences lets them share one pass over the weights
// (Pushing the limits of legacy hardware, "Build the execution path, then
// share the weights"), so the pass should still run at the weight stream's
// speed. Per weight byte the contraction does 2 nb multiply-adds, which the
// matrix cores take; the limit is then how many weight bytes each compute
// unit keeps in flight. Loader waves with LDS-direct loads keep several
// 36 KiB stages in flight independently of the arithmetic, as in the
// batch-1 stream kernel (gemv_stream.hpp), whose ring, loaders and stage
// protocol this kernel shares.
//
// Contraction. As in the register-streaming small-batch kernel
// (gemv_mfma.hpp): v_mfma_f32_16x16x32_bf16 with operand A = activation
// pieces and operand B = 16 weight rows of bf16 codes (0..15, exact), but
// with the pieces of one activation row in adjacent operand rows: row 2n
// holds the top bf16 piece of activation row n, row 2n + 1 its middle
// piece, and a second MFMA gives both rows half the bottom piece, so that
// D[2n] + D[2n + 1] restores the float32 product exactly and is added in
// the lane that holds both (no lane exchange). The scale of a 64-input
// group multiplies the group's MFMA result in float32; the bias term
// sum_g bias[m][g] X[n][g] (X: group sums of the activations, split in
// three pieces like x) is one more pair of MFMAs per tile.
//
// Mapping. Compute wave c owns inputs 256 c .. 256 c + 255 (groups 4c ..
// 4c + 3) of every row; its activation pieces for those inputs stay in
// registers for the whole kernel. Lane (r, q) = (l % 16, l / 16) feeds
// weight row r of the 16-row tile and, for group g, inputs
//     k = 64 g + 16 q + 8 t + {0, 2, 4, 6, 1, 3, 5, 7}    (k-step t = 0, 1)
// (the last term: even-k nibbles first, as the conversion produces them),
// i.e. bytes 32 g + 8 q .. + 7 of the row, one 8-byte LDS read per group.
// The loaders store code row rr with its 16-byte chunks XOR-swizzled by
// rr % 16, so the 16 rows of a tile read 16 different bank groups. A stage
// (32 rows, two tiles) ends with every wave's partial sums of its inputs in
// LDS ([wave][row][activation row], two buffers used in turn); after the
// barrier that opens the next stage, each wave first reads that stage's
// codes and coefficients (both tiles), computes its share of it, and then
// wave n adds the eight partials of activation row n of the previous stage,
// in wave order, writes the 32 outputs and keeps its greedy best. So one
// barrier per stage suffices, and the ring, the two partial buffers and nothing
// else fill the 160 KiB of LDS (the greedy epilogue's scratch reuses the
// ring once the last stage is done).
#pragma once

#include "gemv_mfma.hpp"
#include "gemv_stream.hpp"

namespace qg {

constexpr int kStreamMfmaK = 2048;                 // inputs per row
constexpr int kStreamMfmaRows = 8;                  // activation rows per launch
// partial sums of one stage: [compute wave][32 rows][8 activation rows]
constexpr int kStreamMfmaPartBytes = kStreamComputes * 32 * kStreamMfmaRows * 4;
constexpr int kStreamMfmaLdsBytes = kStreamLdsBytes + 2 * kStreamMfmaPartBytes;   // 160 KiB

struct GemvStreamMfmaParams {
    const uint8_t *codes;
    const uint16_t *scales;
    const uint16_t *biases;
    const float *x;       // [nb][K]
    float *y;             // [nb][M], or nullptr (greedy head without logits)
    GreedyCtl *ctl;       // greedy head control words, or nullptr
    unsigned long long *keys;   // greedy keys, [workgroups][nb]
    int32_t *idx;         // [nb]
    int64_t M;
    int nb;               // 1..8
};

__global__ __launch_bounds__(kStreamThreads) void gemv_stream_mfma_u4_kernel(GemvStreamMfmaParams p)
{
    constexpr int K = kStreamMfmaK;
    constexpr int RS = 32;                          // rows per stage
    constexpr int G = K / 64;                       // groups per row
    static_assert(kStreamComputes * 4 == G, "four groups per compute wave");
    static_assert(RS * G * 2 == kStreamCoefBytes, "one coefficient block per stage");
    extern __shared__ __attribute__((aligned(16))) unsigned char stream_lds[];
    float *const part0 = reinterpret_cast<float *>(stream_lds + kStreamLdsBytes);
    // greedy epilogue scratch, in the ring once the stages are done
    unsigned long long *const s_wkey = reinterpret_cast<unsigned long long *>(stream_lds);
    unsigned long long *const s_best = s_wkey + kStreamMfmaRows;
    unsigned *const s_last = reinterpret_cast<unsigned *>(s_best + 16);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * p.M / gridDim.x;
    const int64_t r1 = static_cast<int64_t>(blockIdx.x + 1) * p.M / gridDim.x;
    const int nstages = static_cast<int>((r1 - r0 + RS - 1) / RS);

    const uint32_t tag = p.ctl != nullptr ? dispatch_tag() : 0u;

    // the loader waves come last: a SIMD gives its oldest waves the first
    // issue slots, and in this kernel the compute waves bound each stage
    // (with the loaders first, as in the batch-1 kernel, the stages of the
    // two SIMDs that host a loader take longest)
    if (wave >= kStreamComputes) {
        stream_loader<1, true, 1>(p.codes, p.scales, p.biases, stream_lds, wave - kStreamComputes, lane, r0, r1,
                                  nstages);
        stream_barrier();   // the compute waves' last reduction
    } else {
        const int c = wave;
        const int r = lane & 15, q = lane >> 4;
        const int n = r >> 1;   // activation row of operand row r (top piece in even rows)

        // 1. activation pieces of this wave's inputs, in operand order, and
        //    the pieces of their group sums (operand A of the bias MFMAs:
        //    group u of this wave at k position u of quarter 0)
        uint4 a_hm[4][2], a_lo[4][2];
        float xs[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float sum = 0.f;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int k0 = 64 * (4 * c + u) + 16 * q + 8 * t;
                float4 va = make_float4(0.f, 0.f, 0.f, 0.f), vb = va;
                if (n < p.nb) {
                    const float4 *src = reinterpret_cast<const float4 *>(p.x + static_cast<int64_t>(n) * K + k0);
                    va = src[0];
                    vb = src[1];
                }
                sum += ((va.x + va.y) + (va.z + va.w)) + ((vb.x + vb.y) + (vb.z + vb.w));
                const float v[8] = {va.x, va.z, vb.x, vb.z, va.y, va.w, vb.y, vb.w};
                uint32_t h[4], md[4], lo[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) split3h_pair(v[2 * j], v[2 * j + 1], h[j], md[j], lo[j]);
                a_hm[u][t] = (r & 1) == 0 ? make_uint4(h[0], h[1], h[2], h[3]) : make_uint4(md[0], md[1], md[2], md[3]);
                a_lo[u][t] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
            }
            // the four quarters hold the group's 64 inputs
            sum += lane_xor_f32(sum, 16);
            sum += lane_xor_f32(sum, 32);
            xs[u] = sum;
        }
        // the dispatch's first workgroup claims the completion word
        if (p.ctl != nullptr && blockIdx.x == 0 && lane == 0 && c == 0) arrival_preclaim(&p.ctl->arrive, tag);
        uint32_t bh[4], bm[4], bl[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) split3h(xs[u], bh[u], bm[u], bl[u]);
        uint4 ab_hm = make_uint4(0u, 0u, 0u, 0u), ab_lo = ab_hm;
        if (q == 0) {
            ab_hm = (r & 1) == 0 ? make_uint4(bh[0] | (bh[1] << 16), bh[2] | (bh[3] << 16), 0u, 0u)
                          : make_uint4(bm[0] | (bm[1] << 16), bm[2] | (bm[3] << 16), 0u, 0u);
            ab_lo = make_uint4(bl[0] | (bl[1] << 16), bl[2] | (bl[3] << 16), 0u, 0u);
        }

        auto mfma = [](uint4 a, bf16x8_t b, floatx4_t acc) {
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), b, acc, 0, 0, 0);
        };
        float best_v = 0.f;
        int64_t best_m = -1;
        // wave c adds the partials of activation row c for the 32 rows of
        // stage st, in wave order
        auto reduce = [&](int st) {
            if (c < p.nb && lane < 32) {
                const float *part = part0 + (st & 1) * (kStreamMfmaPartBytes / 4);
                float sum = 0.f;
#pragma unroll
                for (int w = 0; w < kStreamComputes; ++w) sum += part[(w * 32 + lane) * kStreamMfmaRows + c];
                const int64_t m = r0 + static_cast<int64_t>(st) * RS + lane;
                if (m < r1) {
                    if (p.y) p.y[static_cast<int64_t>(c) * p.M + m] = sum;
                    if (best_m < 0 || sum > best_v) {   // this lane's rows arrive in increasing order
                        best_v = sum;
                        best_m = m;
                    }
                }
            }
        };

        // 2. the stages
        for (int s = 0; s < nstages; ++s) {
            // after this barrier: stage s has landed, and every wave is done
            // with stage s - 1 (its slot, and the partial buffer of stage s - 2)
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            stream_barrier();
            const unsigned char *slot = stream_lds + (s % kStreamStages) * kStreamStageBytes;
            float *part = part0 + (s & 1) * (kStreamMfmaPartBytes / 4);
            // every LDS read of the stage first (both tiles), so that the
            // second tile's codes arrive while the first tile is reduced
            uint2 cw[2][4], sv[2], bv[2];
#pragma unroll
            for (int tile = 0; tile < 2; ++tile) {
                const int row = 16 * tile + r;
                const unsigned char *crow = slot + row * 1024;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int chunk = (2 * (4 * c + u) + (q >> 1)) ^ r;   // row % 16 == r
                    cw[tile][u] = *reinterpret_cast<const uint2 *>(crow + 16 * chunk + 8 * (q & 1));
                }
                sv[tile] = *reinterpret_cast<const uint2 *>(slot + kStreamCodeBytes + row * 2 * G + 8 * c);
                bv[tile] = *reinterpret_cast<const uint2 *>(slot + kStreamCodeBytes + kStreamCoefBytes +
                                                            row * 2 * G + 8 * c);
            }
            float v[2][2];
#pragma unroll
            for (int tile = 0; tile < 2; ++tile) {
                // the bias term (operand B: this row's four biases at k
                // positions 0..3 of quarter 0) on the accumulator, then the
                // four groups as four independent MFMA chains issued in turn,
                // so that no MFMA waits for the one before it
                const uint4 bb = q == 0 ? make_uint4(bv[tile].x, bv[tile].y, 0u, 0u) : make_uint4(0u, 0u, 0u, 0u);
                const floatx4_t zero = {0.f, 0.f, 0.f, 0.f};
                floatx4_t acc = mfma(ab_hm, __builtin_bit_cast(bf16x8_t, bb), zero);
                acc = mfma(ab_lo, __builtin_bit_cast(bf16x8_t, bb), acc);
                bf16x8_t w[4][2];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    w[u][0] = nibbles_to_bf16(cw[tile][u].x);
                    w[u][1] = nibbles_to_bf16(cw[tile][u].y);
                }
                floatx4_t t[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) t[u] = mfma(a_hm[u][0], w[u][0], zero);
#pragma unroll
                for (int u = 0; u < 4; ++u) t[u] = mfma(a_lo[u][0], w[u][0], t[u]);
#pragma unroll
                for (int u = 0; u < 4; ++u) t[u] = mfma(a_hm[u][1], w[u][1], t[u]);
#pragma unroll
                for (int u = 0; u < 4; ++u) t[u] = mfma(a_lo[u][1], w[u][1], t[u]);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t sw = (u < 2) ? sv[tile].x : sv[tile].y;
                    const float sc = (u & 1) ? __uint_as_float(sw & 0xFFFF0000u) : __uint_as_float(sw << 16);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = fmaf(sc, t[u][i], acc[i]);
                }
                // lane (r, q) holds D rows 4q .. 4q + 3 of weight row r:
                // the two pieces of activation rows 2q and 2q + 1
                v[tile][0] = acc[0] + acc[1];
                v[tile][1] = acc[2] + acc[3];
            }
#pragma unroll
            for (int tile = 0; tile < 2; ++tile)
                *reinterpret_cast<float2 *>(part + ((c * 32 + 16 * tile + r) * kStreamMfmaRows + 2 * q)) =
                    make_float2(v[tile][0], v[tile][1]);
            if (s > 0) reduce(s - 1);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        stream_barrier();
        if (nstages > 0) reduce(nstages - 1);
        if (p.ctl != nullptr && c < p.nb) {
            const uint64_t key = wave_max_u64(best_m >= 0 ? argmax_key(best_v, static_cast<uint32_t>(best_m)) : 0ull);
            if (lane == 0) s_wkey[c] = key;
        }
    }

    if (p.ctl != nullptr) {
        __syncthreads();
        greedy_finish_rows_in(s_wkey, p.nb, p.ctl, p.keys, p.idx, static_cast<int>(gridDim.x), tag, s_last, s_best);
    }
}

}  // namespace qg
