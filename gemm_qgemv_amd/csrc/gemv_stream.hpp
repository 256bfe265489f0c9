// gemv_stream.hpp -- batch-1 matrix-vector kernel for the 4-bit format on
// large matrices, with the weight stream driven by dedicated loader waves.
//
// Why. At batch 1 every weight byte is used once, so the kernel is a
// stream (MiniCPM-V-4.6 on a Tesla C2075, section 3.3: decode is bound by
// the weight bytes). A wave that both loads and computes can keep only as
// many bytes in flight as its registers hold, and its loads wait behind its
// own arithmetic. Here the loads go straight from memory into LDS (gfx950's
// LDS-direct loads, 1 KiB per wave instruction, no registers involved), so
// two loader waves keep whole stages of the matrix in flight while eight
// compute waves reduce the stage that has landed.
//
// Mapping. One workgroup per compute unit (the grid is the chip), each a
// contiguous run of rows, cut into stages of 32 KiB of codes (32 / NC rows
// of K = 2048 NC inputs) plus the stage's bf16 scales and biases (2 KiB
// each). A ring of kStreamStages stages lives in LDS. Loader wave L issues
// half of each stage's code rows and one of its two coefficient blocks;
// before the barrier that opens stage s it waits (vector-memory count) until
// only the later stages' loads are outstanding, and after that barrier it
// refills the slot freed by stage s - 1. Compute wave c takes rows
// c RPW .. c RPW + RPW - 1 of every stage: lane l reads its 16-byte slices
// t = l + 64 j of each row (conflict-free LDS reads) and reduces them against
// its activations, kept in registers for the whole kernel, exactly as the
// register-streaming batch-1 kernel does (gemv1.hpp). Rows past the
// workgroup's run are loaded as copies of its last row (every stage issues
// the same number of loads, which keeps the counts exact) and not written.
//
// Greedy head: each writer lane keeps its best (value, index); the
// workgroup reduces them to one key, parks it, and the last workgroup writes
// the index (greedy_finish_rows).
#pragma once

#include "gemv1.hpp"

namespace qg {

typedef const __attribute__((address_space(1))) void *stream_gptr_t;
typedef __attribute__((address_space(3))) void *stream_lptr_t;

constexpr int kStreamLoaders = 2;                 // loader waves per workgroup
constexpr int kStreamComputes = 8;                // compute waves per workgroup
constexpr int kStreamThreads = 64 * (kStreamLoaders + kStreamComputes);
constexpr int kStreamStages = 4;                  // stages in the LDS ring
constexpr int kStreamCodeBytes = 32768;           // codes per stage
constexpr int kStreamCoefBytes = 2048;            // scales (or biases) per stage
constexpr int kStreamStageBytes = kStreamCodeBytes + 2 * kStreamCoefBytes;
constexpr int kStreamLdsBytes = kStreamStages * kStreamStageBytes;   // 144 KiB

struct GemvStreamParams {
    const uint8_t *codes;
    const uint16_t *scales;
    const uint16_t *biases;
    const float *x;       // [K]
    float *y;             // [M], or nullptr (greedy head without logits)
    GreedyCtl *ctl;       // greedy head control words, or nullptr
    unsigned long long *keys;  // greedy keys, one per workgroup
    int32_t *idx;
    int64_t M;
    int64_t K;
};

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt and lgkmcnt at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier that orders no memory by itself: the LDS-direct data is
// ordered by the loaders' vector-memory waits before it, and the compute
// waves' LDS reads are complete before it because their values have been
// used. The memory clobber keeps the compiler from moving LDS accesses or
// loads across it.
__device__ __forceinline__ void stream_barrier()
{
    asm volatile("s_barrier" ::: "memory");
}

// One loader wave's part of stage st (ring slot st % kStreamStages): code
// rows RS = 32 / NC (rows past r1 - 1 repeat row r1 - 1, so every stage
// issues the same number of loads) and one coefficient block (loader 0: the
// scales, loader 1: the biases), 1 KiB per instruction. With SWZ, lane l of
// the load of code row rr fetches the row's 16-byte chunk l ^ (rr % 16), so
// that chunk c of row rr sits at position c ^ (rr % 16) of its LDS row.
template <int NC, bool SWZ>
__device__ __forceinline__ void stream_issue(const uint8_t *codes, const uint16_t *scales,
                                             const uint16_t *biases, unsigned char *lds, int L,
                                             int lane, int st, int64_t r0, int64_t r1)
{
    constexpr int RS = 32 / NC;
    constexpr int GPR = 32 * NC;
    constexpr int CODE_LOADS = RS * NC / kStreamLoaders;
    constexpr int64_t row_bytes = 1024 * NC;
    constexpr int coef_row_bytes = 2 * GPR;
    unsigned char *slot = lds + (st % kStreamStages) * kStreamStageBytes;
    const int64_t rb = r0 + static_cast<int64_t>(st) * RS;
#pragma unroll
    for (int i = 0; i < CODE_LOADS; ++i) {
        const int li = L * CODE_LOADS + i;
        const int rr = li / NC, cc = li % NC;
        const int64_t row = min(rb + rr, r1 - 1);
        const int chunk = SWZ ? (lane ^ (rr & 15)) : lane;
        const uint8_t *g = codes + row * row_bytes + cc * 1024 + 16 * chunk;
        __builtin_amdgcn_global_load_lds((stream_gptr_t)g, (stream_lptr_t)(slot + (rr * NC + cc) * 1024), 16, 0, 2);
    }
    // the stage's coefficients: 2 KiB of consecutive rows, 16 bytes per lane
    const uint16_t *coef = L == 0 ? scales : biases;
    unsigned char *cslot = slot + kStreamCodeBytes + L * kStreamCoefBytes;
#pragma unroll
    for (int i = 0; i < kStreamCoefBytes / 1024; ++i) {
        const int off = 1024 * i + 16 * lane;   // byte within the stage's block
        const int rr = off / coef_row_bytes;
        const int64_t row = min(rb + rr, r1 - 1);
        const int64_t src = row * coef_row_bytes + off % coef_row_bytes;
        __builtin_amdgcn_global_load_lds((stream_gptr_t)(reinterpret_cast<const uint8_t *>(coef) + src),
                                         (stream_lptr_t)(cslot + 1024 * i), 16, 0, 2);
    }
}

// A loader wave's whole life: fill the ring, then for every stage s wait
// (vector-memory count) until only the later stages' loads are outstanding,
// take the barrier that opens stage s, refill the slot that stage s - 1
// freed, and take the BARRIERS - 1 further barriers the compute waves take
// per stage.
template <int NC, bool SWZ, int BARRIERS>
__device__ __forceinline__ void stream_loader(const uint8_t *codes, const uint16_t *scales,
                                              const uint16_t *biases, unsigned char *lds, int L,
                                              int lane, int64_t r0, int64_t r1, int nstages)
{
    constexpr int RS = 32 / NC;
    constexpr int CODE_LOADS = RS * NC / kStreamLoaders;
    constexpr int LPS = CODE_LOADS + kStreamCoefBytes / 1024;   // loads per loader and stage
    constexpr int D = kStreamStages;
    static_assert((D - 2) * LPS < 64, "outstanding loads fit the vector-memory count");
    for (int st = 0; st < D - 1 && st < nstages; ++st)
        stream_issue<NC, SWZ>(codes, scales, biases, lds, L, lane, st, r0, r1);
    for (int s = 0; s < nstages; ++s) {
        // stage s has landed once only the later stages' loads are outstanding
        const int later = min(D - 2, nstages - 1 - s);
        if (later >= 2) wait_vmcnt<2 * LPS>();
        else if (later == 1) wait_vmcnt<LPS>();
        else wait_vmcnt<0>();
        stream_barrier();
        if (s + D - 1 < nstages) stream_issue<NC, SWZ>(codes, scales, biases, lds, L, lane, s + D - 1, r0, r1);
#pragma unroll
        for (int b = 1; b < BARRIERS; ++b) stream_barrier();
    }
}

// NC: 1 KiB chunks of codes per row (K = 2048 NC).
template <int NC>
__global__ __launch_bounds__(kStreamThreads) void gemv_stream_u4_kernel(GemvStreamParams p)
{
    constexpr int RS = 32 / NC;                    // rows per stage
    constexpr int RPW = RS / kStreamComputes;      // rows per compute wave and stage
    constexpr int GPR = 32 * NC;                   // groups of 64 inputs per row
    constexpr int D = kStreamStages;
    static_assert(RPW >= 1 && RS * NC == 32, "32 KiB of codes per stage");
    static_assert(RS * GPR * 2 == kStreamCoefBytes, "one coefficient block per stage");
    extern __shared__ __attribute__((aligned(16))) unsigned char stream_lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * p.M / gridDim.x;
    const int64_t r1 = static_cast<int64_t>(blockIdx.x + 1) * p.M / gridDim.x;
    const int nstages = static_cast<int>((r1 - r0 + RS - 1) / RS);

    const uint32_t tag = p.ctl != nullptr ? dispatch_tag() : 0u;
    __shared__ unsigned long long s_key;   // the workgroup's greedy key
    if (tid == 0) {
        s_key = 0ull;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // done before this wave's first barrier
    }

    float best_v = 0.f;
    int64_t best_m = -1;
    bool writer = false;

    if (wave < kStreamLoaders) {
        stream_loader<NC, false, 1>(p.codes, p.scales, p.biases, stream_lds, wave, lane, r0, r1, nstages);
    } else {
        // ---- compute wave ---------------------------------------------
        const int c = wave - kStreamLoaders;
        const int own = dpp_owner<RPW>(lane);
        writer = dpp_writer<RPW>(lane);

        // this lane's activations of slices t = lane + 64 j (odd k
        // pre-divided by 16) and their sums
        float4 xv[NC][8];
        float xs[NC];
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const float4 *src = reinterpret_cast<const float4 *>(p.x + static_cast<int64_t>(lane + 64 * j) * 32);
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                float4 v = src[q];
                s += (v.x + v.y) + (v.z + v.w);
                v.y *= 0.0625f;
                v.w *= 0.0625f;
                xv[j][q] = v;
            }
            xs[j] = s;
        }
        // the dispatch's first workgroup claims the completion word (this
        // wave only reads LDS from here on, so the wait costs the stream
        // nothing beyond this wave's start)
        if (p.ctl != nullptr && blockIdx.x == 0 && lane == 0 && c == 0) arrival_preclaim(&p.ctl->arrive, tag);

        for (int s = 0; s < nstages; ++s) {
            // the previous stage's LDS reads are complete before its slot
            // can be refilled after this barrier
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            stream_barrier();
            const unsigned char *slot = stream_lds + (s % D) * kStreamStageBytes;
            const int rw = c * RPW;                        // this wave's first row in the stage
            uint4 cw[RPW][NC];
            uint32_t sw[RPW][NC], bw[RPW][NC];
#pragma unroll
            for (int r = 0; r < RPW; ++r)
#pragma unroll
                for (int j = 0; j < NC; ++j) {
                    cw[r][j] = *reinterpret_cast<const uint4 *>(slot + ((rw + r) * NC + j) * 1024 + 16 * lane);
                    const int ci = ((rw + r) * GPR + (lane + 64 * j) / 2) * 2;
                    sw[r][j] = *reinterpret_cast<const uint16_t *>(slot + kStreamCodeBytes + ci);
                    bw[r][j] = *reinterpret_cast<const uint16_t *>(slot + kStreamCodeBytes + kStreamCoefBytes + ci);
                }
            // the RPW rows' dot products as independent chains advanced in
            // turn (a single chain would make every instruction wait for
            // the one before it)
            float acc[RPW];
#pragma unroll
            for (int r = 0; r < RPW; ++r) acc[r] = 0.f;
#pragma unroll
            for (int j = 0; j < NC; ++j) {
                float d[RPW];
#pragma unroll
                for (int r = 0; r < RPW; ++r) d[r] = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    uint32_t dw[RPW];
#pragma unroll
                    for (int r = 0; r < RPW; ++r) dw[r] = word_of(cw[r][j], w);
                    dot_u4x8_mix_rows<RPW>(dw, xv[j][2 * w], xv[j][2 * w + 1], d);
                }
#pragma unroll
                for (int r = 0; r < RPW; ++r)
                    acc[r] = fmaf(bf16_bits_to_f32(sw[r][j]), d[r] * kMixScale,
                                  fmaf(bf16_bits_to_f32(bw[r][j]), xs[j], acc[r]));
            }
            wave_reduce_dpp<RPW>(acc, lane);
            const int64_t m = r0 + static_cast<int64_t>(s) * RS + rw + own;
            if (writer && m < r1) {
                const float v = acc[0];
                if (p.y) p.y[m] = v;
                if (best_m < 0 || v > best_v) {   // this lane's rows arrive in increasing order
                    best_v = v;
                    best_m = m;
                }
            }
        }
    }

    if (p.ctl != nullptr) {
        // the writer lanes' bests straight into the workgroup's key (s_key
        // was cleared before the first stage barrier)
        if (writer && best_m >= 0) atomicMax(&s_key, argmax_key(best_v, static_cast<uint32_t>(best_m)));
        __syncthreads();
        greedy_finish_rows(&s_key, 1, p.ctl, p.keys, p.idx, static_cast<int>(gridDim.x), tag);
    }
}

}  // namespace qg
