// gemv.hpp -- dequantize-fused low-bit matrix-vector kernels (batch 1..16)
// for gfx950, plus the split-K combine and the fused greedy selection.
//
// Mapping. A workgroup of 4 waves owns a contiguous range of output rows and
// one K range (one "split"). The activations of that K range are staged
// once into LDS; each wave then walks blocks of R rows. Within a row the 64
// lanes walk the packed row in 16-byte slices (slice t goes to lane t mod
// 64), so every wave instruction reads 64 consecutive 16-byte pieces of a
// row: fully coalesced 1 KiB loads. The codes are unpacked and dequantized
// in registers and never written anywhere (I Built an LLM Inference Engine
// on a 15 year old GPU..., "Optimization 4: Quantized Kernels"). Each
// activation value read from LDS serves all R rows of the block.
//
// Per format, one 16-byte slice holds:
//   QG_I8_ROW   16 weights (k .. k+15), row scale applied once per row;
//   QG_I8_G64   16 weights of one group of 64 (its fp32 scale);
//   QG_U4_G64   32 weights = half a group of 64: one (scale, bias) pair.
// The affine format is evaluated per slice as s * sum(q * x) + b * sum(x),
// with sum(x) over the slice precomputed once per workgroup. (The 1-bit
// format has its own kernels: gemv_b1.hpp, gemv_mfma16.hpp, gemm.hpp.)
#pragma once

#include "arrive.hpp"
#include "qg_device.hpp"

namespace qg {

enum { FMT_I8_ROW = 1, FMT_U4_G64 = 2, FMT_B1_G128 = 3, FMT_I8_G64 = 4 };

template <int FMT> struct Fmt;
template <> struct Fmt<FMT_I8_ROW>  { static constexpr int KPS = 16;  static constexpr bool kXsum = false; };
template <> struct Fmt<FMT_U4_G64>  { static constexpr int KPS = 32;  static constexpr bool kXsum = true; };
template <> struct Fmt<FMT_B1_G128> { static constexpr int KPS = 128; static constexpr bool kXsum = true; };
template <> struct Fmt<FMT_I8_G64>  { static constexpr int KPS = 16;  static constexpr bool kXsum = false; };

struct GemvParams {
    const uint8_t *codes;
    const void *scales;
    const void *biases;
    const float *x;       // [nb][K]
    float *y;             // [nb][M] final output (used when nsplit == 1)
    float *part;          // [nsplit][nb][M] partial sums (used when nsplit > 1)
    GreedyCtl *ctl;       // control words (greedy head), or nullptr
    unsigned long long *keys;  // greedy keys [nkeys][nb] in the workspace
    int32_t *idx;         // [nb] greedy indices
    int64_t M;
    int64_t K;
    int64_t x_stride;     // floats between activation rows (== K)
    int64_t rows_per_wg;  // multiple of 4 * R
    int64_t kc;           // K per split, multiple of the slice width
    int nb;               // actual batch (<= template B)
    int nsplit;
    int nkeys;            // workgroups of the kernel that finishes the greedy head
};

// Chunk (float4) swizzle inside an activation plane. Lanes reading chunk
// j of consecutive slices would all hit the same LDS banks; flipping the
// low 3 chunk-index bits by the slice number spreads 8 consecutive lanes
// over all 8 16-byte bank groups. It permutes chunks only within aligned
// groups of 8, so planes are padded to a multiple of 32 floats.
template <int CPS>
__device__ __forceinline__ int swz(int c)
{
    return c ^ ((c / CPS) & 7);
}

__host__ __device__ constexpr int64_t plane_floats(int64_t kc)
{
    return (kc + 31) / 32 * 32;
}

template <int FMT>
__host__ __device__ constexpr int64_t xsum_floats(int64_t kc)
{
    return Fmt<FMT>::kXsum ? (kc / Fmt<FMT>::KPS + 3) / 4 * 4 : 0;
}

// Stage x[b][k0 : k0+kc] into LDS planes (swizzled, zero beyond nb), with
// odd k of the 4-bit format pre-divided by 16 (exact: a power of two) so that
// the high nibble can be used without a shift. Then per-slice sums of the
// unscaled activations.
template <int FMT, int B>
__device__ __forceinline__ void stage_x(const GemvParams &p, int64_t k0, int kc,
                                        float4 *xl, float *xs)
{
    constexpr int KPS = Fmt<FMT>::KPS;
    constexpr int CPS = KPS / 4;
    const int pc = static_cast<int>(plane_floats(kc) / 4);  // chunks per plane
    const int nchunk = kc / 4;
    for (int i = threadIdx.x; i < B * pc; i += blockDim.x) {
        const int b = i / pc, c = i % pc;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (b < p.nb && c < nchunk)
            v = *reinterpret_cast<const float4 *>(p.x + b * p.x_stride + k0 + 4 * c);
        if (FMT == FMT_U4_G64) {
            v.y *= 0.0625f;
            v.w *= 0.0625f;
        }
        xl[b * pc + swz<CPS>(c)] = v;
    }
    if (Fmt<FMT>::kXsum) {
        const int ns = kc / KPS;
        const int xsp = static_cast<int>(xsum_floats<FMT>(kc));
        for (int i = threadIdx.x; i < B * ns; i += blockDim.x) {
            const int b = i / ns, t = i % ns;
            float s = 0.f;
            if (b < p.nb) {
                const float4 *src =
                    reinterpret_cast<const float4 *>(p.x + b * p.x_stride + k0 + t * KPS);
#pragma unroll 4
                for (int j = 0; j < CPS; ++j) {
                    float4 v = src[j];
                    s += (v.x + v.y) + (v.z + v.w);
                }
            }
            xs[b * xsp + t] = s;
        }
    }
}

// sum_i q_i * x_i for one dword of 4 int8 codes and 4 activations.
__device__ __forceinline__ float dot_i8x4(uint32_t d, float4 x, float acc)
{
    acc = fmaf(static_cast<float>(static_cast<int8_t>(d & 0xff)), x.x, acc);
    acc = fmaf(static_cast<float>(static_cast<int8_t>((d >> 8) & 0xff)), x.y, acc);
    acc = fmaf(static_cast<float>(static_cast<int8_t>((d >> 16) & 0xff)), x.z, acc);
    acc = fmaf(static_cast<float>(static_cast<int8_t>(d >> 24)), x.w, acc);
    return acc;
}

// sum_i q_i * x_i for one dword of 8 nibbles (k = 8j .. 8j+7), given the
// two activation chunks of those k with odd k pre-divided by 16: the low
// nibbles (even k) are masked in place, the high nibbles (odd k) are masked
// in place as 16*q; each byte then converts to float in one instruction.
__device__ __forceinline__ float dot_u4x8(uint32_t d, float4 xa, float4 xb, float acc)
{
    // The masks go through opaque instructions: if the compiler could see
    // them it would fold each "mask, then take byte i" into a bit-field
    // extract plus a convert (two instructions per weight) instead of one
    // byte-select convert (v_cvt_f32_ubyte0..3).
    uint32_t lo, hi;
    asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(lo) : "v"(d));
    asm("v_and_b32 %0, 0xf0f0f0f0, %1" : "=v"(hi) : "v"(d));
    acc = fmaf(static_cast<float>(lo & 0xff), xa.x, acc);
    acc = fmaf(static_cast<float>(hi & 0xff), xa.y, acc);
    acc = fmaf(static_cast<float>((lo >> 8) & 0xff), xa.z, acc);
    acc = fmaf(static_cast<float>((hi >> 8) & 0xff), xa.w, acc);
    acc = fmaf(static_cast<float>((lo >> 16) & 0xff), xb.x, acc);
    acc = fmaf(static_cast<float>((hi >> 16) & 0xff), xb.y, acc);
    acc = fmaf(static_cast<float>(lo >> 24), xb.z, acc);
    acc = fmaf(static_cast<float>(hi >> 24), xb.w, acc);
    return acc;
}

// 2^-24 sum_i q_i * x_i for one dword of 8 nibbles, same activation layout
// as dot_u4x8 (odd k pre-divided by 16). A 16-bit half that holds only a
// nibble in bits 0..3 (or 4..7) is the fp16 subnormal q 2^-24 (or 16 q
// 2^-24), exactly, so masking both halves of the dword at once yields two
// weights, and the mixed-precision FMA widens the selected half inside the
// multiply-add: one instruction per weight plus five per dword for the
// masks and the shift, instead of a convert and an FMA per weight. Products
// and sums are the fp32 ones of dot_u4x8 scaled by 2^-24 (exact, fp16 and
// fp32 subnormals are kept); the caller multiplies by 2^24.
__device__ __forceinline__ float h16_lo(uint32_t v)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v)));
}
__device__ __forceinline__ float h16_hi(uint32_t v)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v >> 16)));
}
constexpr float kMixScale = 16777216.f;   // 2^24

__device__ __forceinline__ float dot_u4x8_mix(uint32_t d, float4 xa, float4 xb, float acc)
{
    const uint32_t e = d >> 8;
    const uint32_t q04 = d & 0x000F000Fu;   // k = 0 and 4
    const uint32_t q15 = d & 0x00F000F0u;   // k = 1 and 5 (times 16)
    const uint32_t q26 = e & 0x000F000Fu;   // k = 2 and 6
    const uint32_t q37 = e & 0x00F000F0u;   // k = 3 and 7 (times 16)
    acc = fmaf(h16_lo(q04), xa.x, acc);
    acc = fmaf(h16_lo(q15), xa.y, acc);
    acc = fmaf(h16_lo(q26), xa.z, acc);
    acc = fmaf(h16_lo(q37), xa.w, acc);
    acc = fmaf(h16_hi(q04), xb.x, acc);
    acc = fmaf(h16_hi(q15), xb.y, acc);
    acc = fmaf(h16_hi(q26), xb.z, acc);
    acc = fmaf(h16_hi(q37), xb.w, acc);
    return acc;
}

// dot_u4x8_mix for R rows at once (dword dw[r] of row r, the same eight
// activations), each row's chain in the same order as dot_u4x8_mix, the
// chains advanced in turn: consecutive instructions belong to different
// rows, so none waits for the result of the one before it.
template <int R>
__device__ __forceinline__ void dot_u4x8_mix_rows(const uint32_t (&dw)[R], float4 xa, float4 xb, float (&acc)[R])
{
    uint32_t q04[R], q15[R], q26[R], q37[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t e = dw[r] >> 8;
        q04[r] = dw[r] & 0x000F000Fu;
        q15[r] = dw[r] & 0x00F000F0u;
        q26[r] = e & 0x000F000Fu;
        q37[r] = e & 0x00F000F0u;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = fmaf(h16_lo(q04[r]), xa.x, acc[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = fmaf(h16_lo(q15[r]), xa.y, acc[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = fmaf(h16_lo(q26[r]), xa.z, acc[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = fmaf(h16_lo(q37[r]), xa.w, acc[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = fmaf(h16_hi(q04[r]), xb.x, acc[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = fmaf(h16_hi(q15[r]), xb.y, acc[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = fmaf(h16_hi(q26[r]), xb.z, acc[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = fmaf(h16_hi(q37[r]), xb.w, acc[r]);
}

__device__ __forceinline__ uint32_t word_of(const uint4 &c, int j)
{
    return j == 0 ? c.x : j == 1 ? c.y : j == 2 ? c.z : c.w;
}

// Main kernel. B: batch rounded up to a power of two (x rows >= nb are
// zero in LDS and their outputs are not written). R: rows per block.
template <int FMT, int B, int R>
__global__ __launch_bounds__(256) void gemv_kernel(GemvParams p)
{
    constexpr int KPS = Fmt<FMT>::KPS;
    constexpr int CPS = KPS / 4;
    constexpr int V = R * B;
    static_assert(V <= 64, "R * B must not exceed the wave width");

    extern __shared__ float4 lds[];
    const int split = blockIdx.y;
    const int64_t k0 = static_cast<int64_t>(split) * p.kc;
    const int kc = static_cast<int>(min(p.kc, p.K - k0));
    const int pc = static_cast<int>(plane_floats(kc) / 4);
    const int xsp = static_cast<int>(xsum_floats<FMT>(kc));
    float4 *xl = lds;
    float *xs = reinterpret_cast<float *>(lds + B * pc);

    // greedy head: read the completion word as it stands at the start
    const bool greedy = p.ctl != nullptr && p.nsplit == 1;
    const uint32_t tag = greedy ? dispatch_tag() : 0u;
    if (greedy && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) arrival_preclaim(&p.ctl->arrive, tag);

    stage_x<FMT, B>(p, k0, kc, xl, xs);
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int S = kc / KPS;                       // slices in this split
    const int64_t row_bytes =
        (FMT == FMT_I8_ROW || FMT == FMT_I8_G64) ? p.K : FMT == FMT_U4_G64 ? p.K / 2 : p.K / 8;
    const int64_t slice0 = k0 / KPS;              // first global slice of this split
    const int64_t m_begin = static_cast<int64_t>(blockIdx.x) * p.rows_per_wg;
    const int64_t m_end = min(p.M, m_begin + p.rows_per_wg);

    // value index this lane ends up owning after the cross-lane reduction
    // (DPP exchanges up to 16 values, the LDS butterfly beyond)
    constexpr int P = V == 1 ? 0 : V == 2 ? 1 : V == 4 ? 2 : V == 8 ? 3 : V == 16 ? 4 : V == 32 ? 5 : 6;
    const int own = V <= 16 ? dpp_owner<V <= 16 ? V : 1>(lane) : lane >> (6 - P);
    const bool writer = V <= 16 ? dpp_writer<V <= 16 ? V : 1>(lane)
                                : (lane & ((1 << (6 - P)) - 1)) == 0;
    const int own_r = own / B, own_b = own % B;
    float best_v = 0.f;
    int64_t best_m = -1;

    for (int64_t rb = m_begin + wave * R; rb < m_end; rb += 4 * R) {
        float acc[V];
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = 0.f;

        for (int t = lane; t < S; t += kWave) {
            const int64_t gslice = slice0 + t;
            uint4 c[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int64_t m = rb + r;
                c[r] = make_uint4(0, 0, 0, 0);
                if (m < m_end)
                    c[r] = *reinterpret_cast<const uint4 *>(p.codes + m * row_bytes + gslice * 16);
            }
            if constexpr (FMT == FMT_I8_ROW) {
                // each dword of codes is converted once and used for every
                // activation row
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float qv[R][4];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const uint32_t d = word_of(c[r], j);
                        qv[r][0] = static_cast<float>(static_cast<int8_t>(d & 0xff));
                        qv[r][1] = static_cast<float>(static_cast<int8_t>((d >> 8) & 0xff));
                        qv[r][2] = static_cast<float>(static_cast<int8_t>((d >> 16) & 0xff));
                        qv[r][3] = static_cast<float>(static_cast<int8_t>(d >> 24));
                    }
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const float4 xv = xl[b * pc + swz<CPS>(t * CPS + j)];
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            float a = acc[r * B + b];
                            a = fmaf(qv[r][0], xv.x, a);
                            a = fmaf(qv[r][1], xv.y, a);
                            a = fmaf(qv[r][2], xv.z, a);
                            a = fmaf(qv[r][3], xv.w, a);
                            acc[r * B + b] = a;
                        }
                    }
                }
            } else if constexpr (FMT == FMT_I8_G64) {
                // a 16-input slice lies inside one 64-input group: its dot
                // products are scaled by the group's float32 scale
                float sc[R];
                const float *sp = static_cast<const float *>(p.scales);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int64_t m = rb + r;
                    sc[r] = sp[(m < m_end ? m : m_begin) * (p.K / 64) + gslice / 4];
                }
                float dot[R][B];
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int b = 0; b < B; ++b) dot[r][b] = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float qv[R][4];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const uint32_t d = word_of(c[r], j);
                        qv[r][0] = static_cast<float>(static_cast<int8_t>(d & 0xff));
                        qv[r][1] = static_cast<float>(static_cast<int8_t>((d >> 8) & 0xff));
                        qv[r][2] = static_cast<float>(static_cast<int8_t>((d >> 16) & 0xff));
                        qv[r][3] = static_cast<float>(static_cast<int8_t>(d >> 24));
                    }
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const float4 xv = xl[b * pc + swz<CPS>(t * CPS + j)];
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            float a = dot[r][b];
                            a = fmaf(qv[r][0], xv.x, a);
                            a = fmaf(qv[r][1], xv.y, a);
                            a = fmaf(qv[r][2], xv.z, a);
                            a = fmaf(qv[r][3], xv.w, a);
                            dot[r][b] = a;
                        }
                    }
                }
#pragma unroll
                for (int b = 0; b < B; ++b)
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        acc[r * B + b] = fmaf(sc[r], dot[r][b], acc[r * B + b]);
            } else if constexpr (FMT == FMT_U4_G64) {
                float sc[R], bi[R];
                const uint16_t *sp = static_cast<const uint16_t *>(p.scales);
                const uint16_t *bp = static_cast<const uint16_t *>(p.biases);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int64_t m = rb + r;
                    const int64_t gi = (m < m_end ? m : m_begin) * (p.K / 64) + gslice / 2;
                    sc[r] = bf16_bits_to_f32(sp[gi]);
                    bi[r] = bf16_bits_to_f32(bp[gi]);
                }
                // dot[r][b] over this slice; each dword of codes is converted
                // once (low nibbles in place, high nibbles as 16*q against
                // activations pre-divided by 16) and used for every row b
                float dot[R][B];
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int b = 0; b < B; ++b) dot[r][b] = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float qv[R][8];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const uint32_t d = word_of(c[r], j);
                        uint32_t lo, hi;
                        asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(lo) : "v"(d));
                        asm("v_and_b32 %0, 0xf0f0f0f0, %1" : "=v"(hi) : "v"(d));
                        qv[r][0] = static_cast<float>(lo & 0xff);
                        qv[r][1] = static_cast<float>(hi & 0xff);
                        qv[r][2] = static_cast<float>((lo >> 8) & 0xff);
                        qv[r][3] = static_cast<float>((hi >> 8) & 0xff);
                        qv[r][4] = static_cast<float>((lo >> 16) & 0xff);
                        qv[r][5] = static_cast<float>((hi >> 16) & 0xff);
                        qv[r][6] = static_cast<float>(lo >> 24);
                        qv[r][7] = static_cast<float>(hi >> 24);
                    }
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const float4 *xp = xl + b * pc;
                        const float4 xa = xp[swz<CPS>(t * CPS + 2 * j)];
                        const float4 xb = xp[swz<CPS>(t * CPS + 2 * j + 1)];
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            float a = dot[r][b];
                            a = fmaf(qv[r][0], xa.x, a);
                            a = fmaf(qv[r][1], xa.y, a);
                            a = fmaf(qv[r][2], xa.z, a);
                            a = fmaf(qv[r][3], xa.w, a);
                            a = fmaf(qv[r][4], xb.x, a);
                            a = fmaf(qv[r][5], xb.y, a);
                            a = fmaf(qv[r][6], xb.z, a);
                            a = fmaf(qv[r][7], xb.w, a);
                            dot[r][b] = a;
                        }
                    }
                }
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const float xsum = xs[b * xsp + t];
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        acc[r * B + b] = fmaf(sc[r], dot[r][b], fmaf(bi[r], xsum, acc[r * B + b]));
                }
            }
        }

        if constexpr (V <= 16) wave_reduce_dpp<V>(acc, lane);
        else wave_transpose_reduce<V>(acc, lane);

        if (writer) {
            const int64_t m = rb + own_r;
            if (m < m_end && own_b < p.nb) {
                float v = acc[0];
                if (FMT == FMT_I8_ROW)
                    v *= static_cast<const float *>(p.scales)[m];
                if (p.nsplit == 1) {
                    if (p.y) p.y[own_b * p.M + m] = v;
                    if (best_m < 0 || v > best_v || (v == best_v && m < best_m)) {
                        best_v = v;
                        best_m = m;
                    }
                } else {
                    p.part[(static_cast<int64_t>(split) * p.nb + own_b) * p.M + m] = v;
                }
            }
        }
    }

    if (greedy) {
        __shared__ unsigned long long wg_key[B];
        __syncthreads();
        if (threadIdx.x < B) wg_key[threadIdx.x] = 0ull;
        __syncthreads();
        if (writer && best_m >= 0)
            atomicMax(&wg_key[own_b], static_cast<unsigned long long>(
                                          argmax_key(best_v, static_cast<uint32_t>(best_m))));
        __syncthreads();
        greedy_finish_rows(wg_key, p.nb, p.ctl, p.keys, p.idx, p.nkeys, tag);
    }
}

// y[b][m] = sum over splits of part[s][b][m], in split order; optionally
// the per-workgroup argmax keys of the combined rows.
__global__ __launch_bounds__(256) void gemv_combine_kernel(GemvParams p)
{
    __shared__ unsigned long long wg_key[16];
    const uint32_t tag = p.ctl != nullptr ? dispatch_tag() : 0u;
    if (p.ctl != nullptr && blockIdx.x == 0 && threadIdx.x == 0) arrival_preclaim(&p.ctl->arrive, tag);
    if (threadIdx.x < 16) wg_key[threadIdx.x] = 0ull;
    __syncthreads();
    const int64_t m_begin = static_cast<int64_t>(blockIdx.x) * p.rows_per_wg;
    const int64_t m_end = min(p.M, m_begin + p.rows_per_wg);
    for (int b = 0; b < p.nb; ++b) {
        uint64_t best = 0;
        for (int64_t m = m_begin + threadIdx.x; m < m_end; m += blockDim.x) {
            float v = 0.f;
            for (int s = 0; s < p.nsplit; ++s)
                v += p.part[(static_cast<int64_t>(s) * p.nb + b) * p.M + m];
            if (p.y) p.y[b * p.M + m] = v;
            const uint64_t key = argmax_key(v, static_cast<uint32_t>(m));
            best = key > best ? key : best;
        }
        if (p.ctl != nullptr)
            atomicMax(&wg_key[b], static_cast<unsigned long long>(best));
    }
    if (p.ctl != nullptr) {
        __syncthreads();
        greedy_finish_rows(wg_key, p.nb, p.ctl, p.keys, p.idx, p.nkeys, tag);
    }
}

}  // namespace qg
