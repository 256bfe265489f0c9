// gemm.hpp -- prefill product Y[n][m] = sum_k w[m][k] X[n][k] on the gfx950
// matrix cores (MFMA), with the packed weights dequantized in registers.
//
// Precision. The activations are float32 and the result must stay within
// 1e-5 of sum|w x|, so X cannot be rounded to bf16. Each X value is split
// exactly into three bf16 pieces, X = hi + mid + lo (truncation: hi takes the
// top 8 significant bits, mid the next 8, lo the last 8), and the product runs
// as three bf16 MFMAs accumulating in float32. The weight operand is exact in
// bf16 for both formats: int8 codes (|q| <= 128 needs 8 bits) and the signs
// +-1 of the 1-bit format. Per-row (int8) and per-group (1-bit, 128 k) scales
// are applied in float32 outside the MFMA.
// (MiniCPM-V-4.6 on a Tesla C2075, academ.us 2607.14568, section 3.1:
// prefill projections are genuine matrix-matrix products; this kernel keeps
// the weights packed instead of dequantizing them to a float scratch first.)
//
// Tiling. A workgroup of 4 waves computes a 128 (m) x 128 (n) tile of Y; the
// waves form a 2 x 2 grid of 64 x 64 sub-tiles, i.e. 4 x 4 MFMA 16x16 tiles
// per wave. Each k-step stages 32 k of W (converted to bf16) and X (split
// into 3 bf16 planes) in LDS; rows are padded to 80 bytes so that the
// 16-byte fragment reads of 8 consecutive lanes hit 8 distinct bank groups.
// The next k-step's global loads are issued before the current MFMAs.
//
// MFMA 16x16x32 bf16 operand layout (lane l of 64):
//   A (16 x 32, here W rows):    row l % 16, k = 8 * (l / 16) .. + 7
//   B (32 x 16, here X rows):    col l % 16, k = 8 * (l / 16) .. + 7
//   D (16 x 16 float):           col l % 16, rows 4 * (l / 16) .. + 3
// so D holds Y[n][m .. m+3] for 4 consecutive m of one token row n.
#pragma once

#include "gemv.hpp"
#include "qg_device.hpp"

namespace qg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

struct GemmParams {
    const uint8_t *codes;
    const void *scales;
    const float *x;   // [N][K]
    float *y;         // [N][M]
    int64_t M, K, N;
    int tiles_m, tiles_n;
};

constexpr int GT_M = 128, GT_N = 128, GT_K = 32;
constexpr int G_ROW = 40;  // bf16 per padded LDS row (32 + 8 pad)

// Exact three-way bf16 split of float32 values a, b (two consecutive k):
// returns packed bf16x2 words (a in the low half) for each piece.
__device__ __forceinline__ void split3_pair(float a, float b, uint32_t &hi, uint32_t &mid,
                                            uint32_t &lo)
{
    const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
    const uint32_t ha = ua & 0xFFFF0000u, hb = ub & 0xFFFF0000u;
    const float ra = a - __uint_as_float(ha), rb = b - __uint_as_float(hb);     // exact
    const uint32_t ma = __float_as_uint(ra) & 0xFFFF0000u, mb = __float_as_uint(rb) & 0xFFFF0000u;
    const float la = ra - __uint_as_float(ma), lb = rb - __uint_as_float(mb);   // exact
    hi = (ha >> 16) | hb;
    mid = (ma >> 16) | mb;
    lo = (__float_as_uint(la) >> 16) | (__float_as_uint(lb) & 0xFFFF0000u);
}

// int8 code pair -> packed bf16x2 (exact).
__device__ __forceinline__ uint32_t i8pair_to_bf16x2(uint32_t d, int byte0)
{
    const float a = static_cast<float>(static_cast<int8_t>((d >> (8 * byte0)) & 0xff));
    const float b = static_cast<float>(static_cast<int8_t>((d >> (8 * byte0 + 8)) & 0xff));
    return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
}

// Two sign bits (bit0 -> low half) -> packed bf16x2 of +-1: bit 1 -> +1.0
// (0x3F80), bit 0 -> -1.0 (0xBF80). `nbits` holds the inverted bits, so
// the multiply moves inverted bit 0 to bit 15 and inverted bit 1 to bit 31.
__device__ __forceinline__ uint32_t signpair_to_bf16x2(uint32_t nbits2)
{
    return ((nbits2 * 0x40008000u) & 0x80008000u) | 0x3F803F80u;
}

template <int FMT>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmParams p)
{
    __shared__ __attribute__((aligned(16))) uint16_t lw[GT_M * G_ROW];
    __shared__ __attribute__((aligned(16))) uint16_t lx[3][GT_N * G_ROW];

    // XCD-aware order: consecutive workgroup ids go round-robin to the 8
    // XCDs; give each XCD a contiguous run of tiles (m fastest) so the tiles
    // that share an X block meet in the same L2.
    const int ntiles = p.tiles_m * p.tiles_n;
    int bid = blockIdx.x;
    if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);
    const int tm = bid % p.tiles_m, tn = bid / p.tiles_m;
    const int64_t m0 = static_cast<int64_t>(tm) * GT_M, n0 = static_cast<int64_t>(tn) * GT_N;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = (wave & 1) * 64, wn = (wave >> 1) * 64;

    // staging assignment: thread -> (row, half of the 32-k step)
    const int sr = tid >> 1, sh = tid & 1;
    const int64_t wrow = m0 + sr, xrow = n0 + sr;
    const bool wvalid = wrow < p.M, xvalid = xrow < p.N;
    const int64_t row_bytes = FMT == FMT_I8_ROW ? p.K : p.K / 8;
    const uint8_t *wsrc = p.codes + (wvalid ? wrow : 0) * row_bytes;
    const float *xsrc = p.x + (xvalid ? xrow : 0) * p.K;

    const int nk = static_cast<int>((p.K + GT_K - 1) / GT_K);

    // prefetch registers
    uint4 wreg;          // I8: 16 codes; B1: low 16 bits = 16 sign bits
    float4 xreg[4];

    auto load = [&](int kt) {
        const int64_t k = static_cast<int64_t>(kt) * GT_K + 16 * sh;
        const bool kin = k < p.K;  // K is a multiple of 16
        if (FMT == FMT_I8_ROW) {
            wreg = (wvalid && kin) ? *reinterpret_cast<const uint4 *>(wsrc + k) : make_uint4(0, 0, 0, 0);
        } else {
            wreg.x = (wvalid && kin) ? *reinterpret_cast<const uint16_t *>(wsrc + k / 8) : 0u;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            xreg[j] = (xvalid && kin) ? *reinterpret_cast<const float4 *>(xsrc + k + 4 * j)
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
    };

    auto stage = [&]() {
        uint32_t wv[8];
        if (FMT == FMT_I8_ROW) {
            const uint32_t d[4] = {wreg.x, wreg.y, wreg.z, wreg.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                wv[2 * j] = i8pair_to_bf16x2(d[j], 0);
                wv[2 * j + 1] = i8pair_to_bf16x2(d[j], 2);
            }
        } else {
            // rows beyond M carry no codes: their (unused) weights become -1
            const uint32_t nb = ~wreg.x;
#pragma unroll
            for (int j = 0; j < 8; ++j) wv[j] = signpair_to_bf16x2((nb >> (2 * j)) & 3u);
        }
        uint4 *dw = reinterpret_cast<uint4 *>(lw + sr * G_ROW + 16 * sh);
        dw[0] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        dw[1] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
        uint32_t h[8], md[8], lo[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            split3_pair(xreg[j].x, xreg[j].y, h[2 * j], md[2 * j], lo[2 * j]);
            split3_pair(xreg[j].z, xreg[j].w, h[2 * j + 1], md[2 * j + 1], lo[2 * j + 1]);
        }
        uint4 *d0 = reinterpret_cast<uint4 *>(lx[0] + sr * G_ROW + 16 * sh);
        uint4 *d1 = reinterpret_cast<uint4 *>(lx[1] + sr * G_ROW + 16 * sh);
        uint4 *d2 = reinterpret_cast<uint4 *>(lx[2] + sr * G_ROW + 16 * sh);
        d0[0] = make_uint4(h[0], h[1], h[2], h[3]);
        d0[1] = make_uint4(h[4], h[5], h[6], h[7]);
        d1[0] = make_uint4(md[0], md[1], md[2], md[3]);
        d1[1] = make_uint4(md[4], md[5], md[6], md[7]);
        d2[0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        d2[1] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
    };

    floatx4_t acc[4][4];
    floatx4_t gacc[4][4];  // 1-bit format: sums of the current 128-k group
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            gacc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        }

    const int fr = lane & 15, fk = 8 * (lane >> 4);
    load(0);
    for (int kt = 0; kt < nk; ++kt) {
        __syncthreads();
        stage();
        __syncthreads();
        if (kt + 1 < nk) load(kt + 1);

        bf16x8_t a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = __builtin_bit_cast(bf16x8_t,
                                      *reinterpret_cast<const uint4 *>(lw + (wm + 16 * i + fr) * G_ROW + fk));
#pragma unroll
        for (int pc = 0; pc < 3; ++pc) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8_t b = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const uint4 *>(lx[pc] + (wn + 16 * j + fr) * G_ROW + fk));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (FMT == FMT_I8_ROW)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b, acc[i][j], 0, 0, 0);
                    else
                        gacc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b, gacc[i][j], 0, 0, 0);
                }
            }
        }

        if (FMT == FMT_B1_G128 && ((kt & 3) == 3 || kt + 1 == nk)) {
            // close the 128-k group: acc += scale[m][g] * group sum
            const int64_t g = kt >> 2;
            const uint16_t *sp = static_cast<const uint16_t *>(p.scales);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t m = m0 + wm + 16 * i + 4 * (lane >> 4) + r;
                    const float s = m < p.M ? fp16_bits_to_f32(sp[m * (p.K / 128) + g]) : 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc[i][j][r] = fmaf(s, gacc[i][j][r], acc[i][j][r]);
                        gacc[i][j][r] = 0.f;
                    }
                }
            }
        }
    }

    // epilogue: row scale (int8), store Y[n][m .. m+3]
    const bool vec = (p.M & 3) == 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t mb = m0 + wm + 16 * i + 4 * (lane >> 4);
        float s[4] = {1.f, 1.f, 1.f, 1.f};
        if (FMT == FMT_I8_ROW) {
            const float *sp = static_cast<const float *>(p.scales);
#pragma unroll
            for (int r = 0; r < 4; ++r) s[r] = mb + r < p.M ? sp[mb + r] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + wn + 16 * j + fr;
            if (n >= p.N) continue;
            float *dst = p.y + n * p.M + mb;
            const float v0 = s[0] * acc[i][j][0], v1 = s[1] * acc[i][j][1];
            const float v2 = s[2] * acc[i][j][2], v3 = s[3] * acc[i][j][3];
            if (vec && mb + 3 < p.M) {
                *reinterpret_cast<float4 *>(dst) = make_float4(v0, v1, v2, v3);
            } else {
                if (mb < p.M) dst[0] = v0;
                if (mb + 1 < p.M) dst[1] = v1;
                if (mb + 2 < p.M) dst[2] = v2;
                if (mb + 3 < p.M) dst[3] = v3;
            }
        }
    }
}

}  // namespace qg
