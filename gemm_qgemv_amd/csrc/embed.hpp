// embed.hpp -- embedding rows gathered from the tied 4-bit matrix.
//
// out[t][k] is the float32 value of weight (ids[t], k) produced the way the
// pages' decoder does it: scale * code (exact in float32: 8 x 4 significant
// bits) plus the bias, one float32 rounding to nearest even, then a
// round-trip through IEEE binary16 (nearest even, subnormals and the sign of
// zero kept). (Pushing the limits of legacy hardware, "Half a billion
// values, and one negative zero": that decoder multiplies and adds in two
// steps and passes each value through FP16 on its way to FP32, and the
// lookup on the GPU had to reproduce denormals, the sign of zero and
// round-to-nearest-even exactly.) On gfx950 the default floating-point mode already rounds to
// nearest even and keeps binary16 denormals; this library is built without
// float32 denormal flushing. The product and the sum stay two operations:
// the product is exact unless it overflows, and there a fused multiply-add
// could bring a sum back into range that the two steps leave infinite.
//
// A workgroup per kEmbedRows rows (a grid-stride loop over rows). Rows
// outside [0, M) come out as quiet NaN (the ids live in device memory, so
// the host cannot check them before the launch).
#pragma once

#include "qg_device.hpp"

namespace qg {

struct EmbedParams {
    const uint8_t *codes;     // [M][K/2] bytes of 2 nibbles
    const uint16_t *scales;   // bf16 [M][K/64]
    const uint16_t *biases;   // bf16 [M][K/64]
    const int32_t *ids;       // [n]
    float *out;               // [n][K]
    int64_t M, K, n;
};

constexpr int kEmbedThreads = 256;

// Rows gathered per workgroup, and whether the output rows are written with
// non-temporal stores (they are read by the next kernel, not by this one).
// Measured on the 2048-id prompt from the 151936 x 2048 table: one row per
// workgroup with streaming stores writes faster than a plain fill kernel of
// the same output (4.7 us); two or four rows per workgroup, or ordinary
// stores, are slower (5.1 - 7.5 us).
constexpr int kEmbedRows = 1;

__device__ __forceinline__ float embed_value(float s, float b, uint32_t q)
{
#pragma clang fp contract(off)
    const float prod = s * static_cast<float>(q);
    return static_cast<float>(static_cast<_Float16>(prod + b));
}

__device__ __forceinline__ void embed_store(float4 *dst, float4 v)
{
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<f32x4 *>(dst));
}

// Each thread produces float4 f of a row (inputs 4f .. 4f+3: two code bytes)
// so one store instruction of a wave covers 1 KiB of contiguous output.
__global__ __launch_bounds__(kEmbedThreads) void embed_u4_kernel(EmbedParams p)
{
    const int64_t quads = p.K / 4, groups = p.K / 64;
    const auto *codes16 = reinterpret_cast<const uint16_t *>(p.codes);
    for (int64_t t0 = int64_t(blockIdx.x) * kEmbedRows; t0 < p.n;
         t0 += int64_t(gridDim.x) * kEmbedRows) {
        int64_t id[kEmbedRows];
        bool inside[kEmbedRows], live[kEmbedRows];
#pragma unroll
        for (int r = 0; r < kEmbedRows; ++r) {
            live[r] = t0 + r < p.n;
            id[r] = live[r] ? p.ids[t0 + r] : -1;
            inside[r] = id[r] >= 0 && id[r] < p.M;
        }
        for (int64_t f = threadIdx.x; f < quads; f += kEmbedThreads) {
#pragma unroll
            for (int r = 0; r < kEmbedRows; ++r) {
                float4 v = make_float4(__builtin_nanf(""), __builtin_nanf(""),
                                       __builtin_nanf(""), __builtin_nanf(""));
                if (inside[r]) {
                    const uint32_t d = codes16[id[r] * quads + f];
                    const float s = bf16_bits_to_f32(p.scales[id[r] * groups + f / 16]);
                    const float b = bf16_bits_to_f32(p.biases[id[r] * groups + f / 16]);
                    v = make_float4(embed_value(s, b, d & 15u), embed_value(s, b, (d >> 4) & 15u),
                                    embed_value(s, b, (d >> 8) & 15u), embed_value(s, b, d >> 12));
                }
                if (live[r])
                    embed_store(reinterpret_cast<float4 *>(p.out + (t0 + r) * p.K) + f, v);
            }
        }
    }
}

}  // namespace qg
