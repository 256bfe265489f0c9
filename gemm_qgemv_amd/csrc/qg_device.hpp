// qg_device.hpp -- small device helpers shared by the libqg kernels:
// half-precision decoding, the order-preserving argmax key, and wavefront
// reductions for 64-wide waves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

constexpr int kWave = 64;

// bf16 bit pattern -> float32 (the pattern is the top half of a binary32).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16)
{
    return __uint_as_float(bits16 << 16);
}

// fp16 bit pattern -> float32 (hardware conversion; fp16 subnormals are
// preserved on gfx950 in the default floating-point mode).
__device__ __forceinline__ float fp16_bits_to_f32(uint16_t bits)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, bits));
}

// Order-preserving map of a float32 onto uint32: a < b  <=>  ord(a) < ord(b)
// for all non-NaN values, after -0 has been folded onto +0.
__device__ __forceinline__ uint32_t float_order_bits(float v)
{
    v = v + 0.0f;  // -0 + +0 = +0 under round-to-nearest-even
    uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Argmax key: larger value wins; for equal values the lower index wins.
// Key 0 is below every real key.
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t index)
{
    return (static_cast<uint64_t>(float_order_bits(v)) << 32) |
           static_cast<uint64_t>(0xFFFFFFFFu - index);
}

__device__ __forceinline__ uint32_t argmax_key_index(uint64_t key)
{
    return 0xFFFFFFFFu - static_cast<uint32_t>(key & 0xFFFFFFFFu);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask)
{
    uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
    lo = __shfl_xor(lo, mask);
    hi = __shfl_xor(hi, mask);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Reduce V = 2^P per-lane values across the 64 lanes of a wave in one
// butterfly: at each of the first P exchange steps every lane hands half of
// its values to its partner and keeps the other half, so the work is about
// V shuffles instead of 6 * V. On return vals[0] of lane l holds the total
// of value index (l >> (6 - P)); the order of additions is fixed, so the
// result is deterministic.
template <int V>
__device__ __forceinline__ void wave_transpose_reduce(float (&vals)[V], int lane)
{
    static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V must be a power of two <= 64");
    int n = V;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        if (n > 1) {
            const bool upper = (lane & o) != 0;
#pragma unroll
            for (int i = 0; i < V / 2; ++i) {
                if (i < n / 2) {
                    float send = upper ? vals[i] : vals[i + n / 2];
                    float keep = upper ? vals[i + n / 2] : vals[i];
                    vals[i] = keep + __shfl_xor(send, o);
                }
            }
            n >>= 1;
        } else {
            vals[0] += __shfl_xor(vals[0], o);
        }
    }
}

}  // namespace qg
