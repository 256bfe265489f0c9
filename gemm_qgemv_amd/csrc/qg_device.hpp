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

// Value of lane (this lane ^ mask) of the wave, 0 < mask < 64 (a plain
// ds_bpermute: the partner always exists in a 64-lane wave, so no width
// check is needed).
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v, int mask)
{
    const int src = static_cast<int>(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u))) ^ mask;
    return static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src << 2, static_cast<int>(v)));
}

__device__ __forceinline__ float lane_xor_f32(float v, int mask)
{
    return __uint_as_float(lane_xor_u32(__float_as_uint(v), mask));
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask)
{
    const uint32_t lo = lane_xor_u32(static_cast<uint32_t>(v), mask);
    const uint32_t hi = lane_xor_u32(static_cast<uint32_t>(v >> 32), mask);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Reduce V = 2^P per-lane values across the 64 lanes of a wave in one
// butterfly: at each of the first P exchange steps every lane hands half of
// its values to its partner and keeps the other half, so the work is about
// V shuffles instead of 6 * V. On return vals[0] of lane l holds the total
// of value index (l >> (6 - P)); the order of additions is fixed, so the
// result is deterministic. Every step is instantiated at compile time, so
// all register indices are constants.
template <int V, int O, int N>
__device__ __forceinline__ void transpose_step(float (&vals)[V], int lane)
{
    if constexpr (O >= 1) {
        if constexpr (N > 1) {
            const bool upper = (lane & O) != 0;
#pragma unroll
            for (int i = 0; i < N / 2; ++i) {
                const float send = upper ? vals[i] : vals[i + N / 2];
                const float keep = upper ? vals[i + N / 2] : vals[i];
                vals[i] = keep + __shfl_xor(send, O);
            }
            transpose_step<V, O / 2, N / 2>(vals, lane);
        } else {
            vals[0] += __shfl_xor(vals[0], O);
            transpose_step<V, O / 2, 1>(vals, lane);
        }
    }
}

template <int V>
__device__ __forceinline__ void wave_transpose_reduce(float (&vals)[V], int lane)
{
    static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V must be a power of two <= 64");
    transpose_step<V, 32, V>(vals, lane);
}

// ---------------------------------------------------------------------------
// Cross-lane sums without LDS: DPP and the gfx950 permlane swaps.
//
// pair_sum<S>(x) adds to x the value of another lane at exchange step S:
//   S=0  DPP quad_perm [1,0,3,2]        lane ^ 1
//   S=1  DPP quad_perm [2,3,0,1]        lane ^ 2
//   S=2  DPP row_ror:4                  lane rotated by 4 within its 16-lane row
//   S=3  DPP row_ror:8                  lane rotated by 8 within its 16-lane row
//   S=4  v_permlane16_swap              lane ^ 16
//   S=5  v_permlane32_swap              lane ^ 32
// S=0,1,4,5 pair each lane with its xor partner. S=2 followed by S=3 sums
// the four lanes that differ only in bits 2 and 3 (as a cyclic sum), so the
// two are only ever used together, on values that do not depend on those
// bits. The swap steps return both halves of the exchange; their sum is the
// lane's value plus its partner's on every lane.
// ---------------------------------------------------------------------------

template <int S>
__device__ __forceinline__ float pair_sum(float x)
{
    if constexpr (S <= 3) {
        constexpr int ctrl = S == 0 ? 0xB1 : S == 1 ? 0x4E : S == 2 ? 0x124 : 0x128;
        return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xF, 0xF, false));
    } else if constexpr (S == 4) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}

// The larger of a 64-bit key and its partner's at exchange step S (the
// steps of pair_sum; S=2 and S=3 together give the maximum over the four
// lanes that differ in bits 2 and 3, as max is idempotent).
template <int S>
__device__ __forceinline__ uint64_t pair_max_u64(uint64_t k)
{
    const uint32_t lo = static_cast<uint32_t>(k), hi = static_cast<uint32_t>(k >> 32);
    uint64_t a, b;
    if constexpr (S <= 3) {
        constexpr int ctrl = S == 0 ? 0xB1 : S == 1 ? 0x4E : S == 2 ? 0x124 : 0x128;
        const uint32_t plo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(lo), ctrl, 0xF, 0xF, false));
        const uint32_t phi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(hi), ctrl, 0xF, 0xF, false));
        a = k;
        b = (static_cast<uint64_t>(phi) << 32) | plo;
    } else {
        const auto rl = S == 4 ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                               : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
        const auto rh = S == 4 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                               : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
        a = (static_cast<uint64_t>(rh[0]) << 32) | rl[0];
        b = (static_cast<uint64_t>(rh[1]) << 32) | rl[1];
    }
    return a > b ? a : b;
}

// Maximum of a 64-bit key over the 64 lanes of the wave, in every lane
// (DPP and permlane swaps: no LDS round trips).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k)
{
    k = pair_max_u64<0>(k);
    k = pair_max_u64<1>(k);
    k = pair_max_u64<2>(k);
    k = pair_max_u64<3>(k);
    k = pair_max_u64<4>(k);
    return pair_max_u64<5>(k);
}

// Exchange steps used to halve the value count: partners must hold the same
// value indices, so only the xor steps (bits 0, 1, 4, 5) qualify. The other
// steps then sum the single remaining value.
template <int V> struct Halving;
template <> struct Halving<1>  { static constexpr int n = 0; static constexpr int bits[1] = {0}; };
template <> struct Halving<2>  { static constexpr int n = 1; static constexpr int bits[1] = {0}; };
template <> struct Halving<4>  { static constexpr int n = 2; static constexpr int bits[2] = {0, 1}; };
template <> struct Halving<8>  { static constexpr int n = 3; static constexpr int bits[3] = {0, 1, 4}; };
template <> struct Halving<16> { static constexpr int n = 4; static constexpr int bits[4] = {0, 1, 4, 5}; };

template <int V>
__host__ __device__ constexpr int halving_mask()
{
    int m = 0;
    for (int h = 0; h < Halving<V>::n; ++h) m |= 1 << Halving<V>::bits[h];
    return m;
}

template <int V, int H>
__device__ __forceinline__ void halving_step(float (&v)[V], int lane)
{
    if constexpr (H < Halving<V>::n) {
        constexpr int S = Halving<V>::bits[H];
        constexpr int n = V >> H;
        const bool upper = (lane >> S) & 1;
#pragma unroll
        for (int i = 0; i < n / 2; ++i) {
            const float lo = pair_sum<S>(v[i]);
            const float hi = pair_sum<S>(v[i + n / 2]);
            v[i] = upper ? hi : lo;
        }
        halving_step<V, H + 1>(v, lane);
    }
}

template <int V, int S>
__device__ __forceinline__ void plain_steps(float &x)
{
    if constexpr (S <= 5) {
        if constexpr (((halving_mask<V>() >> S) & 1) == 0) x = pair_sum<S>(x);
        plain_steps<V, S + 1>(x);
    }
}

// Reduce V <= 16 per-lane values across the wave. On return v[0] of lane l
// holds the total of value index dpp_owner<V>(l); lanes with
// dpp_writer<V>(l) true hold V distinct indices, one each. The order of the
// additions is fixed and the same for every value index.
template <int V>
__device__ __forceinline__ void wave_reduce_dpp(float (&v)[V], int lane)
{
    halving_step<V, 0>(v, lane);
    plain_steps<V, 0>(v[0]);
}

template <int V>
__device__ __forceinline__ int dpp_owner(int lane)
{
    int own = 0;
#pragma unroll
    for (int h = 0; h < Halving<V>::n; ++h)
        own += ((lane >> Halving<V>::bits[h]) & 1) * (V >> (h + 1));
    return own;
}

template <int V>
__device__ __forceinline__ bool dpp_writer(int lane)
{
    return (lane & (63 & ~halving_mask<V>())) == 0;
}

}  // namespace qg
