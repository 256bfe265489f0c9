// probe.hip -- libqgprobe: two plain streaming kernels used only to measure
// the machine, never by the product path.
//   qg_probe_read  reads `bytes` with 16-byte loads (grid-stride, 256 threads
//                  per workgroup) and writes one word per workgroup: the
//                  achievable HBM read rate for a given size.
//   qg_probe_read_blocked  the same with one contiguous range per workgroup
//                  and 8 non-temporal loads in flight per thread.
//   qg_probe_copy  copies `bytes` with 16-byte loads and stores: a kernel of
//                  known traffic for calibrating the FETCH_SIZE / WRITE_SIZE
//                  counters.
//   qg_probe_stream  one contiguous range per wave, 16-byte non-temporal loads
//                  in batches of 8 KiB per wave with two batches in flight,
//                  in one of four modes: 0 LDS-direct loads only, 1 the same
//                  with each batch read back from LDS into registers, 2 each
//                  batch read back and given the arithmetic of a matrix-core
//                  batch-1 4-bit kernel (unpack to bf16 through the FP8
//                  converter, one 16x16x32 bf16 MFMA per dword, a scale fold
//                  per two), 3 that arithmetic on loads into registers.
#include <hip/hip_runtime.h>
#include <stdint.h>

__global__ __launch_bounds__(256) void qg_probe_read_kernel(const uint4 *p, int64_t n, uint32_t *out)
{
    // four independent 16-byte loads in flight per thread per iteration
    uint32_t acc = 0;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const uint4 a = p[i];
        const uint4 b = p[i + stride];
        const uint4 c = p[i + 2 * stride];
        const uint4 d = p[i + 3 * stride];
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < n; i += stride) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // keep the loads: one word per workgroup (xor over lanes via LDS atomics)
    __shared__ uint32_t s;
    if (threadIdx.x == 0) s = 0;
    __syncthreads();
    atomicXor(&s, acc);
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = s;
}

// Blocked variant: workgroup w reads the contiguous range [w, w + 1) * n /
// grid; each thread keeps 8 non-temporal 16-byte loads in flight and every
// wave instruction covers 1 KiB of consecutive bytes.
typedef unsigned probe_u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void qg_probe_read_blocked_kernel(const uint4 *p, int64_t n, uint32_t *out)
{
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * n / gridDim.x;
    const int64_t hi = static_cast<int64_t>(blockIdx.x + 1) * n / gridDim.x;
    const auto *q = reinterpret_cast<const probe_u32x4 *>(p);
    uint32_t acc = 0;
    int64_t i = lo + threadIdx.x;
    for (; i + 7 * 256 < hi; i += 8 * 256) {
        probe_u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(q + i + 256 * u);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < hi; i += 256) {
        const probe_u32x4 v = __builtin_nontemporal_load(q + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t s;
    if (threadIdx.x == 0) s = 0;
    __syncthreads();
    atomicXor(&s, acc);
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = s;
}

__global__ __launch_bounds__(256) void qg_probe_copy_kernel(const uint4 *src, uint4 *dst, int64_t n)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

typedef const __attribute__((address_space(1))) void *probe_gptr_t;
typedef __attribute__((address_space(3))) void *probe_lptr_t;
typedef __bf16 probe_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float probe_f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kProbeBatch = 8;                                     // 1 KiB loads per wave and batch
constexpr int kProbeStreamLds = 4 * 2 * kProbeBatch * 1024;        // 4 waves, two batches each

__device__ __forceinline__ probe_bf16x8_t probe_nibbles_to_bf16(uint32_t d)
{
    const uint32_t lo = d & 0x0f0f0f0fu, hi = (d >> 4) & 0x0f0f0f0fu;
    probe_u32x4 v;
    v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, false));
    v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, true));
    v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, false));
    v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, true));
    return __builtin_bit_cast(probe_bf16x8_t, v);
}

template <int MODE>
__global__ __launch_bounds__(256) void qg_probe_stream_kernel(const probe_u32x4 *q, int64_t n, uint32_t *out)
{
    constexpr int U = kProbeBatch;
    extern __shared__ __attribute__((aligned(16))) unsigned char probe_lds[];
    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + w, nw = static_cast<int64_t>(gridDim.x) * 4;
    const int64_t lo = wid * n / nw, hi = (wid + 1) * n / nw;   // this wave's 16-byte elements
    unsigned char *mine = probe_lds + w * (2 * U * 1024);
    const uint32_t a0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((probe_lptr_t)mine)) + 16 * l;
    const int64_t step = U * 64;
    probe_f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    uint32_t x = 0;
    const probe_bf16x8_t xa = __builtin_bit_cast(
        probe_bf16x8_t, probe_u32x4{0x3f803f80u ^ static_cast<uint32_t>(l), 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
    auto work = [&](probe_u32x4 (&v)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (MODE >= 2) {
#pragma unroll
                for (int k = 0; k < 4; k += 2) {
                    probe_f32x4_t tt = {0.f, 0.f, 0.f, 0.f};
                    tt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, probe_nibbles_to_bf16(v[u][k]), tt, 0, 0, 0);
                    tt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, probe_nibbles_to_bf16(v[u][k + 1]), tt, 0, 0, 0);
                    const float sc = __uint_as_float(0x3f800000u | (v[u][k] & 0xff00u));
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = fmaf(sc, tt[i], acc[i]);
                }
            } else {
                x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
            }
        }
    };
    if constexpr (MODE <= 2) {
        // batch at element i into buffer h: lane l's 16 bytes of load u land
        // at mine + (h U + u) KiB + 16 l
        auto issue = [&](int64_t i, int h) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t e = i + u * 64 + l;
                if (e < hi)
                    __builtin_amdgcn_global_load_lds((probe_gptr_t)(q + e), (probe_lptr_t)(mine + (h * U + u) * 1024),
                                                     16, 0, 2);
            }
        };
        issue(lo, 0);
        if (lo + step < hi) issue(lo + step, 1);
        int h = 0;
        for (int64_t i = lo; i < hi; i += step) {
            // the batch at i is complete when only the next one (if full) is pending
            if (i + 2 * step <= hi) __builtin_amdgcn_s_waitcnt(0x0F70 | U);
            else __builtin_amdgcn_s_waitcnt(0x0F70);
            if constexpr (MODE >= 1) {
                probe_u32x4 v[U];
#pragma unroll
                for (int u = 0; u < U; ++u)
                    asm volatile("ds_read_b128 %0, %1" : "=v"(v[u]) : "v"(a0 + (h * U + u) * 1024));
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int u = 0; u < U; ++u) asm volatile("" : "+v"(v[u]));
                if (i + 2 * step < hi) issue(i + 2 * step, h);
                work(v);
            } else if (i + 2 * step < hi) {
                issue(i + 2 * step, h);
            }
            h ^= 1;
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);
    } else {
        probe_u32x4 A[U], B[U];
        auto ld = [&](int64_t i, probe_u32x4 (&v)[U]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t e = i + u * 64 + l;
                v[u] = e < hi ? __builtin_nontemporal_load(q + e) : probe_u32x4{0u, 0u, 0u, 0u};
            }
        };
        int64_t i = lo;
        ld(i, A);
        for (; i < hi; i += 2 * step) {
            if (i + step < hi) ld(i + step, B);
            work(A);
            if (i + step < hi) {
                if (i + 2 * step < hi) ld(i + 2 * step, A);
                work(B);
            }
        }
    }
    // keep the work: one word per workgroup, written only on an impossible value
    const bool impossible = MODE >= 2 ? (acc[0] == 1.25f && acc[1] == -7.f) : x == 0x12345u;
    if (impossible) out[blockIdx.x] = static_cast<uint32_t>(t);
}

extern "C" {

// out must hold `grid` words. bytes must be a multiple of 16; pointers 16-byte aligned.
int qg_probe_read(const void *p, int64_t bytes, uint32_t *out, int grid, hipStream_t stream)
{
    if (!p || !out || bytes < 16 || bytes % 16 || grid < 1) return -1;
    (void)hipGetLastError();
    hipLaunchKernelGGL(qg_probe_read_kernel, dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint4 *>(p), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

// The blocked variant of qg_probe_read (same arguments and limits).
int qg_probe_read_blocked(const void *p, int64_t bytes, uint32_t *out, int grid, hipStream_t stream)
{
    if (!p || !out || bytes < 16 || bytes % 16 || grid < 1) return -1;
    (void)hipGetLastError();
    hipLaunchKernelGGL(qg_probe_read_blocked_kernel, dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint4 *>(p), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

int qg_probe_copy(const void *src, void *dst, int64_t bytes, int grid, hipStream_t stream)
{
    if (!src || !dst || bytes < 16 || bytes % 16 || grid < 1) return -1;
    (void)hipGetLastError();
    hipLaunchKernelGGL(qg_probe_copy_kernel, dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

// The streaming variants of qg_probe_read (same arguments and limits; mode
// 0..3 as listed at the top; out is written only in an impossible case).
int qg_probe_stream(const void *p, int64_t bytes, uint32_t *out, int grid, int mode, hipStream_t stream)
{
    if (!p || !out || bytes < 16 || bytes % 16 || grid < 1 || mode < 0 || mode > 3) return -1;
    (void)hipGetLastError();
    const auto *q = static_cast<const probe_u32x4 *>(p);
    const int64_t n = bytes / 16;
    const dim3 g(grid), b(256);
    switch (mode) {
    case 0: hipLaunchKernelGGL(qg_probe_stream_kernel<0>, g, b, kProbeStreamLds, stream, q, n, out); break;
    case 1: hipLaunchKernelGGL(qg_probe_stream_kernel<1>, g, b, kProbeStreamLds, stream, q, n, out); break;
    case 2: hipLaunchKernelGGL(qg_probe_stream_kernel<2>, g, b, kProbeStreamLds, stream, q, n, out); break;
    default: hipLaunchKernelGGL(qg_probe_stream_kernel<3>, g, b, 0, stream, q, n, out); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"
