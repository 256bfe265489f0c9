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

}  // extern "C"
