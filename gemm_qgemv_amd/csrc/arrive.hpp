// arrive.hpp -- cross-workgroup completion for the greedy head and the
// in-kernel split-K combine, robust to whatever the workspace's control
// words hold when a call starts.
//
// Completion word. A 64-bit word whose high half is the tag of the dispatch
// that owns it and whose low half counts the workgroups of that dispatch that
// have arrived. The tag is derived from the dispatch's AQL packet index and
// its queue, so two dispatches that use the same workspace one after the
// other carry different tags. A workgroup that arrives increments the word
// and looks at the value it returns. If that value carries this dispatch's
// tag, the low half is the number of workgroups that arrived before it, and
// the one that sees total - 1 is the last. Otherwise the word still held
// something else (leftovers of an earlier call, a call that never finished,
// uninitialised memory) and the increment did not count: the workgroup then
// claims the word with a compare-and-swap of the value it expects there for
// (tag, 1), which counts it in as the first; if the swap fails because the
// word changed, it retries against the new value, or, once the word carries
// the tag (another workgroup claimed it), counts itself in with a second
// increment. A claim only ever replaces a word without the tag, so counted
// increments are never lost, and every workgroup is counted exactly once.
// The dispatch's first workgroup claims the word as it starts
// (arrival_preclaim), long before any workgroup arrives, so normally no
// arrival takes the slow path, no swap reaches the word at the end, and the
// last workgroup's path to the end of the kernel is its data atomics, one
// increment and the final reads. Nothing has to be zero on
// entry, nothing is cleared on exit, and a call that was cut short or raced
// with another on the same workspace cannot disturb the calls after it.
//
// Ordering. Data moves between workgroups only through device-scope atomics
// (the parked keys and partial sums, the counters), which are performed at
// the device's coherence point rather than in an XCD's own L2. A returning
// atomic has been performed when its value comes back. Each workgroup issues
// its counter increment with an address that depends, through one vector
// AND with zero, on the values returned by every atomic that carried its
// data (or after a barrier that all those values have passed); the
// increment therefore cannot be performed before them. The last workgroup reads the parked data with device-scope atomic
// loads issued after its increment has returned, so it sees every value
// that was performed before the other workgroups counted themselves in. No
// cache writeback or invalidate is needed, because no plain store or load
// carries data between workgroups.
#pragma once

#include "qg_device.hpp"

namespace qg {

// Packet index of this dispatch in its queue (an implicit input of every
// kernel that asks for it).
extern "C" __device__ unsigned long long qg_llvm_dispatch_id() __asm("llvm.amdgcn.dispatch.id");

// 32-bit tag of this dispatch: its packet index mixed with its queue's
// address (dispatches on different queues count from the same start).
__device__ __forceinline__ uint32_t dispatch_tag()
{
    const uint64_t id = qg_llvm_dispatch_id();
    const uint64_t q = reinterpret_cast<uint64_t>(__builtin_amdgcn_queue_ptr());
    const uint64_t h = (q >> 6) * 0x9E3779B97F4A7C15ull;
    return static_cast<uint32_t>(id) ^ static_cast<uint32_t>(h >> 32);
}

// Control words at the start of every workspace: the greedy head's
// completion word, then one completion word per row tile for the in-kernel
// split-K combine.
struct GreedyCtl {
    unsigned long long arrive;
};
constexpr int kCtlBytes = 8192;
constexpr int kCtlTileOffset = 256;
constexpr int kCtlTileCounters = (kCtlBytes - kCtlTileOffset) / 8;

__device__ __forceinline__ unsigned long long *tile_counters(GreedyCtl *ctl)
{
    return reinterpret_cast<unsigned long long *>(reinterpret_cast<char *>(ctl) + kCtlTileOffset);
}

// Claim `word` for this dispatch as the kernel starts: one thread of one
// workgroup per word (the dispatch's first workgroup, which starts before
// the others arrive), so that the arrivals find the word claimed and take
// the fast path. Swaps only a word without the tag; a failed swap means the
// word changed, and the loop retries against the new value (it ends, since
// every change is one of the dispatch's few increments or claims).
__device__ __forceinline__ void arrival_preclaim(unsigned long long *word, uint32_t tag)
{
    unsigned long long cur = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (static_cast<uint32_t>(cur >> 32) != tag) {
        if (__hip_atomic_compare_exchange_strong(word, &cur, static_cast<unsigned long long>(tag) << 32,
                                                 __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            break;
    }
}

// Count the calling workgroup in (one thread); true for the last of `total`.
// `dep` folds together the values returned by the atomics that carried the
// workgroup's data: the increment's address depends on them (through one
// vector AND with zero), so it cannot be performed before them.
__device__ __forceinline__ bool arrival_last(unsigned long long *word, uint32_t tag, uint32_t dep,
                                             unsigned total)
{
    uint32_t zero;
    asm volatile("v_and_b32 %0, 0, %1" : "=v"(zero) : "v"(dep));
    unsigned long long old =
        __hip_atomic_fetch_add(word + zero, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (static_cast<uint32_t>(old >> 32) != tag) {
        // the word was not claimed for this dispatch yet: claim it, counted
        // as the first, or count again once another workgroup has claimed it
        unsigned long long cur = old + 1ull;
        for (;;) {
            if (static_cast<uint32_t>(cur >> 32) == tag) {
                old = __hip_atomic_fetch_add(word, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            if (__hip_atomic_compare_exchange_strong(word, &cur, (static_cast<unsigned long long>(tag) << 32) | 1ull,
                                                     __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT)) {
                old = static_cast<unsigned long long>(tag) << 32;
                break;
            }
            // cur now holds the word's current value
        }
    }
    return static_cast<uint32_t>(old) == total - 1u;
}

// ---------------------------------------------------------------------------
// In-kernel split-K combine: several workgroups own the same rows, each for
// a different chunk of K. splitk_put stores one partial sum with a returning
// device-scope exchange and waits for its return; splitk_arrive (all threads
// of the workgroup) then counts the workgroup in on its row tile's word, so
// the count moves only after every partial of the workgroup is in place. The
// workgroup that completes the count reads all partials back with
// device-scope atomic loads, in split order (splitk_sum).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void splitk_put(float *dst, float v)
{
    const float old = __hip_atomic_exchange(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::"v"(old));   // the exchange has returned
}

__device__ __forceinline__ float splitk_get(const float *src)
{
    return __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum of the nsplit partials part[s * stride], s = 0 .. nsplit-1, added in
// split order. The device-scope loads go out in batches of 8 before any of
// them is used (a plain loop would wait for each one in turn); a batch
// past the last split re-reads the last partial and drops it.
__device__ __forceinline__ float splitk_sum(const float *part, int64_t stride, int nsplit)
{
    constexpr int kBatch = 8;
    float acc = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += kBatch) {
        float v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) v[i] = splitk_get(part + min(s0 + i, nsplit - 1) * stride);
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (s0 + i < nsplit) acc += v[i];
    }
    return acc;
}

// All threads, after their splitk_put calls.
__device__ __forceinline__ bool splitk_arrive(unsigned long long *word, int nsplit, uint32_t tag)
{
    __shared__ unsigned s_last;
    __syncthreads();   // every thread's exchanges have returned
    if (threadIdx.x == 0) s_last = arrival_last(word, tag, 0u, static_cast<unsigned>(nsplit));
    __syncthreads();
    return s_last != 0;
}

// ---------------------------------------------------------------------------
// Greedy selection across workgroups. wg_key[b] (b < nb <= 16, in LDS) is
// this workgroup's best (value, index) key of activation row b. Each
// workgroup parks its nb keys in its own row of `keys` ([nwg][nb], any
// initial contents) with returning device-scope exchanges and counts itself
// in once; the last one reads every row back, reduces them and writes the
// indices. Must be reached by all threads of the workgroup. `lds_last` and `lds_best` (16 keys) are LDS scratch of the
// caller's choosing (greedy_finish_rows below brings its own).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void greedy_finish_rows_in(const unsigned long long *wg_key, int nb,
                                                      GreedyCtl *ctl, unsigned long long *keys,
                                                      int32_t *idx, int nwg, uint32_t tag,
                                                      unsigned *lds_last, unsigned long long *lds_best)
{
    unsigned &s_last = *lds_last;
    unsigned long long *s_best = lds_best;
    if (threadIdx.x == 0) {
        uint32_t dep = 0;
        for (int b = 0; b < nb; ++b) {
            const unsigned long long old = __hip_atomic_exchange(
                &keys[static_cast<int64_t>(blockIdx.x) * nb + b], wg_key[b], __ATOMIC_RELAXED,
                __HIP_MEMORY_SCOPE_AGENT);
            dep |= static_cast<uint32_t>(old) | static_cast<uint32_t>(old >> 32);
        }
        s_last = arrival_last(&ctl->arrive, tag, dep, static_cast<unsigned>(nwg));
    }
    if (threadIdx.x < 16) s_best[threadIdx.x] = 0ull;
    __syncthreads();
    if (!s_last) return;
    const int total = nwg * nb;
    if (nb == 1) {
        // one key per workgroup: the first wave alone reads them (each lane
        // a few, all requests in flight at once) and reduces them across
        // its lanes; no further barrier
        if (threadIdx.x >= 64) return;
        constexpr int kBatch = 8;   // loads per lane issued before any is used
        unsigned long long best = 0ull;
        for (int i0 = threadIdx.x; i0 < total; i0 += 64 * kBatch) {
            unsigned long long k[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                k[u] = __hip_atomic_load(&keys[min(i0 + 64 * u, total - 1)], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int u = 0; u < kBatch; ++u) best = k[u] > best ? k[u] : best;
        }
        best = wave_max_u64(best);
        if (threadIdx.x == 0) idx[0] = static_cast<int32_t>(argmax_key_index(best));
        return;
    } else if ((nb & (nb - 1)) == 0 && nb <= 8 && blockDim.x % 64 == 0) {
        // nb = 2, 4, 8: key i belongs to row i % nb = threadIdx.x % nb for
        // every key a thread reads (blockDim.x is a multiple of nb), so each
        // lane keeps one maximum, the lanes of a row meet across the wave
        // (DPP and permlane swaps), and each wave adds nb keys to LDS
        constexpr int kBatch = 4;   // loads per lane issued before any is used
        unsigned long long best = 0ull;
        for (int i0 = threadIdx.x; i0 < total; i0 += static_cast<int>(blockDim.x) * kBatch) {
            unsigned long long k[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int i = i0 + static_cast<int>(blockDim.x) * u;
                k[u] = __hip_atomic_load(&keys[i < total ? i : i0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) best = k[u] > best ? k[u] : best;
        }
        if (nb <= 2) best = pair_max_u64<1>(best);
        if (nb <= 4) best = pair_max_u64<2>(best);
        best = pair_max_u64<3>(best);
        best = pair_max_u64<4>(best);
        best = pair_max_u64<5>(best);
        if ((threadIdx.x & 63) < nb) atomicMax(&s_best[threadIdx.x & 63], best);
    } else {
        for (int i = threadIdx.x; i < total; i += blockDim.x) {
            const unsigned long long k =
                __hip_atomic_load(&keys[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            atomicMax(&s_best[i % nb], k);
        }
    }
    __syncthreads();
    if (threadIdx.x < nb) idx[threadIdx.x] = static_cast<int32_t>(argmax_key_index(s_best[threadIdx.x]));
}

__device__ __forceinline__ void greedy_finish_rows(const unsigned long long *wg_key, int nb,
                                                   GreedyCtl *ctl, unsigned long long *keys,
                                                   int32_t *idx, int nwg, uint32_t tag)
{
    __shared__ unsigned s_last;
    __shared__ unsigned long long s_best[16];
    greedy_finish_rows_in(wg_key, nb, ctl, keys, idx, nwg, tag, &s_last, s_best);
}

}  // namespace qg
