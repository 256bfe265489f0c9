// qg.hip -- libqg: host-side validation, shape dispatch and launches behind
// the C ABI declared in include/qg.h. All arithmetic runs in the kernels of
// gemv.hpp / gemm.hpp; this file only checks arguments, plans the launch
// geometry from (format, M, K, rows) and enqueues work on the caller's
// stream. It never allocates, copies or synchronizes.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/qg.h"
#include "embed.hpp"
#include "gemm.hpp"
#include "gemv.hpp"
#include "gemv1.hpp"
#include "gemv_b1.hpp"
#include "gemv_mfma.hpp"
#include "gemv_mfma16.hpp"
#include "gemv_stream.hpp"
#include "gemv_stream_mfma.hpp"

namespace {

using qg::GemvParams;

constexpr int64_t kMaxM = 0x7fffffffLL;
constexpr int64_t kMaxK = int64_t(1) << 30;
constexpr int64_t kMaxN = 0x7fffffffLL;
// Dynamic LDS a GEMV workgroup may use for its activation tile (gfx950 has
// 160 KiB per compute unit; this leaves room for two workgroups' worth of
// smaller tiles or one large one).
constexpr int64_t kLdsBudget = 96 * 1024;
// All of a compute unit's LDS: the small-batch matrix-core kernel runs one
// workgroup per compute unit and keeps the whole activation operand there.
constexpr int64_t kLdsMax = 160 * 1024;
constexpr int64_t kLdsStaticReserve = 1024;   // static LDS of a kernel (keys, flags)
// Compute units of the MI355X (one small-batch matrix-core workgroup each).
constexpr int64_t kComputeUnits = 256;
constexpr int64_t kAlign = 16;
constexpr int kThreads = 256;

bool known_format(int fmt)
{
    return fmt == QG_I8_ROW || fmt == QG_U4_G64 || fmt == QG_B1_G128 || fmt == QG_I8_G64;
}
int k_unit(int fmt)
{
    return fmt == QG_I8_ROW ? 16 : (fmt == QG_U4_G64 || fmt == QG_I8_G64) ? 64 : 128;
}
int k_per_slice(int fmt)
{
    return (fmt == QG_I8_ROW || fmt == QG_I8_G64) ? 16 : fmt == QG_U4_G64 ? 32 : 128;
}

int64_t row_bytes(int fmt, int64_t K)
{
    return (fmt == QG_I8_ROW || fmt == QG_I8_G64) ? K : fmt == QG_U4_G64 ? K / 2 : K / 8;
}
int64_t scale_bytes(int fmt, int64_t M, int64_t K)
{
    return fmt == QG_I8_ROW    ? 4 * M
           : fmt == QG_I8_G64  ? 4 * M * (K / 64)
           : fmt == QG_U4_G64  ? 2 * M * (K / 64)
                               : 2 * M * (K / 128);
}
int64_t bias_bytes(int fmt, int64_t M, int64_t K)
{
    return fmt == QG_U4_G64 ? 2 * M * (K / 64) : 0;
}

bool aligned(const void *p, int64_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// ---------------------------------------------------------------------------
// argument checks (host only, before anything is enqueued)
// ---------------------------------------------------------------------------

int check_weights(int fmt, const void *codes, const void *scales, const void *biases,
                  const float *x, int64_t M, int64_t K)
{
    if (!known_format(fmt)) return QG_ERR_FORMAT;
    if (!codes || !scales || !x) return QG_ERR_NULL;
    if ((fmt == QG_U4_G64) != (biases != nullptr)) return QG_ERR_NULL;
    if (M < 1 || M > kMaxM || K < 1 || K > kMaxK || K % k_unit(fmt) != 0) return QG_ERR_SHAPE;
    if (!aligned(codes, kAlign) || !aligned(scales, kAlign) || !aligned(x, kAlign) ||
        (biases && !aligned(biases, kAlign)))
        return QG_ERR_ALIGN;
    return QG_OK;
}

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void *p, int64_t bytes)
{
    uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + static_cast<uintptr_t>(bytes)};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

// Every written range must be disjoint from every input range and from
// every other written range (an exact alias such as y == x is an overlap
// like any other).
int check_alias(const Range *inputs, int n_inputs, const Range *written, int n_written)
{
    for (int i = 0; i < n_written; ++i)
        for (int j = 0; j < n_inputs; ++j)
            if (overlap(written[i], inputs[j])) return QG_ERR_ALIAS;
    for (int i = 0; i < n_written; ++i)
        for (int j = i + 1; j < n_written; ++j)
            if (overlap(written[i], written[j])) return QG_ERR_ALIAS;
    return QG_OK;
}

int launch_status()
{
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

// ---------------------------------------------------------------------------
// GEMV plan: a pure function of (fmt, M, K, batch, argmax)
// ---------------------------------------------------------------------------

// Batch-1 kernel tuning (compile-time; the plan is a pure function of the
// call's shape).
constexpr int64_t kGemv1Waves = 2048;     // waves the rows are spread over (at most)
constexpr bool kGemv1Nt = true;           // non-temporal weight loads (streamed once)
constexpr int kGemv1R = 4;                // rows per block when K fits in one or two slices per lane
constexpr int64_t kGemv1MinWaves = 1024;  // fewer rows per block until this many waves

// Workspace: the first kCtlBytes are completion words (the greedy head's,
// then one per row tile of the in-kernel split-K combine), claimed by each
// dispatch that counts on them whatever they hold; the rest is scratch.
constexpr size_t kCtlBytes = qg::kCtlBytes;
static_assert(kCtlBytes == QG_WS_CONTROL_BYTES, "control area and header disagree");
static_assert(sizeof(qg::GreedyCtl) <= qg::kCtlTileOffset, "greedy control words exceed their area");

// K per workgroup of the 1-bit lookup kernel: 1024 (26 KiB of LDS, six
// workgroups per compute unit) or 2048 (50 KiB, three). The larger chunk
// halves the partial sums to combine, and is taken when K is long and its
// grid still fits in one round of resident workgroups (5120 x 17408: 11.2
// against 13.7 us; 17408 x 5120 would need 816 workgroups and stays at
// 1024: 10.2 against 13.1 us).
constexpr int kB1Chunk = 1024;
constexpr int kB1ChunkLong = 2048;
constexpr int kB1ChunkWide = 512;        // chunk of the 8-row tables (64 KiB of LDS)
constexpr int64_t kB1LongResident = 3;   // workgroups per compute unit at the long chunk

struct GemvPlan {
    bool gemm;           // small batch run as the prefill product on narrow tiles
    bool mfma;           // small-batch 4-bit kernel on the matrix cores
    bool mfma16;         // 9..16 rows of the 4-bit format in one pass (K cut across waves)
    int gw;              // mfma16: groups of 64 inputs per wave (K / 512)
    int passes;          // small-batch kernel: launches of up to 8 activation rows each
    bool lut;            // batch-1 1-bit kernel (table lookup, lanes along rows)
    bool fused;          // split-K combined inside the kernel (per-tile counters);
                         // small-batch kernel: outputs staged in LDS
    bool stream;         // batch-1 4-bit kernel with loader waves (large M, K = 2048 nc)
    int nc;              // stream kernel: 1 KiB code chunks per row
    bool smfma;          // 2..8 rows, 4-bit, K = 2048: loader waves + matrix cores
    bool one;            // batch-1 kernel (8-bit / 4-bit, activations in registers)
    int ns;              // batch-1 kernel: slices per lane
    bool full;           // batch-1 kernel: every lane owns all NS slices
    int64_t rows_per_wave;
    int wg_waves;          // batch 1: waves per workgroup
    int B, R;
    int64_t kc;
    int nsplit;
    int64_t rows_per_wg, grid_x;
    size_t lds_bytes;
    int64_t comb_rows_per_wg, comb_grid;
    int nkeys;
    size_t part_off, key_off, ws_bytes;
};

// The matrix-core prefill product over N token rows, K split when its grid
// is small (defined below), and the workspace that needs.
size_t gemm_mfma_workspace(int fmt, int64_t M, int64_t K, int64_t N);
void run_gemm_mfma(int fmt, const void *codes, const void *scales, const void *biases,
                   const float *x, float *y, int64_t M, int64_t K, int64_t N, void *ws,
                   hipStream_t s);

// The 4-bit small-batch matrix-core kernel stages all of K in LDS.
bool u4_mfma_ok(int fmt, int64_t K)
{
    return fmt == QG_U4_G64 && K % (64 * qg::kMfmaChunk) == 0 &&
           K <= static_cast<int64_t>(qg::kStageItems) * qg::kMfmaThreads &&
           static_cast<int64_t>(qg::gemv_mfma_lds_bytes(K)) + kLdsStaticReserve <= kLdsMax;
}

// The one-pass kernel for up to 16 rows keeps each wave's share of K (a
// multiple of 128 inputs) for all 16 rows in registers: K = 1024 or 2048,
// 4-bit and both 8-bit formats.
bool mfma16_ok(int fmt, int64_t K)
{
    return known_format(fmt) && (K == 1024 || K == 2048);
}

// Fewest rows for the one-pass kernel: 8-bit and 1-bit 3 (the vector-ALU
// and lookup kernels are as fast at 2; 1-bit 4096 x 2048 at 3 / 16 rows
// 9.5 / 14.3 -> 6.3 / 9.6 us), 4-bit 2.
int one_pass_min_rows(int fmt)
{
    return fmt == QG_U4_G64 ? 2 : 3;
}

// 4-bit: it takes 9..16 rows (one pass instead of two launches of 8), and
// 2..8 rows when the 8-row kernel (each wave its own run of tiles) would
// leave compute units without a workgroup: 6144 x 2048 at 2..8 rows
// 15.2-15.8 -> 7.7-8.8 us; on the 151936 x 2048 head the 8-row kernel stays
// ~6% ahead. 8-bit: 3..16 rows, in place of the vector-ALU kernel (3584 x
// 1024 at 16 rows 9.5 -> 6.8 us, 4096 x 2048 25.6 -> 9.6 us, 151936 x 1024
// 123 -> 46 us); at 2 rows that kernel is as fast or faster.
bool one_pass(int fmt, int64_t M, int64_t K, int nb)
{
    if (nb < one_pass_min_rows(fmt) || !mfma16_ok(fmt, K)) return false;
    if (fmt != QG_U4_G64) return true;
    return nb > 8 || ceil_div(ceil_div(M, 16), qg::kMfmaWaves) < kComputeUnits;
}

// Other K for the one-pass kernel: slices of 2048 (or 1024, or 512) inputs over a
// second grid dimension, each writing partial outputs to the workspace,
// which the split-K combine kernel adds in slice order. 0: not available.
// Matrix-vector calls only (the greedy head keeps its own kernels).
int64_t one_pass_slice(int fmt, int64_t K)
{
    if (!known_format(fmt) || mfma16_ok(fmt, K)) return 0;
    if (K % 2048 == 0 && K / 2048 <= 8) return 2048;
    if (K % 1024 == 0 && K / 1024 <= 8) return 1024;
    // 8-bit: slices of 512 (one group per wave; 1024 x 3584 in 7)
    if ((fmt == QG_I8_ROW || fmt == QG_I8_G64) && K % 512 == 0 && K / 512 <= 8) return 512;
    return 0;
}

// From 3 rows (at 2 the vector-ALU kernel is as fast or faster): 4-bit
// 4096 x 4096 at 16 rows 69 -> 20.6 us, 17408 x 16384 484 -> 122 us, 8-bit
// 4096 x 4096 63 -> 20 us. 1-bit from 6 rows (the lookup kernel is faster
// at 3..4): 17408 x 5120 at 6 / 16 rows 37.2 / 47.9 -> 29.3 / 38.8 us. At
// most 8 slices (17 slices of 5120 x 17408 ran at half the lookup kernel's
// speed).
// 8-bit in several slices of 512 from 6 rows as well (4096 x 1536 and
// 14336 x 2560 at 3..4 rows: 7.4 -> 9.1 and 18.8 -> 20.8 us, at 16 rows
// 24.4 -> 12.8 and 97.8 -> 27.2 us; 1024 x 3584 at 16 rows 15.4 -> 10.1).
bool split_pass(int fmt, int64_t K, int nb, bool argmax)
{
    const int64_t slice = one_pass_slice(fmt, K);
    const int min_rows = fmt == QG_B1_G128 || (slice == 512 && K > 512) ? 6 : 3;
    return !argmax && slice > 0 && nb >= min_rows;
}

// Whether nb (2..16) activation rows run faster as the prefill product on
// narrow tiles (weights read once, 16 token rows of matrix-core work) than
// on the matrix-vector kernels. Estimates in microseconds, fitted to
// MI355X measurements (8-bit 3584 x 1024 and 1024 x 3584, 4-bit 6144 x 2048,
// 2048 x 6144 and 151936 x 2048, 1-bit 17408 x 5120 and 5120 x 17408):
//   prefill, narrow tiles     10 + 96 M K / R, R = 220e6 flop/us (1-bit, on
//                             128-row tiles with K split four ways per
//                             compute unit: 280e6)
//   4-bit matrix-core matvec  one pass (K = 1024 or 2048): the weight bytes
//                             at 3.4 TB/s, at least 8; else per launch of up
//                             to 8 rows the weight bytes at 4.4 TB/s, at
//                             least 14
//   1-bit lookup kernel       8 + nb M K / 14e6
// and the vector-ALU and lookup kernels lose from 6 rows on matrices wider
// than tall, whose few rows leave their grids small.
bool batch_on_gemm(int fmt, int64_t M, int64_t K, int nb)
{
    if (nb < 2 || K > qg::kGemmMaxK) return false;
    const double w = static_cast<double>(M) * static_cast<double>(K);
    const double t_gemm = 10.0 + 96.0 * w / (fmt == QG_B1_G128 ? 280e6 : 220e6);
    if (one_pass(fmt, M, K, nb)) {
        const double bytes = static_cast<double>(M) * (row_bytes(fmt, K) + 4 * (K / 64));
        return t_gemm < std::max(8.0, bytes / 3.4e6);
    }
    if (split_pass(fmt, K, nb, false)) {
        const double bytes = static_cast<double>(M) * (row_bytes(fmt, K) + 4 * (K / 64));
        return t_gemm < std::max(8.0, bytes / 3.4e6) + 2.0;
    }
    if (u4_mfma_ok(fmt, K)) {
        const double bytes = static_cast<double>(M) * (row_bytes(fmt, K) + 4 * (K / 64));
        return t_gemm < static_cast<double>(ceil_div(nb, 8)) * std::max(14.0, bytes / 4.4e6);
    }
    if (M < K && nb >= 6) return true;
    return fmt == QG_B1_G128 && t_gemm < 8.0 + nb * w / 14e6;
}

// The batch-1 stream kernel: 4-bit rows of 1, 2 or 4 KiB of codes (K =
// 2048, 4096, 8192), and at least four stages of rows per workgroup when
// each compute unit takes one workgroup (fewer leave the ring unfilled; the
// register-streaming kernel serves those).
bool stream_ok(int fmt, int64_t M, int64_t K)
{
    if (fmt != QG_U4_G64 || (K != 2048 && K != 4096 && K != 8192)) return false;
    const int64_t rows_per_stage = 32 / (K / 2048);
    return M >= kComputeUnits * rows_per_stage * 4;
}

// The small-batch stream kernel: 4-bit rows of K = 2048 inputs, 2..8
// activation rows, at least four stages of 32 rows per workgroup.
bool stream_mfma_ok(int fmt, int64_t M, int64_t K, int nb)
{
    return fmt == QG_U4_G64 && K == qg::kStreamMfmaK && nb >= 2 && nb <= qg::kStreamMfmaRows &&
           M >= kComputeUnits * 32 * 4;
}

GemvPlan plan_gemv(int fmt, int64_t M, int64_t K, int nb, bool argmax)
{
    GemvPlan pl{};
    if (!argmax && nb >= 2 && batch_on_gemm(fmt, M, K, nb)) {
        pl.gemm = true;
        pl.ws_bytes = gemm_mfma_workspace(fmt, M, K, nb);
        return pl;
    }
    if (nb == 1 && stream_ok(fmt, M, K)) {
        // batch 1, 4-bit, large M: one workgroup per compute unit, loader
        // waves streaming the rows through LDS
        pl.stream = true;
        pl.nc = static_cast<int>(K / 2048);
        pl.grid_x = kComputeUnits;
        pl.nsplit = 1;
        if (argmax) {
            pl.nkeys = static_cast<int>(pl.grid_x);
            pl.key_off = kCtlBytes;
            pl.ws_bytes = align256(kCtlBytes + static_cast<size_t>(pl.grid_x) * 8);
        }
        return pl;
    }
    if (stream_mfma_ok(fmt, M, K, nb)) {
        // a few rows, 4-bit, large M: one workgroup per compute unit, loader
        // waves streaming the rows through LDS, matrix cores reducing them
        pl.smfma = true;
        pl.grid_x = kComputeUnits;
        pl.nsplit = 1;
        if (argmax) {
            pl.nkeys = static_cast<int>(pl.grid_x);
            pl.key_off = kCtlBytes;
            pl.ws_bytes = align256(kCtlBytes + static_cast<size_t>(pl.grid_x) * nb * 8);
        }
        return pl;
    }
    const int64_t S = K / k_per_slice(fmt);
    if (nb == 1 && fmt != QG_B1_G128 && ceil_div(S, 64) <= 4) {
        // batch 1: workgroups of 4 independent waves, each wave a
        // contiguous run of rows
        pl.one = true;
        pl.ns = static_cast<int>(ceil_div(S, 64));
        pl.full = S % 64 == 0;
        pl.R = pl.ns >= 3 ? 2 : kGemv1R;
        while (pl.R > 1 && ceil_div(M, pl.R) < kGemv1MinWaves) pl.R /= 2;
        pl.rows_per_wave = round_up(ceil_div(M, kGemv1Waves), pl.R);
        // greedy head: 8-wave workgroups where K takes one or two slices per
        // lane (half the workgroups folding their keys into the shared slot
        // at the end: 6144 x 2048 4-bit 11.0 -> 8.9 us); the 3- and 4-slice
        // kernels keep more, smaller workgroups
        pl.wg_waves = argmax && pl.ns <= 2 ? 8 : 4;
        pl.grid_x = ceil_div(ceil_div(M, pl.rows_per_wave), pl.wg_waves);
        pl.nsplit = 1;
        if (argmax) {
            // one parked greedy key per workgroup after the control words
            pl.nkeys = static_cast<int>(pl.grid_x);
            pl.key_off = kCtlBytes;
            pl.ws_bytes = align256(kCtlBytes + static_cast<size_t>(pl.grid_x) * 8);
        }
        return pl;
    }
    const bool split = split_pass(fmt, K, nb, argmax);
    if (split || one_pass(fmt, M, K, nb)) {
        // one pass over the weights with K cut across the 8 waves of a
        // workgroup per compute unit, each workgroup a run of 16-row tiles;
        // longer K in slices over the second grid dimension
        pl.mfma16 = true;
        const int64_t slice = split ? one_pass_slice(fmt, K) : K;
        pl.gw = static_cast<int>(slice / 512);
        pl.nsplit = static_cast<int>(K / slice);
        const int64_t ntiles = ceil_div(M, 16);
        pl.grid_x = std::min<int64_t>(kComputeUnits, ntiles);
        pl.lds_bytes = qg::gemv_mfma16_lds_bytes();
        const size_t out_bytes = static_cast<size_t>(ceil_div(ntiles, pl.grid_x)) * qg::k16TileOutBytes;
        pl.fused = static_cast<int64_t>(pl.lds_bytes + out_bytes) + kLdsStaticReserve <= kLdsMax;
        if (pl.fused) pl.lds_bytes += out_bytes;
        if (pl.nsplit > 1) {
            // partial outputs after the control words
            pl.part_off = kCtlBytes;
            pl.ws_bytes = align256(kCtlBytes + static_cast<size_t>(pl.nsplit) * nb * M * 4);
        }
        if (argmax) {
            // per-workgroup greedy keys (up to 16 per workgroup) after the control words
            pl.nkeys = static_cast<int>(pl.grid_x);
            pl.key_off = kCtlBytes;
            pl.ws_bytes = align256(kCtlBytes + static_cast<size_t>(pl.grid_x) * 16 * 8);
        }
        return pl;
    }
    if (fmt == QG_B1_G128) {
        // 1-bit, 1..16 activation rows: 64 weight rows x one K chunk per
        // workgroup, a lookup table per activation row, partial sums of the
        // K chunks combined in order. Launches take up to 8 activation rows
        // (tables for 1, 2, 4 or 8 rows); one chunk size for all launches of
        // a call: 512 inputs when a launch has 8-row tables (64 KiB of LDS),
        // else 1024, or 2048 for one row and long K.
        pl.lut = true;
        pl.B = nb == 1 ? 1 : nb <= 2 ? 2 : nb <= 4 ? 4 : 8;   // tables of the widest launch
        pl.passes = static_cast<int>(ceil_div(nb, 8));
        pl.grid_x = ceil_div(M, qg::kB1Rows);
        if (pl.B == 1) {
            const bool long_chunk = K >= 2 * kB1ChunkLong &&
                                    pl.grid_x * ceil_div(K, kB1ChunkLong) <= kB1LongResident * kComputeUnits;
            pl.kc = long_chunk ? kB1ChunkLong : kB1Chunk;
        } else {
            pl.kc = pl.B == 8 ? kB1ChunkWide : kB1Chunk;
        }
        pl.nsplit = static_cast<int>(ceil_div(K, pl.kc));
        pl.fused = pl.nsplit > 1 && pl.grid_x <= qg::kCtlTileCounters;
        size_t off = kCtlBytes;
        if (pl.nsplit > 1) {
            pl.comb_rows_per_wg = round_up(ceil_div(M, 1024), 256);
            pl.comb_grid = ceil_div(M, pl.comb_rows_per_wg);
            pl.part_off = off;
            off = align256(off + static_cast<size_t>(pl.nsplit) * std::min(nb, 8) * M * 4);
        }
        if (argmax) {
            // parked greedy keys (up to 8 per workgroup and launch) after the partials
            pl.nkeys = static_cast<int>(pl.nsplit > 1 && !pl.fused ? pl.comb_grid : pl.grid_x);
            pl.key_off = off;
            off = align256(off + static_cast<size_t>(pl.nkeys) * 8 * 8);
        }
        pl.ws_bytes = (off > kCtlBytes || argmax) ? off : 0;
        return pl;
    }
    if (nb >= 2 && u4_mfma_ok(fmt, K)) {
        // 2..16 rows, 4-bit: matrix cores, one workgroup of 8 waves per
        // compute unit, at least one 16-row tile per wave; a launch takes up
        // to 8 activation rows (9..16 rows: two launches, each reading the
        // weights once, which is far cheaper than the vector-ALU kernel at
        // 16 rows: 151936 x 2048 at 16 rows took 761 us there)
        pl.mfma = true;
        pl.passes = static_cast<int>(ceil_div(nb, 8));
        const int64_t ntiles = ceil_div(M, 16);
        pl.grid_x = std::min<int64_t>(kComputeUnits, ceil_div(ntiles, qg::kMfmaWaves));
        pl.lds_bytes = qg::gemv_mfma_lds_bytes(K);
        // stage the outputs in LDS when the workgroup's tiles fit
        const size_t out_bytes = static_cast<size_t>(ceil_div(ntiles, pl.grid_x)) * qg::kMfmaTileOutBytes;
        pl.fused = static_cast<int64_t>(pl.lds_bytes + out_bytes) + kLdsStaticReserve <= kLdsMax;
        if (pl.fused) pl.lds_bytes += out_bytes;
        pl.nsplit = 1;
        if (argmax) {
            // per-workgroup greedy keys (up to 8 per workgroup) after the control words
            pl.nkeys = static_cast<int>(pl.grid_x);
            pl.key_off = kCtlBytes;
            pl.ws_bytes = align256(kCtlBytes + static_cast<size_t>(pl.grid_x) * 8 * 8);
        }
        return pl;
    }
    pl.B = nb <= 1 ? 1 : nb <= 2 ? 2 : nb <= 4 ? 4 : nb <= 8 ? 8 : 16;
    const int kps = k_per_slice(fmt);
    const bool xsum = fmt == QG_U4_G64 || fmt == QG_B1_G128;   // per-slice activation sums
    // activation planes (+ per-slice sums) must fit the LDS budget
    const double bytes_per_k = pl.B * 4.0 * (1.0 + (xsum ? 1.0 / kps : 0.0));
    int64_t kc_max = static_cast<int64_t>((kLdsBudget - 64 * pl.B) / bytes_per_k);
    kc_max = kc_max / 128 * 128;
    pl.nsplit = static_cast<int>(ceil_div(K, kc_max));
    pl.kc = round_up(ceil_div(K, pl.nsplit), kps);
    pl.nsplit = static_cast<int>(ceil_div(K, pl.kc));
    // rows per block: as many as the wave width allows, fewer when the
    // grid would leave compute units idle
    pl.R = 64 / pl.B < 4 ? 64 / pl.B : 4;
    while (pl.R > 1 && ceil_div(M, 4 * pl.R) * pl.nsplit < 256) pl.R /= 2;
    const int64_t wg_target = 1024 / pl.nsplit > 0 ? 1024 / pl.nsplit : 1;
    pl.rows_per_wg = round_up(ceil_div(M, wg_target), 4 * pl.R);
    pl.grid_x = ceil_div(M, pl.rows_per_wg);
    const int64_t pf = (pl.kc + 31) / 32 * 32;
    const int64_t xsf = xsum ? (pl.kc / kps + 3) / 4 * 4 : 0;
    pl.lds_bytes = static_cast<size_t>(pl.B * (pf + xsf) * 4);
    // scratch (partial sums, keys) always starts after the control words
    size_t off = kCtlBytes;
    if (pl.nsplit > 1) {
        pl.comb_rows_per_wg = round_up(ceil_div(M, 1024), 256);
        pl.comb_grid = ceil_div(M, pl.comb_rows_per_wg);
        pl.part_off = off;
        off = align256(off + static_cast<size_t>(pl.nsplit) * nb * M * 4);
    }
    if (argmax) {
        // parked greedy keys (nb per workgroup) after the partials
        pl.nkeys = static_cast<int>(pl.nsplit > 1 ? pl.comb_grid : pl.grid_x);
        pl.key_off = off;
        off = align256(off + static_cast<size_t>(pl.nkeys) * nb * 8);
    }
    pl.ws_bytes = (off > kCtlBytes || argmax) ? off : 0;
    return pl;
}

// Allow a kernel the full dynamic LDS budget (set once per kernel).
template <typename Kernel>
void allow_lds(Kernel k)
{
    static const bool done = [&] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                  static_cast<int>(kLdsBudget));
        return true;
    }();
    (void)done;
}

template <int FMT, int B, int R>
void launch_gemv_r(const GemvPlan &pl, const GemvParams &p, hipStream_t s)
{
    allow_lds(qg::gemv_kernel<FMT, B, R>);
    dim3 grid(static_cast<unsigned>(pl.grid_x), static_cast<unsigned>(pl.nsplit));
    hipLaunchKernelGGL((qg::gemv_kernel<FMT, B, R>), grid, dim3(kThreads), pl.lds_bytes, s, p);
}

template <int FMT, int B>
void launch_gemv_b(const GemvPlan &pl, const GemvParams &p, hipStream_t s)
{
    switch (pl.R) {
    case 4: launch_gemv_r<FMT, B, 4>(pl, p, s); break;
    case 2: launch_gemv_r<FMT, B, 2>(pl, p, s); break;
    default: launch_gemv_r<FMT, B, 1>(pl, p, s); break;
    }
}

template <int FMT>
void launch_gemv_fmt(const GemvPlan &pl, const GemvParams &p, hipStream_t s)
{
    switch (pl.B) {
    case 1: launch_gemv_b<FMT, 1>(pl, p, s); break;
    case 2: launch_gemv_b<FMT, 2>(pl, p, s); break;
    case 4: launch_gemv_b<FMT, 4>(pl, p, s); break;
    case 8: launch_gemv_b<FMT, 8>(pl, p, s); break;
    default: launch_gemv_b<FMT, 16>(pl, p, s); break;
    }
}

template <int FMT, int NS, bool FULL, int WGW>
void launch_gemv1_wg(const GemvPlan &pl, const qg::Gemv1Params &p, hipStream_t s)
{
    constexpr bool NT = kGemv1Nt;
    const dim3 grid(static_cast<unsigned>(pl.grid_x)), block(64 * WGW);
    switch (pl.R) {
    case 4: hipLaunchKernelGGL((qg::gemv1_kernel<FMT, NS, 4, FULL, NT, WGW>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((qg::gemv1_kernel<FMT, NS, 2, FULL, NT, WGW>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((qg::gemv1_kernel<FMT, NS, 1, FULL, NT, WGW>), grid, block, 0, s, p); break;
    }
}

template <int FMT, int NS, bool FULL>
void launch_gemv1_full(const GemvPlan &pl, const qg::Gemv1Params &p, hipStream_t s)
{
    if constexpr (NS <= 2) {
        if (pl.wg_waves == 8) {
            launch_gemv1_wg<FMT, NS, FULL, 8>(pl, p, s);
            return;
        }
    }
    launch_gemv1_wg<FMT, NS, FULL, 4>(pl, p, s);
}

template <int FMT, int NS>
void launch_gemv1_ns(const GemvPlan &pl, const qg::Gemv1Params &p, hipStream_t s)
{
    if (pl.full) launch_gemv1_full<FMT, NS, true>(pl, p, s);
    else launch_gemv1_full<FMT, NS, false>(pl, p, s);
}

template <int FMT>
void launch_gemv1_fmt(const GemvPlan &pl, const qg::Gemv1Params &p, hipStream_t s)
{
    switch (pl.ns) {
    case 1: launch_gemv1_ns<FMT, 1>(pl, p, s); break;
    case 2: launch_gemv1_ns<FMT, 2>(pl, p, s); break;
    case 3: launch_gemv1_ns<FMT, 3>(pl, p, s); break;
    default: launch_gemv1_ns<FMT, 4>(pl, p, s); break;
    }
}

template <int NC>
void launch_stream(const GemvPlan &pl, const qg::GemvStreamParams &q, hipStream_t s)
{
    static const bool lds_set = [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(qg::gemv_stream_u4_kernel<NC>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, qg::kStreamLdsBytes);
        return true;
    }();
    (void)lds_set;
    hipLaunchKernelGGL((qg::gemv_stream_u4_kernel<NC>), dim3(static_cast<unsigned>(pl.grid_x)),
                       dim3(qg::kStreamThreads), qg::kStreamLdsBytes, s, q);
}

// Enqueue one planned GEMV (+ split-K combine). The greedy selection
// finishes inside the last kernel.
// Launch the one-pass kernel for GW groups of 64 inputs per wave (8-bit: 1,
// 2 or 4; 4-bit and 1-bit: 2 or 4), with dynamic LDS above the default.
template <int FMT, int GW>
void launch_mfma16_gw(dim3 grid, size_t lds, hipStream_t s, const qg::GemvMfmaParams &q)
{
    static const bool lds_set = [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(qg::gemv_mfma16_kernel<FMT, GW>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                  static_cast<int>(kLdsMax - kLdsStaticReserve));
        return true;
    }();
    (void)lds_set;
    hipLaunchKernelGGL((qg::gemv_mfma16_kernel<FMT, GW>), grid, dim3(64 * qg::kMfmaWaves), lds, s, q);
}

template <int FMT>
void launch_mfma16(int gw, dim3 grid, size_t lds, hipStream_t s, const qg::GemvMfmaParams &q)
{
    if (gw == 2) {
        launch_mfma16_gw<FMT, 2>(grid, lds, s, q);
    } else if (gw == 4) {
        launch_mfma16_gw<FMT, 4>(grid, lds, s, q);
    } else if constexpr (FMT == qg::FMT_I8_ROW || FMT == qg::FMT_I8_G64) {
        launch_mfma16_gw<FMT, 1>(grid, lds, s, q);
    }
}

void run_gemv(int fmt, const GemvPlan &pl, const void *codes, const void *scales,
              const void *biases, const float *x, float *y, int32_t *idx, int64_t M,
              int64_t K, int nb, void *ws, hipStream_t s)
{
    if (pl.gemm) {
        run_gemm_mfma(fmt, codes, scales, biases, x, y, M, K, nb, ws, s);
        return;
    }
    if (pl.mfma16) {
        qg::GemvMfmaParams q{};
        q.codes = static_cast<const uint8_t *>(codes);
        q.scales = static_cast<const uint16_t *>(scales);
        q.biases = static_cast<const uint16_t *>(biases);
        q.x = x;
        q.y = y;
        q.ctl = idx ? static_cast<qg::GreedyCtl *>(ws) : nullptr;
        q.keys = idx ? reinterpret_cast<unsigned long long *>(static_cast<char *>(ws) + pl.key_off) : nullptr;
        q.idx = idx;
        q.M = M;
        q.K = K;
        q.nb = nb;
        q.stage_out = pl.fused;
        q.part = pl.nsplit > 1 ? reinterpret_cast<float *>(static_cast<char *>(ws) + pl.part_off) : nullptr;
        const dim3 grid(static_cast<unsigned>(pl.grid_x), static_cast<unsigned>(pl.nsplit));
        if (fmt == QG_U4_G64) launch_mfma16<qg::FMT_U4_G64>(pl.gw, grid, pl.lds_bytes, s, q);
        else if (fmt == QG_I8_ROW) launch_mfma16<qg::FMT_I8_ROW>(pl.gw, grid, pl.lds_bytes, s, q);
        else if (fmt == QG_I8_G64) launch_mfma16<qg::FMT_I8_G64>(pl.gw, grid, pl.lds_bytes, s, q);
        else launch_mfma16<qg::FMT_B1_G128>(pl.gw, grid, pl.lds_bytes, s, q);
        if (pl.nsplit > 1) {
            const int64_t quads = ceil_div(M * nb, 4);
            hipLaunchKernelGGL(qg::gemm_splitk_combine_kernel, dim3(static_cast<unsigned>(ceil_div(quads, 256))),
                               dim3(256), 0, s, q.part, y, M, static_cast<int64_t>(nb), pl.nsplit);
        }
        return;
    }
    if (pl.mfma) {
        qg::GemvMfmaParams q{};
        q.codes = static_cast<const uint8_t *>(codes);
        q.scales = static_cast<const uint16_t *>(scales);
        q.biases = static_cast<const uint16_t *>(biases);
        q.x = x;
        q.y = y;
        q.ctl = idx ? static_cast<qg::GreedyCtl *>(ws) : nullptr;
        q.keys = idx ? reinterpret_cast<unsigned long long *>(static_cast<char *>(ws) + pl.key_off) : nullptr;
        q.idx = idx;
        q.M = M;
        q.K = K;
        q.stage_out = pl.fused;
        // dynamic LDS up to the plan's limit (the kernel's few static bytes
        // come on top, within the compute unit's 160 KiB)
        static const bool lds_set = [] {
            (void)hipFuncSetAttribute(reinterpret_cast<const void *>(qg::gemv_mfma_u4_kernel),
                                      hipFuncAttributeMaxDynamicSharedMemorySize,
                                      static_cast<int>(kLdsMax - kLdsStaticReserve));
            return true;
        }();
        (void)lds_set;
        // rows 8 h .. 8 h + 7 in pass h; the passes share the workspace in
        // stream order (each dispatch claims the completion word for itself)
        for (int h = 0; h < pl.passes; ++h) {
            qg::GemvMfmaParams qh = q;
            qh.x = x + static_cast<int64_t>(8) * h * K;
            qh.y = y ? y + static_cast<int64_t>(8) * h * M : nullptr;
            qh.idx = idx ? idx + 8 * h : nullptr;
            qh.nb = std::min(8, nb - 8 * h);
            hipLaunchKernelGGL(qg::gemv_mfma_u4_kernel, dim3(static_cast<unsigned>(pl.grid_x)),
                               dim3(64 * qg::kMfmaWaves), pl.lds_bytes, s, qh);
        }
        return;
    }
    if (pl.smfma) {
        qg::GemvStreamMfmaParams q{};
        q.codes = static_cast<const uint8_t *>(codes);
        q.scales = static_cast<const uint16_t *>(scales);
        q.biases = static_cast<const uint16_t *>(biases);
        q.x = x;
        q.y = y;
        q.ctl = idx ? static_cast<qg::GreedyCtl *>(ws) : nullptr;
        q.keys = idx ? reinterpret_cast<unsigned long long *>(static_cast<char *>(ws) + pl.key_off) : nullptr;
        q.idx = idx;
        q.M = M;
        q.nb = nb;
        static const bool lds_set = [] {
            (void)hipFuncSetAttribute(reinterpret_cast<const void *>(qg::gemv_stream_mfma_u4_kernel),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, qg::kStreamMfmaLdsBytes);
            return true;
        }();
        (void)lds_set;
        hipLaunchKernelGGL(qg::gemv_stream_mfma_u4_kernel, dim3(static_cast<unsigned>(pl.grid_x)),
                           dim3(qg::kStreamThreads), qg::kStreamMfmaLdsBytes, s, q);
        return;
    }
    if (pl.stream) {
        qg::GemvStreamParams q{};
        q.codes = static_cast<const uint8_t *>(codes);
        q.scales = static_cast<const uint16_t *>(scales);
        q.biases = static_cast<const uint16_t *>(biases);
        q.x = x;
        q.y = y;
        q.ctl = idx ? static_cast<qg::GreedyCtl *>(ws) : nullptr;
        q.keys = idx ? reinterpret_cast<unsigned long long *>(static_cast<char *>(ws) + pl.key_off) : nullptr;
        q.idx = idx;
        q.M = M;
        q.K = K;
        if (pl.nc == 1) launch_stream<1>(pl, q, s);
        else if (pl.nc == 2) launch_stream<2>(pl, q, s);
        else launch_stream<4>(pl, q, s);
        return;
    }
    if (pl.one) {
        qg::Gemv1Params q{};
        q.codes = static_cast<const uint8_t *>(codes);
        q.scales = scales;
        q.biases = biases;
        q.x = x;
        q.y = y;
        q.ctl = idx ? static_cast<qg::GreedyCtl *>(ws) : nullptr;
        q.keys = idx ? reinterpret_cast<unsigned long long *>(static_cast<char *>(ws) + pl.key_off) : nullptr;
        q.idx = idx;
        q.M = M;
        q.K = K;
        q.rows_per_wave = pl.rows_per_wave;
        if (fmt == QG_I8_ROW) launch_gemv1_fmt<qg::FMT_I8_ROW>(pl, q, s);
        else if (fmt == QG_I8_G64) launch_gemv1_fmt<qg::FMT_I8_G64>(pl, q, s);
        else launch_gemv1_fmt<qg::FMT_U4_G64>(pl, q, s);
        return;
    }
    if (pl.lut) {
        // activation rows 8 h .. 8 h + 7 in pass h; the passes share the
        // workspace in stream order (each dispatch claims the completion
        // words for itself)
        for (int h = 0; h < pl.passes; ++h) {
            const int rows = std::min(8, nb - 8 * h);
            float *yh = y ? y + static_cast<int64_t>(8) * h * M : nullptr;
            int32_t *ih = idx ? idx + 8 * h : nullptr;
            qg::B1LutParams q{};
            q.codes = static_cast<const uint8_t *>(codes);
            q.scales = static_cast<const uint16_t *>(scales);
            q.x = x + static_cast<int64_t>(8) * h * K;
            q.y = yh;
            q.part = pl.nsplit > 1 ? reinterpret_cast<float *>(static_cast<char *>(ws) + pl.part_off) : nullptr;
            q.ctl = static_cast<qg::GreedyCtl *>(ws);
            q.keys = idx ? reinterpret_cast<unsigned long long *>(static_cast<char *>(ws) + pl.key_off) : nullptr;
            q.idx = (pl.nsplit == 1 || pl.fused) ? ih : nullptr;
            q.M = M;
            q.K = K;
            q.nb = rows;
            q.nsplit = pl.nsplit;
            q.fused = pl.fused;
            const dim3 grid(static_cast<unsigned>(pl.grid_x), static_cast<unsigned>(pl.nsplit));
            const int tb = rows == 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : 8;   // this launch's tables
            if (pl.kc == kB1ChunkWide) {
                if (tb == 8) hipLaunchKernelGGL((qg::gemv_b1_lut_kernel<kB1ChunkWide, 8>), grid, dim3(256), 0, s, q);
                else if (tb == 4) hipLaunchKernelGGL((qg::gemv_b1_lut_kernel<kB1ChunkWide, 4>), grid, dim3(256), 0, s, q);
                else if (tb == 2) hipLaunchKernelGGL((qg::gemv_b1_lut_kernel<kB1ChunkWide, 2>), grid, dim3(256), 0, s, q);
                else hipLaunchKernelGGL((qg::gemv_b1_lut_kernel<kB1ChunkWide, 1>), grid, dim3(256), 0, s, q);
            } else if (pl.kc == kB1ChunkLong) {
                hipLaunchKernelGGL((qg::gemv_b1_lut_kernel<kB1ChunkLong, 1>), grid, dim3(256), 0, s, q);
            } else {
                if (tb == 4) hipLaunchKernelGGL((qg::gemv_b1_lut_kernel<kB1Chunk, 4>), grid, dim3(256), 0, s, q);
                else if (tb == 2) hipLaunchKernelGGL((qg::gemv_b1_lut_kernel<kB1Chunk, 2>), grid, dim3(256), 0, s, q);
                else hipLaunchKernelGGL((qg::gemv_b1_lut_kernel<kB1Chunk, 1>), grid, dim3(256), 0, s, q);
            }
            if (pl.nsplit > 1 && !pl.fused) {
                GemvParams c{};
                c.y = yh;
                c.part = q.part;
                c.ctl = idx ? static_cast<qg::GreedyCtl *>(ws) : nullptr;
                c.keys = q.keys;
                c.idx = ih;
                c.M = M;
                c.K = K;
                c.rows_per_wg = pl.comb_rows_per_wg;
                c.nb = rows;
                c.nsplit = pl.nsplit;
                c.nkeys = pl.nkeys;
                hipLaunchKernelGGL(qg::gemv_combine_kernel, dim3(static_cast<unsigned>(pl.comb_grid)),
                                   dim3(kThreads), 0, s, c);
            }
        }
        return;
    }
    GemvParams p{};
    p.codes = static_cast<const uint8_t *>(codes);
    p.scales = scales;
    p.biases = biases;
    p.x = x;
    p.y = y;
    p.part = pl.nsplit > 1 ? reinterpret_cast<float *>(static_cast<char *>(ws) + pl.part_off) : nullptr;
    p.ctl = idx ? static_cast<qg::GreedyCtl *>(ws) : nullptr;
    p.keys = idx ? reinterpret_cast<unsigned long long *>(static_cast<char *>(ws) + pl.key_off) : nullptr;
    p.idx = idx;
    p.M = M;
    p.K = K;
    p.x_stride = K;
    p.rows_per_wg = pl.rows_per_wg;
    p.kc = pl.kc;
    p.nb = nb;
    p.nsplit = pl.nsplit;
    p.nkeys = pl.nkeys;
    // (1-bit calls never get here: the planner sends them to the lookup,
    // one-pass or prefill kernels)
    if (fmt == QG_I8_ROW) launch_gemv_fmt<qg::FMT_I8_ROW>(pl, p, s);
    else if (fmt == QG_I8_G64) launch_gemv_fmt<qg::FMT_I8_G64>(pl, p, s);
    else launch_gemv_fmt<qg::FMT_U4_G64>(pl, p, s);
    if (pl.nsplit > 1) {
        GemvParams c = p;
        c.rows_per_wg = pl.comb_rows_per_wg;
        hipLaunchKernelGGL(qg::gemv_combine_kernel, dim3(static_cast<unsigned>(pl.comb_grid)),
                           dim3(kThreads), 0, s, c);
    }
}

int gemv_entry(int fmt, const void *codes, const void *scales, const void *biases,
               const float *x, float *y, int32_t *idx, int64_t M, int64_t K, int batch,
               void *ws, size_t ws_bytes, hipStream_t stream)
{
    int st = check_weights(fmt, codes, scales, biases, x, M, K);
    if (st != QG_OK) return st;
    const bool argmax = idx != nullptr;
    if (!y && !argmax) return QG_ERR_NULL;   // the greedy head may skip its logits
    if (batch < 1 || batch > QG_MAX_GEMV_BATCH) return QG_ERR_SHAPE;
    if (y && !aligned(y, kAlign)) return QG_ERR_ALIGN;
    if (argmax && !aligned(idx, 4)) return QG_ERR_ALIGN;
    const GemvPlan pl = plan_gemv(fmt, M, K, batch, argmax);
    if (pl.ws_bytes > 0) {
        if (!ws || ws_bytes < pl.ws_bytes) return QG_ERR_WORKSPACE;
        if (!aligned(ws, kAlign)) return QG_ERR_ALIGN;
    }
    Range inputs[4];
    int n = 0;
    inputs[n++] = range_of(codes, M * row_bytes(fmt, K));
    inputs[n++] = range_of(scales, scale_bytes(fmt, M, K));
    if (biases) inputs[n++] = range_of(biases, bias_bytes(fmt, M, K));
    inputs[n++] = range_of(x, int64_t(batch) * K * 4);
    Range wr[3];
    int nw = 0;
    if (y) wr[nw++] = range_of(y, int64_t(batch) * M * 4);
    if (argmax) wr[nw++] = range_of(idx, int64_t(batch) * 4);
    if (pl.ws_bytes > 0) wr[nw++] = range_of(ws, static_cast<int64_t>(pl.ws_bytes));
    st = check_alias(inputs, n, wr, nw);
    if (st != QG_OK) return st;

    (void)hipGetLastError();
    run_gemv(fmt, pl, codes, scales, biases, x, y, idx, M, K, batch, ws, stream);
    return launch_status();
}

// ---------------------------------------------------------------------------
// GEMM: up to 16 token rows go through the matrix-vector kernel (one pass
// over the weights serves all rows); more rows go to the MFMA kernel.
// ---------------------------------------------------------------------------

constexpr int kGemmViaGemv = 16;

void gemm_tile(int fmt, int64_t M, int64_t N, int &bm, int &bn, int &wn);

// Split of K for prefill grids too small for the chip: with fewer tiles than
// compute units, each tile's K range is cut into nsplit pieces of kt_split
// steps (a multiple of 4, so that group boundaries do not move) to give
// about two workgroups per compute unit; the partial products go to the
// workspace and a second launch adds them in split order. The 1-bit format
// does the most work per k-step beside its MFMAs (sign unpacking and a
// barrier for few MFMAs), so it splits grids of up to four tiles per
// compute unit, into about four workgroups per compute unit (17408 x 5120,
// 128 token rows: 148 -> 131 us; 64 rows: 101 -> 75 us); the 8-bit per-row
// format splits grids of up to two tiles per compute unit into about two
// workgroups per unit (its 128 x 64 tile runs four to a unit; 1024 x 3584,
// N = 2048, 256 tiles: 65 -> 56 us; three or four pieces: 59, 63 us), the
// 8-bit group-64 format into about as many as its tile runs to a unit
// (three for 128 x 64; 77 -> 67 -> 64 us for two, then three pieces); the 1-bit format's 5120 x 17408, N = 512
// (320 tiles) takes 277 us in four pieces, 285 in three, 295 in eight;
// deeper splits lose (8-bit 3584 x 1024, 128 rows, four workgroups per
// compute unit instead of two: 16.7 -> 21.6 us).
// kt_split = 0: no split.
// Workgroups of the prefill kernel per compute unit (gemm_occupancy).
int gemm_wg_per_cu(int fmt, int bm, int bn)
{
    const bool i8 = fmt == QG_I8_ROW || fmt == QG_I8_G64;
    return fmt == QG_I8_ROW && bm == 128 && bn == 64 ? 4
           : i8 && bn == 64 && (bm == 128 || (fmt == QG_I8_ROW && bm == 256)) ? 3 : 2;
}

void gemm_split(int fmt, int64_t M, int64_t K, int64_t N, int &kt_split, int &nsplit)
{
    kt_split = 0;
    nsplit = 1;
    int bm, bn, wn;
    gemm_tile(fmt, M, N, bm, bn, wn);
    const int64_t tiles = ceil_div(M, bm) * ceil_div(N, bn);
    const int64_t nk = ceil_div(K, 32);
    const int below = fmt == QG_B1_G128 ? 4 : fmt == QG_I8_ROW || fmt == QG_I8_G64 ? 2 : 1;
    const int per_cu = fmt == QG_B1_G128 ? 4 : fmt == QG_I8_G64 ? gemm_wg_per_cu(fmt, bm, bn) : 2;
    if (tiles >= below * kComputeUnits || nk < 8) return;
    const int64_t want = std::min(ceil_div(per_cu * kComputeUnits, tiles), nk / 4);
    if (want < 2) return;
    kt_split = static_cast<int>(round_up(ceil_div(nk, want), 4));
    nsplit = static_cast<int>(ceil_div(nk, kt_split));
    if (nsplit < 2) kt_split = 0, nsplit = 1;
}

// Split tail of grids of at least one full round (two workgroups per
// compute unit): when the last round would be at most a quarter full, its
// tiles are cut along K into tsplit pieces (of kt_tail steps, a multiple of
// 4) that fill it, the full rounds keep whole tiles, and a second launch
// adds the pieces (17408 x 5120 1-bit, 512 token rows: 320 -> 273 us;
// 1024 x 3584 8-bit, 10240 rows: 227 -> 210 us). A fuller last round gains
// less than the partial stores and the second launch cost (3584 x 1024
// 8-bit, 10240 rows, last round 3/8 full: 217 -> 240 us).
// nfull: tiles computed whole. tsplit = 0: no split tail.
struct GemmTail {
    int nfull = 0, ntail = 0, tsplit = 0, kt_tail = 0;
};

GemmTail gemm_tail(int fmt, int64_t M, int64_t K, int64_t N)
{
    GemmTail t;
    int kt_split, nsplit, bm, bn, wn;
    gemm_split(fmt, M, K, N, kt_split, nsplit);
    if (nsplit > 1) return t;
    gemm_tile(fmt, M, N, bm, bn, wn);
    const int64_t tiles = ceil_div(M, bm) * ceil_div(N, bn);
    const int64_t slots = int64_t(gemm_wg_per_cu(fmt, bm, bn)) * kComputeUnits;
    const int64_t ntail = tiles % slots;
    if (tiles < slots || ntail == 0 || 4 * ntail > slots) return t;
    const int64_t nk = ceil_div(K, 32);
    const int64_t want = std::min(slots / ntail, nk / 4);
    if (want < 2) return t;
    const int64_t kt = round_up(ceil_div(nk, want), 4);
    const int64_t pieces = ceil_div(nk, kt);
    if (pieces < 2) return t;
    t.nfull = static_cast<int>(tiles - ntail);
    t.ntail = static_cast<int>(ntail);
    t.tsplit = static_cast<int>(pieces);
    t.kt_tail = static_cast<int>(kt);
    return t;
}

size_t gemm_mfma_workspace(int fmt, int64_t M, int64_t K, int64_t N)
{
    int kt_split, nsplit;
    gemm_split(fmt, M, K, N, kt_split, nsplit);
    // partial products after the control words
    if (nsplit > 1) return align256(kCtlBytes + static_cast<size_t>(nsplit) * N * M * 4);
    const GemmTail t = gemm_tail(fmt, M, K, N);
    if (t.tsplit == 0) return 0;
    int bm, bn, wn;
    gemm_tile(fmt, M, N, bm, bn, wn);
    return align256(kCtlBytes + static_cast<size_t>(t.tsplit) * t.ntail * bm * bn * 4);
}

// 17..48 rows of the 4-bit format at K = 1024 or 2048 as launches of up to
// 16 rows each (the one-pass matrix-vector kernel, or the batch-1 kernel for
// a last single row), where reading the weights once per 16 rows costs less
// than the prefill kernel's matrix-core work on rows padded to a multiple
// of 32 (an estimate fitted to the 151936 x 2048 head: 10 us + 6 M K
// round_up(N, 32) flop at 560 TFLOP/s, against ~51.5 us per launch of 16
// rows). Returns the number of launches, or 0 for the prefill kernel.
int u4_row_launches(int fmt, int64_t M, int64_t K, int64_t N)
{
    if (N <= kGemmViaGemv || N > 48 || fmt != QG_U4_G64 || !mfma16_ok(fmt, K)) return 0;
    const int n = static_cast<int>(ceil_div(N, 16));
    const double w = static_cast<double>(M) * static_cast<double>(K);
    const double bytes = static_cast<double>(M) * (row_bytes(fmt, K) + 4 * (K / 64));
    const double t_gemm = 10.0 + 6.0 * w * static_cast<double>(round_up(N, 32)) / 560e6;
    return n * std::max(8.0, bytes / 3.4e6) < t_gemm ? n : 0;
}

// Workspace of those launches: the largest of their plans (they run in
// stream order, each dispatch claiming the completion words for itself).
size_t row_launches_workspace(int fmt, int64_t M, int64_t K, int64_t N, bool argmax)
{
    size_t ws = 0;
    for (int64_t r0 = 0; r0 < N; r0 += kGemmViaGemv) {
        const int nb = static_cast<int>(std::min<int64_t>(kGemmViaGemv, N - r0));
        ws = std::max(ws, plan_gemv(fmt, M, K, nb, argmax).ws_bytes);
    }
    return ws;
}

void run_row_launches(int fmt, const void *codes, const void *scales, const void *biases,
                      const float *x, float *y, int32_t *idx, int64_t M, int64_t K, int64_t N,
                      void *ws, hipStream_t s)
{
    for (int64_t r0 = 0; r0 < N; r0 += kGemmViaGemv) {
        const int nb = static_cast<int>(std::min<int64_t>(kGemmViaGemv, N - r0));
        const GemvPlan pl = plan_gemv(fmt, M, K, nb, idx != nullptr);
        run_gemv(fmt, pl, codes, scales, biases, x + r0 * K, y ? y + r0 * M : nullptr,
                 idx ? idx + r0 : nullptr, M, K, nb, ws, s);
    }
}

size_t gemm_workspace(int fmt, int64_t M, int64_t K, int64_t N)
{
    if (N <= kGemmViaGemv) return plan_gemv(fmt, M, K, static_cast<int>(N), false).ws_bytes;
    if (u4_row_launches(fmt, M, K, N)) return row_launches_workspace(fmt, M, K, N, false);
    return gemm_mfma_workspace(fmt, M, K, N);
}

bool gemm_shape_ok(int64_t M, int64_t K, int64_t N)
{
    if (N <= kGemmViaGemv) return true;
    return K <= qg::kGemmMaxK && ceil_div(M, 64) * ceil_div(N, 64) <= 0x7fffffffLL;   // smallest tile
}

// The largest tile that still gives every compute unit a workgroup
// (4-bit and 1-bit: at most 64 x 128, their per-group accumulators double
// the accumulator registers). wn: waves along n (4, or 2 and 1 for the
// narrow tiles of up to 32 token rows).
void gemm_tile(int fmt, int64_t M, int64_t N, int &bm, int &bn, int &wn)
{
    auto tiles = [&](int tm, int tn) { return ceil_div(M, tm) * ceil_div(N, tn); };
    bm = 64;
    bn = 64;
    wn = 4;
    if (N <= 32) {
        // a few token rows: 16 or 32 tokens wide (a 64-wide tile would spend
        // most of its MFMAs on padding), the waves split the weight rows;
        // 128 rows once every compute unit still gets two tiles, and always
        // for the 1-bit format, whose k-steps cost the most beside the MFMAs
        // (K is split to fill the chip; 17408 x 5120, 17 rows: 54 -> 44 us)
        bn = N <= 16 ? 16 : 32;
        wn = bn / 16;
        if (fmt == QG_B1_G128 || tiles(128, bn) >= 2 * kComputeUnits) bm = 128;
        return;
    }
    // the grouped formats: 128 weight rows by 64 token rows (each activation
    // split feeds twice the MFMAs of a 64-row tile; 128 x 128 would spill
    // their second set of accumulators), for the 1-bit format always
    // (17408 x 5120, N = 512: 431 -> 318 us), for the 8-bit group-64 format
    // (three to a compute unit) once every compute unit gets a tile, with K
    // split below two (1024 x 3584, N = 2048: 77 -> 67 us against 512 tiles
    // of 64 x 64), for the 4-bit format once every compute unit gets two
    if (fmt != QG_I8_ROW && (fmt == QG_B1_G128 || tiles(128, 64) >= 2 * kComputeUnits ||
                             (fmt == QG_I8_G64 && tiles(128, 64) >= kComputeUnits))) {
        bm = 128;
        return;
    }
    // the 8-bit per-row format: 256 x 64 (three workgroups per compute unit)
    // once every compute unit gets two tiles, else 128 x 64 (four per unit)
    // once every compute unit gets a tile (gemm_occupancy)
    if (fmt == QG_I8_ROW && tiles(256, 64) >= 2 * kComputeUnits) {
        bm = 256;
        return;
    }
    if (fmt == QG_I8_ROW && tiles(128, 64) >= kComputeUnits) {
        bm = 128;
        return;
    }
    // 128 token rows per tile only where that pads no more than 64 would
    // (64 token rows with 128-row tiles would halve the useful MFMA work)
    const bool n128 = N % 128 == 0 || N % 128 > 64;
    if (!n128) return;
    // 128 x 128 only for the per-row 8-bit format (the grouped formats keep a
    // second set of accumulators, which would not fit in registers), once
    // every compute unit gets a tile; 64 x 128 only once every compute unit
    // gets two, since a single workgroup per compute unit leaves one wave
    // per SIMD, which cannot keep the matrix pipe busy (1024 x 3584, N =
    // 2048: 99 us on 256 tiles of 64 x 128, 80 us on 512 of 64 x 64)
    if (fmt == QG_I8_ROW && tiles(128, 128) >= kComputeUnits) bm = 128, bn = 128;
    else if (tiles(64, 128) >= 2 * kComputeUnits) bn = 128;
}

template <int FMT>
void launch_gemm_fmt(int bm, int bn, dim3 grid, hipStream_t s, const qg::GemmParams &p)
{
    const dim3 block(qg::kGemmThreads);
    if (bn == 16) {
        if (bm == 128) hipLaunchKernelGGL((qg::gemm_kernel<FMT, 128, 16, 1>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((qg::gemm_kernel<FMT, 64, 16, 1>), grid, block, 0, s, p);
    } else if (bn == 32) {
        if (bm == 128) hipLaunchKernelGGL((qg::gemm_kernel<FMT, 128, 32, 2>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((qg::gemm_kernel<FMT, 64, 32, 2>), grid, block, 0, s, p);
    } else if (bn == 64) {
        if constexpr (FMT == qg::FMT_I8_ROW) {
            if (bm == 256) {
                hipLaunchKernelGGL((qg::gemm_kernel<FMT, 256, 64>), grid, block, 0, s, p);
                return;
            }
        }
        if (bm == 128) hipLaunchKernelGGL((qg::gemm_kernel<FMT, 128, 64>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((qg::gemm_kernel<FMT, 64, 64>), grid, block, 0, s, p);
    } else if constexpr (FMT == qg::FMT_I8_ROW) {
        if (bm == 128) hipLaunchKernelGGL((qg::gemm_kernel<FMT, 128, 128>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((qg::gemm_kernel<FMT, 64, 128>), grid, block, 0, s, p);
    } else {
        hipLaunchKernelGGL((qg::gemm_kernel<FMT, 64, 128>), grid, block, 0, s, p);
    }
}

// Enqueue the matrix-core prefill kernel; with `keys`, the greedy head's
// keys [N][tiles_m x waves along m] as well (y may then be nullptr).
void launch_gemm(int fmt, const void *codes, const void *scales, const void *biases,
                 const float *x, float *y, unsigned long long *keys, int64_t M, int64_t K,
                 int64_t N, hipStream_t s, float *part = nullptr, int kt_split = 0, int nsplit = 1,
                 const GemmTail &tail = GemmTail{})
{
    qg::GemmParams p{};
    p.part = part;
    p.kt_split = kt_split;
    p.tpart = tail.tsplit > 0 ? part : nullptr;
    p.nfull = tail.nfull;
    p.tsplit = tail.tsplit;
    p.kt_tail = tail.kt_tail;
    p.codes = static_cast<const uint8_t *>(codes);
    p.scales = scales;
    p.biases = static_cast<const uint16_t *>(biases);
    p.x = x;
    p.y = y;
    p.keys = keys;
    p.M = M;
    p.K = K;
    p.N = N;
    int bm, bn, wn;
    gemm_tile(fmt, M, N, bm, bn, wn);
    p.tiles_m = static_cast<int>(ceil_div(M, bm));
    p.tiles_n = static_cast<int>(ceil_div(N, bn));
    p.keys_m = p.tiles_m * (4 / wn);
    const int64_t wgs = tail.tsplit > 0 ? int64_t(tail.nfull) + int64_t(tail.ntail) * tail.tsplit
                                        : int64_t(p.tiles_m) * p.tiles_n;
    const dim3 grid(static_cast<unsigned>(wgs), static_cast<unsigned>(nsplit));
    if (fmt == QG_I8_ROW) launch_gemm_fmt<qg::FMT_I8_ROW>(bm, bn, grid, s, p);
    else if (fmt == QG_I8_G64) launch_gemm_fmt<qg::FMT_I8_G64>(bm, bn, grid, s, p);
    else if (fmt == QG_U4_G64) launch_gemm_fmt<qg::FMT_U4_G64>(bm, bn, grid, s, p);
    else launch_gemm_fmt<qg::FMT_B1_G128>(bm, bn, grid, s, p);
}

void run_gemm_mfma(int fmt, const void *codes, const void *scales, const void *biases,
                   const float *x, float *y, int64_t M, int64_t K, int64_t N, void *ws,
                   hipStream_t s)
{
    int kt_split, nsplit;
    gemm_split(fmt, M, K, N, kt_split, nsplit);
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + kCtlBytes);
    if (nsplit == 1) {
        const GemmTail t = gemm_tail(fmt, M, K, N);
        if (t.tsplit == 0) {
            launch_gemm(fmt, codes, scales, biases, x, y, nullptr, M, K, N, s);
            return;
        }
        launch_gemm(fmt, codes, scales, biases, x, y, nullptr, M, K, N, s, part, 0, 1, t);
        int bm, bn, wn;
        gemm_tile(fmt, M, N, bm, bn, wn);
        const int64_t quads = static_cast<int64_t>(t.ntail) * bm * bn / 4;
        hipLaunchKernelGGL(qg::gemm_tail_combine_kernel, dim3(static_cast<unsigned>(ceil_div(quads, 256))),
                           dim3(256), 0, s, part, y, M, N, static_cast<int>(ceil_div(M, bm)), t.nfull,
                           t.ntail, t.tsplit, bm, bn);
        return;
    }
    launch_gemm(fmt, codes, scales, biases, x, nullptr, nullptr, M, K, N, s, part, kt_split, nsplit);
    const int64_t quads = ceil_div(M * N, 4);
    hipLaunchKernelGGL(qg::gemm_splitk_combine_kernel, dim3(static_cast<unsigned>(ceil_div(quads, 256))),
                       dim3(256), 0, s, part, y, M, N, nsplit);
}

void run_gemm(int fmt, const void *codes, const void *scales, const void *biases, const float *x,
              float *y, int64_t M, int64_t K, int64_t N, void *ws, hipStream_t s)
{
    if (N <= kGemmViaGemv) {
        const int nb = static_cast<int>(N);
        const GemvPlan pl = plan_gemv(fmt, M, K, nb, false);
        run_gemv(fmt, pl, codes, scales, biases, x, y, nullptr, M, K, nb, ws, s);
        return;
    }
    if (u4_row_launches(fmt, M, K, N)) {
        run_row_launches(fmt, codes, scales, biases, x, y, nullptr, M, K, N, ws, s);
        return;
    }
    run_gemm_mfma(fmt, codes, scales, biases, x, y, M, K, N, ws, s);
}

// ---------------------------------------------------------------------------
// Greedy head over more than QG_MAX_GEMV_BATCH rows: the prefill kernel with
// tile keys in the workspace (after the control words), then one workgroup
// per row reduces its keys. The logits may be skipped (y == nullptr).
// ---------------------------------------------------------------------------

// Greedy-head keys per token row: one per tile and wave along m.
int64_t wide_argmax_keys(int fmt, int64_t M, int64_t N)
{
    int bm, bn, wn;
    gemm_tile(fmt, M, N, bm, bn, wn);
    return ceil_div(M, bm) * (4 / wn);
}

size_t wide_argmax_workspace(int fmt, int64_t M, int64_t K, int64_t N)
{
    if (u4_row_launches(fmt, M, K, N)) return row_launches_workspace(fmt, M, K, N, true);
    return align256(kCtlBytes + static_cast<size_t>(N) * wide_argmax_keys(fmt, M, N) * 8);
}

int wide_argmax_entry(int fmt, const void *codes, const void *scales, const void *biases,
                      const float *x, float *y, int32_t *idx, int64_t M, int64_t K, int64_t N,
                      void *ws, size_t ws_bytes, hipStream_t stream)
{
    int st = check_weights(fmt, codes, scales, biases, x, M, K);
    if (st != QG_OK) return st;
    if (N < 1 || N > QG_MAX_ARGMAX_BATCH || K > qg::kGemmMaxK) return QG_ERR_SHAPE;
    if ((y && !aligned(y, kAlign)) || !aligned(idx, 4)) return QG_ERR_ALIGN;
    const size_t need = wide_argmax_workspace(fmt, M, K, N);
    if (!ws || ws_bytes < need) return QG_ERR_WORKSPACE;
    if (!aligned(ws, kAlign)) return QG_ERR_ALIGN;
    Range inputs[4];
    int n = 0;
    inputs[n++] = range_of(codes, M * row_bytes(fmt, K));
    inputs[n++] = range_of(scales, scale_bytes(fmt, M, K));
    if (biases) inputs[n++] = range_of(biases, bias_bytes(fmt, M, K));
    inputs[n++] = range_of(x, N * K * 4);
    Range wr[3];
    int nw = 0;
    if (y) wr[nw++] = range_of(y, N * M * 4);
    wr[nw++] = range_of(idx, N * 4);
    wr[nw++] = range_of(ws, static_cast<int64_t>(need));
    st = check_alias(inputs, n, wr, nw);
    if (st != QG_OK) return st;

    (void)hipGetLastError();
    if (u4_row_launches(fmt, M, K, N)) {
        run_row_launches(fmt, codes, scales, biases, x, y, idx, M, K, N, ws, stream);
        return launch_status();
    }
    auto *keys = reinterpret_cast<unsigned long long *>(static_cast<char *>(ws) + kCtlBytes);
    launch_gemm(fmt, codes, scales, biases, x, y, keys, M, K, N, stream);
    hipLaunchKernelGGL(qg::argmax_keys_kernel, dim3(static_cast<unsigned>(N)), dim3(256), 0, stream,
                       keys, static_cast<int>(wide_argmax_keys(fmt, M, N)), idx);
    return launch_status();
}

int gemm_entry(int fmt, const void *codes, const void *scales, const void *biases,
               const float *x, float *y, int64_t M, int64_t K, int64_t N, void *ws,
               size_t ws_bytes, hipStream_t stream)
{
    int st = check_weights(fmt, codes, scales, biases, x, M, K);
    if (st != QG_OK) return st;
    if (!y) return QG_ERR_NULL;
    if (N < 1 || N > kMaxN || !gemm_shape_ok(M, K, N)) return QG_ERR_SHAPE;
    if (!aligned(y, kAlign)) return QG_ERR_ALIGN;
    const size_t need = gemm_workspace(fmt, M, K, N);
    if (need > 0) {
        if (!ws || ws_bytes < need) return QG_ERR_WORKSPACE;
        if (!aligned(ws, kAlign)) return QG_ERR_ALIGN;
    }
    Range inputs[4];
    int n = 0;
    inputs[n++] = range_of(codes, M * row_bytes(fmt, K));
    inputs[n++] = range_of(scales, scale_bytes(fmt, M, K));
    if (biases) inputs[n++] = range_of(biases, bias_bytes(fmt, M, K));
    inputs[n++] = range_of(x, N * K * 4);
    Range wr[2];
    int nw = 0;
    wr[nw++] = range_of(y, N * M * 4);
    if (need > 0) wr[nw++] = range_of(ws, static_cast<int64_t>(need));
    st = check_alias(inputs, n, wr, nw);
    if (st != QG_OK) return st;

    (void)hipGetLastError();
    run_gemm(fmt, codes, scales, biases, x, y, M, K, N, ws, stream);
    return launch_status();
}

// Workgroups of the embedding gather: enough to fill the chip several times
// over; more rows are taken by the grid-stride loop.
constexpr int64_t kEmbedMaxGrid = 65536;

int embed_entry(int fmt, const void *codes, const void *scales, const void *biases,
                const int32_t *ids, float *out, int64_t M, int64_t K, int64_t n,
                hipStream_t stream)
{
    if (!known_format(fmt)) return QG_ERR_FORMAT;
    if (!codes || !scales || !ids || !out) return QG_ERR_NULL;
    if ((fmt == QG_U4_G64) != (biases != nullptr)) return QG_ERR_NULL;
    if (fmt != QG_U4_G64) return QG_ERR_UNSUPPORTED;
    if (M < 1 || M > kMaxM || K < 1 || K > kMaxK || K % k_unit(fmt) != 0 || n < 1 ||
        n > kMaxN)
        return QG_ERR_SHAPE;
    if (!aligned(codes, kAlign) || !aligned(scales, kAlign) || !aligned(biases, kAlign) ||
        !aligned(out, kAlign) || !aligned(ids, 4))
        return QG_ERR_ALIGN;
    Range inputs[4];
    int nr = 0;
    inputs[nr++] = range_of(codes, M * row_bytes(fmt, K));
    inputs[nr++] = range_of(scales, scale_bytes(fmt, M, K));
    inputs[nr++] = range_of(biases, bias_bytes(fmt, M, K));
    inputs[nr++] = range_of(ids, n * 4);
    Range wr[1];
    wr[0] = range_of(out, n * K * 4);
    const int st = check_alias(inputs, nr, wr, 1);
    if (st != QG_OK) return st;

    (void)hipGetLastError();
    qg::EmbedParams p{static_cast<const uint8_t *>(codes), static_cast<const uint16_t *>(scales),
                      static_cast<const uint16_t *>(biases), ids, out, M, K, n};
    const auto grid = static_cast<unsigned>(std::min(ceil_div(n, qg::kEmbedRows), kEmbedMaxGrid));
    hipLaunchKernelGGL(qg::embed_u4_kernel, dim3(grid), dim3(qg::kEmbedThreads), 0, stream, p);
    return launch_status();
}

// ---------------------------------------------------------------------------
// The library's own scratch, for callers that cannot allocate
// (qgemv_argmax_noalloc): one array per GPU, in the code object's device
// memory, held until the process ends. Kernels receive its device address,
// looked up once per device with that device current; the array's name in
// host code is only a handle for that lookup, never an address.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[QG_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (looked up on the
// first call on that device).
int static_scratch(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QG_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return QG_ERR_LAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QG_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

int qgemv(int fmt, const void *codes, const void *scales, const void *biases,
          const float *x, float *y, int64_t M, int64_t K, int batch, void *ws,
          size_t ws_bytes, hipStream_t stream)
{
    return gemv_entry(fmt, codes, scales, biases, x, y, nullptr, M, K, batch, ws, ws_bytes, stream);
}

int qgemv_argmax(int fmt, const void *codes, const void *scales, const void *biases,
                 const float *x, float *logits, int32_t *idx, int64_t M, int64_t K,
                 int batch, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (!idx) return QG_ERR_NULL;
    if (batch > QG_MAX_GEMV_BATCH)
        return wide_argmax_entry(fmt, codes, scales, biases, x, logits, idx, M, K, batch, ws,
                                 ws_bytes, stream);
    return gemv_entry(fmt, codes, scales, biases, x, logits, idx, M, K, batch, ws, ws_bytes,
                      stream);
}

int qgemv_argmax_noalloc(int fmt, const void *codes, const void *scales, const void *biases,
                         const float *x, float *logits, int32_t *idx, int64_t M, int64_t K,
                         int batch, hipStream_t stream)
{
    // the argument checks of qgemv_argmax that come before its workspace,
    // so that they are reported before the scratch is looked up
    if (!idx) return QG_ERR_NULL;
    const int st0 = check_weights(fmt, codes, scales, biases, x, M, K);
    if (st0 != QG_OK) return st0;
    if (batch < 1 || batch > QG_MAX_ARGMAX_BATCH) return QG_ERR_SHAPE;
    if ((logits && !aligned(logits, kAlign)) || !aligned(idx, 4)) return QG_ERR_ALIGN;
    // the workspace qgemv_argmax would need (0 for the arguments it still
    // rejects, which it then reports without the scratch)
    const size_t need = qg_workspace_bytes(QG_OP_GEMV_ARGMAX, fmt, M, K, batch);
    if (need > QG_STATIC_SCRATCH_BYTES) return QG_ERR_SCRATCH;
    void *ws = nullptr;
    if (need > 0) {
        const int st = static_scratch(&ws);
        if (st != QG_OK) return st;
    }
    return qgemv_argmax(fmt, codes, scales, biases, x, logits, idx, M, K, batch, ws,
                        need > 0 ? static_cast<size_t>(QG_STATIC_SCRATCH_BYTES) : 0, stream);
}

int qgemm(int fmt, const void *codes, const void *scales, const void *biases,
          const float *x, float *y, int64_t M, int64_t K, int64_t N, void *ws,
          size_t ws_bytes, hipStream_t stream)
{
    return gemm_entry(fmt, codes, scales, biases, x, y, M, K, N, ws, ws_bytes, stream);
}

int qembed(int fmt, const void *codes, const void *scales, const void *biases,
           const int32_t *ids, float *out, int64_t M, int64_t K, int64_t n, hipStream_t stream)
{
    return embed_entry(fmt, codes, scales, biases, ids, out, M, K, n, stream);
}

size_t qg_workspace_bytes(int op, int fmt, int64_t M, int64_t K, int64_t rows)
{
    if (!known_format(fmt)) return 0;
    if (M < 1 || M > kMaxM || K < 1 || K > kMaxK || K % k_unit(fmt) != 0) return 0;
    if (op == QG_OP_GEMV_ARGMAX && rows > QG_MAX_GEMV_BATCH && rows <= QG_MAX_ARGMAX_BATCH)
        return K <= qg::kGemmMaxK ? wide_argmax_workspace(fmt, M, K, rows) : 0;
    if (op == QG_OP_GEMV || op == QG_OP_GEMV_ARGMAX) {
        if (rows < 1 || rows > QG_MAX_GEMV_BATCH) return 0;
        return plan_gemv(fmt, M, K, static_cast<int>(rows), op == QG_OP_GEMV_ARGMAX).ws_bytes;
    }
    if (op == QG_OP_GEMM) {
        if (rows < 1 || rows > kMaxN || !gemm_shape_ok(M, K, rows)) return 0;
        return gemm_workspace(fmt, M, K, rows);
    }
    return 0;
}

const char *qg_status_str(int status)
{
    switch (status) {
    case QG_OK: return "ok";
    case QG_ERR_NULL: return "a required pointer is NULL (or biases given for a format without them)";
    case QG_ERR_FORMAT: return "unknown weight format";
    case QG_ERR_SHAPE: return "M, K or rows out of range, or K not a multiple of the format's unit";
    case QG_ERR_ALIGN: return "a pointer is not aligned as required";
    case QG_ERR_WORKSPACE: return "workspace missing or smaller than qg_workspace_bytes()";
    case QG_ERR_ALIAS: return "a written buffer overlaps another buffer";
    case QG_ERR_LAUNCH: return "kernel launch failed";
    case QG_ERR_UNSUPPORTED: return "format not implemented by this entry point";
    case QG_ERR_SCRATCH:
        return "the call needs more scratch than the library's static array holds "
               "(QG_STATIC_SCRATCH_BYTES); use the entry point with a caller workspace";
    default: return "unknown status";
    }
}

int qg_abi_version(void) { return QG_ABI_VERSION; }

}  // extern "C"
