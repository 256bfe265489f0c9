// gemm.hpp -- prefill product Y[n][m] = sum_k w[m][k] X[n][k] on the gfx950
// matrix cores (MFMA), with the packed weights dequantized in registers.
//
// Precision. The activations are float32 and the result must stay within
// 1e-5 of sum|w x|, so X cannot be rounded to bf16. Each X value is split
// exactly into three bf16 pieces, X = hi + mid + lo (truncation: hi takes the
// top 8 significant bits, mid the next 8, lo the last 8), and the product runs
// as three bf16 MFMAs accumulating in float32. The weight operand is exact in
// bf16 for every format: int8 codes (|q| <= 128 needs 8 bits), 4-bit codes
// and the signs +-1 of the 1-bit format. Per-row (int8) and per-group (int8
// and 4-bit: 64 k, 1-bit: 128 k) scales are applied in float32 outside the
// MFMA.
// (MiniCPM-V-4.6 on a Tesla C2075, academ.us 2607.14568, section 3.1:
// the prompt's projections contract whole matrices, not vectors; this kernel keeps
// the weights packed instead of dequantizing them to a float scratch first.)
//
// Tiling. A workgroup of 4 waves computes a BM (m) x BN (n) tile of Y
// (256 x 64, 128 x 128, 128 x 64, 64 x 128 or 64 x 64, chosen by the host
// so that the grid fills the 256 compute units); the waves sit side by side
// along n, each covering
// all BM weight rows, so a wave reads BM / 16 weight fragments and 3 * BN / 64
// activation fragments per k-step for 3 * BM * BN / 1024 MFMAs. For up to 32
// token rows the tile is 16 or 32 tokens wide and the waves split the
// weight rows instead (see gemm_kernel). A k-step stages 32 k of W
// (converted to bf16) in LDS, double-buffered: the step after the current
// one is staged from registers while the current MFMAs run, and the loads of
// the step after that are issued behind it, so one barrier per step
// suffices. LDS rows are 64 bytes with an XOR swizzle of their four 16-byte
// chunks (conflict-free fragment reads). The activations go from global
// memory straight into registers in the MFMA operand layout (each token row
// is used by one wave only) and are split there into their three bf16 pieces.
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
    const uint16_t *biases;   // 4-bit format: bf16 [M][K/64]
    const float *x;   // [N][K]
    float *y;         // [N][M], or nullptr (greedy head without logits)
    unsigned long long *keys;  // greedy head: [N][keys_m] keys of the waves' row blocks, or nullptr
    float *part;      // split K: [nsplit][N][M] partial products (y and keys unused)
    int64_t M, K, N;
    int tiles_m, tiles_n;
    int keys_m;       // greedy head: keys per token row (tiles_m x waves along m)
    int kt_split;     // 32-input steps per split of K (a multiple of 4), or 0: no split
    // Split tail: workgroups 0 .. nfull-1 each take one of tiles 0 .. nfull-1
    // over all of K; the workgroups after them take the remaining tiles in
    // tsplit pieces of kt_tail steps each (a multiple of 4) and store their
    // partial tiles in tpart [tsplit][tiles - nfull][BN][BM] (y unused for
    // them). tsplit = 0: no split tail.
    float *tpart;
    int nfull, tsplit, kt_tail;
};

// 8 nibbles of one dword (8 consecutive inputs, even k in the low nibbles)
// -> 8 bf16 codes in the order k = 0, 2, 4, 6, 1, 3, 5, 7. A byte holding one
// code (0..15) is, read as an OCP e4m3 number, exactly code * 2^-9; the
// gfx950 scaled fp8 -> bf16 conversion turns two such bytes into two exact
// bf16 codes in one instruction.
__device__ __forceinline__ bf16x8_t nibbles_to_bf16(uint32_t d)
{
    const uint32_t lo = d & 0x0f0f0f0fu, hi = (d >> 4) & 0x0f0f0f0fu;
    uint4 v;
    v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, false));
    v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, true));
    v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, false));
    v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, true));
    return __builtin_bit_cast(bf16x8_t, v);
}

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
    // each piece is the high half of its float32: one byte permute packs a
    // pair (bytes 2, 3 of the a word low, of the b word high)
    hi = __builtin_amdgcn_perm(ub, ua, 0x07060302u);
    mid = __builtin_amdgcn_perm(__float_as_uint(rb), __float_as_uint(ra), 0x07060302u);
    lo = __builtin_amdgcn_perm(__float_as_uint(lb), __float_as_uint(la), 0x07060302u);
}

// int8 code pair -> packed bf16x2 (exact: integers of at most 8 bits,
// converted with the packing conversion, whose rounding leaves them as they are).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t i8pair_to_bf16x2(uint32_t d, int byte0)
{
    const float a = static_cast<float>(static_cast<int8_t>((d >> (8 * byte0)) & 0xff));
    const float b = static_cast<float>(static_cast<int8_t>((d >> (8 * byte0 + 8)) & 0xff));
    const float2v_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Two sign bits (bit0 -> low half) -> packed bf16x2 of +-1: bit 1 -> +1.0
// (0x3F80), bit 0 -> -1.0 (0xBF80). `nbits` holds the inverted bits, so
// the multiply moves inverted bit 0 to bit 15 and inverted bit 1 to bit 31.
__device__ __forceinline__ uint32_t signpair_to_bf16x2(uint32_t nbits2)
{
    return ((nbits2 * 0x40008000u) & 0x80008000u) | 0x3F803F80u;
}

constexpr int GT_K = 32;    // k per step
constexpr int kGemmThreads = 256;
// k-steps of loads in flight (register sets), per format, as measured. With
// every load issued unconditionally two steps cover the latency for the
// byte formats (8-bit 3584 x 1024, N = 10240: 252 us at depth 2, 266 at 3);
// for the grouped formats a depth equal to the steps of one group also puts
// the group close at the same place of every unrolled pass. The 1-bit
// format keeps 4 (one 128-input group; 514 us at depth 2, 461 at 4 for
// 17408 x 5120, N = 512).
template <int FMT> struct GemmDepth { static constexpr int value = 2; };
template <> struct GemmDepth<FMT_B1_G128> { static constexpr int value = 4; };
// Workgroups per compute unit the register budget is set for: four for the
// 8-bit per-row 128 x 64 tile (110 VGPRs; 3584 x 1024, N = 2048: 62 -> 58
// us against three), three for the other 8-bit tiles of 64 token rows
// (group-64 128 x 64: 168 VGPRs; per-row 256 x 64: 164), so that further
// waves per SIMD hide the activation loads and splits (3584 x 1024, N =
// 10240: 245 -> 233 us at 128 x 64 against 128 x 128; 232 -> 201 us at
// 256 x 64, where each activation split feeds twice the MFMAs); two for
// every other tile (the 4-bit and 1-bit 128 x 64 tiles need 202 and 204;
// the 1-bit tile at prefetch depth 2 fits three, but 17408 x 5120, N = 512
// then takes 336 us instead of 269).
template <int FMT, int BM, int BN>
constexpr int gemm_occupancy()
{
    if (FMT == FMT_I8_ROW && BM == 128 && BN == 64) return 4;
    constexpr bool i8 = FMT == FMT_I8_ROW || FMT == FMT_I8_G64;
    return i8 && BN == 64 && (BM == 128 || (FMT == FMT_I8_ROW && BM == 256)) ? 3 : 2;
}
constexpr int kGemmInterleave = 5;   // VALU instructions issued after each MFMA

// Largest K of the matrix-core prefill: the buffer loads below address a
// tile's activation rows (128 rows of 4 K bytes) with 32-bit offsets, and
// every range stays below 2^30 bytes.
constexpr int64_t kGemmMaxK = int64_t(1) << 21;

// Raw buffer resource over [base, base + bytes) (gfx9 family descriptor
// word 3: 32-bit data format, untyped). A load whose offset lies outside
// the range returns zeros, so tile edges need no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0,
                                             static_cast<int>(bytes), 0x00020000);
}
constexpr uint32_t kOutOfRange = 0x80000000u;   // above every range used here

// `off`, or an offset out of range when i >= n, by arithmetic only: a select
// here would be turned into a branch around the load.
__device__ __forceinline__ uint32_t in_range_or_out(uint32_t off, int64_t i, int64_t n)
{
    uint32_t out = static_cast<uint32_t>(static_cast<uint64_t>(n - 1 - i) >> 63) << 31;
    asm("" : "+v"(out));
    return off | out;
}

// Physical 16-byte chunk of logical chunk c (0..3) in LDS row r (rows of
// 64 bytes). Under this XOR swizzle both access patterns are free of bank
// conflicts, whether the LDS serves a 16-byte-per-lane access 16 lanes per
// 256-byte cycle or 8 lanes per 128-byte cycle: the fragment reads (16
// consecutive rows from a multiple of 16, one logical chunk) and the
// staging writes (8 consecutive rows from a multiple of 8, logical chunks
// c and c ^ 2 on alternate lanes). The earlier swizzle c ^ ((r/2 ^ r/8) & 3)
// left the staging writes 2-way conflicted in 16-lane cycles.
__device__ __forceinline__ int swz_chunk(int r, int c)
{
    return c ^ ((((r >> 1) ^ (r >> 2)) & 1) | ((((r >> 2) ^ (r >> 3)) & 1) << 1));
}

// Workgroup tile BM (weight rows m) x BN (token rows n); the 4 waves form a
// WM x WN grid: WN side by side along n, each covering BM / WM rows and
// BN / WN tokens. Wide tiles put all 4 along n (every wave reads all BM
// weight rows from LDS); the narrow tiles of a few token rows (BN = 16 or
// 32) put 4 or 2 along m, so that no MFMA works on more padding than the
// last 16-token block holds.
template <int FMT, int BM, int BN, int WN = 4>
__global__ __launch_bounds__(kGemmThreads, (gemm_occupancy<FMT, BM, BN>())) void gemm_kernel(GemmParams p)
{
    static_assert(WN == 1 || WN == 2 || WN == 4, "4 waves in a WM x WN grid");
    constexpr int WM = 4 / WN;
    constexpr int TI = BM / (16 * WM);   // 16-row weight blocks per wave
    constexpr int TJ = BN / (16 * WN);   // 16-token blocks per wave
    // staging items per thread: a row half (16 k of the 32-k step) each,
    // rows sr and sr + 128
    constexpr int SI = BM * 2 > kGemmThreads ? BM * 2 / kGemmThreads : 1;
    static_assert(TI >= 1 && TJ >= 1 && BM * 2 <= kGemmThreads * SI && SI <= 2, "staging items");
    // double-buffered weight stages: [buffer][row][4 chunks of 8 bf16]
    __shared__ uint4 lw[2][BM * 4];
    // per-group coefficients of the current and next group: scales (grouped
    // formats) and biases (4-bit)
    constexpr bool GROUPED = FMT != FMT_I8_ROW;
    constexpr int GSTEPS = FMT == FMT_B1_G128 ? 4 : 2;   // 32-k steps per group
    __shared__ float ls[2][BM];
    __shared__ float lb[2][FMT == FMT_U4_G64 ? BM : 1];

    // XCD-aware order: consecutive workgroup ids go round-robin to the 8
    // XCDs; give each XCD a contiguous run of tiles (m fastest) so the tiles
    // that share an X block meet in the same L2.
    const int ntiles = p.tiles_m * p.tiles_n;
    int bid = blockIdx.x;
    int piece = -1;   // split tail: this workgroup's piece of K
    if (p.tsplit > 0 && bid >= p.nfull) {
        piece = (bid - p.nfull) % p.tsplit;
        bid = p.nfull + (bid - p.nfull) / p.tsplit;
    } else {
        const int nmap = p.tsplit > 0 ? p.nfull : ntiles;
        if ((nmap & 7) == 0) bid = (bid & 7) * (nmap >> 3) + (bid >> 3);
    }
    const int tm = bid % p.tiles_m, tn = bid / p.tiles_m;
    const int64_t m0 = static_cast<int64_t>(tm) * BM, n0 = static_cast<int64_t>(tn) * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = (wave % WN) * (BN / WN), wm = (wave / WN) * (BM / WM);
    const int fr = lane & 15, fq = lane >> 4;

    // weight staging assignment: thread -> (row, half of the 32-k step), and
    // row + 128 for the 256-row tile
    const int sr = tid >> 1, sh = tid & 1;
    const bool wst = 2 * BM >= kGemmThreads || sr < BM;   // constant when every thread stages
    constexpr bool I8 = FMT == FMT_I8_ROW || FMT == FMT_I8_G64;   // int8 codes
    const int64_t row_bytes = I8 ? p.K : FMT == FMT_U4_G64 ? p.K / 2 : p.K / 8;
    const int64_t wrows = min(static_cast<int64_t>(BM), p.M - m0);    // valid rows of the tile
    const int64_t xrows = min(static_cast<int64_t>(BN), p.N - n0);    // valid tokens of the tile
    // Buffer views of the tile's weight rows and activation rows: a row
    // beyond M or N lies outside its view and reads as zero. Offsets of
    // inputs beyond K (the last step of an odd number of 16-k halves) are
    // moved out of range explicitly.
    const auto wbuf = buffer_rsrc(p.codes + m0 * row_bytes, wrows * row_bytes);
    const auto xbuf = buffer_rsrc(p.x + n0 * p.K, xrows * p.K * 4);
    uint32_t woff[SI];
#pragma unroll
    for (int it = 0; it < SI; ++it)
        woff[it] = wst ? static_cast<uint32_t>((sr + 128 * it) * row_bytes) : kOutOfRange;
    // activation fragments: this lane feeds the MFMA operand of token
    // n0 + wn + 16 j + fr with inputs 8 fq .. 8 fq + 7 of each step; each
    // token row is used by this wave only, so it goes straight from global
    // memory to registers (no LDS stage)
    uint32_t xoff[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j)
        xoff[j] = static_cast<uint32_t>(((wn + 16 * j + fr) * p.K + 8 * fq) * 4);
    // steps of this workgroup: all of K, or split blockIdx.y of it (kt
    // counts local steps below; loads add ktb; ktb is a multiple of every
    // group's step count, so group boundaries stay where they are)
    const int nk_all = static_cast<int>((p.K + GT_K - 1) / GT_K);   // K is a multiple of 16
    const int kts = piece >= 0 ? p.kt_tail : p.kt_split;
    const int ktb = piece >= 0 ? piece * p.kt_tail : p.kt_split > 0 ? static_cast<int>(blockIdx.y) * p.kt_split : 0;
    const int nk = kts > 0 ? min(kts, nk_all - ktb) : nk_all;
    const int64_t groups = p.K / (32 * GSTEPS);
    constexpr int SBYTES = FMT == FMT_I8_G64 ? 4 : 2;   // bytes per group coefficient
    const auto sbuf = buffer_rsrc(static_cast<const uint8_t *>(p.scales) + m0 * groups * SBYTES,
                                  wrows * groups * SBYTES);
    const auto bbuf = buffer_rsrc(reinterpret_cast<const uint8_t *>(p.biases) + m0 * groups * 2,
                                  FMT == FMT_U4_G64 ? wrows * groups * 2 : 0);
    const uint32_t soff = tid < BM ? static_cast<uint32_t>(tid * groups * SBYTES) : kOutOfRange;
    const uint32_t boff = tid < BM ? static_cast<uint32_t>(tid * groups * 2) : kOutOfRange;

    struct Regs {
        uint4 w[SI];      // per item, I8: 16 codes; U4: w.x, w.y = 16 nibbles; B1: low 16 bits = 16 sign bits
        uint32_t s, b;    // grouped formats, first step of a group: scale (and bias) bits of row m0 + tid
        float4 x[TJ][2];  // this lane's activations of the step (8 consecutive inputs per block)
    };

    // Every load is issued unconditionally (edges read zeros through the
    // buffer range checks), so the compiler can count the loads in flight
    // exactly and waits only for the step it needs.
    auto load_w = [&](Regs &R, int kt) {
        const int64_t k = static_cast<int64_t>(kt + ktb) * GT_K + 16 * sh;
        constexpr int KSHIFT = I8 ? 0 : FMT == FMT_U4_G64 ? 1 : 3;   // input index -> byte in the row
#pragma unroll
        for (int it = 0; it < SI; ++it) {
            const uint32_t off = in_range_or_out(woff[it] + static_cast<uint32_t>(k >> KSHIFT), k, p.K);
            if (I8) {
                R.w[it] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wbuf, off, 0, 0));
            } else if (FMT == FMT_U4_G64) {
                const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(wbuf, off, 0, 0));
                R.w[it].x = v.x;
                R.w[it].y = v.y;
            } else {
                R.w[it].x = __builtin_amdgcn_raw_buffer_load_b16(wbuf, off, 0, 0);
            }
        }
        if (GROUPED && kt % GSTEPS == 0) {
            const uint32_t o = soff + static_cast<uint32_t>(((kt + ktb) / GSTEPS) * SBYTES);
            if (FMT == FMT_I8_G64) {
                R.s = __builtin_amdgcn_raw_buffer_load_b32(sbuf, o, 0, 0);
            } else {
                R.s = __builtin_amdgcn_raw_buffer_load_b16(sbuf, o, 0, 0);
                if (FMT == FMT_U4_G64)
                    R.b = __builtin_amdgcn_raw_buffer_load_b16(
                        bbuf, boff + static_cast<uint32_t>(((kt + ktb) / GSTEPS) * 2), 0, 0);
            }
        }
    };

    auto load_x = [&](Regs &R, int kt) {
        const int64_t k = static_cast<int64_t>(kt + ktb) * GT_K;
        // K is a multiple of 16: a block of 8 inputs is all in or all out
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const uint32_t off = in_range_or_out(xoff[j] + static_cast<uint32_t>(k * 4), k + 8 * fq, p.K);
            R.x[j][0] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xbuf, off, 0, 0));
            R.x[j][1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xbuf, off + 16, 0, 0));
        }
    };

    auto stage = [&](const Regs &R, int kt, int b) {
#pragma unroll
        for (int it = 0; it < SI; ++it) {
            if (!wst) break;
            const uint4 rw = R.w[it];
            const int row = sr + 128 * it;
            uint32_t wv[8];
            if (I8) {
                const uint32_t d[4] = {rw.x, rw.y, rw.z, rw.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    wv[2 * j] = i8pair_to_bf16x2(d[j], 0);
                    wv[2 * j + 1] = i8pair_to_bf16x2(d[j], 2);
                }
            } else if (FMT == FMT_U4_G64) {
                // codes in the order k = 0, 2, 4, 6, 1, 3, 5, 7 of each 8
                const uint4 c0 = __builtin_bit_cast(uint4, nibbles_to_bf16(rw.x));
                const uint4 c1 = __builtin_bit_cast(uint4, nibbles_to_bf16(rw.y));
                wv[0] = c0.x; wv[1] = c0.y; wv[2] = c0.z; wv[3] = c0.w;
                wv[4] = c1.x; wv[5] = c1.y; wv[6] = c1.z; wv[7] = c1.w;
            } else {
                // rows beyond M carry no codes: their (unused) weights become -1
                const uint32_t nbits = ~rw.x;
#pragma unroll
                for (int j = 0; j < 8; ++j) wv[j] = signpair_to_bf16x2((nbits >> (2 * j)) & 3u);
            }
            lw[b][row * 4 + swz_chunk(row, 2 * sh)] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            lw[b][row * 4 + swz_chunk(row, 2 * sh + 1)] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
        }
        if (GROUPED && kt % GSTEPS == 0 && tid < BM) {
            const int gb = (kt / GSTEPS) & 1;
            if (FMT == FMT_B1_G128) {
                ls[gb][tid] = fp16_bits_to_f32(static_cast<uint16_t>(R.s));
            } else if (FMT == FMT_I8_G64) {
                ls[gb][tid] = __uint_as_float(R.s);
            } else {
                ls[gb][tid] = bf16_bits_to_f32(R.s);
                lb[gb][tid] = bf16_bits_to_f32(R.b);
            }
        }
    };

    floatx4_t acc[TI][TJ];
    floatx4_t gacc[TI][TJ];  // grouped formats: sums of the current group
    float xs[TJ];            // 4-bit format: this lane's token's activation sum over the group
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            gacc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
    for (int j = 0; j < TJ; ++j) xs[j] = 0.f;

    // exact three-piece split of this lane's activations of step kt (the
    // 4-bit operand order k = 0, 2, 4, 6, 1, 3, 5, 7 for the 4-bit format),
    // and for the 4-bit format the running group sum of the activations
    auto split = [&](int kt, const Regs &R, bf16x8_t (&bx)[TJ][3]) {
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const float4 u = R.x[j][0], v = R.x[j][1];
            uint32_t h[4], md[4], lo[4];
            if (FMT == FMT_U4_G64) {
                split3_pair(u.x, u.z, h[0], md[0], lo[0]);
                split3_pair(v.x, v.z, h[1], md[1], lo[1]);
                split3_pair(u.y, u.w, h[2], md[2], lo[2]);
                split3_pair(v.y, v.w, h[3], md[3], lo[3]);
                // this lane's 8 inputs, then the other three blocks of the step
                float t = ((u.x + u.y) + (u.z + u.w)) + ((v.x + v.y) + (v.z + v.w));
                t = pair_sum<5>(pair_sum<4>(t));   // the other three blocks (lanes ^ 16, ^ 32)
                xs[j] = kt % GSTEPS == 0 ? t : xs[j] + t;
            } else {
                split3_pair(u.x, u.y, h[0], md[0], lo[0]);
                split3_pair(u.z, u.w, h[1], md[1], lo[1]);
                split3_pair(v.x, v.y, h[2], md[2], lo[2]);
                split3_pair(v.z, v.w, h[3], md[3], lo[3]);
            }
            bx[j][0] = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
            bx[j][1] = __builtin_bit_cast(bf16x8_t, make_uint4(md[0], md[1], md[2], md[3]));
            bx[j][2] = __builtin_bit_cast(bf16x8_t, make_uint4(lo[0], lo[1], lo[2], lo[3]));
        }
    };

    // the MFMAs of step kt on its weights (LDS buffer kt & 1) and its
    // activation pieces bx, then the group close
    auto compute = [&](int kt, const bf16x8_t (&bx)[TJ][3]) {
        const int b = kt & 1;
        // the first MFMA of a group starts its sum from zero (the group's
        // position is known at compile time in the unrolled pipeline)
        const bool first = GROUPED && kt % GSTEPS == 0;
        const floatx4_t zero = {0.f, 0.f, 0.f, 0.f};
        if constexpr (TI >= 8) {
            // the weight fragments two at a time through all three pieces,
            // so that only two are held (registers: the 256-row tile needs
            // this to fit at all, the 128-row tiles need 12 to 43 fewer)
#pragma unroll
            for (int i = 0; i < TI; i += 2) {
                bf16x8_t a2[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int r = wm + 16 * (i + u) + fr;
                    a2[u] = __builtin_bit_cast(bf16x8_t, lw[b][r * 4 + swz_chunk(r, fq)]);
                }
#pragma unroll
                for (int pc = 0; pc < 3; ++pc)
#pragma unroll
                    for (int j = 0; j < TJ; ++j)
#pragma unroll
                        for (int u = 0; u < 2; ++u)
                            if (FMT == FMT_I8_ROW)
                                acc[i + u][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2[u], bx[j][pc], acc[i + u][j], 0, 0, 0);
                            else
                                gacc[i + u][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    a2[u], bx[j][pc], first && pc == 0 ? zero : gacc[i + u][j], 0, 0, 0);
            }
        } else {
        bf16x8_t a[TI];
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            const int r = wm + 16 * i + fr;
            a[i] = __builtin_bit_cast(bf16x8_t, lw[b][r * 4 + swz_chunk(r, fq)]);
        }
#pragma unroll
        for (int pc = 0; pc < 3; ++pc) {
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
#pragma unroll
                for (int i = 0; i < TI; ++i) {
                    if (FMT == FMT_I8_ROW)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bx[j][pc], acc[i][j], 0, 0, 0);
                    else
                        gacc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            a[i], bx[j][pc], first && pc == 0 ? zero : gacc[i][j], 0, 0, 0);
                }
            }
        }
        }
        if (GROUPED && kt % GSTEPS == GSTEPS - 1) {
            // close the group: acc += scale[m][g] * (sum of code * x over the
            // group) [+ bias[m][g] * (sum of x over the group), 4-bit]
            const int gb = (kt / GSTEPS) & 1;
#pragma unroll
            for (int i = 0; i < TI; ++i) {
                const float4 s4 = *reinterpret_cast<const float4 *>(&ls[gb][wm + 16 * i + 4 * fq]);
                const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
                float bv[4] = {0.f, 0.f, 0.f, 0.f};
                if (FMT == FMT_U4_G64) {
                    const float4 b4 = *reinterpret_cast<const float4 *>(&lb[gb][wm + 16 * i + 4 * fq]);
                    bv[0] = b4.x; bv[1] = b4.y; bv[2] = b4.z; bv[3] = b4.w;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int j = 0; j < TJ; ++j) {
                        float a = acc[i][j][r];
                        if (FMT == FMT_U4_G64) a = fmaf(bv[r], xs[j], a);
                        acc[i][j][r] = fmaf(sv[r], gacc[i][j][r], a);
                    }
            }
        }
    };

    // pipeline: LDS buffer kt & 1 holds the weights of step kt; register set
    // s % D holds the weights and activations of step s from their load (D
    // steps ahead) until the step before s, when the weights are staged and
    // the activations split; the split pieces of the step being computed
    // stay in registers (bx), so a step's MFMAs never wait for its own
    // VALU work, which runs beside the previous step's MFMAs
    constexpr int D = GemmDepth<FMT>::value;
    Regs R[D];
#pragma unroll
    for (int u = 0; u < D; ++u)
        if (u < nk) {
            load_w(R[u], u);
            load_x(R[u], u);
        }
    bf16x8_t bx[TJ][3];
    split(0, R[0], bx);
    stage(R[0], 0, 0);
    if (D < nk) {
        load_x(R[0], D);
        load_w(R[0], D);
    }
    __syncthreads();
    int kt0 = 0;
    // steady state: every step computes, splits and stages the next step
    // and loads D + 1 steps ahead
    for (; kt0 + 2 * D < nk; kt0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int kt = kt0 + u;
            Regs &N = R[(u + 1) % D];
            compute(kt, bx);
            bf16x8_t bn[TJ][3];
            split(kt + 1, N, bn);
            load_x(N, kt + 1 + D);
            stage(N, kt + 1, (kt + 1) & 1);
            load_w(N, kt + 1 + D);
#pragma unroll
            for (int j = 0; j < TJ; ++j)
#pragma unroll
                for (int c = 0; c < 3; ++c) bx[j][c] = bn[j][c];
            // issue order: the fragment reads, then each MFMA followed by a
            // few VALU instructions (the next step's split and staging), so
            // that they run while the matrix pipe is busy
            __builtin_amdgcn_sched_group_barrier(0x100, TI, 0);
#pragma unroll
            for (int i = 0; i < 3 * TI * TJ; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, kGemmInterleave, 0);
            }
            __syncthreads();
        }
    }
    // drain
    for (; kt0 < nk; kt0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int kt = kt0 + u;
            if (kt < nk) {
                Regs &N = R[(u + 1) % D];
                compute(kt, bx);
                if (kt + 1 < nk) {
                    bf16x8_t bn[TJ][3];
                    split(kt + 1, N, bn);
                    if (kt + 1 + D < nk) load_x(N, kt + 1 + D);
                    stage(N, kt + 1, (kt + 1) & 1);
                    if (kt + 1 + D < nk) load_w(N, kt + 1 + D);
#pragma unroll
                    for (int j = 0; j < TJ; ++j)
#pragma unroll
                        for (int c = 0; c < 3; ++c) bx[j][c] = bn[j][c];
                }
                __syncthreads();
            }
        }
    }

    // epilogue: row scale (int8), store Y[n][m .. m+3]; greedy head: the
    // best (value, lowest index) key of the wave's rows per token row
    const bool vec = (p.M & 3) == 0;
    uint64_t best[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j) best[j] = 0ull;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
        const int64_t mb = m0 + wm + 16 * i + 4 * fq;
        float s[4] = {1.f, 1.f, 1.f, 1.f};
        if (FMT == FMT_I8_ROW) {
            const float *sp = static_cast<const float *>(p.scales);
#pragma unroll
            for (int r = 0; r < 4; ++r) s[r] = mb + r < p.M ? sp[mb + r] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int64_t n = n0 + wn + 16 * j + fr;
            if (n >= p.N) continue;
            const float v[4] = {s[0] * acc[i][j][0], s[1] * acc[i][j][1], s[2] * acc[i][j][2],
                                s[3] * acc[i][j][3]};
            if (piece >= 0) {
                // partial tile, stored whole ([token][row] within the tile)
                float *dst = p.tpart + ((static_cast<int64_t>(piece) * (ntiles - p.nfull) + (bid - p.nfull)) * BN +
                                        (n - n0)) * BM + (mb - m0);
                *reinterpret_cast<float4 *>(dst) = make_float4(v[0], v[1], v[2], v[3]);
                continue;
            }
            if (p.keys != nullptr) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (mb + r < p.M) {
                        const uint64_t k = argmax_key(v[r], static_cast<uint32_t>(mb + r));
                        best[j] = k > best[j] ? k : best[j];
                    }
            }
            float *out = p.kt_split > 0 ? p.part + static_cast<int64_t>(blockIdx.y) * p.N * p.M : p.y;
            if (out == nullptr) continue;
            float *dst = out + n * p.M + mb;
            if (vec && mb + 3 < p.M) {
                *reinterpret_cast<float4 *>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
                if (mb < p.M) dst[0] = v[0];
                if (mb + 1 < p.M) dst[1] = v[1];
                if (mb + 2 < p.M) dst[2] = v[2];
                if (mb + 3 < p.M) dst[3] = v[3];
            }
        }
    }
    if (p.keys != nullptr) {
        // lanes fr, fr + 16, fr + 32, fr + 48 hold the same token rows
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            uint64_t k = best[j];
            uint64_t o = shfl_xor_u64(k, 16);
            k = o > k ? o : k;
            o = shfl_xor_u64(k, 32);
            k = o > k ? o : k;
            const int64_t n = n0 + wn + 16 * j + fr;
            if (fq == 0 && n < p.N) p.keys[n * p.keys_m + tm * WM + wave / WN] = k;
        }
    }
}

// Split K: y[n][m] = sum over splits s of part[s][n][m], added in split
// order (one thread per 4 outputs; M a multiple of 4 takes 16-byte accesses).
__global__ __launch_bounds__(256) void gemm_splitk_combine_kernel(const float *part, float *y,
                                                                  int64_t M, int64_t N, int nsplit)
{
    const int64_t total = M * N;
    const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
    if (i >= total) return;
    if ((M & 3) == 0) {
        float4 a = *reinterpret_cast<const float4 *>(part + i);
        for (int s = 1; s < nsplit; ++s) {
            const float4 b = *reinterpret_cast<const float4 *>(part + s * total + i);
            a.x += b.x;
            a.y += b.y;
            a.z += b.z;
            a.w += b.w;
        }
        *reinterpret_cast<float4 *>(y + i) = a;
    } else {
        for (int64_t e = i; e < min(i + 4, total); ++e) {
            float a = part[e];
            for (int s = 1; s < nsplit; ++s) a += part[s * total + e];
            y[e] = a;
        }
    }
}

// Split tail: Y of tiles nfull .. tiles-1 = sum over pieces s of
// tpart[s][t][n][m] (tile-local token n, row m), added in piece order. One
// thread per 4 outputs of a tile, tiles of BM x BN.
__global__ __launch_bounds__(256) void gemm_tail_combine_kernel(const float *tpart, float *y, int64_t M,
                                                                int64_t N, int tiles_m, int nfull, int ntail,
                                                                int tsplit, int bm, int bn)
{
    const int64_t tile_elems = static_cast<int64_t>(bm) * bn;
    const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
    if (i >= ntail * tile_elems) return;
    const int t = static_cast<int>(i / tile_elems);
    const int e = static_cast<int>(i % tile_elems);
    const int tile = nfull + t;
    const int64_t m = static_cast<int64_t>(tile % tiles_m) * bm + e % bm;
    const int64_t n = static_cast<int64_t>(tile / tiles_m) * bn + e / bm;
    if (n >= N || m >= M) return;
    const int64_t stride = static_cast<int64_t>(ntail) * tile_elems;
    float4 a = *reinterpret_cast<const float4 *>(tpart + i);
    for (int s = 1; s < tsplit; ++s) {
        const float4 b = *reinterpret_cast<const float4 *>(tpart + s * stride + i);
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
    }
    float *dst = y + n * M + m;
    if ((M & 3) == 0 && m + 3 < M) {
        *reinterpret_cast<float4 *>(dst) = a;
    } else {
        dst[0] = a.x;
        if (m + 1 < M) dst[1] = a.y;
        if (m + 2 < M) dst[2] = a.z;
        if (m + 3 < M) dst[3] = a.w;
    }
}

// Greedy selection over the keys of the prefill-shaped head: one workgroup
// per token row n reduces keys[n][0 .. nkeys) and writes idx[n] (the key
// order makes the result the lowest index of the maximum).
__global__ __launch_bounds__(256) void argmax_keys_kernel(const unsigned long long *keys, int nkeys,
                                                          int32_t *idx)
{
    __shared__ unsigned long long s_best[4];
    const int64_t n = blockIdx.x;
    uint64_t best = 0ull;
    for (int t = threadIdx.x; t < nkeys; t += blockDim.x) {
        const uint64_t k = keys[n * nkeys + t];
        best = k > best ? k : best;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint64_t other = shfl_xor_u64(best, o);
        best = other > best ? other : best;
    }
    if ((threadIdx.x & 63) == 0) s_best[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 4; ++w) best = s_best[w] > best ? s_best[w] : best;
        idx[n] = static_cast<int32_t>(argmax_key_index(best));
    }
}

}  // namespace qg
