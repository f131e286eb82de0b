// Batched-token (prefill) product on the matrix cores: y[t][i] = sum_j W[i][j] x[t][j]
// for n_tok > 1 with W in any of the five formats, and the fused first half of
// the SwiGLU block, h = silu(Wg x) * (Wu x).
//
// With several tokens every weight read is shared by all of them, so the work
// is a dense contraction and belongs on the matrix units (llmoxide blog,
// section 11 "Prefill and decode": a tile of weights is dequantized once and
// run as a real GEMM).  Here:
//   * each wave owns MTR 16-row tiles of every matrix (NMAT of them) and the
//     workgroup NTW 16-token tiles; K advances by super-steps of 4Q blocks;
//   * weights are read row by row in runs of 64Q bytes (128Q for the 8-bit
//     formats; whole cache lines, one run per row and super-step) into
//     registers, then transposed through a per-wave LDS area into the
//     v_mfma_f32_16x16x32_bf16 A layout (lane l:
//     row l%16, k-group l/16), where each lane dequantizes its block exactly in
//     fp32 (q*D - M via the binary16-subnormal trick and v_fma_mix_f32, as in
//     the GEMV: Q4_0 D = d, M = 8d; Q4_K, whose repacked sub-blocks have the
//     Q4_0 nibble order, D = d*sc and M = dmin*m of the sub-block, both exact;
//     Q6_K, the same nibble order with the two high bits of each code OR-ed
//     in from the high-bit plane, D = d*sc of each 16-column half and M = 32D;
//     Q8_0 and per-row INT8, 32-byte blocks whose signed bytes xor 0x80 are
//     q + 128, D = d or 1 and M = 128D, the INT8 row scale multiplying the
//     fp32 sums) and rounds to bf16 (nearest even);
//   * the workgroup stages the x tile of the super-step in LDS as bf16 (nearest
//     even), in natural column order: the decode emits 8 consecutive columns
//     per operand, so A and B agree on k without any shuffle;
//   * fp32 accumulation; the epilogue writes y, or silu(g)*u for the gate/up
//     pair (tiles of Wg and Wu with the same rows sit in the same lanes), or
//     raw partial sums when K is split over workgroups.
// Every weight is decoded once per token group (once per kernel when the
// group spans all tokens), and x never needs a staging buffer in HBM.
//
// This header holds the kernel and its launch; prefill_<format>.hip
// instantiates it per format (compiled in parallel) and prefill.hip holds the
// tile choice, the split-K reduce and the RMSNorm launch.
#pragma once

#include <hip/hip_ext.h>

#include <atomic>
#include <cstdint>
#include <type_traits>

#include "qg_internal.h"

namespace qg {

struct PrefillParams {
    const uint8_t *q[2];
    const float *x;  // [n_tok][cols] fp32
    float *y;        // [n_tok][rows], or the partials [ksplit][NMAT][n_tok][rows] when ksplit > 1
    int64_t rows;
    int64_t row_qbytes;
    int64_t soff;
    int64_t row_groups;
    int nb;          // 32-weight blocks per row (cols / 32): Q4_0 blocks or Q4_K sub-blocks
    int cols;
    int ssteps;      // super-steps (Q K steps each) covering the row
    int n_tok;
    int tok_groups;
    int ksplit;      // K ranges, one per workgroup of a (row group, token group)
    int spk;         // super-steps per K range; every range is non-empty
    const float *resid;  // NMAT 1: residual [n_tok][rows] added to y (may be y itself), or null
    int64_t hoff;    // Q6_K: offsets of the high-bit plane and the f16 d plane
    int64_t doff;
    const uint16_t *xb;  // null, or x already rounded to bf16 (nearest even) [n_tok][cols]: read instead of x
    uint16_t *yb;        // NMAT 2 without a K split: null, or where y is also written rounded to bf16
};

// Split-K sum of the partials (prefill.hip): y = sum over the ksplit ranges
// (range order) of part, plus resid for one matrix, or silu(g) * u for the
// pair; n = n_tok * rows; stop (may be null) is recorded when it ends.
hipError_t launch_prefill_reduce(int nmat, const float *part, float *y, int64_t n, int ksplit, const float *resid,
                                 hipStream_t s, hipEvent_t stop, uint16_t *yb = nullptr);
// One format's built shapes (prefill_<format>.hip).
hipError_t prefill_dispatch_q4_0(const PrefillCfg &c, int nmat, const PrefillParams &p, float *y, hipStream_t s);
hipError_t prefill_dispatch_q4_k(const PrefillCfg &c, int nmat, const PrefillParams &p, float *y, hipStream_t s);
hipError_t prefill_dispatch_q6_k(const PrefillCfg &c, int nmat, const PrefillParams &p, float *y, hipStream_t s);
hipError_t prefill_dispatch_q8_0(const PrefillCfg &c, int nmat, const PrefillParams &p, float *y, hipStream_t s);
hipError_t prefill_dispatch_i8row(const PrefillCfg &c, int nmat, const PrefillParams &p, float *y, hipStream_t s);

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));


template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (N > 0) {
        static_for<N - 1>(f);
        f(std::integral_constant<int, N - 1>{});
    }
}

__device__ __forceinline__ float half_lo(uint32_t v)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t v)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two fp32 -> two bf16 (nearest even) in one v_cvt_pk_bf16_f32; a in the low half
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Columns 8c .. 8c+7 of a block as 8 bf16 weights q*D - M, c = 0..3.
// Column j < 16 is the low nibble of byte j, column j >= 16 the high nibble of
// byte j-16; so c = 0, 1 take the low nibbles of words (2c, 2c+1) and c = 2, 3
// the high nibbles of words (2c-4, 2c-3).  A masked nibble pair read as two
// binary16 subnormals is q*2^-24 (low) or q*2^-20 (high); with ds = D*2^24 or
// D*2^20 and n8 = -M, fma(that, ds, n8) is q*D - M exactly in fp32 (for Q4_0
// (q-8)*d; for Q4_K d*sc*q - dmin*m, whose two products are exact and whose
// difference rounds once, as the format's own fp32 value does).
__device__ __forceinline__ bf16x8 decode8(uint32_t wa, uint32_t wb, uint32_t mask, float ds, float n8)
{
    const uint32_t ea = wa & mask, oa = (wa >> 8) & mask;   // bytes (0, 2) and (1, 3)
    const uint32_t eb = wb & mask, ob = (wb >> 8) & mask;
    uint4 u;
    u.x = pack_bf16(__builtin_fmaf(half_lo(ea), ds, n8), __builtin_fmaf(half_lo(oa), ds, n8));
    u.y = pack_bf16(__builtin_fmaf(half_hi(ea), ds, n8), __builtin_fmaf(half_hi(oa), ds, n8));
    u.z = pack_bf16(__builtin_fmaf(half_lo(eb), ds, n8), __builtin_fmaf(half_lo(ob), ds, n8));
    u.w = pack_bf16(__builtin_fmaf(half_hi(eb), ds, n8), __builtin_fmaf(half_hi(ob), ds, n8));
    return __builtin_bit_cast(bf16x8, u);
}

// Q6_K: as decode8, the codes' two high bits OR-ed in from the high-bit words
// of the two code words (ha for wa, hb for wb; each already shifted by 2 for
// an odd code word), at bit 4 of each half for the low nibbles (the code is
// q*2^-24) or at bit 8 for the high nibbles (q*2^-20); ds = D*2^24 or D*2^20,
// n8 = -32D.
__device__ __forceinline__ bf16x8 decode8_q6(uint32_t wa, uint32_t wb, uint32_t ha, uint32_t hb, bool high, float ds,
                                            float n8)
{
    uint32_t ea, oa, eb, ob;
    if (high) {
        ea = (wa & 0x00F000F0u) | (ha & 0x03000300u);
        oa = ((wa >> 8) & 0x00F000F0u) | ((ha << 8) & 0x03000300u);
        eb = (wb & 0x00F000F0u) | (hb & 0x03000300u);
        ob = ((wb >> 8) & 0x00F000F0u) | ((hb << 8) & 0x03000300u);
    } else {
        ea = (wa & 0x000F000Fu) | (ha & 0x00300030u);
        oa = ((wa >> 8) & 0x000F000Fu) | ((ha >> 8) & 0x00300030u);
        eb = (wb & 0x000F000Fu) | (hb & 0x00300030u);
        ob = ((wb >> 8) & 0x000F000Fu) | ((hb >> 8) & 0x00300030u);
    }
    uint4 u;
    u.x = pack_bf16(__builtin_fmaf(half_lo(ea), ds, n8), __builtin_fmaf(half_lo(oa), ds, n8));
    u.y = pack_bf16(__builtin_fmaf(half_hi(ea), ds, n8), __builtin_fmaf(half_hi(oa), ds, n8));
    u.z = pack_bf16(__builtin_fmaf(half_lo(eb), ds, n8), __builtin_fmaf(half_lo(ob), ds, n8));
    u.w = pack_bf16(__builtin_fmaf(half_hi(eb), ds, n8), __builtin_fmaf(half_hi(ob), ds, n8));
    return __builtin_bit_cast(bf16x8, u);
}

// Q4_K: (D, M) = (d*sc, dmin*m) of sub-block s (0..7) from a super-block
// header (d, dmin as binary16 in h.x; the 12-byte six-bit scale/min field in
// h.y, h.z, h.w, unpacked as the llamini.cpp post's get_scale_min_k4 does).
__device__ __forceinline__ f32x2 q4k_dm(u32x4 h, int s)
{
    const uint32_t sh = 8u * (uint32_t)(s & 3);
    const uint32_t a = h.y >> sh, b = h.z >> sh, c = h.w >> sh;
    const bool upper = s >= 4;
    const uint32_t sc = upper ? ((c & 0xFu) | ((a >> 2) & 0x30u)) : (a & 63u);
    const uint32_t m = upper ? (((c >> 4) & 0xFu) | ((b >> 2) & 0x30u)) : (b & 63u);
    return f32x2{half_lo(h.x) * (float)sc, half_hi(h.x) * (float)m};
}

// One workgroup: W waves, each with MTR 16-row tiles of every matrix (NMAT),
// over NTW 16-token tiles and the K range [k0, k1) of super-steps of 4Q
// blocks.  Super-step S's weight runs and x pieces travel together in ring
// slot S % 2: the loads of the next super-step are in flight while this one
// is computed.
template <int FMT, int NMAT, int MTR, int NTW, int W, int Q, int XB>
__global__ __launch_bounds__(W * 64) void prefill_mfma_kernel(PrefillParams p)
{
    constexpr bool KQ = FMT == QG_Q4_K;
    constexpr bool K6 = FMT == QG_Q6_K;
    constexpr bool K8 = FMT == QG_Q8_0 || FMT == QG_I8ROW;   // 32 code bytes per block
    constexpr bool KR = FMT == QG_I8ROW;    // one fp32 scale per row, applied to the sums
    constexpr int BB = K8 ? 32 : 16;        // code bytes per block
    constexpr int MT = MTR * NMAT;          // 16-row tiles per wave
    constexpr int NT = W * 64;              // threads
    constexpr int SB = 4 * Q;               // blocks per super-step
    constexpr int SCOLS = 32 * SB;          // columns per super-step
    constexpr int RPI = 16 / Q;             // tile rows per weight load instruction (4Q lanes per row)
    // LDS: two x tiles (bf16, token rows padded by 16 B), then one weight
    // area per wave (codes [tile][row][block] and scales [tile][row][block],
    // rows padded so that the 16 rows of a read fall in different banks)
    constexpr int XROW = SCOLS * 2 + 16;
    constexpr int XTILE = NTW * 16 * XROW;
    constexpr int AROW = SB * BB + 16;
    // Q4_0, Q8_0: f16 d; Q4_K: (D, M) as two floats; Q6_K: the two halves' D;
    // I8ROW: none
    constexpr int SROW = (KQ || K6) ? SB * 8 + 8 : (KR ? 0 : SB * 2 + 4);
    constexpr int HROW = K6 ? SB * 8 + 8 : 0;           // Q6_K: 8 bytes of high bits per block
    constexpr int AWAVE = MT * 16 * (AROW + SROW + HROW);
    constexpr int XF4 = NTW * 16 * SCOLS / 4;   // float4 pieces of x per super-step
    constexpr int PT = XF4 / NT;
    static_assert(XF4 % NT == 0 && PT >= 1 && PT <= 16, "x pieces must split evenly over the threads");
    extern __shared__ float4 pf_lds[];
    uint8_t *lds = reinterpret_cast<uint8_t *>(pf_lds);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    uint8_t *aw = lds + 2 * XTILE + wave * AWAVE;           // this wave's weight area
    uint8_t *sw = aw + MT * 16 * AROW;
    uint8_t *hw = sw + MT * 16 * SROW;                      // Q6_K: high bits

    // work item (row group, K range, token group), token group fastest;
    // consecutive items share an XCD, so the token groups of one row group
    // find its weights in the same L2
    const int64_t items = p.row_groups * p.ksplit * p.tok_groups;
    int64_t item = blockIdx.x;
    if (items % 8 == 0) item = (int64_t)(blockIdx.x % 8) * (items / 8) + blockIdx.x / 8;
    const int tg = (int)(item % p.tok_groups);
    const int64_t rest = item / p.tok_groups;
    const int ks = (int)(rest % p.ksplit);
    const int64_t rg = rest / p.ksplit;
    const int64_t row_base = (rg * W + wave) * (MTR * 16);
    const int tok_base = tg * NTW * 16;
    const int k0 = ks * p.spk;
    const int k1 = k0 + p.spk < p.ssteps ? k0 + p.spk : p.ssteps;

    // weight loads: instruction i of tile m reads row i*RPI + lane/(4Q) of the
    // tile, block lane%(4Q) of the super-step (16 code bytes + its f16 scale).
    // Every loop over a register array below is a static_for: its indices must
    // be compile-time constants, or the arrays would live in scratch memory.
    const int lrow = lane / (4 * Q), lblk = lane % (4 * Q);
    // row offsets (in rows) of load instruction i: row_base + (m % MTR)*16 + i*RPI + lrow, clamped
    auto arow = [&](int m, int i) __attribute__((always_inline)) -> int64_t {
        int64_t row = row_base + (m % MTR) * 16 + i * RPI + lrow;
        return row < p.rows ? row : p.rows - 1;   // rows past the end read a valid row; never stored
    };

    f32x4 acc[MT][NTW];
    static_for<MT>([&](auto mc) __attribute__((always_inline)) {
        static_for<NTW>([&](auto nc) __attribute__((always_inline)) {
            acc[decltype(mc)::value][decltype(nc)::value] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        });
    });

    // the ring: weight runs, scales, x pieces and liveness (bit k: x piece k
    // inside x; bit 31: the lane's weight block inside the row)
    u32x4 qa[2][MT][Q];
    u32x4 qb[2][K8 ? MT : 1][K8 ? Q : 1];         // 8-bit: the second 16-byte piece
    uint32_t da[2][MT][Q];                        // Q4_0: the block's f16 scale
    u32x4 ha[2][KQ ? MT : 1][KQ ? Q : 1];         // Q4_K: the super-block header
    uint2 h6[2][K6 ? MT : 1][K6 ? Q : 1];         // Q6_K: the block's high bits
    uint32_t d6[2][K6 ? MT : 1][K6 ? Q : 1];      // Q6_K: the super-block's f16 d (da: the two int8 scales)
    int sub[2];                                   // Q4_K: the lane's sub-block (0..7)
    f32x4 xv[2][PT];
    uint32_t live[2];

    // x pieces of 16 bytes: 4 fp32 values, or (XB) 8 bf16 values from the
    // bf16 copy (half as many pieces: those of k < PT/2, the last one partly)
    constexpr bool xb16 = XB != 0;
    auto issue = [&](auto jc, int ss) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        uint32_t lv = 0;
        if constexpr (xb16) {
            static_for<PT>([&](auto kc) __attribute__((always_inline)) {
                constexpr int k = decltype(kc)::value;
                if constexpr (2 * k < PT) {
                    const int piece = threadIdx.x + k * NT;
                    const int t = piece / (SCOLS / 8), c8 = piece % (SCOLS / 8);
                    const int tok = tok_base + t;
                    const int col = ss * SCOLS + 8 * c8;
                    const bool alive = piece < XF4 / 2 && tok < p.n_tok && col < p.cols;
                    lv |= alive ? (1u << k) : 0u;
                    const int64_t off = alive ? (int64_t)tok * p.cols + col : 0;
                    xv[J][k] = __builtin_bit_cast(f32x4, *reinterpret_cast<const u32x4 *>(p.xb + off));
                }
            });
        } else {
            static_for<PT>([&](auto kc) __attribute__((always_inline)) {
                constexpr int k = decltype(kc)::value;
                const int piece = threadIdx.x + k * NT;
                const int t = piece / (SCOLS / 4), c4 = piece % (SCOLS / 4);
                const int tok = tok_base + t;
                const int col = ss * SCOLS + 4 * c4;
                const bool alive = tok < p.n_tok && col < p.cols;
                lv |= alive ? (1u << k) : 0u;
                // dead pieces (tokens past n_tok, columns past the row) all read
                // the first 16 bytes of x: one cache line per wave, stored as 0
                const int64_t off = alive ? (int64_t)tok * p.cols + col : 0;
                xv[J][k] = *reinterpret_cast<const f32x4 *>(p.x + off);
            });
        }
        int blk = ss * SB + lblk;
        lv |= blk < p.nb ? (1u << 31) : 0u;
        blk = blk < p.nb ? blk : p.nb - 1;   // past the row: a valid block, weighted 0
        static_for<MT>([&](auto mc) __attribute__((always_inline)) {
            constexpr int m = decltype(mc)::value;
            static_for<Q>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                const int64_t row = arow(m, i);
                const uint8_t *base = p.q[m / MTR];
                if constexpr (K8) {
                    // 8-bit: the row's 2SB 16-byte pieces of the super-step,
                    // pieces lblk and lblk + 4Q (each instruction reads 64Q
                    // consecutive bytes of the row); pieces past the row read
                    // the last one and meet x = 0
                    const u32x4 *rp = reinterpret_cast<const u32x4 *>(base + row * p.row_qbytes);
                    const int pa = ss * 2 * SB + lblk, pb = pa + 4 * Q;
                    qa[J][m][i] = rp[pa < 2 * p.nb ? pa : 2 * p.nb - 1];
                    qb[J][m][i] = rp[pb < 2 * p.nb ? pb : 2 * p.nb - 1];
                } else {
                    qa[J][m][i] = reinterpret_cast<const u32x4 *>(base + row * p.row_qbytes)[blk];
                }
                if constexpr (KR) {
                    // the row scale is applied to the sums
                } else if constexpr (KQ) {
                    ha[J][m][i] = reinterpret_cast<const u32x4 *>(base + p.soff)[row * (p.nb / 8) + blk / 8];
                } else {
                    da[J][m][i] = (reinterpret_cast<const uint16_t *>(base + p.soff) + row * p.nb)[blk];
                    if constexpr (K6) {
                        h6[J][m][i] = reinterpret_cast<const uint2 *>(base + p.hoff)[row * p.nb + blk];
                        d6[J][m][i] = (reinterpret_cast<const uint16_t *>(base + p.doff) + row * (p.nb / 8))[blk / 8];
                    }
                }
            });
        });
        live[J] = lv;
        sub[J] = blk & 7;
    };

    auto consume = [&](auto jc, int nxt, bool refill) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        const uint32_t lv = live[J];
        uint8_t *xt = lds + J * XTILE;
        // x of this super-step -> bf16 tile, natural column order
        if constexpr (xb16) {
            static_for<PT>([&](auto kc) __attribute__((always_inline)) {
                constexpr int k = decltype(kc)::value;
                if constexpr (2 * k < PT) {
                    const int piece = threadIdx.x + k * NT;
                    const int t = piece / (SCOLS / 8), c8 = piece % (SCOLS / 8);
                    u32x4 v = __builtin_bit_cast(u32x4, xv[J][k]);
                    if (!((lv >> k) & 1u)) v = u32x4{0u, 0u, 0u, 0u};
                    if (piece < XF4 / 2) *reinterpret_cast<u32x4 *>(xt + t * XROW + c8 * 16) = v;
                }
            });
        } else {
            static_for<PT>([&](auto kc) __attribute__((always_inline)) {
                constexpr int k = decltype(kc)::value;
                const int piece = threadIdx.x + k * NT;
                const int t = piece / (SCOLS / 4), c4 = piece % (SCOLS / 4);
                const f32x4 a = xv[J][k];
                uint2 v = make_uint2(pack_bf16(a.x, a.y), pack_bf16(a.z, a.w));
                if (!((lv >> k) & 1u)) v = make_uint2(0u, 0u);
                *reinterpret_cast<uint2 *>(xt + t * XROW + c4 * 8) = v;
            });
        }
        // this wave's weight runs -> its LDS area (a block past the row gets scale 0)
        static_for<MT>([&](auto mc) __attribute__((always_inline)) {
            constexpr int m = decltype(mc)::value;
            static_for<Q>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                const int row = i * RPI + lrow;
                *reinterpret_cast<u32x4 *>(aw + (m * 16 + row) * AROW + lblk * 16) = qa[J][m][i];
                if constexpr (K8)
                    *reinterpret_cast<u32x4 *>(aw + (m * 16 + row) * AROW + (lblk + 4 * Q) * 16) = qb[J][m][i];
                if constexpr (KR) {
                } else if constexpr (KQ) {
                    const f32x2 dm = q4k_dm(ha[J][m][i], sub[J]);
                    *reinterpret_cast<f32x2 *>(sw + (m * 16 + row) * SROW + lblk * 8) =
                        (lv >> 31) ? dm : f32x2{0.0f, 0.0f};
                } else if constexpr (K6) {
                    // the two 16-column halves' D = d * sc (exact: 11-bit by 8-bit)
                    const float d = half_lo(d6[J][m][i]);
                    const uint32_t sc = da[J][m][i];
                    const f32x2 dd{d * (float)(int8_t)(sc & 0xFFu), d * (float)(int8_t)((sc >> 8) & 0xFFu)};
                    *reinterpret_cast<f32x2 *>(sw + (m * 16 + row) * SROW + lblk * 8) =
                        (lv >> 31) ? dd : f32x2{0.0f, 0.0f};
                    *reinterpret_cast<uint2 *>(hw + (m * 16 + row) * HROW + lblk * 8) = h6[J][m][i];
                } else {
                    *reinterpret_cast<uint16_t *>(sw + (m * 16 + row) * SROW + lblk * 2) =
                        (lv >> 31) ? (uint16_t)da[J][m][i] : (uint16_t)0;
                }
            });
        });
        __syncthreads();
        // K step q multiplies blocks 4q .. 4q+3 of the super-step, block 4q+g in
        // lane group g; operand c covers its columns 8c .. 8c+7
        static_for<Q>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            const int b = 4 * q + g;
            bf16x8 af[MT][4];
            static_for<MT>([&](auto mc) __attribute__((always_inline)) {
                constexpr int m = decltype(mc)::value;
                if constexpr (K8) {
                    // q + 128 (the byte xor 0x80) as a binary16 subnormal is
                    // (q + 128)*2^-24; fma with D*2^24 and -128D gives q*D,
                    // exact in fp32 for Q8_0 (an 8-bit code by an 11-bit d)
                    // and for I8ROW (D = 1: the code itself)
                    const uint8_t *ap = aw + (m * 16 + r16) * AROW + b * 32;
                    const u32x4 w0 = *reinterpret_cast<const u32x4 *>(ap);
                    const u32x4 w1 = *reinterpret_cast<const u32x4 *>(ap + 16);
                    float d = 1.0f;
                    if constexpr (!KR) d = half_lo(*reinterpret_cast<const uint16_t *>(sw + (m * 16 + r16) * SROW + b * 2));
                    const float d24 = d * 0x1p24f, nd = -128.0f * d;
                    constexpr uint32_t F = 0x80808080u, M8 = 0x00FF00FFu;
                    af[m][0] = decode8(w0.x ^ F, w0.y ^ F, M8, d24, nd);
                    af[m][1] = decode8(w0.z ^ F, w0.w ^ F, M8, d24, nd);
                    af[m][2] = decode8(w1.x ^ F, w1.y ^ F, M8, d24, nd);
                    af[m][3] = decode8(w1.z ^ F, w1.w ^ F, M8, d24, nd);
                    return;
                }
                const u32x4 w = *reinterpret_cast<const u32x4 *>(aw + (m * 16 + r16) * AROW + b * 16);
                if constexpr (K6) {
                    // code words 0, 1 take high-bit word 0 (shifted 0, 2), words 2, 3 word 1
                    const uint2 hv = *reinterpret_cast<const uint2 *>(hw + (m * 16 + r16) * HROW + b * 8);
                    const f32x2 dd = *reinterpret_cast<const f32x2 *>(sw + (m * 16 + r16) * SROW + b * 8);
                    const float a24 = dd.x * 0x1p24f, na = -32.0f * dd.x;
                    const float b20 = dd.y * 0x1p20f, nb = -32.0f * dd.y;
                    af[m][0] = decode8_q6(w.x, w.y, hv.x, hv.x >> 2, false, a24, na);
                    af[m][1] = decode8_q6(w.z, w.w, hv.y, hv.y >> 2, false, a24, na);
                    af[m][2] = decode8_q6(w.x, w.y, hv.x, hv.x >> 2, true, b20, nb);
                    af[m][3] = decode8_q6(w.z, w.w, hv.y, hv.y >> 2, true, b20, nb);
                    return;
                }
                float d, n8;
                if constexpr (KQ) {
                    const f32x2 dm = *reinterpret_cast<const f32x2 *>(sw + (m * 16 + r16) * SROW + b * 8);
                    d = dm.x;
                    n8 = -dm.y;
                } else {
                    d = half_lo(*reinterpret_cast<const uint16_t *>(sw + (m * 16 + r16) * SROW + b * 2));
                    n8 = -8.0f * d;
                }
                const float d24 = d * 0x1p24f, d20 = d * 0x1p20f;
                af[m][0] = decode8(w.x, w.y, 0x000F000Fu, d24, n8);
                af[m][1] = decode8(w.z, w.w, 0x000F000Fu, d24, n8);
                af[m][2] = decode8(w.x, w.y, 0x00F000F0u, d20, n8);
                af[m][3] = decode8(w.z, w.w, 0x00F000F0u, d20, n8);
            });
            static_for<NTW>([&](auto nc) __attribute__((always_inline)) {
                constexpr int n = decltype(nc)::value;
                const uint8_t *rowp = xt + (n * 16 + r16) * XROW + b * 64;
                bf16x8 bf[4];
                static_for<4>([&](auto cc) __attribute__((always_inline)) {
                    bf[decltype(cc)::value] = *reinterpret_cast<const bf16x8 *>(rowp + decltype(cc)::value * 16);
                });
                static_for<4>([&](auto cc) __attribute__((always_inline)) {
                    constexpr int c = decltype(cc)::value;
                    static_for<MT>([&](auto mc) __attribute__((always_inline)) {
                        constexpr int m = decltype(mc)::value;
                        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m][c], bf[c], acc[m][n], 0, 0, 0);
                    });
                });
            });
        });
        // refill after the products: issued earlier, the register allocator
        // parks the new loads in other registers and copies them back at the
        // loop latch, which makes the loop wait for the whole ring
        __builtin_amdgcn_sched_barrier(0);
        if (refill) issue(jc, nxt);
        __builtin_amdgcn_sched_barrier(0);
    };

    // prologue: super-steps k0, k0+1 (past k1: the last one again, never consumed)
    issue(std::integral_constant<int, 0>{}, k0);
    issue(std::integral_constant<int, 1>{}, k0 + 1 < k1 ? k0 + 1 : k1 - 1);
    int k = k0;
    for (; k + 2 <= k1; k += 2) {
        consume(std::integral_constant<int, 0>{}, k + 2 < k1 ? k + 2 : k1 - 1, true);
        consume(std::integral_constant<int, 1>{}, k + 3 < k1 ? k + 3 : k1 - 1, true);
    }
    if (k < k1) consume(std::integral_constant<int, 0>{}, 0, false);   // uniform branch

    // epilogue: the lane holds rows 4*(lane/16)+i of each tile for token lane%16
    const bool partial = p.ksplit > 1;
    auto store4 = [&](float *dst, int64_t row, float v0, float v1, float v2, float v3) __attribute__((always_inline)) {
        if ((p.rows & 3) == 0 && row + 3 < p.rows) {
            *reinterpret_cast<float4 *>(dst) = make_float4(v0, v1, v2, v3);
        } else {
            if (row < p.rows) dst[0] = v0;
            if (row + 1 < p.rows) dst[1] = v1;
            if (row + 2 < p.rows) dst[2] = v2;
            if (row + 3 < p.rows) dst[3] = v3;
        }
    };
    // I8ROW: the sums of matrix mo's rows row .. row+3 times their row scales
    auto rscale = [&](int mo, int64_t row, f32x4 a) __attribute__((always_inline)) -> f32x4 {
        if constexpr (KR) {
            const float *sp = reinterpret_cast<const float *>(p.q[mo] + p.soff);
#pragma unroll
            for (int i = 0; i < 4; i++) a[i] *= sp[row + i < p.rows ? row + i : p.rows - 1];
        }
        return a;
    };
    static_for<NTW>([&](auto nc) __attribute__((always_inline)) {
        constexpr int n = decltype(nc)::value;
        const int tok = tok_base + n * 16 + r16;
        if (tok < p.n_tok) {
            static_for<MTR>([&](auto rc) __attribute__((always_inline)) {
                constexpr int mr = decltype(rc)::value;
                const int64_t row = row_base + mr * 16 + 4 * g;
                if (partial) {
                    // raw sums of this K range: [ks][matrix][token][row]
                    static_for<NMAT>([&](auto oc) __attribute__((always_inline)) {
                        constexpr int mo = decltype(oc)::value;
                        const f32x4 a = rscale(mo, row, acc[mo * MTR + mr][n]);
                        store4(p.y + (((int64_t)(ks * NMAT + mo) * p.n_tok + tok) * p.rows + row), row, a[0], a[1],
                               a[2], a[3]);
                    });
                } else if (NMAT == 1) {
                    f32x4 a = rscale(0, row, acc[mr][n]);
                    if (p.resid) {   // the residual stream: read before this thread overwrites it
                        const float *rp = p.resid + (int64_t)tok * p.rows + row;
#pragma unroll
                        for (int i = 0; i < 4; i++) a[i] += row + i < p.rows ? rp[i] : 0.0f;
                    }
                    store4(p.y + (int64_t)tok * p.rows + row, row, a[0], a[1], a[2], a[3]);
                } else {
                    const f32x4 gg = rscale(0, row, acc[mr][n]), uu = rscale(NMAT - 1, row, acc[(NMAT - 1) * MTR + mr][n]);
                    float v[4];
                    for (int i = 0; i < 4; i++) v[i] = gg[i] / (1.0f + expf(-gg[i])) * uu[i];
                    store4(p.y + (int64_t)tok * p.rows + row, row, v[0], v[1], v[2], v[3]);
                    if (p.yb) {   // the bf16 copy of h for the next product, the kernel's own rounding
                        uint16_t *yb = p.yb + (int64_t)tok * p.rows + row;
                        if ((p.rows & 3) == 0 && row + 3 < p.rows) {
                            *reinterpret_cast<uint2 *>(yb) = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
                        } else {
                            for (int i = 0; i < 4; i++)
                                if (row + i < p.rows) yb[i] = (uint16_t)(pack_bf16(v[i], 0.0f) & 0xFFFFu);
                        }
                    }
                }
            });
        }
    });
}

// LDS of a workgroup: two bf16 x tiles plus one weight area per wave (codes,
// 16 bytes per block or 32 for the 8-bit formats, and per-block scales: f16
// d for Q4_0 and Q8_0, the (D, M) pair for Q4_K, the two halves' D for Q6_K,
// which also stages 8 bytes of high bits per block; none for I8ROW)
constexpr size_t pf_lds_bytes(int fmt, int nmat, int mtr, int ntw, int waves, int run)
{
    const size_t bb = (fmt == QG_Q8_0 || fmt == QG_I8ROW) ? 32 : 16;
    const size_t srow = (fmt == QG_Q4_K || fmt == QG_Q6_K) ? (size_t)run * 32 + 8
                        : fmt == QG_I8ROW                  ? 0
                                                           : (size_t)run * 8 + 4;
    const size_t hrow = fmt == QG_Q6_K ? (size_t)run * 32 + 8 : 0;
    return 2 * (size_t)ntw * 16 * (run * 256 + 16) +
           (size_t)waves * nmat * mtr * 16 * ((run * 4 * bb + 16) + srow + hrow);
}

template <int FMT, int NMAT, int MTR, int NTW, int W, int Q, int XB>
hipError_t go_prefill(PrefillParams p, float *y, hipStream_t s)
{
    const size_t lds = pf_lds_bytes(FMT, NMAT, MTR, NTW, W, Q);
    const int64_t grid = p.row_groups * p.tok_groups * p.ksplit;
    if (grid >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    auto kern = prefill_mfma_kernel<FMT, NMAT, MTR, NTW, W, Q, XB>;
    if (lds > 65536) {
        // the attribute is per device and per instantiation: set it once
        static std::atomic<bool> configured[64];
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
        if (!configured[dev].load(std::memory_order_relaxed)) {
            hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            configured[dev].store(true, std::memory_order_relaxed);
        }
    }
    // measurement hook: the start event rides on this launch, the stop event
    // on the last launch of the product (this one, or the reduce)
    hipEvent_t t0 = nullptr, t1 = nullptr;
    const bool timed = take_launch_timing(&t0, &t1);
    hipError_t e;
    if (timed) {
        void *args[] = {&p};
        e = hipExtLaunchKernel((const void *)kern, dim3((unsigned)grid), dim3(64 * W), args, lds, s, t0,
                               p.ksplit == 1 ? t1 : nullptr, 0);
    } else {
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * W), lds, s, p);
        e = hipGetLastError();
    }
    if (e != hipSuccess || p.ksplit == 1) return e;
    return launch_prefill_reduce(NMAT, p.y, y, (int64_t)p.n_tok * p.rows, p.ksplit, p.resid, s, timed ? t1 : nullptr,
                                 p.yb);
}

// Tile shapes that are built, per format: those whose ring, operands and
// accumulators fit the register file without spilling (checked in the
// compiled code), whose x pieces split evenly over the threads and whose LDS
// fits a CU.  Code: nmat*10000 + mtr*1000 + ntw*100 + waves*10 + run.
constexpr int kBuiltShapes[] = {
    11141, 11142, 11144, 11181, 11182, 11184, 11241, 11242, 11244,
    11281, 11282, 11284, 11441, 11442, 11481, 11482, 11841, 11881,
    12141, 12142, 12144, 12181, 12182, 12184, 12241, 12242, 12244,
    12281, 12282, 12441, 12442, 12481, 12482, 12841, 12881, 21141,
    21142, 21144, 21181, 21182, 21184, 21241, 21242, 21244, 21281,
    21282, 21441, 21442, 21481, 21482, 21841, 21881, 22141, 22142,
    22182, 22241, 22242, 22281, 22441, 22481, 22841,
    11561, 11961,   // 16 waves (waves * 10 = 160), one matrix only: two spill
};

constexpr int kBuiltShapesK[] = {
    11141, 11142, 11144, 11181, 11182, 11184, 11241, 11242, 11244,
    11281, 11282, 11284, 11441, 11442, 11481, 11482, 11561, 11841,
    11881, 11961, 12141, 12142, 12144, 12181, 12182, 12241, 12242,
    12281, 12282, 12441, 12442, 12481, 12482, 12841, 12881, 21141,
    21142, 21144, 21181, 21182, 21241, 21242, 21281, 21282, 21441,
    21442, 21481, 21482, 21841, 21881, 22141, 22142, 22181, 22241,
    22242, 22281, 22441, 22442, 22841,
};

constexpr int kBuiltShapes6[] = {
    11141, 11142, 11144, 11181, 11182, 11184, 11241, 11242, 11244,
    11281, 11282, 11284, 11441, 11442, 11481, 11482, 11561, 11841,
    11881, 11961, 12141, 12142, 12144, 12181, 12182, 12241, 12242,
    12281, 12282, 12441, 12442, 12481, 12841, 12881, 21141,
    21142, 21144, 21181, 21182, 21241, 21242, 21281, 21282,
    21441, 21442, 21481, 21841, 21881, 22141, 22142, 22181, 22241,
    22242, 22281, 22441, 22841,
};

constexpr int kBuiltShapes8[] = {
    11141, 11142, 11144, 11181, 11182, 11184, 11241, 11242, 11244,
    11281, 11282, 11284, 11441, 11442, 11481, 11482, 11561, 11841,
    11881, 11961, 12141, 12142, 12144, 12181, 12182, 12241, 12242,
    12244, 12281, 12282, 12441, 12442, 12481, 12841, 12881, 21141,
    21142, 21144, 21181, 21182, 21241, 21242, 21244, 21281, 21282,
    21441, 21442, 21481, 21841, 21881, 22141, 22142, 22181, 22241,
    22242, 22281, 22441, 22841,
};

constexpr int kBuiltShapesR[] = {
    11141, 11142, 11144, 11181, 11182, 11184, 11241, 11242, 11244,
    11281, 11282, 11284, 11441, 11442, 11481, 11482, 11561, 11841,
    11881, 11961, 12141, 12142, 12144, 12181, 12182, 12241, 12242,
    12244, 12281, 12282, 12441, 12442, 12481, 12482, 12561, 12841,
    12881, 21141, 21142, 21144, 21181, 21182, 21241, 21242, 21244,
    21281, 21282, 21441, 21442, 21481, 21482, 21841, 21881, 22141,
    22142, 22181, 22182, 22241, 22242, 22281, 22441, 22442, 22481,
    22841,
};

constexpr bool pf_fits(int fmt, int nmat, int mtr, int ntw, int waves, int run)
{
    const int code = nmat * 10000 + mtr * 1000 + ntw * 100 + waves * 10 + run;
    const bool geometry = pf_lds_bytes(fmt, nmat, mtr, ntw, waves, run) <= 160 * 1024 &&
                          ntw * 512 * run >= waves * 64 && ntw * 512 * run <= 16 * waves * 64;
    if (fmt == QG_Q8_0) {
        for (int c : kBuiltShapes8)
            if (c == code) return geometry;
        return false;
    }
    if (fmt == QG_I8ROW) {
        for (int c : kBuiltShapesR)
            if (c == code) return geometry;
        return false;
    }
    if (fmt == QG_Q6_K) {
        for (int c : kBuiltShapes6)
            if (c == code) return geometry;
        return false;
    }
    if (fmt == QG_Q4_K) {
        for (int c : kBuiltShapesK)
            if (c == code) return geometry;
        return false;
    }
    for (int c : kBuiltShapes)
        if (c == code) return geometry;
    return false;
}

// Every built shape has both x variants: fp32 x, or its bf16 copy when given.
template <int FMT, int NM, int MR, int NT, int WV, int RN>
hipError_t go_prefill_x(const PrefillParams &p, float *y, hipStream_t s)
{
    if (p.xb) return go_prefill<FMT, NM, MR, NT, WV, RN, 1>(p, y, s);
    return go_prefill<FMT, NM, MR, NT, WV, RN, 0>(p, y, s);
}

// The built shapes of one format, dispatched on the chosen tile.
template <int FMT>
hipError_t prefill_dispatch(const PrefillCfg &c, int nmat, const PrefillParams &p, float *y, hipStream_t s)
{
#define QG_PF(NM, MR, NT, WV, RN)                                                                  \
    if constexpr (pf_fits(FMT, NM, MR, NT, WV, RN))                                                \
        if (nmat == NM && c.mtr == MR && c.ntw == NT && c.waves == WV && c.run == RN)              \
            return go_prefill_x<FMT, NM, MR, NT, WV, RN>(p, y, s);
#define QG_PF_R(NM, MR, NT, WV) QG_PF(NM, MR, NT, WV, 1) QG_PF(NM, MR, NT, WV, 2) QG_PF(NM, MR, NT, WV, 4)
#define QG_PF_W(NM, MR) QG_PF_R(NM, MR, 1, 4) QG_PF_R(NM, MR, 2, 4) QG_PF_R(NM, MR, 4, 4) QG_PF_R(NM, MR, 8, 4) \
    QG_PF(NM, MR, 4, 16, 1) QG_PF(NM, MR, 8, 16, 1) \
    QG_PF_R(NM, MR, 1, 8) QG_PF_R(NM, MR, 2, 8) QG_PF_R(NM, MR, 4, 8) QG_PF_R(NM, MR, 8, 8)
    QG_PF_W(1, 1) QG_PF_W(1, 2) QG_PF_W(2, 1) QG_PF_W(2, 2)
#undef QG_PF_W
#undef QG_PF_R
#undef QG_PF
    return hipErrorInvalidValue;
}

} // namespace

} // namespace qg
