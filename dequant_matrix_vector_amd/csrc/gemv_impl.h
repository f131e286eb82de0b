// Fused dequant-dot GEMV kernels for gfx950 (wave64, fp32 accumulation).
//
// y = W x with W block-quantized, one token: the decode-time product that sets
// decode speed because every weight is streamed once for one multiply-add
// (llmoxide blog, section 11 "Prefill and decode"); each dot product decodes
// its row's blocks on the fly and never materializes floats (llmoxide blog,
// section 10 "Loading weights").
//
// Work decomposition
//   * A 32-weight "chunk" (a Q4_0 or Q8_0 block, a Q4_K sub-block, 32 int8 of
//     an I8ROW row) is the unit of decode; a lane takes CPL adjacent chunks
//     (a "group") per pass, so the group's CPL scales arrive in one 2-, 4- or
//     8-byte load.
//   * LPR lanes share a row: lane `sl` takes group sl, sl+LPR, ...;
//     consecutive lanes read consecutive pieces of the quant plane.
//   * Each lane group owns R rows (times NMAT matrices for the fused gate/up),
//     so one staged x chunk read from LDS feeds R*NMAT chunks of weights.
//   * The workgroup stages x once into LDS (36 floats per chunk: the 32
//     values, the chunk sum, padding that spreads consecutive chunks over all
//     LDS banks), then each wave streams its rows; partial sums are combined
//     across the LPR lanes by a fixed xor-shuffle tree (deterministic: no
//     atomics).
//
// 4-bit decode (Q4_0, Q4_K): a 32-bit word of packed nibbles is masked with
// 0x000F000F / 0x00F000F0 (and again after a byte shift) so that each 16-bit
// half holds one code in its low mantissa bits: as a binary16 subnormal its
// value is q*2^-24 (or q*2^-20 for the nibble one position up).  x was staged
// pre-multiplied by 2^24 (first 16 elements of a chunk) or 2^20 (last 16), so
// v_fma_mix_f32 (binary16 operand converted exactly inside the fma) adds
// exactly q*x before its single rounding.  Five integer ops decode eight codes.
// The Q4_0 offset of 8 and the Q4_K minimum are folded in per chunk through the
// staged chunk sum, accumulated in the same order as the codes so that all-8
// codes cancel exactly.
//
// 6-bit decode (Q6_K): the low four bits of each code sit in a word laid out
// like Q4_0's, the top two bits in a second plane, placed so that one AND
// moves them next to the nibble they extend (bits 4-5 / 20-21 for the first
// mask, 8-9 / 24-25 for the second), giving q*2^-24 or q*2^-20 as before.
// A 32-weight chunk spans two 16-weight sub-blocks with their own int8
// scales: the first mask's codes (columns 0-15 of the chunk) and the second
// mask's (16-31) go to two sums, and the offset of 32 is folded in through
// two staged half-chunk sums.
//
// 8-bit decode (Q8_0, I8ROW): each signed byte converts with one SDWA
// v_cvt_f32_i32 (sign-extending byte select) and feeds one fma.
//
// Q8_0 activations (format code + kQ8Act, Q4_0 and Q8_0 weights): the
// workgroup quantizes each staged chunk of x to Q8_0 (q8act.h) and stores its
// 32 codes, its binary16 scale and its code sum; a chunk's dot product is then
// exact integer arithmetic (v_dot4_i32_i8 on the codes; Q4_0 nibbles are
// 0..15 bytes, the offset of 8 folded in through the code sum), scaled once
// by d_w * d_x (exact in binary32) into the fp32 accumulator.
//
// Epilogue variants (EPI): 0 plain; 1 (gate/up) the input is RMS-normalized
// with a per-element gain (llmoxide blog, section 4 "Keeping the numbers in
// range"): the workgroup stages x*gamma and sums x^2 while staging, and the
// per-token scale 1/sqrt(mean(x^2) + eps) multiplies the finished dot products
// (it factors out of every row's sum); 2 (down) adds the residual stream
// (section 7 "The block, and the residual stream").
#pragma once
#include <atomic>
#include <type_traits>

#include <hip/hip_ext.h>

#include "q8act.h"
#include "qg_internal.h"

namespace qg {

namespace gemv_detail {

struct GemvParams {
    const uint8_t *q[2];  // packed tensors (quant plane at offset 0)
    const float *x;       // [cols]
    float *y;             // [rows]
    int64_t rows;
    int64_t row_qbytes;
    int64_t soff;         // scale plane offset inside each packed tensor
    int nchunk;           // cols / 32
    const float *gamma;   // EPI 1: RMSNorm gain [cols]
    float eps;            // EPI 1: RMSNorm epsilon
    const float *resid;   // EPI 2: residual [rows], added to y (may be y itself)
    int64_t hoff;         // Q6_K: offsets of the high-bit plane and the f16 d plane
    int64_t doff;
    uint2 *am_cand;       // EPI 3: one (value bits, index) candidate per workgroup
    int64_t am_max;       // EPI 3: room for candidates (workgroups) in am_cand
    uint32_t *am_count;   // EPI 3: where workgroup 0 stores the number of candidates
    int64_t *am_grid;     // EPI 3, host memory: the launcher records its grid there (not read by the kernel)
};

enum { kEpiPlain = 0, kEpiNorm = 1, kEpiResid = 2, kEpiArgmax = 3 };

// Greedy sampling fused into the product (EPI 3; the Go "llm" package's
// Argmax, which runs on the GPU so that only the token leaves it): the first
// index of the largest y.  An in-order scan's result has a closed form that
// any order of comparisons reaches -- if y[0] is NaN the answer is 0 (nothing
// compares greater); otherwise NaN never wins and the answer is the smallest
// index whose value equals the maximum (-0 equal to +0) -- so each thread
// keeps (value, index) under "greater value, or equal value and smaller
// index" over the rows it writes, and candidates combine by the same rule.
__device__ __forceinline__ void am_take(float &bv, int &bi, float v, int i)
{
    if (v > bv || (v == bv && i < bi)) {   // NaN v: both false, never taken
        bv = v;
        bi = i;
    }
}

// The workgroup's candidate: the (value, index) of the rows it wrote, kept
// under the rule above through a fixed xor tree and the waves in order, is
// stored at cand[blockIdx.x] (index 0xFFFFFFFF: this workgroup wrote row 0
// and it is NaN); workgroup 0 also stores the number of candidates at
// *count.  A second, one-workgroup launch (am_combine) reduces them to the
// token: the boundary between the launches orders every candidate store
// before its loads, so no counter, fence or wait is needed here.  Every
// thread of the workgroup calls this once, after its last row; nan0: this
// thread wrote row 0 and it is NaN.
__device__ __forceinline__ void am_finish(float bv, int bi, bool nan0, uint2 *cand, uint32_t *count)
{
    __shared__ float am_v[16];
    __shared__ int am_i[16];
    __shared__ int am_n[16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        nan0 = __shfl_xor((int)nan0, off, 64) != 0 || nan0;
        am_take(bv, bi, ov, oi);
    }
    if (lane == 0) {
        am_v[wave] = bv;
        am_i[wave] = bi;
        am_n[wave] = nan0;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float v = am_v[0];
        int i = am_i[0];
        bool n = am_n[0] != 0;
        for (int w = 1; w < nw; w++) {
            am_take(v, i, am_v[w], am_i[w]);
            n = n || am_n[w] != 0;
        }
        cand[blockIdx.x] = make_uint2(__builtin_bit_cast(uint32_t, v), n ? 0xFFFFFFFFu : (uint32_t)i);
        if (blockIdx.x == 0) *count = gridDim.x;
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

// sum_l q_l * x_l over one chunk of 4-bit codes, x pre-scaled as described
// above.  Element order of the sum: for word k, 4k, 4k+2, 4k+16, 4k+18, 4k+1,
// 4k+3, 4k+17, 4k+19 -- the staging of the chunk sum uses the same order.
__device__ __forceinline__ float dot_q4_chunk(uint4 q, const float4 (&xv)[8])
{
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float t = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t t0 = w[k] & 0x000F000Fu;
        const uint32_t t1 = w[k] & 0x00F000F0u;
        const uint32_t s = w[k] >> 8;
        const uint32_t t2 = s & 0x000F000Fu;
        const uint32_t t3 = s & 0x00F000F0u;
        const float4 xl = xv[k], xh = xv[4 + k];
        t = __builtin_fmaf(half_lo(t0), xl.x, t);
        t = __builtin_fmaf(half_hi(t0), xl.z, t);
        t = __builtin_fmaf(half_lo(t1), xh.x, t);
        t = __builtin_fmaf(half_hi(t1), xh.z, t);
        t = __builtin_fmaf(half_lo(t2), xl.y, t);
        t = __builtin_fmaf(half_hi(t2), xl.w, t);
        t = __builtin_fmaf(half_lo(t3), xh.y, t);
        t = __builtin_fmaf(half_hi(t3), xh.w, t);
    }
    return t;
}

__device__ __forceinline__ float dot_i8_word(uint32_t w, float4 xv, float t)
{
    t = __builtin_fmaf((float)(int8_t)(w), xv.x, t);
    t = __builtin_fmaf((float)(int8_t)(w >> 8), xv.y, t);
    t = __builtin_fmaf((float)(int8_t)(w >> 16), xv.z, t);
    t = __builtin_fmaf((float)(int8_t)(w >> 24), xv.w, t);
    return t;
}

// t + sum_l q_l * x_l over 32 int8 codes in column order.
__device__ __forceinline__ float dot_i8_chunk(uint4 a, uint4 b, const float4 (&xv)[8], float t)
{
    t = dot_i8_word(a.x, xv[0], t);
    t = dot_i8_word(a.y, xv[1], t);
    t = dot_i8_word(a.z, xv[2], t);
    t = dot_i8_word(a.w, xv[3], t);
    t = dot_i8_word(b.x, xv[4], t);
    t = dot_i8_word(b.y, xv[5], t);
    t = dot_i8_word(b.z, xv[6], t);
    t = dot_i8_word(b.w, xv[7], t);
    return t;
}

// kSums: staged sums of x per chunk (0: none, x not prescaled; 1: the chunk
// sum; 2: the sums of its two 16-element halves).  kWords: 16-byte quant words
// per chunk.
template <int FMT> struct Fmt;
template <> struct Fmt<QG_Q4_0> { static constexpr int kSums = 1; static constexpr int kWords = 1; };
template <> struct Fmt<QG_Q4_K> { static constexpr int kSums = 1; static constexpr int kWords = 1; };
template <> struct Fmt<QG_Q6_K> { static constexpr int kSums = 2; static constexpr int kWords = 1; };
template <> struct Fmt<QG_Q8_0> { static constexpr int kSums = 0; static constexpr int kWords = 2; };
template <> struct Fmt<QG_I8ROW> { static constexpr int kSums = 0; static constexpr int kWords = 2; };
// kSums = -1: x staged as Q8_0 codes (8 words), the binary16 scale and the code sum
template <> struct Fmt<QG_Q4_0 | kQ8Act> { static constexpr int kSums = -1; static constexpr int kWords = 1; };
template <> struct Fmt<QG_Q8_0 | kQ8Act> { static constexpr int kSums = -1; static constexpr int kWords = 2; };

// ------------------------------------------------------------ x staging --
// Per chunk: 32 values (scaled by 2^24 / 2^20 for the 4- and 6-bit formats)
// and, for those, the chunk sum (Q6_K: the two half sums) in the decode order.  A thread issues the loads of
// its first two chunks before anything else (so they are not queued behind
// the weight stream) and finishes them after the first weight loads are out.
template <bool NORM> struct XStage {
    float4 v[2][8];
};
template <> struct XStage<true> {
    float4 v[2][8];
    float4 gm[2][8];   // the gain of the same chunks
};

template <bool NORM>
__device__ __forceinline__ void stage_issue(const float *__restrict__ x, const float *__restrict__ gamma, int nchunk,
                                            XStage<NORM> &st)
{
#pragma unroll
    for (int u = 0; u < 2; u++) {
        int c = (int)threadIdx.x + u * (int)blockDim.x;
        c = c < nchunk ? c : nchunk - 1;   // valid address; the duplicate is not stored
        const float4 *src = reinterpret_cast<const float4 *>(x + (int64_t)c * kChunk);
#pragma unroll
        for (int k = 0; k < 8; k++) st.v[u][k] = src[k];
        if constexpr (NORM) {
            const float4 *gs = reinterpret_cast<const float4 *>(gamma + (int64_t)c * kChunk);
#pragma unroll
            for (int k = 0; k < 8; k++) st.gm[u][k] = gs[k];
        }
    }
}

// sum of the squares of one chunk (raw x), in column order
__device__ __forceinline__ float chunk_sumsq(const float4 (&v)[8])
{
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; k++) {
        s = __builtin_fmaf(v[k].x, v[k].x, s);
        s = __builtin_fmaf(v[k].y, v[k].y, s);
        s = __builtin_fmaf(v[k].z, v[k].z, s);
        s = __builtin_fmaf(v[k].w, v[k].w, s);
    }
    return s;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int SUMS>
__device__ __forceinline__ void stage_store(float4 (&v)[8], float *xs, int c)
{
    if constexpr (SUMS < 0) {
        Q8Chunk qc;
        quantize_chunk_q8_0(v, qc);
        u32x4 *dq = reinterpret_cast<u32x4 *>(xs + c * kXStride);
        dq[0] = u32x4{qc.q[0], qc.q[1], qc.q[2], qc.q[3]};
        dq[1] = u32x4{qc.q[4], qc.q[5], qc.q[6], qc.q[7]};
        *reinterpret_cast<f32x2 *>(xs + c * kXStride + 8) = f32x2{qc.d, (float)qc.qsum};
        return;
    }
    // stores through a native vector type: a whole-struct float4 copy becomes a
    // memcpy, which keeps the staging registers out of registers (in scratch)
    f32x4 *dst = reinterpret_cast<f32x4 *>(xs + c * kXStride);
    if constexpr (SUMS == 1) {
        // in the order the codes are summed (see dot_q4_chunk)
        float sum = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            sum = sum + v[k].x;
            sum = sum + v[k].z;
            sum = sum + v[4 + k].x;
            sum = sum + v[4 + k].z;
            sum = sum + v[k].y;
            sum = sum + v[k].w;
            sum = sum + v[4 + k].y;
            sum = sum + v[4 + k].w;
        }
        xs[c * kXStride + 32] = sum;
    } else if constexpr (SUMS == 2) {
        // each half in the order its codes are summed (columns 4k, 4k+2, 4k+1, 4k+3)
        float a = 0.0f, b = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            a = a + v[k].x;
            a = a + v[k].z;
            b = b + v[4 + k].x;
            b = b + v[4 + k].z;
            a = a + v[k].y;
            a = a + v[k].w;
            b = b + v[4 + k].y;
            b = b + v[4 + k].w;
        }
        *reinterpret_cast<f32x2 *>(xs + c * kXStride + 32) = f32x2{a, b};
    }
    if constexpr (SUMS > 0) {
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const float sc = k < 4 ? 0x1p24f : 0x1p20f;
            v[k].x *= sc;
            v[k].y *= sc;
            v[k].z *= sc;
            v[k].w *= sc;
        }
    }
#pragma unroll
    for (int k = 0; k < 8; k++) dst[k] = f32x4{v[k].x, v[k].y, v[k].z, v[k].w};
}

// x (times the gain, NORM) -> chunk c of the staging area; NORM adds the raw
// chunk's sum of squares to ss when `count` (false for the clamped duplicate)
template <int SUMS, bool NORM>
__device__ __forceinline__ void stage_chunk(float4 (&v)[8], const float4 *gm, float *xs, int c, bool count, float &ss)
{
    if constexpr (NORM) {
        const float q = chunk_sumsq(v);
        ss += count ? q : 0.0f;
#pragma unroll
        for (int k = 0; k < 8; k++) {
            v[k].x *= gm[k].x;
            v[k].y *= gm[k].y;
            v[k].z *= gm[k].z;
            v[k].w *= gm[k].w;
        }
    }
    stage_store<SUMS>(v, xs, c);
}

template <int SUMS, bool NORM>
__device__ __forceinline__ void stage_finish(float *xs, int nchunk, XStage<NORM> &st, float &ss)
{
    // Branch-free for the first two chunks of each thread (an out-of-range
    // thread writes to the spare slot after the last chunk): a divergent
    // branch here would make the compiler wait for every load in flight,
    // including the weight stream issued after x's loads.
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const int c = (int)threadIdx.x + u * (int)blockDim.x;
        const float4 *gm = nullptr;
        if constexpr (NORM) gm = st.gm[u];
        stage_chunk<SUMS, NORM>(st.v[u], gm, xs, c < nchunk ? c : nchunk, c < nchunk, ss);
    }
}

// Chunks from the thread's first + `from` blocks of the workgroup on, staged
// synchronously before any weight load is issued.
template <int SUMS, bool NORM>
__device__ __forceinline__ void stage_rest_from(const float *__restrict__ x, const float *__restrict__ gamma,
                                                float *xs, int nchunk, float &ss, int from)
{
    for (int c = (int)threadIdx.x + from * (int)blockDim.x; c < nchunk; c += blockDim.x) {
        const float4 *src = reinterpret_cast<const float4 *>(x + (int64_t)c * kChunk);
        float4 v[8];
#pragma unroll
        for (int k = 0; k < 8; k++) v[k] = src[k];
        stage_chunk<SUMS, NORM>(v, reinterpret_cast<const float4 *>(gamma + (int64_t)c * kChunk), xs, c, true, ss);
    }
}

// Chunks beyond the first two per thread (only when nchunk > 2 * threads).
template <int SUMS, bool NORM>
__device__ __forceinline__ void stage_rest(const float *__restrict__ x, const float *__restrict__ gamma, float *xs,
                                           int nchunk, float &ss)
{
    stage_rest_from<SUMS, NORM>(x, gamma, xs, nchunk, ss, 2);
}

// ------------------------------------------------------- weight groups --
// Registers of CPL adjacent chunks of one row.  f16 scales of two chunks
// share a 32-bit word (low half = even chunk).
template <int FMT, int CPL> struct Group;
template <int CPL> struct Group<QG_Q4_0, CPL> { uint4 q[CPL]; uint32_t d[(CPL + 1) / 2]; };
template <int CPL> struct Group<QG_Q8_0, CPL> { uint4 q[2 * CPL]; uint32_t d[(CPL + 1) / 2]; };
template <int CPL> struct Group<QG_Q4_K, CPL> { uint4 q[CPL]; uint4 h; };
// Q6_K: low nibbles, 8 bytes of high bits and two int8 scales per chunk, and
// the super-block's f16 d (a group never crosses a super-block: CPL | 8)
template <int CPL> struct Group<QG_Q6_K, CPL> {
    uint4 q[CPL];
    uint32_t h[2 * CPL];
    uint32_t sc[(2 * CPL + 3) / 4];
    uint32_t d;
};
template <int CPL> struct Group<QG_I8ROW, CPL> { uint4 q[2 * CPL]; };

// Load the group starting at chunk c0 (c0 a multiple of CPL).  hrow and drow
// (the Q6_K high-bit and d planes) are unused by the other formats.
template <int FMT, int CPL>
__device__ __forceinline__ void load_group(Group<FMT, CPL> &o, const uint8_t *qrow, const uint8_t *srow,
                                           const uint8_t *hrow, const uint8_t *drow, int c0, int nchunk)
{
    constexpr int W = Fmt<FMT>::kWords;
    const uint4 *qp = reinterpret_cast<const uint4 *>(qrow + (int64_t)c0 * 16 * W);
    (void)nchunk;
#pragma unroll
    for (int j = 0; j < CPL * W; j++) o.q[j] = qp[j];
    if constexpr (FMT == QG_Q4_0 || FMT == QG_Q8_0) {
        if constexpr (CPL == 1) {
            o.d[0] = reinterpret_cast<const uint16_t *>(srow)[c0];
        } else if constexpr (CPL == 2) {
            o.d[0] = reinterpret_cast<const uint32_t *>(srow)[c0 >> 1];
        } else {
            const uint2 v = reinterpret_cast<const uint2 *>(srow)[c0 >> 2];
            o.d[0] = v.x;
            o.d[1] = v.y;
        }
    } else if constexpr (FMT == QG_Q4_K) {
        o.h = reinterpret_cast<const uint4 *>(srow)[c0 >> 3];
    } else if constexpr (FMT == QG_Q6_K) {
        if constexpr (CPL == 1) {
            const uint2 v = reinterpret_cast<const uint2 *>(hrow)[c0];
            o.h[0] = v.x;
            o.h[1] = v.y;
            o.sc[0] = reinterpret_cast<const uint16_t *>(srow)[c0];
        } else {
#pragma unroll
            for (int j = 0; j < CPL / 2; j++) {
                const uint4 v = reinterpret_cast<const uint4 *>(hrow)[(c0 >> 1) + j];
                o.h[4 * j] = v.x;
                o.h[4 * j + 1] = v.y;
                o.h[4 * j + 2] = v.z;
                o.h[4 * j + 3] = v.w;
            }
            if constexpr (CPL == 2) {
                o.sc[0] = reinterpret_cast<const uint32_t *>(srow)[c0 >> 1];
            } else {
                const uint2 v = reinterpret_cast<const uint2 *>(srow)[c0 >> 2];
                o.sc[0] = v.x;
                o.sc[1] = v.y;
            }
        }
        o.d = reinterpret_cast<const uint16_t *>(drow)[c0 >> 3];
    }
}

// Q4_K: position of sub-block s = chunk mod 8 inside the 12-byte scale field.
struct Q4KSub {
    uint32_t shift; // 8 * (s mod 4)
    bool upper;     // s >= 4
};

__device__ __forceinline__ Q4KSub q4k_sub(int s)
{
    Q4KSub k;
    k.shift = 8u * (uint32_t)(s & 3);
    k.upper = (s & 7) >= 4;
    return k;
}

// Q6_K: sum over one chunk of q*x for its two 16-column halves (columns 0-15
// into ta, 16-31 into tb), codes of low word k extended by high word k/2
// shifted by 2*(k mod 2); the same column order as the staged half sums.
__device__ __forceinline__ void dot_q6_chunk(uint4 q, const uint32_t *h, const float4 (&xv)[8], float &ta,
                                             float &tb)
{
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    ta = 0.0f;
    tb = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t H = h[k >> 1] >> (2 * (k & 1));
        const uint32_t pa = (w[k] & 0x000F000Fu) | (H & 0x00300030u);
        const uint32_t pb = (w[k] & 0x00F000F0u) | (H & 0x03000300u);
        const uint32_t s = w[k] >> 8;
        const uint32_t pc = (s & 0x000F000Fu) | ((H >> 8) & 0x00300030u);
        const uint32_t pd = (s & 0x00F000F0u) | ((H << 8) & 0x03000300u);
        const float4 xl = xv[k], xh = xv[4 + k];
        ta = __builtin_fmaf(half_lo(pa), xl.x, ta);
        ta = __builtin_fmaf(half_hi(pa), xl.z, ta);
        tb = __builtin_fmaf(half_lo(pb), xh.x, tb);
        tb = __builtin_fmaf(half_hi(pb), xh.z, tb);
        ta = __builtin_fmaf(half_lo(pc), xl.y, ta);
        ta = __builtin_fmaf(half_hi(pc), xl.w, ta);
        tb = __builtin_fmaf(half_lo(pd), xh.y, tb);
        tb = __builtin_fmaf(half_hi(pd), xh.w, tb);
    }
}

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c)
{
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// acc += contribution of chunk j of the group, x chunk in xv (+ its staged
// sums: xsum.x the chunk sum or the first half's, xsum.y the second half's;
// Q8_0 activations: xv[0..1] the codes, xsum = (d_x, code sum)).
template <int FMT, int CPL, int J>
__device__ __forceinline__ float consume(const Group<(FMT & 7), CPL> &g, const float4 (&xv)[8], f32x2 xsum,
                                         float acc, const Q4KSub &ks)
{
    if constexpr ((FMT & kQ8Act) != 0) {
        const uint32_t qx[8] = {__builtin_bit_cast(uint32_t, xv[0].x), __builtin_bit_cast(uint32_t, xv[0].y),
                                __builtin_bit_cast(uint32_t, xv[0].z), __builtin_bit_cast(uint32_t, xv[0].w),
                                __builtin_bit_cast(uint32_t, xv[1].x), __builtin_bit_cast(uint32_t, xv[1].y),
                                __builtin_bit_cast(uint32_t, xv[1].z), __builtin_bit_cast(uint32_t, xv[1].w)};
        int isum = 0;
        if constexpr ((FMT & 7) == QG_Q4_0) {
            // word k: low nibbles are columns 4k..4k+3, high nibbles 16+4k..16+4k+3
            const uint32_t w[4] = {g.q[J].x, g.q[J].y, g.q[J].z, g.q[J].w};
#pragma unroll
            for (int k = 0; k < 4; k++) {
                isum = dot4(w[k] & 0x0F0F0F0Fu, qx[k], isum);
                isum = dot4((w[k] >> 4) & 0x0F0F0F0Fu, qx[4 + k], isum);
            }
            isum -= 8 * (int)xsum.y;   // sum (q - 8) q_x
        } else {
            const uint4 a = g.q[2 * J], b = g.q[2 * J + 1];
            isum = dot4(a.x, qx[0], isum);
            isum = dot4(a.y, qx[1], isum);
            isum = dot4(a.z, qx[2], isum);
            isum = dot4(a.w, qx[3], isum);
            isum = dot4(b.x, qx[4], isum);
            isum = dot4(b.y, qx[5], isum);
            isum = dot4(b.z, qx[6], isum);
            isum = dot4(b.w, qx[7], isum);
        }
        const float dw = (J & 1) ? half_hi(g.d[J >> 1]) : half_lo(g.d[J >> 1]);
        return __builtin_fmaf(dw * xsum.x, (float)isum, acc);   // dw * d_x exact: two binary16 significands
    } else if constexpr (FMT == QG_Q4_0 || FMT == QG_Q8_0) {
        const float d = (J & 1) ? half_hi(g.d[J >> 1]) : half_lo(g.d[J >> 1]);
        if constexpr (FMT == QG_Q4_0) {
            const float t = dot_q4_chunk(g.q[J], xv);
            const float u = __builtin_fmaf(-8.0f, xsum.x, t);  // sum (q-8) x
            return __builtin_fmaf(d, u, acc);
        } else {
            const float t = dot_i8_chunk(g.q[2 * J], g.q[2 * J + 1], xv, 0.0f);
            return __builtin_fmaf(d, t, acc);
        }
    } else if constexpr (FMT == QG_Q4_K) {
        const float t = dot_q4_chunk(g.q[J], xv);
        // (sc, m) of this sub-block from the 12-byte field (get_scale_min_k4 of
        // the llamini.cpp post): bytes 0-3 in h.y, 4-7 in h.z, 8-11 in h.w.
        const uint32_t a = g.h.y >> ks.shift, b = g.h.z >> ks.shift, c = g.h.w >> ks.shift;
        const uint32_t sc = ks.upper ? ((c & 0xFu) | ((a >> 2) & 0x30u)) : (a & 63u);
        const uint32_t m = ks.upper ? (((c >> 4) & 0xFu) | ((b >> 2) & 0x30u)) : (b & 63u);
        const float D = half_lo(g.h.x) * (float)sc;   // exact
        const float M = half_hi(g.h.x) * (float)m;    // exact
        acc = __builtin_fmaf(D, t, acc);
        return __builtin_fmaf(-M, xsum.x, acc);
    } else if constexpr (FMT == QG_Q6_K) {
        float ta, tb;
        dot_q6_chunk(g.q[J], &g.h[2 * J], xv, ta, tb);
        // int8 scales of the chunk's two sub-blocks: bytes 2J and 2J+1 of the group's run
        const uint32_t sw = g.sc[J >> 1] >> (16 * (J & 1));
        const float d = half_lo(g.d);
        const float da = d * (float)(int8_t)(sw & 0xFFu);           // exact: 11-bit x 8-bit
        const float db = d * (float)(int8_t)((sw >> 8) & 0xFFu);
        acc = __builtin_fmaf(da, __builtin_fmaf(-32.0f, xsum.x, ta), acc);   // sum (q-32) x
        return __builtin_fmaf(db, __builtin_fmaf(-32.0f, xsum.y, tb), acc);
    } else {
        return dot_i8_chunk(g.q[2 * J], g.q[2 * J + 1], xv, acc);
    }
}

__device__ __forceinline__ float silu_mul(float g, float u)
{
    return g / (1.0f + expf(-g)) * u;
}

template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (N > 0) {
        static_for<N - 1>(f);
        f(std::integral_constant<int, N - 1>{});
    }
}

// NMAT = 1: y = W x.  NMAT = 2: y = silu(Wg x) * (Wu x) (the SwiGLU gate/up
// half, with q[0] = Wg and q[1] = Wu sharing the lane's staged x).
//
// A lane makes P = nchunk / (LPR*CPL) full passes over its row (group sl +
// k*LPR in pass k); the remaining chunks are one partial pass handled chunk by
// chunk.  The full passes run through a ring of D register stages: the loop
// body is straight-line code over the D stages (no branches, so the
// compiler's wait counts stay exact), and the refill of a stage is issued
// right after the stage is consumed, D-1 stage computations before it is
// needed.  Refill indices are clamped to the last full pass, so the final
// refills re-read (cached) valid data instead of branching.  The first stages
// are issued right after x's loads and before the workgroup waits for x to be
// staged, and the next row batch's stages before the current batch's
// reduction.  Batches of G*R rows go to waves in grid-stride order.
template <int FMT, int LPR, int R, int NMAT, int D, int CPL, int EPI>
__global__ __launch_bounds__(512) void gemv_kernel(GemvParams p)
{
    constexpr bool NORM = EPI == kEpiNorm;
    constexpr int BF = FMT & 7;   // the weight format (FMT may carry kQ8Act)
    static_assert((FMT & kQ8Act) == 0 || EPI == kEpiPlain, "Q8_0 activations: plain epilogue only");
    static_assert(EPI != kEpiArgmax || NMAT == 1, "argmax of one product");
    extern __shared__ float4 qg_lds[];
    float *xs = reinterpret_cast<float *>(qg_lds);

    constexpr int G = 64 / LPR;
    constexpr int GS = LPR * CPL;        // chunks covered by one pass of a row
    const int lane = threadIdx.x & 63;
    const int g = lane / LPR, sl = lane % LPR;
    const int waves = blockDim.x >> 6;
    const int64_t nbatch = (p.rows + G * R - 1) / (G * R);
    const int64_t bstride = (int64_t)gridDim.x * waves;
    int64_t batch = (int64_t)blockIdx.x * waves + (threadIdx.x >> 6);
    const int P = p.nchunk / GS;         // full passes (uniform)

    Q4KSub ks[CPL];
#pragma unroll
    for (int j = 0; j < CPL; j++) ks[j] = q4k_sub(sl * CPL + j);   // GS is a multiple of 8

    const uint8_t *qrow[NMAT][R];
    const uint8_t *srow[NMAT][R];
    const uint8_t *hrow[NMAT][R];   // Q6_K only
    const uint8_t *drow[NMAT][R];   // Q6_K only
    Group<BF, CPL> st[D][NMAT][R];

    auto set_rows = [&](int64_t b) {
        const int64_t row0 = b * (G * R) + (int64_t)g * R;
#pragma unroll
        for (int m = 0; m < NMAT; m++) {
#pragma unroll
            for (int r = 0; r < R; r++) {
                int64_t row = row0 + r;
                row = row < p.rows ? row : p.rows - 1;   // ragged tail: read a valid row, store nothing
                qrow[m][r] = p.q[m] + row * p.row_qbytes;
                const uint8_t *sp = p.q[m] + p.soff;
                if (BF == QG_Q4_0 || BF == QG_Q8_0 || BF == QG_Q6_K) srow[m][r] = sp + row * p.nchunk * 2;
                else if (BF == QG_Q4_K) srow[m][r] = sp + row * (p.nchunk / 8) * 16;
                else srow[m][r] = sp + row * 4;
                if constexpr (BF == QG_Q6_K) {
                    hrow[m][r] = p.q[m] + p.hoff + row * p.nchunk * 8;
                    drow[m][r] = p.q[m] + p.doff + row * (p.nchunk / 8) * 2;
                } else {
                    hrow[m][r] = nullptr;
                    drow[m][r] = nullptr;
                }
            }
        }
    };
    auto load_stage = [&](int s, int pass) {
        // the clamp only matters when P == 0 (a row shorter than one pass):
        // the prologue then reads some valid group that is never consumed
        int c0 = (sl + pass * LPR) * CPL;
        c0 = c0 < p.nchunk - CPL ? c0 : p.nchunk - CPL;
#pragma unroll
        for (int m = 0; m < NMAT; m++)
#pragma unroll
            for (int r = 0; r < R; r++)
                load_group<BF, CPL>(st[s][m][r], qrow[m][r], srow[m][r], hrow[m][r], drow[m][r], c0, p.nchunk);
    };
    auto prologue = [&]() {
        const int last = P > 0 ? P - 1 : 0;
#pragma unroll
        for (int s = 0; s < D; s++) load_stage(s, s < last ? s : last);
    };
    auto read_x = [&](int c, float4 (&xv)[8]) -> f32x2 {
        const float4 *xp = reinterpret_cast<const float4 *>(xs + c * kXStride);
        if constexpr (Fmt<FMT>::kSums < 0) {
            xv[0] = xp[0];   // the 32 codes; xv[2..7] unused
            xv[1] = xp[1];
            return *reinterpret_cast<const f32x2 *>(xs + c * kXStride + 8);
        } else {
#pragma unroll
            for (int k = 0; k < 8; k++) xv[k] = xp[k];
            if constexpr (Fmt<FMT>::kSums == 2) return *reinterpret_cast<const f32x2 *>(xs + c * kXStride + 32);
            else if constexpr (Fmt<FMT>::kSums == 1) return f32x2{xs[c * kXStride + 32], 0.0f};
            else return f32x2{0.0f, 0.0f};
        }
    };
    auto compute = [&](const Group<BF, CPL> (&regs)[NMAT][R], int c0, float (&acc)[NMAT][R]) {
        static_for<CPL>([&](auto jj) {
            constexpr int J = decltype(jj)::value;
            float4 xv[8];
            const f32x2 xsum = read_x(c0 + J, xv);
#pragma unroll
            for (int m = 0; m < NMAT; m++)
#pragma unroll
                for (int r = 0; r < R; r++) acc[m][r] = consume<FMT, CPL, J>(regs[m][r], xv, xsum, acc[m][r], ks[J]);
        });
    };

    float norm_scale = 1.0f;
    {
        // No branches until the barrier: a join here would make the compiler
        // wait for every load in flight, the weight stream included.
        float ss = 0.0f;   // NORM: this thread's sum of x^2, chunks in a fixed order
        XStage<false> xst;
        if constexpr (NORM) {
            // the gain doubles the staging registers, and holding them under
            // the weight ring would halve the waves a SIMD can hold; so the
            // normalized staging runs chunk by chunk before the weight stream
            stage_rest_from<Fmt<FMT>::kSums, true>(p.x, p.gamma, xs, p.nchunk, ss, 0);
        } else {
            stage_issue<false>(p.x, p.gamma, p.nchunk, xst);
            stage_rest<Fmt<FMT>::kSums, false>(p.x, p.gamma, xs, p.nchunk, ss);
        }
        __builtin_amdgcn_sched_barrier(0);
        set_rows(batch < nbatch ? batch : nbatch - 1);   // idle waves read a valid row
        prologue();
        // x's loads went out first, so finishing the staging waits for them
        // only, not for the weight loads behind them
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!NORM) stage_finish<Fmt<FMT>::kSums, false>(xs, p.nchunk, xst, ss);
        if constexpr (NORM) {
            // wave sums (fixed xor tree) into the slots after the spare chunk
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
            if (lane == 0) xs[(p.nchunk + 1) * kXStride + (threadIdx.x >> 6)] = ss;
        }
    }
    __syncthreads();
    if constexpr (NORM) {
        // every workgroup adds the same wave sums in the same order: one scale
        float tot = 0.0f;
        for (int w = 0; w < waves; w++) tot += xs[(p.nchunk + 1) * kXStride + w];
        norm_scale = 1.0f / sqrtf(tot / (float)(p.nchunk * kChunk) + p.eps);
    }

    float am_v = -__builtin_inff();   // EPI 3: this thread's best (value, index) so far
    int am_i = 0x7FFFFFFF;
    bool am_nan0 = false;            // EPI 3: this thread wrote row 0 and it is NaN
    for (; batch < nbatch; batch += bstride) {
        float rv[R];   // EPI 2: the residual of this lane group's rows, loaded before the weight stream's waits
        if constexpr (EPI == kEpiResid) {
            const int64_t rrow = batch * (G * R) + (int64_t)g * R;
#pragma unroll
            for (int r = 0; r < R; r++) rv[r] = p.resid[rrow + r < p.rows ? rrow + r : p.rows - 1];
        }
        float acc[NMAT][R];
#pragma unroll
        for (int m = 0; m < NMAT; m++)
#pragma unroll
            for (int r = 0; r < R; r++) acc[m][r] = 0.0f;

        int k = 0;
        for (; k + D <= P; k += D) {
#pragma unroll
            for (int s = 0; s < D; s++) {
                compute(st[s], (sl + (k + s) * LPR) * CPL, acc);
                const int nxt = k + s + D;
                load_stage(s, nxt < P ? nxt : P - 1);
                // keep the refill here: without this fence the scheduler may
                // sink it past the next stages' arithmetic, shortening the time
                // the loads have to land
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int s = 0; s < D; s++)      // remaining full passes (fewer than D), uniform branch
            if (k + s < P) compute(st[s], (sl + (k + s) * LPR) * CPL, acc);
        // the partial pass, chunk by chunk
#pragma unroll
        for (int j = 0; j < CPL; j++) {
            const int c = (sl + P * LPR) * CPL + j;
            if (c < p.nchunk) {
                Group<BF, 1> tl[NMAT][R];
#pragma unroll
                for (int m = 0; m < NMAT; m++)
#pragma unroll
                    for (int r = 0; r < R; r++)
                        load_group<BF, 1>(tl[m][r], qrow[m][r], srow[m][r], hrow[m][r], drow[m][r], c, p.nchunk);
                float4 xv[8];
                const f32x2 xsum = read_x(c, xv);
                const Q4KSub kt = q4k_sub(c);
#pragma unroll
                for (int m = 0; m < NMAT; m++)
#pragma unroll
                    for (int r = 0; r < R; r++) acc[m][r] = consume<FMT, 1, 0>(tl[m][r], xv, xsum, acc[m][r], kt);
            }
        }

        float scale[NMAT][R];
#pragma unroll
        for (int m = 0; m < NMAT; m++)
#pragma unroll
            for (int r = 0; r < R; r++)
                scale[m][r] = BF == QG_I8ROW ? *reinterpret_cast<const float *>(srow[m][r]) : 1.0f;
        const int64_t row0 = batch * (G * R) + (int64_t)g * R;
        const int64_t nb = batch + bstride;
        if (nb < nbatch) {               // next batch starts streaming before this one is reduced
            set_rows(nb);
            prologue();
        }

        // combine the LPR partial sums of each row (fixed tree)
#pragma unroll
        for (int m = 0; m < NMAT; m++)
#pragma unroll
            for (int r = 0; r < R; r++) {
                float v = acc[m][r];
#pragma unroll
                for (int off = LPR / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
                acc[m][r] = v;
            }
        if (sl == 0) {
#pragma unroll
            for (int r = 0; r < R; r++) {
                const int64_t row = row0 + r;
                if (row < p.rows) {
                    float v[NMAT];
#pragma unroll
                    for (int m = 0; m < NMAT; m++) v[m] = acc[m][r] * scale[m][r];
                    if constexpr (NORM) {
#pragma unroll
                        for (int m = 0; m < NMAT; m++) v[m] *= norm_scale;
                    }
                    if constexpr (EPI == kEpiResid) v[0] += rv[r];
                    if constexpr (EPI == kEpiArgmax) {
                        am_take(am_v, am_i, v[0], (int)row);
                        if (row == 0 && v[0] != v[0]) am_nan0 = true;
                    }
                    if (NMAT == 1) p.y[row] = v[0];
                    else p.y[row] = silu_mul(v[0], v[NMAT - 1]);
                }
            }
        }
    }
    if constexpr (EPI == kEpiArgmax) am_finish(am_v, am_i, am_nan0, p.am_cand, p.am_count);
}

template <int FMT, int LPR, int R, int NMAT, int D, int CPL, int EPI>
hipError_t go(const GemvParams &p, const GemvCfg &c, hipStream_t s)
{
    constexpr int G = 64 / LPR;
    const int64_t batches = (p.rows + G * R - 1) / (G * R);
    int64_t nwg = (batches + c.waves - 1) / c.waves;
    if (c.max_wg > 0 && nwg > c.max_wg) nwg = c.max_wg;
    if (EPI == kEpiArgmax && nwg > p.am_max) return hipErrorInvalidValue;
    if (EPI == kEpiArgmax && p.am_grid) *p.am_grid = nwg;
    // NORM: 16 more floats after the spare chunk for the wave sums of x^2
    const size_t lds = gemv_lds_bytes((int64_t)p.nchunk * kChunk) + (EPI == kEpiNorm ? 64 : 0);
    auto kern = gemv_kernel<FMT, LPR, R, NMAT, D, CPL, EPI>;
    if (lds > 65536) {
        // largest dynamic LDS size already allowed for this instantiation, per device
        static std::atomic<int> configured_lds[64];
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
        if ((int)lds > configured_lds[dev].load(std::memory_order_relaxed)) {
            hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            configured_lds[dev].store((int)lds, std::memory_order_relaxed);
        }
    }
    hipEvent_t t0 = nullptr, t1 = nullptr;
    if (take_launch_timing(&t0, &t1)) {
        // the events take this dispatch's own start and end (no extra packets)
        GemvParams arg = p;
        void *args[] = {&arg};
        return hipExtLaunchKernel((const void *)kern, dim3((unsigned)nwg), dim3(64 * c.waves), args, lds, s, t0, t1,
                                  0);
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(64 * c.waves), lds, s, p);
    return hipGetLastError();
}

template <int FMT, int NMAT, int D, int CPL, int EPI>
hipError_t dispatch_lr(const GemvParams &p, const GemvCfg &c, hipStream_t s)
{
#define QG_CASE(L, RR) \
    if (c.lpr == L && c.r == RR) return go<FMT, L, RR, NMAT, D, CPL, EPI>(p, c, s);
    QG_CASE(8, 1) QG_CASE(16, 1) QG_CASE(32, 1) QG_CASE(64, 1)
    QG_CASE(8, 2) QG_CASE(16, 2) QG_CASE(32, 2) QG_CASE(64, 2)
#undef QG_CASE
    return hipErrorInvalidValue;
}

template <int FMT, int NMAT, int D, int EPI>
hipError_t dispatch_cpl(const GemvParams &p, const GemvCfg &c, hipStream_t s)
{
    switch (c.cpl) {
    case 1: return dispatch_lr<FMT, NMAT, D, 1, EPI>(p, c, s);
    case 2: return dispatch_lr<FMT, NMAT, D, 2, EPI>(p, c, s);
    case 4: return dispatch_lr<FMT, NMAT, D, 4, EPI>(p, c, s);
    }
    return hipErrorInvalidValue;
}

template <int FMT, int NMAT, int EPI>
hipError_t dispatch(const GemvParams &p, const GemvCfg &c, hipStream_t s)
{
    switch (c.depth) {
    case 2: return dispatch_cpl<FMT, NMAT, 2, EPI>(p, c, s);
    case 4: return dispatch_cpl<FMT, NMAT, 4, EPI>(p, c, s);
    }
    return hipErrorInvalidValue;
}

} // namespace gemv_detail

// Per-format entry points, each instantiated in its own translation unit.
// EPI: plain, the normalized-input gate/up (NMAT 2), the residual down (NMAT 1)
// or the product with its argmax (NMAT 1).
template <int FMT, int NMAT, int EPI>
hipError_t gemv_dispatch(const gemv_detail::GemvParams &p, const GemvCfg &c, hipStream_t s);

} // namespace qg
