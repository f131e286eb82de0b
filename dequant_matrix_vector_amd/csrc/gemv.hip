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
//     an I8ROW row) is one lane's work item.
//   * LPR lanes share a row: lane `sl` of the group takes chunks sl, sl+LPR,
//     ...; consecutive lanes read consecutive 16-byte (or 32-byte) pieces of
//     the quant plane, so every wave-wide load is made of whole 128-byte runs.
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
// 8-bit decode (Q8_0, I8ROW): each signed byte converts with one SDWA
// v_cvt_f32_i32 (sign-extending byte select) and feeds one fma.
#include "qg_internal.h"

namespace qg {

namespace {

struct GemvParams {
    const uint8_t *q[2];  // packed tensors (quant plane at offset 0)
    const float *x;       // [cols]
    float *y;             // [rows]
    int64_t rows;
    int64_t row_qbytes;
    int64_t soff;         // scale plane offset inside each packed tensor
    int nchunk;           // cols / 32
};

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

template <int FMT> struct Fmt;
template <> struct Fmt<QG_Q4_0> { static constexpr bool kPrescale = true; };
template <> struct Fmt<QG_Q4_K> { static constexpr bool kPrescale = true; };
template <> struct Fmt<QG_Q8_0> { static constexpr bool kPrescale = false; };
template <> struct Fmt<QG_I8ROW> { static constexpr bool kPrescale = false; };

// Stage x into LDS: per chunk 32 values (scaled by 2^24 / 2^20 for the 4-bit
// formats) and, for those, the chunk sum in the decode order.
template <bool kPrescale>
__device__ __forceinline__ void stage_x(const float *__restrict__ x, float *xs, int nchunk)
{
    for (int c = threadIdx.x; c < nchunk; c += blockDim.x) {
        const float4 *src = reinterpret_cast<const float4 *>(x + (int64_t)c * kChunk);
        float4 v[8];
#pragma unroll
        for (int k = 0; k < 8; k++) v[k] = src[k];
        float4 *dst = reinterpret_cast<float4 *>(xs + c * kXStride);
        if (kPrescale) {
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
#pragma unroll
            for (int k = 0; k < 8; k++) {
                const float sc = k < 4 ? 0x1p24f : 0x1p20f;
                v[k].x *= sc;
                v[k].y *= sc;
                v[k].z *= sc;
                v[k].w *= sc;
            }
            xs[c * kXStride + 32] = sum;
        }
#pragma unroll
        for (int k = 0; k < 8; k++) dst[k] = v[k];
    }
}

template <int FMT> struct ChunkRegs;
template <> struct ChunkRegs<QG_Q4_0> { uint4 q; uint32_t d; };
template <> struct ChunkRegs<QG_Q8_0> { uint4 a, b; uint32_t d; };
template <> struct ChunkRegs<QG_Q4_K> { uint4 q; uint4 h; };
template <> struct ChunkRegs<QG_I8ROW> { uint4 a, b; };

template <int FMT>
__device__ __forceinline__ void load_chunk(ChunkRegs<FMT> &o, const uint8_t *qrow, const uint8_t *srow, int c);

template <>
__device__ __forceinline__ void load_chunk<QG_Q4_0>(ChunkRegs<QG_Q4_0> &o, const uint8_t *qrow, const uint8_t *srow, int c)
{
    o.q = *reinterpret_cast<const uint4 *>(qrow + (int64_t)c * 16);
    o.d = reinterpret_cast<const uint16_t *>(srow)[c];
}
template <>
__device__ __forceinline__ void load_chunk<QG_Q8_0>(ChunkRegs<QG_Q8_0> &o, const uint8_t *qrow, const uint8_t *srow, int c)
{
    const uint4 *p = reinterpret_cast<const uint4 *>(qrow + (int64_t)c * 32);
    o.a = p[0];
    o.b = p[1];
    o.d = reinterpret_cast<const uint16_t *>(srow)[c];
}
template <>
__device__ __forceinline__ void load_chunk<QG_Q4_K>(ChunkRegs<QG_Q4_K> &o, const uint8_t *qrow, const uint8_t *srow, int c)
{
    o.q = *reinterpret_cast<const uint4 *>(qrow + (int64_t)c * 16);
    o.h = reinterpret_cast<const uint4 *>(srow)[c >> 3];
}
template <>
__device__ __forceinline__ void load_chunk<QG_I8ROW>(ChunkRegs<QG_I8ROW> &o, const uint8_t *qrow, const uint8_t *, int c)
{
    const uint4 *p = reinterpret_cast<const uint4 *>(qrow + (int64_t)c * 32);
    o.a = p[0];
    o.b = p[1];
}

// Per-lane constants of the Q4_K six-bit scale unpack: the lane's sub-block
// index s = chunk mod 8 is fixed because LPR is a multiple of 8.
struct Q4KLane {
    uint32_t shift; // 8 * (s mod 4)
    bool upper;     // s >= 4
};

template <int FMT>
__device__ __forceinline__ float consume(const ChunkRegs<FMT> &r, const float4 (&xv)[8], float xsum,
                                         float acc, const Q4KLane &kl);

template <>
__device__ __forceinline__ float consume<QG_Q4_0>(const ChunkRegs<QG_Q4_0> &r, const float4 (&xv)[8],
                                                  float xsum, float acc, const Q4KLane &)
{
    const float t = dot_q4_chunk(r.q, xv);
    const float u = __builtin_fmaf(-8.0f, xsum, t);  // sum (q-8) x
    return __builtin_fmaf(half_lo(r.d), u, acc);
}
template <>
__device__ __forceinline__ float consume<QG_Q8_0>(const ChunkRegs<QG_Q8_0> &r, const float4 (&xv)[8],
                                                  float, float acc, const Q4KLane &)
{
    const float t = dot_i8_chunk(r.a, r.b, xv, 0.0f);
    return __builtin_fmaf(half_lo(r.d), t, acc);
}
template <>
__device__ __forceinline__ float consume<QG_Q4_K>(const ChunkRegs<QG_Q4_K> &r, const float4 (&xv)[8],
                                                  float xsum, float acc, const Q4KLane &kl)
{
    const float t = dot_q4_chunk(r.q, xv);
    // (sc, m) of this sub-block from the 12-byte field (get_scale_min_k4 of
    // the llamini.cpp post): bytes 0-3 in h.y, 4-7 in h.z, 8-11 in h.w.
    const uint32_t a = r.h.y >> kl.shift, b = r.h.z >> kl.shift, c = r.h.w >> kl.shift;
    const uint32_t sc = kl.upper ? ((c & 0xFu) | ((a >> 2) & 0x30u)) : (a & 63u);
    const uint32_t m = kl.upper ? (((c >> 4) & 0xFu) | ((b >> 2) & 0x30u)) : (b & 63u);
    const float D = half_lo(r.h.x) * (float)sc;   // exact
    const float M = half_hi(r.h.x) * (float)m;    // exact
    acc = __builtin_fmaf(D, t, acc);
    return __builtin_fmaf(-M, xsum, acc);
}
template <>
__device__ __forceinline__ float consume<QG_I8ROW>(const ChunkRegs<QG_I8ROW> &r, const float4 (&xv)[8],
                                                   float, float acc, const Q4KLane &)
{
    return dot_i8_chunk(r.a, r.b, xv, acc);
}

__device__ __forceinline__ float silu_mul(float g, float u)
{
    return g / (1.0f + expf(-g)) * u;
}

// NMAT = 1: y = W x.  NMAT = 2: y = silu(Wg x) * (Wu x) (the SwiGLU gate/up
// half, with q[0] = Wg and q[1] = Wu sharing the lane's staged x).
template <int FMT, int LPR, int R, int NMAT>
__global__ __launch_bounds__(512) void gemv_kernel(GemvParams p)
{
    extern __shared__ float4 qg_lds[];
    float *xs = reinterpret_cast<float *>(qg_lds);
    stage_x<Fmt<FMT>::kPrescale>(p.x, xs, p.nchunk);
    __syncthreads();

    constexpr int G = 64 / LPR;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane / LPR, sl = lane % LPR;
    const int64_t batch = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
    if (batch * (G * R) >= p.rows) return;   // uniform per wave; no barrier follows
    const int64_t row0 = batch * (G * R) + (int64_t)g * R;

    const uint8_t *qrow[NMAT][R];
    const uint8_t *srow[NMAT][R];
#pragma unroll
    for (int m = 0; m < NMAT; m++) {
#pragma unroll
        for (int r = 0; r < R; r++) {
            int64_t row = row0 + r;
            row = row < p.rows ? row : p.rows - 1;   // ragged tail: read a valid row, store nothing
            qrow[m][r] = p.q[m] + row * p.row_qbytes;
            const uint8_t *sp = p.q[m] + p.soff;
            if (FMT == QG_Q4_0 || FMT == QG_Q8_0) srow[m][r] = sp + row * p.nchunk * 2;
            else if (FMT == QG_Q4_K) srow[m][r] = sp + row * (p.nchunk / 8) * 16;
            else srow[m][r] = sp + row * 4;
        }
    }
    Q4KLane kl;
    kl.shift = 8u * (uint32_t)(sl & 3);
    kl.upper = (sl & 7) >= 4;

    float acc[NMAT][R];
#pragma unroll
    for (int m = 0; m < NMAT; m++)
#pragma unroll
        for (int r = 0; r < R; r++) acc[m][r] = 0.0f;

    ChunkRegs<FMT> cur[NMAT][R];
    int c = sl;
    if (c < p.nchunk) {
#pragma unroll
        for (int m = 0; m < NMAT; m++)
#pragma unroll
            for (int r = 0; r < R; r++) load_chunk<FMT>(cur[m][r], qrow[m][r], srow[m][r], c);
    }
    while (c < p.nchunk) {
        const int cn = c + LPR;
        ChunkRegs<FMT> nxt[NMAT][R];
        if (cn < p.nchunk) {
#pragma unroll
            for (int m = 0; m < NMAT; m++)
#pragma unroll
                for (int r = 0; r < R; r++) load_chunk<FMT>(nxt[m][r], qrow[m][r], srow[m][r], cn);
        }
        const float4 *xp = reinterpret_cast<const float4 *>(xs + c * kXStride);
        float4 xv[8];
#pragma unroll
        for (int k = 0; k < 8; k++) xv[k] = xp[k];
        const float xsum = Fmt<FMT>::kPrescale ? xs[c * kXStride + 32] : 0.0f;
#pragma unroll
        for (int m = 0; m < NMAT; m++)
#pragma unroll
            for (int r = 0; r < R; r++) acc[m][r] = consume<FMT>(cur[m][r], xv, xsum, acc[m][r], kl);
#pragma unroll
        for (int m = 0; m < NMAT; m++)
#pragma unroll
            for (int r = 0; r < R; r++) cur[m][r] = nxt[m][r];
        c = cn;
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
    if (sl != 0) return;
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int64_t row = row0 + r;
        if (row >= p.rows) break;
        float v[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; m++) {
            v[m] = acc[m][r];
            if (FMT == QG_I8ROW) v[m] *= *reinterpret_cast<const float *>(srow[m][r]);
        }
        if (NMAT == 1) p.y[row] = v[0];
        else p.y[row] = silu_mul(v[0], v[NMAT - 1]);
    }
}

template <int FMT, int LPR, int R, int NMAT>
hipError_t go(const GemvParams &p, int waves, hipStream_t s)
{
    constexpr int G = 64 / LPR;
    const int64_t batches = (p.rows + G * R - 1) / (G * R);
    const int64_t nwg = (batches + waves - 1) / waves;
    const size_t lds = (size_t)p.nchunk * kXStride * sizeof(float);
    auto kern = gemv_kernel<FMT, LPR, R, NMAT>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(64 * waves), lds, s, p);
    return hipGetLastError();
}

template <int FMT, int NMAT>
hipError_t dispatch(const GemvParams &p, const GemvCfg &c, hipStream_t s)
{
#define QG_CASE(L, RR) \
    if (c.lpr == L && c.r == RR) return go<FMT, L, RR, NMAT>(p, c.waves, s);
    QG_CASE(8, 1) QG_CASE(16, 1) QG_CASE(32, 1) QG_CASE(64, 1)
    QG_CASE(8, 2) QG_CASE(16, 2) QG_CASE(32, 2) QG_CASE(64, 2)
    if (NMAT == 1) {
        QG_CASE(8, 4) QG_CASE(16, 4) QG_CASE(32, 4) QG_CASE(64, 4)
    }
#undef QG_CASE
    return hipErrorInvalidValue;
}

template <int NMAT>
hipError_t dispatch_fmt(int fmt, const GemvParams &p, const GemvCfg &c, hipStream_t s)
{
    switch (fmt) {
    case QG_Q4_0: return dispatch<QG_Q4_0, NMAT>(p, c, s);
    case QG_Q8_0: return dispatch<QG_Q8_0, NMAT>(p, c, s);
    case QG_Q4_K: return dispatch<QG_Q4_K, NMAT>(p, c, s);
    case QG_I8ROW: return dispatch<QG_I8ROW, NMAT>(p, c, s);
    }
    return hipErrorInvalidValue;
}

GemvCfg g_override = {0, 0, 0};

} // namespace

extern "C" int qgemv_set_launch_override(int lpr, int r, int waves)
{
    if (lpr == 0) {
        g_override = {0, 0, 0};
        return QG_OK;
    }
    if ((lpr != 8 && lpr != 16 && lpr != 32 && lpr != 64) || (r != 1 && r != 2 && r != 4) || waves < 1 ||
        waves > 8)
        return QG_ERR_SHAPE;
    g_override = {lpr, r, waves};
    return QG_OK;
}

bool launch_override(GemvCfg *c)
{
    if (g_override.lpr == 0) return false;
    *c = g_override;
    return true;
}

size_t gemv_lds_bytes(int64_t cols) { return (size_t)(cols / kChunk) * kXStride * sizeof(float); }

GemvCfg choose_cfg(int fmt, int64_t rows, int64_t cols, int nmat)
{
    GemvCfg c;
    if (launch_override(&c)) {
        if (nmat == 2 && c.r == 4) c.r = 2;
        return c;
    }
    (void)fmt;
    (void)rows;
    const int64_t nchunk = cols / kChunk;
    // lanes per row: the widest group whose last pass over the row is full
    // (ties go to the wider group)
    int best = 8;
    double best_eff = -1.0;
    for (int L : {64, 32, 16, 8}) {
        const int64_t passes = (nchunk + L - 1) / L;
        const double eff = (double)nchunk / (double)(passes * L);
        if (eff > best_eff + 1e-9) {
            best_eff = eff;
            best = L;
        }
    }
    c.lpr = best;
    c.r = nmat == 2 ? 1 : 2;
    c.waves = 4;
    return c;
}

hipError_t launch_gemv(int fmt, const uint8_t *packed, const float *x, float *y, int64_t rows,
                       int64_t cols, hipStream_t s, const GemvCfg &cfg)
{
    Layout L;
    if (!layout_for(fmt, rows, cols, &L)) return hipErrorInvalidValue;
    GemvParams p;
    p.q[0] = packed;
    p.q[1] = packed;
    p.x = x;
    p.y = y;
    p.rows = rows;
    p.row_qbytes = L.row_qbytes;
    p.soff = L.splane_off;
    p.nchunk = (int)(cols / kChunk);
    return dispatch_fmt<1>(fmt, p, cfg, s);
}

hipError_t launch_gate_up(int fmt, const uint8_t *wg, const uint8_t *wu, const float *x, float *h,
                          int64_t ffn, int64_t d_model, hipStream_t s, const GemvCfg &cfg)
{
    Layout L;
    if (!layout_for(fmt, ffn, d_model, &L)) return hipErrorInvalidValue;
    GemvParams p;
    p.q[0] = wg;
    p.q[1] = wu;
    p.x = x;
    p.y = h;
    p.rows = ffn;
    p.row_qbytes = L.row_qbytes;
    p.soff = L.splane_off;
    p.nchunk = (int)(d_model / kChunk);
    return dispatch_fmt<2>(fmt, p, cfg, s);
}

} // namespace qg
