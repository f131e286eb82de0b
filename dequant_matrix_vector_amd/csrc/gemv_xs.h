// Row-streaming GEMV for one token, the activation held in registers.
//
// y = W x with W block-quantized, one token (llmoxide blog, section 11
// "Prefill and decode": every weight is streamed once for one multiply-add, so
// the product runs at the speed the weight bytes arrive; section 10 "Loading
// weights": each dot product decodes its row's blocks on the fly).
//
// Work decomposition ("x-stationary"):
//   * A lane owns one 32-weight chunk position c of the rows (a Q4_0 block).
//     The workgroup stages x once in LDS (coalesced loads issued before the
//     weight stream, chunks 144 bytes apart so that lanes reading consecutive
//     chunks use different banks); each lane then reads its chunk once and
//     keeps it in registers pre-scaled for the
//     binary16-subnormal decode (2^24 for the low nibbles, 2^20 for the high
//     ones) together with its sum in the decode order (the Q4_0 offset of 8
//     folds in through it, and all-8 codes cancel exactly), and then streams
//     chunk c of row after row.
//   * The lanes of a row are 32-lane segments: lprow = 32 * segments >= the
//     chunks of a row (spare lanes read a valid chunk and contribute 0).  A
//     workgroup of rs * lprow threads covers rs rows per row-step (row
//     phases), so each load instruction of a wave reads whole 512-byte or
//     1 KB runs of consecutive chunks of one or two rows.
//   * A workgroup owns nrs row-steps of rs rows: consecutive ones, or every
//     grid-th one so that all workgroups sweep one band of rows together (the
//     order a plain streaming read is fastest in).  Each lane keeps D row-steps
//     of weight loads in flight in a register ring whose refills are issued
//     as soon as a slot is consumed, across row boundaries (no per-row
//     prologue or drain).
//   * After every D row-steps the lane has D * NMAT chunk products; a
//     butterfly over the 32 lanes of the segment (DPP and one swizzle, no
//     atomics) leaves one full segment sum per lane, written to LDS.  After
//     the last row-step one barrier, then one thread per row adds its
//     segments' sums in segment order (deterministic) and applies the
//     epilogue: silu(g) * u for the gate/up pair (NMAT 2), the RMSNorm scale
//     (EPI 1) or the residual (EPI 2).
//   * Q8_0 activations (FMT Q4_0 | kQ8Act, plain epilogue or K halves): the lane
//     quantizes its staged chunk of x to Q8_0 (as every other kernel of the
//     mode does) and keeps its 32 codes, d_x and their sum; a chunk's product
//     is then the exact integer sum of (q_w - 8) * q_x by v_dot4 on the
//     nibbles spread to bytes, times d_w * d_x (exact: two binary16
//     significands).
//   * K halves (EPI 4, one matrix): each workgroup takes one half of the
//     columns of its rows (even workgroups the first, odd ones the second),
//     so it stages half of x, and adds its half-row sums into y, which holds
//     zeros before the launch, with an atomic add (the first half adds the
//     residual too, when there is one).  Each y then takes exactly two adds
//     onto an exact zero, (0 + a) + b = a + b = b + a, so the result does not
//     depend on which half lands first.
//
// Compared with the lane-group kernel (gemv_impl.h) this stages nothing in
// LDS before streaming (a workgroup of the 27B-class down product would
// otherwise read all 68 KB of its input first), reads x once per lane instead
// of once per chunk from LDS, and keeps the weight ring running through rows.
#pragma once
#include "gemv_impl.h"

namespace qg {
namespace xs_detail {

using gemv_detail::dot_q4_chunk;
using gemv_detail::half_lo;
using gemv_detail::silu_mul;
using gemv_detail::f32x4;
using gemv_detail::static_for;
using gemv_detail::am_take;
using gemv_detail::am_finish;
using gemv_detail::dot4;

struct XsParams {
    const uint8_t *q[2];  // packed tensors (quant plane at offset 0)
    const float *x;       // [cols]
    float *y;             // [rows]
    const float *gamma;   // EPI 1: RMSNorm gain [cols]
    const float *resid;   // EPI 2: residual [rows] (may be y itself)
    float eps;            // EPI 1
    int rows;
    int nchunk;           // cols / 32
    uint32_t row_qbytes;  // quant-plane bytes per row
    uint32_t soff;        // scale-plane offset
    uint32_t row_sbytes;  // scale-plane bytes per row (2 * nchunk)
    int lprow;            // lanes per row: 32 * segments >= the chunks of a K part
    int kchunks;          // chunks per K part (EPI 4: the first half's; else nchunk)
    int rs;               // rows per row-step
    int nrs;              // row-steps per workgroup
    int ga, gb;           // global row-step of local step i in workgroup b: i * ga + b * gb
                          // (ga = 1, gb = nrs: consecutive steps; ga = grid, gb = 1: round robin)
    uint2 *am_cand;       // EPI 3: one (value bits, index) candidate per workgroup
    uint32_t *am_count;   // EPI 3: where workgroup 0 stores the number of candidates
    float *zero;          // NMAT 2, EPI 0 or 1: a vector set to zero after the products (may be null)
    int nzero;            // its length
};

enum { kEpiPlain = 0, kEpiNorm = 1, kEpiResid = 2, kEpiArgmax = 3, kEpiKHalf = 4 };

constexpr int kXsMaxWaves = 16;   // waves per workgroup, at most

// One row-step of one matrix in flight: the lane's 16 code bytes and f16 scale.
struct Slot {
    uint4 q;
    uint32_t d;
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Partner value across lane bit k of a 32-lane segment: quad permutations for
// bits 0 and 1, the 8- and 16-lane mirrors for bits 2 and 3 (each pairs every
// lane with one whose bit k differs), a swizzle for bit 4.
template <int K>
__device__ __forceinline__ float partner(float v)
{
    if constexpr (K == 0) return dpp<0xB1>(v);        // quad_perm [1,0,3,2]
    else if constexpr (K == 1) return dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    else if constexpr (K == 2) return dpp<0x141>(v);  // row_half_mirror
    else if constexpr (K == 3) return dpp<0x140>(v);  // row_mirror
    else return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));   // xor 16
}

// Lane bit taken by step S of the butterfly.  The mirrors pair lanes whose
// lower bits differ, so they come first, while every lane still holds every
// value; each later step pairs lanes that agree on the bits already split on.
__device__ __host__ constexpr int bfly_bit(int S) { return S < 4 ? 3 - S : 4; }

// Butterfly over the 32 lanes of a segment: v[0..V) in every lane -> each lane
// holds one complete segment sum, of the value seg_index<V>(lane).
template <int V, int S = 0>
__device__ __forceinline__ float seg_reduce(float (&v)[V], int lane)
{
    if constexpr (S == 5) {
        return v[0];
    } else {
        constexpr int K = bfly_bit(S);
        if constexpr ((1 << S) < V) {
            constexpr int H = V >> (S + 1);   // values left after this step
            const bool up = (lane >> K) & 1;
#pragma unroll
            for (int i = 0; i < H; i++) {
                const float send = up ? v[i] : v[i + H];
                const float keep = up ? v[i + H] : v[i];
                v[i] = keep + partner<K>(send);
            }
        } else {
            v[0] += partner<K>(v[0]);
        }
        return seg_reduce<V, S + 1>(v, lane);
    }
}

// The value a lane holds after seg_reduce, and whether it is the lane of its
// segment that writes it (the lane whose bits not split on are zero).
template <int V>
__device__ __forceinline__ int seg_index(int lane)
{
    int idx = 0;
#pragma unroll
    for (int s = 0; (1 << s) < V; s++) idx += ((lane >> bfly_bit(s)) & 1) * (V >> (s + 1));
    return idx;
}
template <int V>
__device__ __forceinline__ bool seg_writer(int lane)
{
    int split = 0;
#pragma unroll
    for (int s = 0; (1 << s) < V; s++) split |= 1 << bfly_bit(s);
    return (lane & 31 & ~split) == 0;
}

// x chunk -> pre-scaled registers; returns the chunk sum in the order
// dot_q4_chunk adds the codes (so that sum (q - 8) x of all-8 codes is 0).
__device__ __forceinline__ float prep_q4(float4 (&v)[8])
{
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
    return sum;
}

// PX: 16-byte pieces of x staged per thread (PX * threads >= 8 * chunks); the
// pieces are held in registers under the first weight loads, so the smaller
// PX that covers the row keeps more waves resident.
template <int FMT, int NMAT, int EPI, int D, int PX>
__global__ __launch_bounds__(1024) void gemv_xs_kernel(XsParams p)
{
    static_assert((FMT & ~kQ8Act) == QG_Q4_0, "x-stationary GEMV: Q4_0");
    constexpr bool Q8A = (FMT & kQ8Act) != 0;   // Q8_0 activations
    static_assert(!Q8A || EPI == kEpiPlain || EPI == kEpiKHalf, "Q8_0 activations: plain epilogue or K halves");
    static_assert(PX == 4 || PX == 8, "pieces per thread");
    static_assert(EPI != kEpiArgmax || NMAT == 1, "argmax of one product");
    static_assert(EPI != kEpiKHalf || NMAT == 1, "K halves of one product");
    constexpr int V = D * NMAT;   // chunk products per lane between reductions
    static_assert(V >= 2 && V <= 32 && (V & (V - 1)) == 0, "power-of-two batch");
    extern __shared__ float4 xs_lds4[];
    float *xs_part = reinterpret_cast<float *>(xs_lds4);

    const int t = threadIdx.x;
    const int lane = t & 63;
    // EPI 4: K half kh of the rows of workgroup bid; else the whole row
    constexpr bool KH = EPI == kEpiKHalf;
    const int kh = KH ? (int)(blockIdx.x & 1u) : 0;
    const int bid = KH ? (int)(blockIdx.x >> 1) : (int)blockIdx.x;
    const int c0 = kh * p.kchunks;                                  // first chunk of the part
    const int nck = KH ? min(p.kchunks, p.nchunk - c0) : p.nchunk;  // chunks of the part
    const int phase = t / p.lprow;
    const int craw = t - phase * p.lprow;
    const bool live = craw < nck;
    const int c = live ? craw : nck - 1;   // spare lanes read a valid chunk, contribute 0
    const int seg = t >> 5;
    const int nseg = p.lprow >> 5;
    const int row0 = bid * p.gb * p.rs + phase;   // row of local step i: row0 + i * ga * rs
    const int rstep = p.ga * p.rs;
    const int last = p.rows - 1;

    // LDS: x's part (EPI 1: x times the gain) staged [kchunks + 1][36]
    // (chunks 144 bytes apart, so the lanes' 16-byte reads of consecutive
    // chunks fall in different banks; one spare chunk slot), then (EPI 1) one
    // sum of squares per wave, then the partial row sums [segments][nrs][NMAT]
    float *xsx = xs_part;
    float *wsq = xsx + (p.kchunks + 1) * kXStride;
    float *part = wsq + (EPI == kEpiNorm ? kXsMaxWaves : 0);

    // x (and the gain) in 16-byte pieces, consecutive threads reading
    // consecutive pieces, at most PX per thread; issued before the weight
    // stream so that waiting for them waits for nothing else
    const int npiece = nck * 8;
    const float4 *xpart = reinterpret_cast<const float4 *>(p.x) + c0 * 8;
    float4 xp[PX], gp[PX];
#pragma unroll
    for (int k = 0; k < PX; k++) {
        int j = t + k * (int)blockDim.x;
        j = j < npiece ? j : npiece - 1;
        xp[k] = xpart[j];
        if constexpr (EPI == kEpiNorm) gp[k] = reinterpret_cast<const float4 *>(p.gamma)[j];
    }

    // EPI 2: the residual of the row this thread finishes first, read now so
    // that its latency hides under the weight stream (y may be the residual
    // itself: only this workgroup writes its rows, after this read)
    float rpre = 0.0f;
    if constexpr (EPI == kEpiResid) {
        // branch-free, as the x loads: a clamped row, used only where valid
        const int ph = t % p.rs, i = t / p.rs;
        int row = bid * p.gb * p.rs + i * p.ga * p.rs + ph;
        row = row < p.rows - 1 ? row : p.rows - 1;
        rpre = p.resid[row];
    }

    Slot st[D][NMAT];
    const uint32_t qcol = (uint32_t)(c0 + c) * 16u, scol = p.soff + (uint32_t)(c0 + c) * 2u;
    auto load_step = [&](int s, int i) {
        int row = row0 + i * rstep;
        row = row < last ? row : last;
        const uint32_t qo = __umul24((uint32_t)row, p.row_qbytes) + qcol;
        // one 24-bit multiply-add each (a wider form made the compiler wait for
        // the loads in flight before every refill)
        const uint32_t so = __umul24((uint32_t)row, p.row_sbytes) + scol;
#pragma unroll
        for (int m = 0; m < NMAT; m++) {
            st[s][m].q = *reinterpret_cast<const uint4 *>(p.q[m] + qo);
            st[s][m].d = *reinterpret_cast<const uint16_t *>(p.q[m] + so);
        }
    };
#pragma unroll
    for (int s = 0; s < D; s++) load_step(s, s < p.nrs ? s : p.nrs - 1);
    __builtin_amdgcn_sched_barrier(0);

    // branch-free (a divergent branch here would make the compiler wait for
    // the weight stream too, and keep the pieces in scratch): a piece past the
    // end goes to the spare slot after the last chunk.  EPI 1: the sum of x^2
    // over this thread's pieces (a repeated piece past the end adds 0), and
    // x times the gain is what is staged.
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < PX; k++) {
        const int j = t + k * (int)blockDim.x;
        const int at = j < npiece ? (j >> 3) * kXStride + (j & 7) * 4 : nck * kXStride;
        float4 v = xp[k];
        if constexpr (EPI == kEpiNorm) {
            float q = v.x * v.x;
            q = __builtin_fmaf(v.y, v.y, q);
            q = __builtin_fmaf(v.z, v.z, q);
            q = __builtin_fmaf(v.w, v.w, q);
            ss += j < npiece ? q : 0.0f;
            v.x *= gp[k].x;
            v.y *= gp[k].y;
            v.z *= gp[k].z;
            v.w *= gp[k].w;
        }
        *reinterpret_cast<f32x4 *>(xsx + at) = f32x4{v.x, v.y, v.z, v.w};
    }
    if constexpr (EPI == kEpiNorm) {
        // wave sum by an xor butterfly (partners add the same two values, so
        // every lane ends with the same bits), one slot per wave
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
        if (lane == 0) wsq[t >> 6] = ss;
    }
    __syncthreads();
    float4 xv[8];
#pragma unroll
    for (int k = 0; k < 8; k++) xv[k] = *reinterpret_cast<const float4 *>(xsx + c * kXStride + k * 4);
#pragma unroll
    for (int k = 0; k < 8; k++) {
        xv[k].x = live ? xv[k].x : 0.0f;
        xv[k].y = live ? xv[k].y : 0.0f;
        xv[k].z = live ? xv[k].z : 0.0f;
        xv[k].w = live ? xv[k].w : 0.0f;
    }
    // fp32 activations: x pre-scaled and its chunk sum; Q8_0 activations:
    // the chunk's codes, d_x and code sum (spare lanes: all zero)
    float xsum = 0.0f;
    uint32_t qx[Q8A ? 8 : 1];
    float dx = 0.0f;
    int qxs = 0;
    if constexpr (Q8A) {
        Q8Chunk qc;
        quantize_chunk_q8_0(xv, qc);
#pragma unroll
        for (int k = 0; k < 8; k++) qx[k] = qc.q[k];
        dx = qc.d;
        qxs = qc.qsum;
    } else {
        xsum = prep_q4(xv);
    }

    float norm_scale = 1.0f;
    if constexpr (EPI == kEpiNorm) {
        // the wave sums in wave order: the same scale in every workgroup
        float tot = 0.0f;
        const int nw = (int)blockDim.x >> 6;
        for (int w = 0; w < nw; w++) tot += wsq[w];
        norm_scale = 1.0f / sqrtf(tot / (float)(p.nchunk * kChunk) + p.eps);
    }

    const bool writer = seg_writer<V>(lane);
    const int widx = seg_index<V>(lane);
    // R <= D row-steps from i0, then their reduction (values of steps past R
    // are 0 and not written); REFILL: issue the loads D steps ahead (full
    // batches before the last; the last batch has nothing more to fetch)
    auto batch = [&](int i0, auto refill, auto nsteps) {
        constexpr int R = decltype(nsteps)::value;
        float v[V];
#pragma unroll
        for (int s = 0; s < D; s++) {
#pragma unroll
            for (int m = 0; m < NMAT; m++) {
                if (s < R) {
                    if constexpr (Q8A) {
                        // word k: low nibbles are columns 4k..4k+3, high nibbles 16+4k..16+4k+3
                        const uint32_t w[4] = {st[s][m].q.x, st[s][m].q.y, st[s][m].q.z, st[s][m].q.w};
                        int isum = 0;
#pragma unroll
                        for (int k = 0; k < 4; k++) {
                            isum = dot4(w[k] & 0x0F0F0F0Fu, qx[k], isum);
                            isum = dot4((w[k] >> 4) & 0x0F0F0F0Fu, qx[4 + k], isum);
                        }
                        isum -= 8 * qxs;   // sum (q - 8) q_x, exact
                        v[s * NMAT + m] = live ? (half_lo(st[s][m].d) * dx) * (float)isum : 0.0f;
                    } else {
                        const float tq = dot_q4_chunk(st[s][m].q, xv);
                        const float u = __builtin_fmaf(-8.0f, xsum, tq);   // sum (q - 8) x
                        v[s * NMAT + m] = live ? half_lo(st[s][m].d) * u : 0.0f;   // spare lanes: exactly 0
                    }
                } else {
                    v[s * NMAT + m] = 0.0f;
                }
            }
            if constexpr (decltype(refill)::value) {
                const int nxt = i0 + s + D;
                load_step(s, nxt < p.nrs ? nxt : p.nrs - 1);
            }
            // keep the refill here, right after its slot is consumed
            __builtin_amdgcn_sched_barrier(0);
        }
        const float r = seg_reduce<V>(v, lane);
        if (writer && widx < R * NMAT) part[(seg * p.nrs + i0) * NMAT + widx] = r;   // widx = step * NMAT + matrix
    };
    int i0 = 0;
    for (; i0 + D < p.nrs; i0 += D) batch(i0, std::true_type{}, std::integral_constant<int, D>{});
    // the last 1..D row-steps
    static_for<D>([&](auto rr) {
        constexpr int R = decltype(rr)::value + 1;
        if (p.nrs - i0 == R) batch(i0, std::false_type{}, std::integral_constant<int, R>{});
    });
    __syncthreads();

    // one thread per row: the row phase's segments in order
    float am_v = -__builtin_inff();   // EPI 3: this thread's best (value, index)
    int am_i = 0x7FFFFFFF;
    bool am_nan0 = false;            // EPI 3: this thread wrote row 0 and it is NaN
    for (int j = t; j < p.rs * p.nrs; j += blockDim.x) {
        const int ph = j % p.rs, i = j / p.rs;
        const int row = bid * p.gb * p.rs + i * rstep + ph;
        if (row > last) continue;
        float a[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; m++) a[m] = 0.0f;
        for (int sg = ph * nseg; sg < (ph + 1) * nseg; sg++) {
#pragma unroll
            for (int m = 0; m < NMAT; m++) a[m] += part[(sg * p.nrs + i) * NMAT + m];
        }
        if constexpr (EPI == kEpiNorm) {
#pragma unroll
            for (int m = 0; m < NMAT; m++) a[m] *= norm_scale;
        }
        if constexpr (EPI == kEpiResid) a[0] += j == t ? rpre : p.resid[row];
        if constexpr (EPI == kEpiArgmax) {
            am_take(am_v, am_i, a[0], row);
            if (row == 0 && a[0] != a[0]) am_nan0 = true;
        }
        if constexpr (KH) {
            // the first half carries the residual (y and the residual are
            // disjoint here: y held zeros before the launch)
            if (kh == 0 && p.resid != nullptr) a[0] += p.resid[row];
            __hip_atomic_fetch_add(p.y + row, a[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        else if constexpr (NMAT == 1) p.y[row] = a[0];
        else p.y[row] = silu_mul(a[0], a[NMAT - 1]);
    }
    if constexpr (EPI == kEpiArgmax) am_finish(am_v, am_i, am_nan0, p.am_cand, p.am_count);
    if constexpr (NMAT == 2 && (EPI == kEpiPlain || EPI == kEpiNorm)) {
        // the next product's output, cleared for its K halves' adds
        if (p.zero != nullptr) {
            const int stride = (int)(gridDim.x * blockDim.x);
            for (int j = (int)(blockIdx.x * blockDim.x) + t; j < p.nzero; j += stride) p.zero[j] = 0.0f;
        }
    }
}

} // namespace xs_detail

// Launch configuration of the x-stationary kernel.
struct XsCfg {
    int rs;     // rows per row-step (row phases)
    int seg;    // 32-lane segments per row (>= chunks / 32)
    int depth;  // row-steps in flight per lane (ring depth, also the reduction batch)
    int nrs;    // row-steps per workgroup
    int rr;     // 1: row-steps dealt to workgroups round robin; 0: consecutive
    int wpc;    // > 0: exactly wpc workgroups per CU (nrs follows), at most wpc resident per CU
    int kp;     // K parts: 2 = each row's two column halves in different workgroups (EPI 4), else 1
};

// The calling thread's forced fields (mode 1 of qgemv_set_xs_override; 0 or
// -1 fields: built-in), or false.
bool xs_forced(XsCfg *c);

// Host side (gemv_xs.hip): the configuration for a shape, or false when the
// x-stationary kernel does not take it.  khalf (one matrix, no norm): the
// K-halves form, whose y must hold zeros before the launch (a residual, if
// any, must not overlap y).
bool xs_choose(int fmt, int64_t rows, int64_t cols, int nmat, bool norm, XsCfg *c, bool khalf = false);
// zero (gate/up pair, may be null): nzero floats set to zero after the
// products.
hipError_t launch_xs(int fmt, int nmat, const uint8_t *w0, const uint8_t *w1, const float *x, float *y,
                     int64_t rows, int64_t cols, const XsCfg &c, hipStream_t s, const float *gamma, float eps,
                     const float *resid, const ArgmaxOut *am = nullptr, float *zero = nullptr, int64_t nzero = 0);

} // namespace qg
