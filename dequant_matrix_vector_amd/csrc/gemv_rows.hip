// Row-packed GEMV for one token over Q8_0 matrices with short rows (the
// SmolLM2-135M-shaped vocab head, 576 columns: 18 blocks per row).
//
// y = W x with W block-quantized, one token (llmoxide blog, section 11
// "Prefill and decode": the product runs at the speed the weight bytes
// arrive).  When a row holds fewer blocks than a wave has lanes, neither a
// lane group per row (a remainder pass of idle lanes) nor 32-lane segments
// per row (idle lanes in every segment) fill the lanes.  Here a lane owns one
// block position c of the row (nchunk lanes per row, packed without gaps:
// lane t takes row phase t / nchunk, block t % nchunk), so one wave's two
// 16-byte loads cover a contiguous run of rows (the rows of the quant plane
// are contiguous) and no lane idles while rows remain.
//   * The lane keeps x's block c in registers (read once) and streams block c
//     of row after row: a workgroup owns nrs row-steps of rps = threads /
//     nchunk rows, dealt round robin over the grid (all workgroups sweep one
//     band of rows together), with D row-steps of loads in flight per lane.
//   * Each block product (32 sign-extended byte converts and fmas, times the
//     block's binary16 scale) goes to LDS; after the last row-step one
//     barrier, then one thread per row adds its row's nchunk products in
//     block order (deterministic) and applies the epilogue: plain, the
//     residual, or greedy sampling (the workgroup's argmax candidate and the
//     last workgroup's token, as the other GEMV kernels do).
#include "gemv_xs.h"

namespace qg {
namespace rows_detail {

using gemv_detail::am_finish;
using gemv_detail::am_take;
using gemv_detail::dot_i8_chunk;
using gemv_detail::half_lo;

struct RowsParams {
    const uint8_t *q;     // packed Q8_0 tensor (quant plane at offset 0)
    const float *x;       // [cols]
    float *y;             // [rows]
    const float *resid;   // EPI 2: residual [rows] (may be y itself)
    int rows;
    int nchunk;           // blocks per row
    uint32_t soff;        // scale-plane offset
    int rps;              // rows per row-step (threads / nchunk)
    int nrs;              // row-steps per workgroup
    uint2 *am_cand;       // EPI 3: one (value bits, index) candidate per workgroup
    uint32_t *am_count;   // EPI 3: where workgroup 0 stores the number of candidates
};

enum { kEpiPlain = 0, kEpiResid = 2, kEpiArgmax = 3 };

template <int EPI, int D>
__global__ __launch_bounds__(1024) void gemv_rows_q8_kernel(RowsParams p)
{
    extern __shared__ float rows_part[];   // [nrs][threads] block products
    const int t = threadIdx.x;
    const int nt = (int)blockDim.x;
    const int phase = t / p.nchunk;
    const int c = t - phase * p.nchunk;
    const bool live = phase < p.rps;        // threads past rps * nchunk idle (they read valid rows)
    const int grid = (int)gridDim.x;
    const int last = p.rows - 1;

    // the lane's block of x, read once
    float4 xv[8];
    const float4 *xp = reinterpret_cast<const float4 *>(p.x) + c * 8;
#pragma unroll
    for (int k = 0; k < 8; k++) xv[k] = xp[k];

    uint4 qa[D], qb[D];
    uint32_t sd[D];
    const uint32_t rowb = (uint32_t)p.nchunk * 32u;
    auto load_step = [&](int s, int i) {
        int row = (i * grid + (int)blockIdx.x) * p.rps + phase;
        row = row < last ? row : last;
        const uint8_t *b = p.q + (size_t)row * rowb + (size_t)c * 32;
        qa[s] = *reinterpret_cast<const uint4 *>(b);
        qb[s] = *reinterpret_cast<const uint4 *>(b + 16);
        sd[s] = *reinterpret_cast<const uint16_t *>(p.q + p.soff + ((size_t)row * p.nchunk + c) * 2);
    };
#pragma unroll
    for (int s = 0; s < D; s++) load_step(s, s < p.nrs ? s : p.nrs - 1);
    __builtin_amdgcn_sched_barrier(0);

    // D row-steps from i0: products to LDS, then (REFILL) the loads D steps
    // ahead, issued as soon as each slot is consumed
    auto batch = [&](int i0, auto refill, auto nsteps) {
        constexpr int R = decltype(nsteps)::value;
#pragma unroll
        for (int s = 0; s < R; s++) {
            const float v = dot_i8_chunk(qa[s], qb[s], xv, 0.0f) * half_lo(sd[s]);
            rows_part[(i0 + s) * nt + t] = live ? v : 0.0f;
            if constexpr (decltype(refill)::value) {
                const int nxt = i0 + s + D;
                load_step(s, nxt < p.nrs ? nxt : p.nrs - 1);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    int i0 = 0;
    for (; i0 + D < p.nrs; i0 += D) batch(i0, std::true_type{}, std::integral_constant<int, D>{});
    gemv_detail::static_for<D>([&](auto rr) {
        constexpr int R = decltype(rr)::value + 1;
        if (p.nrs - i0 == R) batch(i0, std::false_type{}, std::integral_constant<int, R>{});
    });
    __syncthreads();

    // one thread per row: its blocks' products in block order
    float am_v = -__builtin_inff();
    int am_i = 0x7FFFFFFF;
    bool am_nan0 = false;
    for (int j = t; j < p.rps * p.nrs; j += nt) {
        const int i = j / p.rps, ph = j - i * p.rps;
        const int row = (i * grid + (int)blockIdx.x) * p.rps + ph;
        if (row > last) continue;
        const float *pp = rows_part + i * nt + ph * p.nchunk;
        float a = 0.0f;
        for (int cc = 0; cc < p.nchunk; cc++) a += pp[cc];
        if constexpr (EPI == kEpiResid) a += p.resid[row];
        if constexpr (EPI == kEpiArgmax) {
            am_take(am_v, am_i, a, row);
            if (row == 0 && a != a) am_nan0 = true;
        }
        p.y[row] = a;
    }
    if constexpr (EPI == kEpiArgmax) am_finish(am_v, am_i, am_nan0, p.am_cand, p.am_count);
}

constexpr int kRowsMaxLds = 64 * 1024;

template <int EPI, int D>
hipError_t go(const RowsParams &p, int threads, int64_t grid, size_t lds, hipStream_t s)
{
    auto kern = gemv_rows_q8_kernel<EPI, D>;
    hipEvent_t t0 = nullptr, t1 = nullptr;
    if (take_launch_timing(&t0, &t1)) {
        RowsParams arg = p;
        void *args[] = {&arg};
        return hipExtLaunchKernel((const void *)kern, dim3((unsigned)grid), dim3(threads), args, lds, s, t0, t1, 0);
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), lds, s, p);
    return hipGetLastError();
}

} // namespace rows_detail

// The shapes it takes: Q8_0 rows of at most 64 blocks (a row-step of whole
// rows fits a workgroup of up to 16 waves), offsets below 2^32.  The
// workgroup: the fewest whole waves (4 to 16) whose threads hold whole rows
// with the fewest idle lanes; about one workgroup per CU, at least 4
// row-steps each; the products of all its row-steps fit 64 KB of LDS.
bool rows_choose(int fmt, int64_t rows, int64_t cols, RowsCfg *out)
{
    if (fmt != QG_Q8_0 || xs_mode() < 0) return false;
    Layout L;
    if (!layout_for(fmt, rows, cols, &L) || L.total >= (int64_t(1) << 32)) return false;
    const int nchunk = (int)(cols / kChunk);
    if (nchunk > 64) return false;
    int best = 4, best_spare = 256;
    for (int w = 4; w <= 16; w++) {
        const int nt = 64 * w, spare = nt - (nt / nchunk) * nchunk;
        if (spare * 64 * best < best_spare * nt) {   // a smaller idle fraction
            best = w;
            best_spare = spare;
        }
    }
    const int nt = 64 * best, rps = nt / nchunk;
    const int64_t steps = (rows + rps - 1) / rps;
    int64_t grid = cu_count();
    int64_t nrs = (steps + grid - 1) / grid;
    if (nrs < 4) {
        nrs = 4;
        grid = (steps + nrs - 1) / nrs;
    }
    if ((size_t)nrs * nt * 4 > (size_t)rows_detail::kRowsMaxLds) {
        nrs = rows_detail::kRowsMaxLds / (nt * 4);
        grid = (steps + nrs - 1) / nrs;
    }
    // two row-steps in flight (a sweep of the SmolLM2-135M Q8_0 head over
    // ring depth 2, 4, 8, row-steps per workgroup 2 to 24 and 1 to 4
    // workgroups per CU: 8.1 us at depth 2 and the choice above, 8.6-9.2 for
    // the others)
    int depth = 2;
    XsCfg f;
    if (xs_forced(&f)) {
        // tuning: row-steps per workgroup (nrs), workgroups per CU (wg_per_cu), ring depth
        if (f.nrs > 0) nrs = f.nrs;
        grid = (steps + nrs - 1) / nrs;
        if (f.wpc > 0) {
            grid = (int64_t)f.wpc * cu_count();
            nrs = (steps + grid - 1) / grid;
        }
        if (f.depth == 2 || f.depth == 4 || f.depth == 8) depth = f.depth;
        if ((size_t)nrs * nt * 4 > (size_t)rows_detail::kRowsMaxLds) return false;
    }
    if (nrs < 1 || grid < 1 || grid >= (int64_t(1) << 31)) return false;
    out->depth = depth;
    out->threads = nt;
    out->rps = rps;
    out->nrs = (int)nrs;
    out->grid = (int)grid;
    return true;
}

hipError_t launch_rows(int fmt, const uint8_t *packed, const float *x, float *y, int64_t rows, int64_t cols,
                       const RowsCfg &c, hipStream_t s, const float *resid, const ArgmaxOut *am)
{
    Layout L;
    if (fmt != QG_Q8_0 || !layout_for(fmt, rows, cols, &L)) return hipErrorInvalidValue;
    rows_detail::RowsParams p;
    p.q = packed;
    p.x = x;
    p.y = y;
    p.resid = resid;
    p.rows = (int)rows;
    p.nchunk = (int)(cols / kChunk);
    p.soff = (uint32_t)L.splane_off;
    p.rps = c.rps;
    p.nrs = c.nrs;
    p.am_cand = am ? am->cand : nullptr;
    p.am_count = am ? am->count : nullptr;
    if (am && (resid || c.grid > am->max_cand)) return hipErrorInvalidValue;
    if (am && am->grid_out) *am->grid_out = c.grid;
    const size_t lds = (size_t)c.nrs * c.threads * 4;
    using namespace rows_detail;
    if (am) {
        if (c.depth == 2) return go<kEpiArgmax, 2>(p, c.threads, c.grid, lds, s);
        if (c.depth == 8) return go<kEpiArgmax, 8>(p, c.threads, c.grid, lds, s);
        return go<kEpiArgmax, 4>(p, c.threads, c.grid, lds, s);
    }
    if (resid) {
        if (c.depth == 2) return go<kEpiResid, 2>(p, c.threads, c.grid, lds, s);
        if (c.depth == 8) return go<kEpiResid, 8>(p, c.threads, c.grid, lds, s);
        return go<kEpiResid, 4>(p, c.threads, c.grid, lds, s);
    }
    if (c.depth == 2) return go<kEpiPlain, 2>(p, c.threads, c.grid, lds, s);
    if (c.depth == 8) return go<kEpiPlain, 8>(p, c.threads, c.grid, lds, s);
    return go<kEpiPlain, 4>(p, c.threads, c.grid, lds, s);
}

} // namespace qg
