// Host side of the x-stationary GEMV (gemv_xs.h): which shapes it takes, its
// launch configuration and the per-variant dispatch.
#include <algorithm>
#include <atomic>

#include "gemv_xs.h"

namespace qg {

using xs_detail::XsParams;

namespace {

// tuning override of the calling thread (qgemv_set_xs_override): mode 0 =
// built-in, -1 = never take the x-stationary kernel, 1 = take it with the
// fields below (0 = built-in value)
thread_local int g_xs_mode = 0;
thread_local XsCfg g_xs_force = {0, 0, 0, 0, -1, 0, 0};

template <int FMT, int NMAT, int EPI, int D, int PX>
hipError_t go(const XsParams &p, int waves, int64_t nwg, size_t lds, hipStream_t s)
{
    auto kern = xs_detail::gemv_xs_kernel<FMT, NMAT, EPI, D, PX>;
    if (lds > 65536) {
        static std::atomic<int> configured[64];
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
        if ((int)lds > configured[dev].load(std::memory_order_relaxed)) {
            hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            configured[dev].store((int)lds, std::memory_order_relaxed);
        }
    }
    hipEvent_t t0 = nullptr, t1 = nullptr;
    if (take_launch_timing(&t0, &t1)) {
        XsParams arg = p;
        void *args[] = {&arg};
        return hipExtLaunchKernel((const void *)kern, dim3((unsigned)nwg), dim3(64 * waves), args, lds, s, t0, t1, 0);
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(64 * waves), lds, s, p);
    return hipGetLastError();
}

template <int FMT, int NMAT, int EPI, int PX>
hipError_t by_depth(const XsParams &p, int depth, int waves, int64_t nwg, size_t lds, hipStream_t s)
{
    switch (depth) {
    case 2: return go<FMT, NMAT, EPI, 2, PX>(p, waves, nwg, lds, s);
    case 4: return go<FMT, NMAT, EPI, 4, PX>(p, waves, nwg, lds, s);
    case 8:
        if constexpr (NMAT == 1) return go<FMT, NMAT, EPI, 8, PX>(p, waves, nwg, lds, s);
        break;
    }
    return hipErrorInvalidValue;
}

// x's pieces per thread: 4 when they cover the row's part, else 8 (threads >= chunks)
template <int FMT, int NMAT, int EPI>
hipError_t by_pieces(const XsParams &p, int depth, int waves, int64_t nwg, size_t lds, hipStream_t s)
{
    if ((int64_t)p.kchunks * 8 <= (int64_t)4 * 64 * waves) return by_depth<FMT, NMAT, EPI, 4>(p, depth, waves, nwg, lds, s);
    return by_depth<FMT, NMAT, EPI, 8>(p, depth, waves, nwg, lds, s);
}

// LDS of a workgroup: x (its K part: nchunk chunks) staged with a spare
// chunk slot, (normalized input) one sum of squares per wave, and the partial
// row sums of every segment.
size_t xs_lds_bytes(const XsCfg &c, int nmat, int64_t nchunk, bool norm)
{
    const size_t staged = (size_t)(nchunk + 1) * kXStride + (norm ? (size_t)xs_detail::kXsMaxWaves : 0);
    return (staged + (size_t)c.rs * c.seg * c.nrs * nmat) * sizeof(float);
}

// a workgroup's LDS may use all of a CU's 160 KB (x of a row of 1024 chunks
// alone takes 144 KB)
constexpr size_t kXsMaxLds = 160 * 1024;

int64_t steps_of(const XsCfg &c, int64_t rows) { return (rows + c.rs - 1) / c.rs; }

// chunks of a K part (the first half's when the columns are split in two)
int64_t part_chunks(const XsCfg &c, int64_t nchunk) { return c.kp == 2 ? (nchunk + 1) / 2 : nchunk; }

bool valid_cfg(const XsCfg &c, int nmat, int64_t nchunk, bool norm)
{
    if (c.wpc > 0 && xs_lds_bytes(c, nmat, nchunk, norm) > kXsMaxLds / c.wpc) return false;
    if (c.rs < 1 || c.rs > 8 || (c.rs & (c.rs - 1))) return false;
    if (c.seg * 32 < nchunk || c.seg > 32) return false;
    if ((c.rs * c.seg) % 2 || c.rs * c.seg / 2 > xs_detail::kXsMaxWaves) return false;
    if (!(c.depth == 2 || c.depth == 4 || (c.depth == 8 && nmat == 1))) return false;
    return c.nrs >= 1 && xs_lds_bytes(c, nmat, nchunk, norm) <= kXsMaxLds;
}

} // namespace

int xs_mode() { return g_xs_mode; }

bool xs_forced(XsCfg *c)
{
    if (g_xs_mode != 1) return false;
    *c = g_xs_force;
    return true;
}

extern "C" int qgemv_set_xs_override(int mode, int rs, int seg, int depth, int nrs, int order, int wg_per_cu)
{
    if (mode == 0 || mode == -1) {
        g_xs_mode = mode;
        g_xs_force = {0, 0, 0, 0, -1, 0, 0};
        return QG_OK;
    }
    if (mode != 1 || rs < 0 || seg < 0 || depth < 0 || nrs < 0 || order < -1 || order > 1 || wg_per_cu < -1 ||
        wg_per_cu > 8)
        return QG_ERR_SHAPE;
    g_xs_mode = 1;
    g_xs_force = {rs, seg, depth, nrs, order, wg_per_cu, 0};
    return QG_OK;
}

// The shapes the kernel takes: Q4_0, a row of at most 1024 chunks (32
// segments), offsets inside one packed tensor below 2^32 and rows below 2^24
// (24-bit multiplies form the addresses).
bool xs_choose(int fmt, int64_t rows, int64_t cols, int nmat, bool norm, XsCfg *out, bool khalf)
{
    // Q4_0 weights, with fp32 or (plain products only) Q8_0 activations
    if (g_xs_mode < 0 || (fmt & ~kQ8Act) != QG_Q4_0) return false;
    if ((fmt & kQ8Act) && norm) return false;
    if (khalf && (nmat != 1 || norm)) return false;
    fmt &= ~kQ8Act;
    Layout L;
    if (!layout_for(fmt, rows, cols, &L) || L.total >= (int64_t(1) << 32) || rows >= (1 << 24) ||
        L.row_qbytes >= (1 << 24))
        return false;
    const int64_t nchunk = cols / kChunk;
    if (khalf && nchunk < 2) return false;
    const int64_t pchunk = khalf ? (nchunk + 1) / 2 : nchunk;   // chunks of a K part
    const int seg0 = (int)((pchunk + 31) / 32);
    if (seg0 > 32) return false;
    // The built-in choice: rows per row-step and segments (padded by one when
    // needed) for a whole number of waves, at most 16; row-steps
    // per workgroup for about three workgroups per CU (pair) or one (single
    // matrix, whose workgroups are wider).
    XsCfg c = {0, 0, 0, 0, 1, 0, khalf ? 2 : 1};
    for (int rs : {2, 1, 4, 8}) {
        for (int seg : {seg0, seg0 + 1}) {
            if ((rs * seg) % 2 == 0 && rs * seg / 2 <= 16 && rs * seg / 2 >= 2 && c.rs == 0) {
                c.rs = rs;
                c.seg = seg;
            }
        }
    }
    if (c.rs == 0) return false;
    // ring depth 2 and several workgroups per CU, from back-to-back sweeps
    // of the 27B-class matrices: the pair three per CU; one matrix as many as
    // its staged x leaves room for in the LDS, at most three (the gate alone,
    // 23 KB: three, 11.7 against 13.7 us at one per CU and depth 4; the down
    // on whole rows, 78 KB: two, 13.5 against 14.3); K halves two per CU over
    // both halves, each staging half of x (the 27B-class block 31.9 against
    // 32.2 us at one per CU)
    c.depth = 2;
    int per_cu = 3;
    if (nmat == 1) {
        const int64_t staged = (pchunk + 1) * kXStride * (int64_t)sizeof(float) + 512;
        per_cu = khalf ? 2 : (int)std::max<int64_t>(1, std::min<int64_t>(3, (int64_t)kXsMaxLds / staged));
    }
    const int64_t steps = steps_of(c, rows);
    const int64_t want_wg = (int64_t)cu_count() * per_cu / c.kp;
    int64_t nrs = (steps + want_wg - 1) / want_wg;
    // tall matrices: more workgroups rather than more LDS per workgroup
    const int64_t room = (int64_t)(kXsMaxLds / sizeof(float)) - (pchunk + 1) * kXStride - (norm ? xs_detail::kXsMaxWaves : 0);
    const int64_t cap = room / ((int64_t)c.rs * c.seg * nmat);
    if (nrs > cap) nrs = cap;
    c.nrs = (int)(nrs < 1 ? 1 : nrs);
    if (g_xs_mode == 1) {
        if (g_xs_force.rs) c.rs = g_xs_force.rs;
        if (g_xs_force.seg) c.seg = g_xs_force.seg;
        if (g_xs_force.depth) c.depth = g_xs_force.depth;
        if (g_xs_force.nrs) c.nrs = g_xs_force.nrs;
        if (g_xs_force.rr >= 0) c.rr = g_xs_force.rr;
        if (g_xs_force.wpc >= 0) c.wpc = g_xs_force.wpc;
    }
    if (c.wpc > 0) {
        // exactly wpc workgroups per CU (over both K halves): the row-steps
        // each one takes follow
        const int64_t grid = (int64_t)c.wpc * cu_count() / c.kp;
        if (grid < 1) return false;
        c.nrs = (int)((steps_of(c, rows) + grid - 1) / grid);
    }
    if (!valid_cfg(c, nmat, pchunk, norm)) return false;
    *out = c;
    return true;
}

hipError_t launch_xs(int fmt, int nmat, const uint8_t *w0, const uint8_t *w1, const float *x, float *y,
                     int64_t rows, int64_t cols, const XsCfg &c, hipStream_t s, const float *gamma, float eps,
                     const float *resid, const ArgmaxOut *am, float *zero, int64_t nzero)
{
    Layout L;
    const bool q8a = (fmt & kQ8Act) != 0;
    if (!layout_for(fmt & ~kQ8Act, rows, cols, &L)) return hipErrorInvalidValue;
    if (q8a && (gamma || resid || am)) return hipErrorInvalidValue;
    const bool khalf = c.kp == 2;
    if (khalf && (nmat != 1 || gamma || am)) return hipErrorInvalidValue;
    if (khalf && resid && resid + rows > y && y + rows > resid) return hipErrorInvalidValue;
    if (zero && (nmat != 2 || nzero < 0 || nzero >= (int64_t(1) << 31))) return hipErrorInvalidValue;
    XsParams p;
    p.q[0] = w0;
    p.q[1] = nmat == 2 ? w1 : w0;
    p.x = x;
    p.y = y;
    p.gamma = gamma;
    p.resid = resid;
    p.eps = eps;
    p.rows = (int)rows;
    p.nchunk = (int)(cols / kChunk);
    p.row_qbytes = (uint32_t)L.row_qbytes;
    p.soff = (uint32_t)L.splane_off;
    p.row_sbytes = (uint32_t)(2 * p.nchunk);
    p.lprow = 32 * c.seg;
    p.kchunks = (int)part_chunks(c, p.nchunk);
    p.rs = c.rs;
    p.nrs = c.nrs;
    const int waves = c.rs * c.seg / 2;
    // workgroups per K part; with K halves, workgroups 2b and 2b + 1 take the
    // two halves of the same rows
    const int64_t nwg = c.wpc > 0 ? (int64_t)c.wpc * cu_count() / c.kp : (steps_of(c, rows) + c.nrs - 1) / c.nrs;
    p.ga = c.rr ? (int)nwg : 1;
    p.gb = c.rr ? 1 : c.nrs;
    p.zero = zero;
    p.nzero = (int)nzero;
    p.am_cand = am ? am->cand : nullptr;
    p.am_count = am ? am->count : nullptr;
    if (am && (nmat != 1 || nwg > am->max_cand)) return hipErrorInvalidValue;
    if (am && am->grid_out) *am->grid_out = nwg;
    size_t lds = xs_lds_bytes(c, nmat, p.kchunks, gamma != nullptr);
    // at most wpc resident per CU: ask for more than a (wpc+1)-th of the LDS
    if (c.wpc > 0 && lds <= kXsMaxLds / (c.wpc + 1)) lds = kXsMaxLds / (c.wpc + 1) + 256;
    const int epi = nmat == 2 ? (gamma ? 1 : 0) : (am ? 3 : (resid ? 2 : 0));
    if (q8a) {
        if (fmt != (QG_Q4_0 | kQ8Act)) return hipErrorInvalidValue;
        if (khalf) return by_pieces<QG_Q4_0 | kQ8Act, 1, 4>(p, c.depth, waves, 2 * nwg, lds, s);
        if (nmat == 1) return by_pieces<QG_Q4_0 | kQ8Act, 1, 0>(p, c.depth, waves, nwg, lds, s);
        return by_pieces<QG_Q4_0 | kQ8Act, 2, 0>(p, c.depth, waves, nwg, lds, s);
    }
    if (fmt != QG_Q4_0) return hipErrorInvalidValue;
    if (khalf) return by_pieces<QG_Q4_0, 1, 4>(p, c.depth, waves, 2 * nwg, lds, s);
    if (nmat == 1) {
        if (epi == 3) return by_pieces<QG_Q4_0, 1, 3>(p, c.depth, waves, nwg, lds, s);
        if (epi == 2) return by_pieces<QG_Q4_0, 1, 2>(p, c.depth, waves, nwg, lds, s);
        return by_pieces<QG_Q4_0, 1, 0>(p, c.depth, waves, nwg, lds, s);
    }
    if (epi == 1) return by_pieces<QG_Q4_0, 2, 1>(p, c.depth, waves, nwg, lds, s);
    return by_pieces<QG_Q4_0, 2, 0>(p, c.depth, waves, nwg, lds, s);
}

} // namespace qg
