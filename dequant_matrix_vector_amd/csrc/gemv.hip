// Host side of the GEMV path: launch-shape choice and per-format dispatch.
// The kernels themselves are in gemv_impl.h (instantiated per format in
// gemv_<format>.hip).
#include "gemv_impl.h"
#include "gemv_xs.h"

namespace qg {

using gemv_detail::GemvParams;

namespace {

template <int NMAT>
hipError_t dispatch_fmt(int fmt, const GemvParams &p, const GemvCfg &c, hipStream_t s)
{
    // NMAT 1 with its argmax or a residual, NMAT 2 with a normalized input, else plain
    const int epi = (NMAT == 1 && p.am_cand) ? 3 : ((NMAT == 1 && p.resid) ? 2 : ((NMAT == 2 && p.gamma) ? 1 : 0));
#define QG_FMT(F)                                                                                  \
    case F:                                                                                        \
        if (epi == 0) return gemv_dispatch<F, NMAT, 0>(p, c, s);                                   \
        if constexpr (NMAT == 2) return gemv_dispatch<F, 2, 1>(p, c, s);                           \
        else if (epi == 3) return gemv_dispatch<F, 1, 3>(p, c, s);                                 \
        else return gemv_dispatch<F, 1, 2>(p, c, s);
    switch (fmt) {
        QG_FMT(QG_Q4_0)
        QG_FMT(QG_Q8_0)
        QG_FMT(QG_Q4_K)
        QG_FMT(QG_I8ROW)
        QG_FMT(QG_Q6_K)
    // Q8_0 activations: plain epilogue only
    case QG_Q4_0 | kQ8Act:
        return epi == 0 ? gemv_dispatch<QG_Q4_0 | kQ8Act, NMAT, 0>(p, c, s) : hipErrorInvalidValue;
    case QG_Q8_0 | kQ8Act:
        return epi == 0 ? gemv_dispatch<QG_Q8_0 | kQ8Act, NMAT, 0>(p, c, s) : hipErrorInvalidValue;
    }
#undef QG_FMT
    return hipErrorInvalidValue;
}

// tuning override of the calling thread (qgemv_set_launch_override)
thread_local GemvCfg g_override = {0, 0, 0, 0, 0, 0};

// CPL must divide the row's chunk count: a group of CPL f16 scales is read
// with one 2*CPL-byte load, which needs the row's scale run (nchunk * 2
// bytes) to keep that alignment, and the kernel's prologue clamps group
// starts to nchunk - CPL.
GemvCfg aligned_cfg(int fmt, int nchunk, GemvCfg c)
{
    (void)fmt;
    while (c.cpl > 1 && nchunk % c.cpl != 0) c.cpl /= 2;
    return c;
}

} // namespace

namespace {
// the calling thread's queued (start, stop) pairs, oldest first
constexpr int kTimedMax = 4;
thread_local hipEvent_t t_ev[kTimedMax][2];
thread_local int t_pending = 0;
} // namespace

bool take_launch_timing(hipEvent_t *start, hipEvent_t *stop)
{
    if (t_pending == 0) return false;
    *start = t_ev[0][0];
    *stop = t_ev[0][1];
    for (int i = 1; i < t_pending; i++) {
        t_ev[i - 1][0] = t_ev[i][0];
        t_ev[i - 1][1] = t_ev[i][1];
    }
    t_pending--;
    return true;
}

extern "C" int qgemv_time_next_launch(void *start_event, void *stop_event)
{
    if ((start_event == nullptr) != (stop_event == nullptr)) return QG_ERR_NULL;
    if (start_event == nullptr) {
        t_pending = 0;
        return QG_OK;
    }
    if (t_pending == kTimedMax) return QG_ERR_SHAPE;
    t_ev[t_pending][0] = static_cast<hipEvent_t>(start_event);
    t_ev[t_pending][1] = static_cast<hipEvent_t>(stop_event);
    t_pending++;
    return QG_OK;
}

extern "C" int qgemv_set_launch_override(int lpr, int r, int waves, int depth, int max_wg, int cpl)
{
    if (lpr == 0) {
        g_override = {0, 0, 0, 0, 0, 0};
        return QG_OK;
    }
    if ((lpr != 8 && lpr != 16 && lpr != 32 && lpr != 64) || (r != 1 && r != 2) || waves < 1 || waves > 8 ||
        (depth != 2 && depth != 4) || max_wg < 0 || (cpl != 1 && cpl != 2 && cpl != 4))
        return QG_ERR_SHAPE;
    g_override = {lpr, r, waves, depth, max_wg, cpl};
    return QG_OK;
}

bool launch_override(GemvCfg *c)
{
    if (g_override.lpr == 0) return false;
    *c = g_override;
    return true;
}

// staged x: 36 floats per chunk plus one spare chunk slot
size_t gemv_lds_bytes(int64_t cols) { return (size_t)(cols / kChunk + 1) * kXStride * sizeof(float); }

// Launch shape from the matrix shape, following launch-shape sweeps on MI355X
// over the five workload families (27B-class FFN, TinyLlama Q4_K layer,
// SmolLM2 layers and heads, stories15M FFN).
GemvCfg choose_cfg(int fmt, int64_t rows, int64_t cols, int nmat)
{
    GemvCfg c;
    if (launch_override(&c)) return c;
    const int64_t nchunk = cols / kChunk;
    const bool eight_bit = fmt == QG_Q8_0 || fmt == QG_I8ROW;
    // Lanes per row and chunks per lane: the widest lane group that still
    // makes enough full passes over the row with no partial pass (a lane then
    // keeps several loads of its own row in flight); otherwise the group whose
    // passes waste the fewest lanes.
    const int64_t min_passes = eight_bit ? 8 : 4;
    c.cpl = 1;
    c.lpr = 0;
    for (int L : {64, 32, 16, 8}) {
        for (int cpl : {1, 2}) {
            const int64_t gs = (int64_t)L * cpl;
            if (nchunk % gs == 0 && nchunk / gs >= min_passes && c.lpr == 0) {
                c.lpr = L;
                c.cpl = cpl;
            }
        }
    }
    if (c.lpr == 0) {
        double best_eff = -1.0;
        for (int L : {64, 32, 16, 8}) {
            const int64_t passes = (nchunk + L - 1) / L;
            const double eff = (double)nchunk / (double)(passes * L);
            if (eff > best_eff + 1e-9) {
                best_eff = eff;
                c.lpr = L;
            }
        }
    }
    const int cus = cu_count();
    if (fmt == QG_Q6_K) {
        // Q6_K (sweeps over the TinyLlama Q6_K vocab head [32000][2048] and
        // down projection [2048][5632]): short rows take narrow lane groups
        // with many rows in flight; long rows take 32 lanes with two chunks
        // each and a deep ring (shallow for the fused pair, which would spill)
        c.r = 1;
        c.max_wg = 4 * cus;
        if (nchunk < 128) {
            c.lpr = 8;
            c.cpl = 1;
            c.waves = 2;
            c.depth = 2;
        } else {
            c.lpr = 32;
            c.cpl = 2;
            c.waves = 4;
            c.depth = nmat == 2 ? 2 : 4;
        }
        return c;
    }
    if (eight_bit) {
        // one row per lane group and 4 waves (sweeps over the SmolLM2-shaped
        // Q8_0 [49152][576] and INT8 [49152][2048] heads and the INT8 FFN
        // [8192][2048] pair and [2048][8192] down); a 4-deep ring for a single
        // matrix, 2 for the pair and the tall heads
        c.max_wg = 4 * cus;
        c.r = 1;
        c.waves = 4;
        c.depth = (nmat == 2 || rows >= 32768) ? 2 : 4;
    } else {
        // long rows want deeper per-lane prefetch
        c.depth = nchunk >= 256 ? 4 : 2;
        c.max_wg = 4 * cus;
        if (nmat == 2) {
            // the fused gate/up kernel already reads two rows per staged x chunk
            c.r = 1;
            c.waves = 2;
        } else {
            // a single matrix: about one workgroup per CU (each stages all of
            // x, so more would repeat the staging; fewer leave CUs idle), two
            // rows per lane group only where rows are plentiful (x reuse from
            // LDS)
            const int64_t g = 64 / c.lpr;
            c.r = rows / g >= 8 * (int64_t)cus ? 2 : 1;
            const int64_t batches = (rows + g * c.r - 1) / (g * c.r);
            const int64_t w = (batches + cus / 2) / cus;
            c.waves = (int)(w < 2 ? 2 : (w > 8 ? 8 : w));
        }
    }
    return c;
}

hipError_t launch_gemv(int fmt, const uint8_t *packed, const float *x, float *y, int64_t rows,
                       int64_t cols, hipStream_t s, const GemvCfg &cfg, const float *resid, const ArgmaxOut *am)
{
    Layout L;
    if (!layout_for(fmt & ~kQ8Act, rows, cols, &L)) return hipErrorInvalidValue;
    if (am && (resid || (fmt & kQ8Act))) return hipErrorInvalidValue;
    GemvCfg forced;
    XsCfg xc;
    RowsCfg rc;
    if (!launch_override(&forced) && xs_choose(fmt, rows, cols, 1, false, &xc))
        return launch_xs(fmt, 1, packed, nullptr, x, y, rows, cols, xc, s, nullptr, 0.0f, resid, am);
    if (!launch_override(&forced) && rows_choose(fmt, rows, cols, &rc))
        return launch_rows(fmt, packed, x, y, rows, cols, rc, s, resid, am);
    GemvParams p;
    p.q[0] = packed;
    p.q[1] = packed;
    p.x = x;
    p.y = y;
    p.rows = rows;
    p.row_qbytes = L.row_qbytes;
    p.soff = L.splane_off;
    p.nchunk = (int)(cols / kChunk);
    p.gamma = nullptr;
    p.eps = 0.0f;
    p.resid = resid;
    p.hoff = L.hplane_off;
    p.doff = L.dplane_off;
    p.am_cand = am ? am->cand : nullptr;
    p.am_max = am ? am->max_cand : 0;
    p.am_count = am ? am->count : nullptr;
    p.am_grid = am ? am->grid_out : nullptr;
    return dispatch_fmt<1>(fmt, p, aligned_cfg(fmt, p.nchunk, cfg), s);
}

namespace {
// tuning switch of the calling thread (qgemv_set_ffn_khalf): 0 built-in, 1 off, 2 on
thread_local int g_khalf_mode = 0;
} // namespace

extern "C" int qgemv_set_ffn_khalf(int mode)
{
    if (mode < 0 || mode > 2) return QG_ERR_SHAPE;
    g_khalf_mode = mode;
    return QG_OK;
}

bool ffn_down_khalf(int fmt, int64_t d_model, int64_t ffn, bool norm)
{
    GemvCfg forced;
    XsCfg a, b;
    if (g_khalf_mode == 1 || launch_override(&forced)) return false;
    // built in from rows of 256 chunks on (the 27B-class down, 544 chunks:
    // half rows of 272)
    if (g_khalf_mode == 0 && ffn / kChunk < 256) return false;
    return xs_choose(fmt, ffn, d_model, 2, norm, &a) && xs_choose(fmt, d_model, ffn, 1, false, &b, true);
}

hipError_t launch_down_khalf(int fmt, const uint8_t *wd, const float *h, float *out, int64_t d_model, int64_t ffn,
                             hipStream_t s, const float *resid)
{
    XsCfg c;
    if (!xs_choose(fmt, d_model, ffn, 1, false, &c, true)) return hipErrorInvalidValue;
    return launch_xs(fmt, 1, wd, nullptr, h, out, d_model, ffn, c, s, nullptr, 0.0f, resid);
}

hipError_t launch_gate_up(int fmt, const uint8_t *wg, const uint8_t *wu, const float *x, float *h,
                          int64_t ffn, int64_t d_model, hipStream_t s, const GemvCfg &cfg, const float *gamma,
                          float eps, float *zero, int64_t nzero)
{
    Layout L;
    if (!layout_for(fmt & ~kQ8Act, ffn, d_model, &L)) return hipErrorInvalidValue;
    GemvCfg forced;
    XsCfg xc;
    const bool on_xs = !launch_override(&forced) && xs_choose(fmt, ffn, d_model, 2, gamma != nullptr, &xc);
    if (zero && !on_xs) return hipErrorInvalidValue;
    if (on_xs) return launch_xs(fmt, 2, wg, wu, x, h, ffn, d_model, xc, s, gamma, eps, nullptr, nullptr, zero, nzero);
    GemvParams p;
    p.q[0] = wg;
    p.q[1] = wu;
    p.x = x;
    p.y = h;
    p.rows = ffn;
    p.row_qbytes = L.row_qbytes;
    p.soff = L.splane_off;
    p.nchunk = (int)(d_model / kChunk);
    p.gamma = gamma;
    p.eps = eps;
    p.resid = nullptr;
    p.hoff = L.hplane_off;
    p.doff = L.dplane_off;
    p.am_cand = nullptr;
    p.am_max = 0;
    p.am_count = nullptr;
    p.am_grid = nullptr;
    return dispatch_fmt<2>(fmt, p, aligned_cfg(fmt, p.nchunk, cfg), s);
}

} // namespace qg
