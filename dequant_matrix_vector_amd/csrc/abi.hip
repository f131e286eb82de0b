// The C-ABI entry points: synchronous argument validation, then kernel
// enqueue on the caller's stream.  Errors are returned as values and nothing
// is enqueued on any error (the refusal discipline of the Go "llm" package's
// tests and of llamini.cpp, which rejects what it cannot read rather than
// misreading it).
#include <atomic>
#include <mutex>

#include "qg_internal.h"

using namespace qg;

namespace {

bool valid_fmt(int fmt) { return fmt >= QG_Q4_0 && fmt <= QG_Q6_K; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void *a, int64_t na, const void *b, int64_t nb)
{
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

constexpr int kMaxDevices = 64;
std::atomic<int64_t> g_max_cols[kMaxDevices];
std::atomic<int> g_cu_count[kMaxDevices];
std::once_flag g_init_flag;

void init_cache()
{
    for (auto &v : g_max_cols) v.store(0);
    for (auto &v : g_cu_count) v.store(0);
}

// Largest cols whose staged activation row fits one workgroup's LDS.
int64_t max_cols_current()
{
    std::call_once(g_init_flag, init_cache);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QG_ERR_DEVICE;
    int64_t v = g_max_cols[dev].load();
    if (v > 0) return v;
    int lds = 0;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || lds <= 0)
        return QG_ERR_DEVICE;
    // 36 floats per 32 columns, plus one spare 36-float slot
    v = ((int64_t)lds / (kXStride * 4) - 1) * kChunk;
    v -= v % 256;
    g_max_cols[dev].store(v);
    return v;
}

// Common checks of a [rows][cols] product with x [n_tok][cols] -> y [n_tok][rows].
int check_product(int fmt, const void *packed, const float *x, const float *y, int64_t rows,
                  int64_t cols, int64_t n_tok, Layout *L)
{
    if (!valid_fmt(fmt)) return QG_ERR_FORMAT;
    if (!packed || !x || !y) return QG_ERR_NULL;
    if (n_tok < 1 || n_tok >= (int64_t(1) << 31) || !layout_for(fmt, rows, cols, L)) return QG_ERR_SHAPE;
    const int64_t mc = max_cols_current();
    if (mc < 0) return (int)mc;
    if (cols > mc) return QG_ERR_SHAPE;
    if (!aligned(packed, kPlaneAlign) || !aligned(x, 16) || !aligned(y, 16)) return QG_ERR_ALIGN;
    if (overlap(x, n_tok * cols * 4, y, n_tok * rows * 4) || overlap(packed, L->total, y, n_tok * rows * 4))
        return QG_ERR_ALIAS;
    return QG_OK;
}

} // namespace

namespace qg {
int cu_count()
{
    std::call_once(g_init_flag, init_cache);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int v = g_cu_count[dev].load();
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    g_cu_count[dev].store(v);
    return v;
}
} // namespace qg

extern "C" {

int qgemv_layout_version(void) { return kLayoutVersion; }

const char *qgemv_status_string(int status)
{
    switch (status) {
    case QG_OK: return "ok";
    case QG_ERR_NULL: return "null pointer argument";
    case QG_ERR_SHAPE: return "invalid shape (rows/cols/n_tok out of range or not a block multiple)";
    case QG_ERR_ALIGN: return "misaligned pointer (packed needs 256 bytes, activations 16 bytes)";
    case QG_ERR_FORMAT: return "unknown format";
    case QG_ERR_ALIAS: return "an output buffer overlaps an input or another output";
    case QG_ERR_SCRATCH: return "scratch buffer too small";
    case QG_ERR_LAUNCH: return "kernel launch failed";
    case QG_ERR_DEVICE: return "no usable HIP device";
    default: return "unknown status";
    }
}

int64_t qgemv_max_cols(void) { return max_cols_current(); }

int64_t qgemv_packed_bytes(int fmt, int64_t rows, int64_t cols)
{
    if (!valid_fmt(fmt)) return QG_ERR_FORMAT;
    Layout L;
    if (!layout_for(fmt, rows, cols, &L)) return QG_ERR_SHAPE;
    return L.total;
}

static int repack_common(int fmt, const void *raw, const float *row_scale, void *packed, int64_t rows,
                         int64_t cols, void *stream)
{
    if (!valid_fmt(fmt)) return QG_ERR_FORMAT;
    if (!raw || !packed || (fmt == QG_I8ROW && !row_scale)) return QG_ERR_NULL;
    Layout L;
    if (!layout_for(fmt, rows, cols, &L)) return QG_ERR_SHAPE;
    if (!aligned(packed, kPlaneAlign)) return QG_ERR_ALIGN;
    if (fmt == QG_I8ROW && (!aligned(raw, 16) || !aligned(row_scale, 4))) return QG_ERR_ALIGN;
    int64_t raw_bytes;
    switch (fmt) {
    case QG_Q4_0: raw_bytes = rows * (cols / 32) * 18; break;
    case QG_Q8_0: raw_bytes = rows * (cols / 32) * 34; break;
    case QG_Q4_K: raw_bytes = rows * (cols / 256) * 144; break;
    case QG_Q6_K: raw_bytes = rows * (cols / 256) * 210; break;
    default: raw_bytes = rows * cols; break;
    }
    if (overlap(raw, raw_bytes, packed, L.total)) return QG_ERR_ALIAS;
    if (fmt == QG_I8ROW && overlap(row_scale, rows * 4, packed, L.total)) return QG_ERR_ALIAS;
    if (launch_repack(fmt, raw, row_scale, static_cast<uint8_t *>(packed), rows, cols, (hipStream_t)stream) !=
        hipSuccess)
        return QG_ERR_LAUNCH;
    return QG_OK;
}

int qgemv_repack_q4_0(const void *raw, void *packed, int64_t rows, int64_t cols, void *stream)
{
    return repack_common(QG_Q4_0, raw, nullptr, packed, rows, cols, stream);
}
int qgemv_repack_q8_0(const void *raw, void *packed, int64_t rows, int64_t cols, void *stream)
{
    return repack_common(QG_Q8_0, raw, nullptr, packed, rows, cols, stream);
}
int qgemv_repack_q4_k(const void *raw, void *packed, int64_t rows, int64_t cols, void *stream)
{
    return repack_common(QG_Q4_K, raw, nullptr, packed, rows, cols, stream);
}
int qgemv_repack_q6_k(const void *raw, void *packed, int64_t rows, int64_t cols, void *stream)
{
    return repack_common(QG_Q6_K, raw, nullptr, packed, rows, cols, stream);
}
int qgemv_repack_i8row(const int8_t *q, const float *row_scale, void *packed, int64_t rows, int64_t cols,
                       void *stream)
{
    return repack_common(QG_I8ROW, q, row_scale, packed, rows, cols, stream);
}

int qgemv(int fmt, const void *packed, const float *x, float *y, int64_t rows, int64_t cols, int64_t n_tok,
          void *stream)
{
    Layout L;
    int st = check_product(fmt, packed, x, y, rows, cols, n_tok, &L);
    if (st) return st;
    if (prefill_format(fmt) && n_tok > 1 && prefill_enabled())
        return launch_prefill(fmt, 1, static_cast<const uint8_t *>(packed), nullptr, x, y, rows, cols, n_tok, nullptr, 0,
                              (hipStream_t)stream) == hipSuccess
                   ? QG_OK
                   : QG_ERR_LAUNCH;
    const GemvCfg cfg = choose_cfg(fmt, rows, cols, 1);
    for (int64_t t = 0; t < n_tok; t++) {
        if (launch_gemv(fmt, static_cast<const uint8_t *>(packed), x + t * cols, y + t * rows, rows, cols,
                        (hipStream_t)stream, cfg) != hipSuccess)
            return QG_ERR_LAUNCH;
    }
    return QG_OK;
}

int qgemv_q4_0(const void *packed, const float *x, float *y, int64_t rows, int64_t cols, int64_t n_tok,
               void *stream)
{
    return qgemv(QG_Q4_0, packed, x, y, rows, cols, n_tok, stream);
}
int qgemv_q8_0(const void *packed, const float *x, float *y, int64_t rows, int64_t cols, int64_t n_tok,
               void *stream)
{
    return qgemv(QG_Q8_0, packed, x, y, rows, cols, n_tok, stream);
}
int qgemv_q4_k(const void *packed, const float *x, float *y, int64_t rows, int64_t cols, int64_t n_tok,
               void *stream)
{
    return qgemv(QG_Q4_K, packed, x, y, rows, cols, n_tok, stream);
}
int qgemv_i8row(const void *packed, const float *x, float *y, int64_t rows, int64_t cols, int64_t n_tok,
                void *stream)
{
    return qgemv(QG_I8ROW, packed, x, y, rows, cols, n_tok, stream);
}
int qgemv_q6_k(const void *packed, const float *x, float *y, int64_t rows, int64_t cols, int64_t n_tok,
               void *stream)
{
    return qgemv(QG_Q6_K, packed, x, y, rows, cols, n_tok, stream);
}

int swiglu_gate_up(int fmt, const void *wg, const void *wu, const float *x, float *h, int64_t d_model,
                   int64_t ffn, int64_t n_tok, void *stream)
{
    Layout L;
    int st = check_product(fmt, wg, x, h, ffn, d_model, n_tok, &L);
    if (st) return st;
    if (!wu) return QG_ERR_NULL;
    if (!aligned(wu, kPlaneAlign)) return QG_ERR_ALIGN;
    if (overlap(wu, L.total, h, n_tok * ffn * 4)) return QG_ERR_ALIAS;
    if (prefill_format(fmt) && n_tok > 1 && prefill_enabled())
        return launch_prefill(fmt, 2, static_cast<const uint8_t *>(wg), static_cast<const uint8_t *>(wu), x, h, ffn,
                              d_model, n_tok, nullptr, 0, (hipStream_t)stream) == hipSuccess
                   ? QG_OK
                   : QG_ERR_LAUNCH;
    const GemvCfg cfg = choose_cfg(fmt, ffn, d_model, 2);
    for (int64_t t = 0; t < n_tok; t++) {
        if (launch_gate_up(fmt, static_cast<const uint8_t *>(wg), static_cast<const uint8_t *>(wu),
                           x + t * d_model, h + t * ffn, ffn, d_model, (hipStream_t)stream, cfg) != hipSuccess)
            return QG_ERR_LAUNCH;
    }
    return QG_OK;
}

// Scratch of swiglu_ffn, in floats: h [n_tok][ffn], then, from the next
// 256-byte boundary, room for the partial sums of a K split on the matrix-core
// path (n_tok > 1) -- the most that the gate/up or the down product uses.
static int64_t ffn_part_offset(int64_t d_model, int64_t ffn, int64_t n_tok)
{
    (void)d_model;
    return align_up(n_tok * ffn, kPlaneAlign / 4);
}

// From this many tokens on, and for matrices of at least this many weights,
// swiglu_ffn's matrix-core products read bf16 copies of x and h (x's made by
// a conversion launch, h's by the gate/up product itself, when the scratch
// holds them): each workgroup re-reads its x tile from L2 for every
// super-step, so halving those bytes outweighs the extra launch (about 2 us)
// only on large matrices (27B-class FFN: 62.9 to 61.9 us at 8 tokens, 69.7 to
// 64.8 at 16, 184.9 to 171 at 128; a 576 x 1536 FFN at 128 tokens with two
// conversion launches: 72 to 76).
static const int64_t kFfnBf16MinTok = 8;
static const int64_t kFfnBf16MinWeights = int64_t(1) << 24;

static bool ffn_bf16_copies(int64_t d_model, int64_t ffn, int64_t n_tok)
{
    return n_tok >= kFfnBf16MinTok && d_model * ffn >= kFfnBf16MinWeights;
}

// Floats of scratch behind the partial sums for the bf16 copies of x
// [n_tok][d_model] and h [n_tok][ffn], each from a 256-byte boundary.
static int64_t ffn_bf16_elems(int64_t d_model, int64_t ffn, int64_t n_tok)
{
    return align_up(n_tok * d_model / 2, kPlaneAlign / 4) + align_up(n_tok * ffn / 2, kPlaneAlign / 4);
}

// Floats of partial sums the built-in tile choice asks for (the larger of
// the gate/up and the down product's).
static int64_t ffn_part_elems(int fmt, int64_t d_model, int64_t ffn, int64_t n_tok)
{
    const int64_t a = prefill_part_elems(fmt, 2, ffn, d_model, n_tok), b = prefill_part_elems(fmt, 1, d_model, ffn, n_tok);
    return a > b ? a : b;
}

int64_t swiglu_ffn_scratch_elems(int fmt, int64_t d_model, int64_t ffn, int64_t n_tok)
{
    if (!valid_fmt(fmt)) return QG_ERR_FORMAT;
    Layout La, Lb;
    if (n_tok < 1 || n_tok >= (int64_t(1) << 31) || !layout_for(fmt, ffn, d_model, &La) ||
        !layout_for(fmt, d_model, ffn, &Lb))
        return QG_ERR_SHAPE;
    if (!prefill_format(fmt) || n_tok == 1 || !prefill_enabled()) return n_tok * ffn;
    const int64_t part = ffn_part_elems(fmt, d_model, ffn, n_tok);
    if (ffn_bf16_copies(d_model, ffn, n_tok))
        return align_up(ffn_part_offset(d_model, ffn, n_tok) + part, kPlaneAlign / 4) + ffn_bf16_elems(d_model, ffn, n_tok);
    return part > 0 ? ffn_part_offset(d_model, ffn, n_tok) + part : n_tok * ffn;
}

// Checks shared by swiglu_ffn and swiglu_ffn_q8act.
static int check_ffn(int fmt, const void *wg, const void *wu, const void *wd, const float *x, const float *out,
                     const float *h_scratch, int64_t h_scratch_elems, int64_t d_model, int64_t ffn, int64_t n_tok,
                     Layout *Lg_out, Layout *Ld_out)
{
    if (!valid_fmt(fmt)) return QG_ERR_FORMAT;
    if (!wg || !wu || !wd || !x || !out || !h_scratch) return QG_ERR_NULL;
    Layout Lg, Ld;
    if (n_tok < 1 || n_tok >= (int64_t(1) << 31) || !layout_for(fmt, ffn, d_model, &Lg) ||
        !layout_for(fmt, d_model, ffn, &Ld))
        return QG_ERR_SHAPE;
    const int64_t mc = max_cols_current();
    if (mc < 0) return (int)mc;
    if (d_model > mc || ffn > mc) return QG_ERR_SHAPE;
    if (h_scratch_elems < n_tok * ffn) return QG_ERR_SCRATCH;
    if (!aligned(wg, kPlaneAlign) || !aligned(wu, kPlaneAlign) || !aligned(wd, kPlaneAlign) || !aligned(x, 16) ||
        !aligned(out, 16) || !aligned(h_scratch, 16))
        return QG_ERR_ALIGN;
    const int64_t xb = n_tok * d_model * 4, hb = h_scratch_elems * 4;
    if (overlap(x, xb, out, xb) || overlap(x, xb, h_scratch, hb) || overlap(out, xb, h_scratch, hb) ||
        overlap(wg, Lg.total, h_scratch, hb) || overlap(wu, Lg.total, h_scratch, hb) ||
        overlap(wd, Ld.total, h_scratch, hb) || overlap(wg, Lg.total, out, xb) || overlap(wu, Lg.total, out, xb) ||
        overlap(wd, Ld.total, out, xb))
        return QG_ERR_ALIAS;
    *Lg_out = Lg;
    *Ld_out = Ld;
    return QG_OK;
}

int swiglu_ffn(int fmt, const void *wg, const void *wu, const void *wd, const float *x, float *out,
               float *h_scratch, int64_t h_scratch_elems, int64_t d_model, int64_t ffn, int64_t n_tok,
               void *stream)
{
    Layout Lg, Ld;
    const int st = check_ffn(fmt, wg, wu, wd, x, out, h_scratch, h_scratch_elems, d_model, ffn, n_tok, &Lg, &Ld);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    if (prefill_format(fmt) && n_tok > 1 && prefill_enabled()) {
        // partial sums of a K split go behind h, when the caller's scratch has
        // room; for large matrices from kFfnBf16MinTok tokens on, and with
        // room for them behind the partials, the bf16 copies of x and h too
        const int64_t po = ffn_part_offset(d_model, ffn, n_tok);
        float *part = h_scratch_elems > po ? h_scratch + po : nullptr;
        int64_t pe = part ? h_scratch_elems - po : 0;
        uint16_t *xb = nullptr, *hb = nullptr;
        if (ffn_bf16_copies(d_model, ffn, n_tok)) {
            const int64_t pn = ffn_part_elems(fmt, d_model, ffn, n_tok);
            const int64_t xo = align_up(po + pn, kPlaneAlign / 4);
            if (h_scratch_elems >= xo + ffn_bf16_elems(d_model, ffn, n_tok)) {
                part = pn > 0 ? h_scratch + po : nullptr;
                pe = pn;
                xb = reinterpret_cast<uint16_t *>(h_scratch + xo);
                hb = reinterpret_cast<uint16_t *>(h_scratch + xo + align_up(n_tok * d_model / 2, kPlaneAlign / 4));
            }
        }
        // the gate/up product writes h's bf16 copy itself (its epilogue or
        // its split-K sum)
        if ((xb && launch_to_bf16(x, xb, n_tok * d_model, s) != hipSuccess) ||
            launch_prefill(fmt, 2, static_cast<const uint8_t *>(wg), static_cast<const uint8_t *>(wu), x, h_scratch, ffn,
                           d_model, n_tok, part, pe, s, nullptr, xb, hb) != hipSuccess ||
            launch_prefill(fmt, 1, static_cast<const uint8_t *>(wd), nullptr, h_scratch, out, d_model, ffn, n_tok, part,
                           pe, s, nullptr, hb) != hipSuccess)
            return QG_ERR_LAUNCH;
        return QG_OK;
    }
    const GemvCfg cg = choose_cfg(fmt, ffn, d_model, 2);
    const GemvCfg cd = choose_cfg(fmt, d_model, ffn, 1);
    // K halves for the down product: the gate/up launch clears its output
    // (out is disjoint from x), each half adds into it
    const bool kh = ffn_down_khalf(fmt, d_model, ffn);
    for (int64_t t = 0; t < n_tok; t++) {
        if (launch_gate_up(fmt, static_cast<const uint8_t *>(wg), static_cast<const uint8_t *>(wu), x + t * d_model,
                           h_scratch + t * ffn, ffn, d_model, s, cg, nullptr, 0.0f, kh ? out + t * d_model : nullptr,
                           kh ? d_model : 0) != hipSuccess)
            return QG_ERR_LAUNCH;
    }
    for (int64_t t = 0; t < n_tok; t++) {
        const hipError_t e =
            kh ? launch_down_khalf(fmt, static_cast<const uint8_t *>(wd), h_scratch + t * ffn, out + t * d_model,
                                   d_model, ffn, s)
               : launch_gemv(fmt, static_cast<const uint8_t *>(wd), h_scratch + t * ffn, out + t * d_model, d_model,
                             ffn, s, cd);
        if (e != hipSuccess) return QG_ERR_LAUNCH;
    }
    return QG_OK;
}

// Scratch of swiglu_ffn_block, in floats: h [n_tok][ffn]; on the matrix-core
// path (n_tok > 1) then the normalized input [n_tok][d_model] and room
// for split-K partial sums, each from a 256-byte boundary.
static bool block_on_matrix_cores(int fmt, int64_t n_tok) { return prefill_format(fmt) && n_tok > 1 && prefill_enabled(); }

static int64_t block_xn_offset(int64_t ffn, int64_t n_tok) { return align_up(n_tok * ffn, kPlaneAlign / 4); }

static int64_t block_part_offset(int64_t d_model, int64_t ffn, int64_t n_tok)
{
    return align_up(block_xn_offset(ffn, n_tok) + n_tok * d_model, kPlaneAlign / 4);
}

int64_t swiglu_ffn_block_scratch_elems(int fmt, int64_t d_model, int64_t ffn, int64_t n_tok)
{
    if (!valid_fmt(fmt)) return QG_ERR_FORMAT;
    Layout La, Lb;
    if (n_tok < 1 || n_tok >= (int64_t(1) << 31) || !layout_for(fmt, ffn, d_model, &La) ||
        !layout_for(fmt, d_model, ffn, &Lb))
        return QG_ERR_SHAPE;
    if (!block_on_matrix_cores(fmt, n_tok)) return n_tok * ffn;
    const int64_t part = ffn_part_elems(fmt, d_model, ffn, n_tok);
    if (ffn_bf16_copies(d_model, ffn, n_tok))
        return align_up(block_part_offset(d_model, ffn, n_tok) + part, kPlaneAlign / 4) + ffn_bf16_elems(d_model, ffn, n_tok);
    return part > 0 ? block_part_offset(d_model, ffn, n_tok) + part : block_xn_offset(ffn, n_tok) + n_tok * d_model;
}

int swiglu_ffn_block(int fmt, const void *wg, const void *wu, const void *wd, const float *gamma, float eps,
                     const float *x, float *out, float *h_scratch, int64_t h_scratch_elems, int64_t d_model,
                     int64_t ffn, int64_t n_tok, void *stream)
{
    if (!valid_fmt(fmt)) return QG_ERR_FORMAT;
    if (!wg || !wu || !wd || !gamma || !x || !out || !h_scratch) return QG_ERR_NULL;
    Layout Lg, Ld;
    if (n_tok < 1 || n_tok >= (int64_t(1) << 31) || !layout_for(fmt, ffn, d_model, &Lg) ||
        !layout_for(fmt, d_model, ffn, &Ld) || !(eps >= 0.0f) || !(eps <= 3.0e38f))
        return QG_ERR_SHAPE;
    const int64_t mc = max_cols_current();
    if (mc < 0) return (int)mc;
    if (d_model > mc || ffn > mc) return QG_ERR_SHAPE;
    const bool mfma = block_on_matrix_cores(fmt, n_tok);
    const int64_t need = mfma ? block_xn_offset(ffn, n_tok) + n_tok * d_model : n_tok * ffn;
    if (h_scratch_elems < need) return QG_ERR_SCRATCH;
    if (!aligned(wg, kPlaneAlign) || !aligned(wu, kPlaneAlign) || !aligned(wd, kPlaneAlign) || !aligned(x, 16) ||
        !aligned(out, 16) || !aligned(h_scratch, 16) || !aligned(gamma, 16))
        return QG_ERR_ALIGN;
    const int64_t xb = n_tok * d_model * 4, hb = h_scratch_elems * 4, gb = d_model * 4;
    // out may be x itself (the residual stream updated in place) but not partly overlap it
    if ((out != x && overlap(x, xb, out, xb)) || overlap(x, xb, h_scratch, hb) || overlap(out, xb, h_scratch, hb) ||
        overlap(gamma, gb, out, xb) || overlap(gamma, gb, h_scratch, hb) || overlap(wg, Lg.total, h_scratch, hb) ||
        overlap(wu, Lg.total, h_scratch, hb) || overlap(wd, Ld.total, h_scratch, hb) || overlap(wg, Lg.total, out, xb) ||
        overlap(wu, Lg.total, out, xb) || overlap(wd, Ld.total, out, xb))
        return QG_ERR_ALIAS;
    hipStream_t s = (hipStream_t)stream;
    if (mfma) {
        // normalized input and partial sums behind h in the scratch; with room
        // behind those (large matrices), the bf16 copies of the normalized
        // input (written by the RMSNorm launch) and of h (by the gate/up
        // product), as in swiglu_ffn
        float *xn = h_scratch + block_xn_offset(ffn, n_tok);
        const int64_t po = block_part_offset(d_model, ffn, n_tok);
        float *part = h_scratch_elems > po ? h_scratch + po : nullptr;
        int64_t pe = part ? h_scratch_elems - po : 0;
        uint16_t *xnb = nullptr, *hb = nullptr;
        if (ffn_bf16_copies(d_model, ffn, n_tok)) {
            const int64_t pn = ffn_part_elems(fmt, d_model, ffn, n_tok);
            const int64_t xo = align_up(po + pn, kPlaneAlign / 4);
            if (h_scratch_elems >= xo + ffn_bf16_elems(d_model, ffn, n_tok)) {
                part = pn > 0 ? h_scratch + po : nullptr;
                pe = pn;
                xnb = reinterpret_cast<uint16_t *>(h_scratch + xo);
                hb = reinterpret_cast<uint16_t *>(h_scratch + xo + align_up(n_tok * d_model / 2, kPlaneAlign / 4));
            }
        }
        if (launch_rmsnorm(x, gamma, eps, xn, d_model, n_tok, s, xnb) != hipSuccess ||
            launch_prefill(fmt, 2, static_cast<const uint8_t *>(wg), static_cast<const uint8_t *>(wu), xn, h_scratch, ffn,
                           d_model, n_tok, part, pe, s, nullptr, xnb, hb) != hipSuccess ||
            launch_prefill(fmt, 1, static_cast<const uint8_t *>(wd), nullptr, h_scratch, out, d_model, ffn, n_tok, part,
                           pe, s, x, hb) != hipSuccess)
            return QG_ERR_LAUNCH;
        return QG_OK;
    }
    GemvCfg cg = choose_cfg(fmt, ffn, d_model, 2);
    const GemvCfg cd = choose_cfg(fmt, d_model, ffn, 1);
    // Every workgroup stages the whole normalized input, x and the gain: twice
    // the plain staging, from every workgroup at once.  Twice the waves in half
    // as many workgroups keep the waves and halve that traffic.
    GemvCfg forced;
    if (!launch_override(&forced) && cg.max_wg >= 2 && cg.waves <= 4) {
        cg.waves *= 2;
        cg.max_wg /= 2;
    }
    // K halves for the down product when out is not x (then it does not
    // overlap x): the gate/up launch clears out, the first half adds the
    // residual with its sums.  In place, the residual is out's own content.
    const bool kh = out != x && ffn_down_khalf(fmt, d_model, ffn, true);
    // every token's gate/up (which read x) before any down (which may overwrite x)
    for (int64_t t = 0; t < n_tok; t++) {
        if (launch_gate_up(fmt, static_cast<const uint8_t *>(wg), static_cast<const uint8_t *>(wu), x + t * d_model,
                           h_scratch + t * ffn, ffn, d_model, s, cg, gamma, eps, kh ? out + t * d_model : nullptr,
                           kh ? d_model : 0) != hipSuccess)
            return QG_ERR_LAUNCH;
    }
    for (int64_t t = 0; t < n_tok; t++) {
        const hipError_t e =
            kh ? launch_down_khalf(fmt, static_cast<const uint8_t *>(wd), h_scratch + t * ffn, out + t * d_model,
                                   d_model, ffn, s, x + t * d_model)
               : launch_gemv(fmt, static_cast<const uint8_t *>(wd), h_scratch + t * ffn, out + t * d_model, d_model,
                             ffn, s, cd, x + t * d_model);
        if (e != hipSuccess) return QG_ERR_LAUNCH;
    }
    return QG_OK;
}

int qgemv_argmax(const float *logits, int32_t *token, int64_t n, int64_t n_tok, void *stream)
{
    if (!logits || !token) return QG_ERR_NULL;
    if (n < 1 || n >= (int64_t(1) << 31) || n_tok < 1 || n_tok >= (int64_t(1) << 31)) return QG_ERR_SHAPE;
    if (!aligned(logits, 4) || !aligned(token, 4)) return QG_ERR_ALIGN;
    if (overlap(logits, n * n_tok * 4, token, n_tok * 4)) return QG_ERR_ALIAS;
    return launch_argmax(logits, token, n, n_tok, (hipStream_t)stream) == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

int qgemv_head_argmax(int fmt, const void *packed, const float *x, float *logits, int32_t *token, int64_t rows,
                      int64_t cols, int64_t n_tok, void *stream)
{
    Layout L;
    int st = check_product(fmt, packed, x, logits, rows, cols, n_tok, &L);
    if (st) return st;
    if (!token) return QG_ERR_NULL;
    if (!aligned(token, 4)) return QG_ERR_ALIGN;
    if (overlap(token, n_tok * 4, logits, n_tok * rows * 4) || overlap(token, n_tok * 4, x, n_tok * cols * 4) ||
        overlap(token, n_tok * 4, packed, L.total))
        return QG_ERR_ALIAS;
    st = qgemv(fmt, packed, x, logits, rows, cols, n_tok, stream);
    if (st) return st;
    return launch_argmax(logits, token, rows, n_tok, (hipStream_t)stream) == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

// Workspace of the fused head, laid out alike for every shape (so one
// workspace serves heads of several shapes): a 256-byte header whose first
// word the product sets to its number of candidates, then one 8-byte
// candidate per workgroup (a workgroup writes at least one row, so rows
// candidates always suffice).
static const int64_t kAmCounterBytes = 256;

int64_t qgemv_head_argmax_workspace_bytes(int fmt, int64_t rows, int64_t cols)
{
    if (!valid_fmt(fmt)) return QG_ERR_FORMAT;
    Layout L;
    if (!layout_for(fmt, rows, cols, &L)) return QG_ERR_SHAPE;
    return kAmCounterBytes + 8 * rows;
}

int qgemv_head_argmax_ws(int fmt, const void *packed, const float *x, float *logits, int32_t *token, int64_t rows,
                         int64_t cols, int64_t n_tok, void *workspace, int64_t workspace_bytes, void *stream)
{
    if (n_tok != 1) return qgemv_head_argmax(fmt, packed, x, logits, token, rows, cols, n_tok, stream);
    Layout L;
    int st = check_product(fmt, packed, x, logits, rows, cols, n_tok, &L);
    if (st) return st;
    if (!token || !workspace) return QG_ERR_NULL;
    if (!aligned(token, 4) || !aligned(workspace, 16)) return QG_ERR_ALIGN;
    const int64_t hdr = kAmCounterBytes;
    if (workspace_bytes < hdr + 8 * rows) return QG_ERR_SCRATCH;
    if (overlap(token, 4, logits, rows * 4) || overlap(token, 4, x, cols * 4) || overlap(token, 4, packed, L.total) ||
        overlap(workspace, workspace_bytes, token, 4) || overlap(workspace, workspace_bytes, logits, rows * 4) ||
        overlap(workspace, workspace_bytes, x, cols * 4) || overlap(workspace, workspace_bytes, packed, L.total))
        return QG_ERR_ALIAS;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    ArgmaxOut am;
    am.count = reinterpret_cast<uint32_t *>(ws);
    am.cand = reinterpret_cast<uint2 *>(ws + hdr);
    am.max_cand = (workspace_bytes - hdr) / 8;
    int64_t ncand = 0;
    am.grid_out = &ncand;
    const GemvCfg cfg = choose_cfg(fmt, rows, cols, 1);
    if (launch_gemv(fmt, static_cast<const uint8_t *>(packed), x, logits, rows, cols, (hipStream_t)stream, cfg,
                    nullptr, &am) != hipSuccess ||
        launch_am_combine(am.cand, ncand, token, (hipStream_t)stream) != hipSuccess)
        return QG_ERR_LAUNCH;
    return QG_OK;
}

// ------------------------------------------------------ Q8_0 activations --
static bool q8act_fmt(int fmt) { return fmt == QG_Q4_0 || fmt == QG_Q8_0; }

int qgemv_q8act(int fmt, const void *packed, const float *x, float *y, int64_t rows, int64_t cols, int64_t n_tok,
                void *stream)
{
    if (!q8act_fmt(fmt)) return QG_ERR_FORMAT;
    Layout L;
    int st = check_product(fmt, packed, x, y, rows, cols, n_tok, &L);
    if (st) return st;
    const GemvCfg cfg = choose_cfg(fmt, rows, cols, 1);
    for (int64_t t = 0; t < n_tok; t++) {
        if (launch_gemv(fmt | kQ8Act, static_cast<const uint8_t *>(packed), x + t * cols, y + t * rows, rows, cols,
                        (hipStream_t)stream, cfg) != hipSuccess)
            return QG_ERR_LAUNCH;
    }
    return QG_OK;
}

int swiglu_ffn_q8act(int fmt, const void *wg, const void *wu, const void *wd, const float *x, float *out,
                     float *h_scratch, int64_t h_scratch_elems, int64_t d_model, int64_t ffn, int64_t n_tok,
                     void *stream)
{
    if (!q8act_fmt(fmt)) return QG_ERR_FORMAT;
    Layout Lg, Ld;
    const int st = check_ffn(fmt, wg, wu, wd, x, out, h_scratch, h_scratch_elems, d_model, ffn, n_tok, &Lg, &Ld);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    if (n_tok > 1 && prefill_enabled()) {
        // the batched path when the scratch holds h, the quantized
        // activations and (if room is left) partial sums
        const int64_t ho = align_up(n_tok * ffn, kPlaneAlign / 4);
        const int64_t xb = q8act_x_bytes(d_model > ffn ? d_model : ffn, n_tok);
        if (h_scratch_elems >= ho + xb / 4) {
            uint8_t *ws = reinterpret_cast<uint8_t *>(h_scratch + ho);
            float *part = h_scratch + ho + xb / 4;
            const int64_t pe = h_scratch_elems - ho - xb / 4;
            const uint8_t *g8 = static_cast<const uint8_t *>(wg), *u8 = static_cast<const uint8_t *>(wu);
            if (launch_q8act_quantize(x, ws, d_model, n_tok, s) != hipSuccess ||
                launch_q8act_mfma(fmt, 2, g8, u8, ws, h_scratch, ffn, d_model, n_tok, part, pe, s) != hipSuccess ||
                launch_q8act_quantize(h_scratch, ws, ffn, n_tok, s) != hipSuccess ||
                launch_q8act_mfma(fmt, 1, static_cast<const uint8_t *>(wd), nullptr, ws, out, d_model, ffn, n_tok,
                                  part, pe, s) != hipSuccess)
                return QG_ERR_LAUNCH;
            return QG_OK;
        }
    }
    const GemvCfg cg = choose_cfg(fmt, ffn, d_model, 2);
    const GemvCfg cd = choose_cfg(fmt, d_model, ffn, 1);
    // K halves for the down product as in swiglu_ffn (each lane quantizes its
    // own chunk of h, so the halves quantize exactly what whole rows would)
    const bool kh = ffn_down_khalf(fmt | kQ8Act, d_model, ffn);
    for (int64_t t = 0; t < n_tok; t++) {
        if (launch_gate_up(fmt | kQ8Act, static_cast<const uint8_t *>(wg), static_cast<const uint8_t *>(wu),
                           x + t * d_model, h_scratch + t * ffn, ffn, d_model, s, cg, nullptr, 0.0f,
                           kh ? out + t * d_model : nullptr, kh ? d_model : 0) != hipSuccess)
            return QG_ERR_LAUNCH;
    }
    for (int64_t t = 0; t < n_tok; t++) {
        const hipError_t e =
            kh ? launch_down_khalf(fmt | kQ8Act, static_cast<const uint8_t *>(wd), h_scratch + t * ffn,
                                   out + t * d_model, d_model, ffn, s)
               : launch_gemv(fmt | kQ8Act, static_cast<const uint8_t *>(wd), h_scratch + t * ffn,
                             out + t * d_model, d_model, ffn, s, cd);
        if (e != hipSuccess) return QG_ERR_LAUNCH;
    }
    return QG_OK;
}

// Partial-sum floats the batched Q8_0-activation product splits K into (0: none).
static int64_t q8act_part_elems(int nmat, int64_t rows, int64_t cols, int64_t n_tok)
{
    const Q8mPlan c = q8act_mfma_plan(nmat, rows, cols, n_tok, INT64_MAX);
    return c.ksplit > 1 ? (int64_t)c.ksplit * nmat * n_tok * rows : 0;
}

int64_t qgemv_q8act_workspace_bytes(int fmt, int64_t rows, int64_t cols, int64_t n_tok)
{
    if (!q8act_fmt(fmt)) return QG_ERR_FORMAT;
    Layout L;
    if (n_tok < 1 || n_tok >= (int64_t(1) << 31) || !layout_for(fmt, rows, cols, &L)) return QG_ERR_SHAPE;
    if (n_tok == 1) return 0;
    return q8act_x_bytes(cols, n_tok) + 4 * q8act_part_elems(1, rows, cols, n_tok);
}

int qgemv_q8act_ws(int fmt, const void *packed, const float *x, float *y, int64_t rows, int64_t cols, int64_t n_tok,
                   void *workspace, int64_t workspace_bytes, void *stream)
{
    if (!q8act_fmt(fmt)) return QG_ERR_FORMAT;
    Layout L;
    int st = check_product(fmt, packed, x, y, rows, cols, n_tok, &L);
    if (st) return st;
    if (n_tok == 1 || !prefill_enabled()) return qgemv_q8act(fmt, packed, x, y, rows, cols, n_tok, stream);
    const int64_t xb = q8act_x_bytes(cols, n_tok);
    if (!workspace) return QG_ERR_NULL;
    if (workspace_bytes < xb) return QG_ERR_SCRATCH;
    if (!aligned(workspace, kPlaneAlign)) return QG_ERR_ALIGN;
    if (overlap(workspace, workspace_bytes, x, n_tok * cols * 4) ||
        overlap(workspace, workspace_bytes, y, n_tok * rows * 4) || overlap(workspace, workspace_bytes, packed, L.total))
        return QG_ERR_ALIAS;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    hipStream_t s = (hipStream_t)stream;
    if (launch_q8act_quantize(x, ws, cols, n_tok, s) != hipSuccess ||
        launch_q8act_mfma(fmt, 1, static_cast<const uint8_t *>(packed), nullptr, ws, y, rows, cols, n_tok,
                          reinterpret_cast<float *>(ws + xb), (workspace_bytes - xb) / 4, s) != hipSuccess)
        return QG_ERR_LAUNCH;
    return QG_OK;
}

int64_t swiglu_ffn_q8act_scratch_elems(int fmt, int64_t d_model, int64_t ffn, int64_t n_tok)
{
    if (!q8act_fmt(fmt)) return QG_ERR_FORMAT;
    Layout Lg, Ld;
    if (n_tok < 1 || n_tok >= (int64_t(1) << 31) || !layout_for(fmt, ffn, d_model, &Lg) ||
        !layout_for(fmt, d_model, ffn, &Ld))
        return QG_ERR_SHAPE;
    if (n_tok == 1) return n_tok * ffn;
    const int64_t pg = q8act_part_elems(2, ffn, d_model, n_tok), pd = q8act_part_elems(1, d_model, ffn, n_tok);
    return align_up(n_tok * ffn, kPlaneAlign / 4) + q8act_x_bytes(d_model > ffn ? d_model : ffn, n_tok) / 4 +
           (pg > pd ? pg : pd);
}

int qquantize_q8_0(const float *x, void *blocks, int64_t n, int64_t n_tok, void *stream)
{
    if (!x || !blocks) return QG_ERR_NULL;
    if (n < 32 || n % 32 || n >= (int64_t(1) << 31) || n_tok < 1 || n_tok >= (int64_t(1) << 31))
        return QG_ERR_SHAPE;
    if (!aligned(x, 16)) return QG_ERR_ALIGN;
    if (overlap(x, n * n_tok * 4, blocks, n_tok * (n / 32) * 34)) return QG_ERR_ALIAS;
    return launch_quantize_q8_0(x, static_cast<uint8_t *>(blocks), n, n_tok, (hipStream_t)stream) == hipSuccess
               ? QG_OK
               : QG_ERR_LAUNCH;
}

int qdequant(int fmt, const void *packed, float *w_out, int64_t rows, int64_t cols, void *stream)
{
    if (!valid_fmt(fmt)) return QG_ERR_FORMAT;
    if (!packed || !w_out) return QG_ERR_NULL;
    Layout L;
    if (!layout_for(fmt, rows, cols, &L)) return QG_ERR_SHAPE;
    if (!aligned(packed, kPlaneAlign) || !aligned(w_out, 16)) return QG_ERR_ALIGN;
    if (overlap(packed, L.total, w_out, rows * cols * 4)) return QG_ERR_ALIAS;
    if (launch_dequant(fmt, static_cast<const uint8_t *>(packed), w_out, rows, cols, (hipStream_t)stream) !=
        hipSuccess)
        return QG_ERR_LAUNCH;
    return QG_OK;
}

} // extern "C"
