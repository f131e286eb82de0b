// Host side of the matrix-core (batched-token) path: the tile choice, the
// split-K reduce, the RMSNorm launch of the FFN block and the dispatch to the
// per-format kernels (prefill_impl.h, instantiated in prefill_<format>.hip).
#include "prefill_impl.h"

namespace qg {

namespace {

// y[t][i] = sum over K ranges of the partials, in range order (NMAT = 1, plus
// the residual when given), or silu(g) * u of the two summed products
// (NMAT = 2; yb, if not null, also gets it rounded to bf16).  V outputs per
// thread (4 when the element count allows 16-byte accesses).
template <int NMAT, int V>
__global__ void prefill_reduce_kernel(const float *__restrict__ part, float *y, int64_t n, int ksplit,
                                      const float *resid, uint16_t *yb)
{
    typedef float fv __attribute__((ext_vector_type(V)));
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * V;
    if (i >= n) return;
    fv s[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; m++) s[m] = fv(0.0f);
    int k = 0;
    for (; k + 4 <= ksplit; k += 4) {   // four ranges' loads in flight, added in range order
        fv v[4][NMAT];
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int m = 0; m < NMAT; m++) v[j][m] = *reinterpret_cast<const fv *>(part + ((int64_t)(k + j) * NMAT + m) * n + i);
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int m = 0; m < NMAT; m++) s[m] += v[j][m];
    }
    for (; k < ksplit; k++)
#pragma unroll
        for (int m = 0; m < NMAT; m++) s[m] += *reinterpret_cast<const fv *>(part + ((int64_t)k * NMAT + m) * n + i);
    fv r;
#pragma unroll
    for (int e = 0; e < V; e++) r[e] = NMAT == 1 ? s[0][e] : s[0][e] / (1.0f + expf(-s[0][e])) * s[NMAT - 1][e];
    if (NMAT == 1 && resid) r += *reinterpret_cast<const fv *>(resid + i);
    *reinterpret_cast<fv *>(y + i) = r;
    if (NMAT == 2 && yb) {
        if constexpr (V == 4) *reinterpret_cast<uint2 *>(yb + i) = make_uint2(pack_bf16(r[0], r[1]), pack_bf16(r[2], r[3]));
        else yb[i] = (uint16_t)(pack_bf16(r[0], 0.0f) & 0xFFFFu);
    }
}

// RMSNorm of one token row per workgroup (llmoxide blog, section 4 "Keeping
// the numbers in range"): xn_j = x_j * gamma_j / sqrt(mean(x^2) + eps).  The
// sum of squares runs in a fixed order (thread stride, xor tree, waves in
// order), so every call gives the same scale.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float *__restrict__ x, const float *__restrict__ gamma,
                                                      float eps, float *__restrict__ xn, int n, uint16_t *xnb)
{
    __shared__ float wsum[4];
    const float *xt = x + (int64_t)blockIdx.x * n;
    float ss = 0.0f;
    for (int j = threadIdx.x; j < n; j += 256) ss = __builtin_fmaf(xt[j], xt[j], ss);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
    const float sc = 1.0f / sqrtf(tot / (float)n + eps);
    float *o = xn + (int64_t)blockIdx.x * n;
    uint16_t *ob = xnb ? xnb + (int64_t)blockIdx.x * n : nullptr;
    for (int j = threadIdx.x; j < n; j += 256) {
        const float v = xt[j] * sc * gamma[j];
        o[j] = v;
        if (ob) ob[j] = (uint16_t)(pack_bf16(v, 0.0f) & 0xFFFFu);
    }
}

// The same for rows of whole 16-byte pieces that fit P pieces per thread
// (n % 4 == 0, 16-byte aligned, n <= 1024 P): x and the gain are loaded once,
// together, and stay in registers between the sum of squares (each thread
// over its pieces in index order, then the xor tree and the waves in order)
// and the scaling.  xnb (may be null) also gets xn rounded to bf16.
template <int P>
__global__ __launch_bounds__(256) void rmsnorm4_kernel(const float *__restrict__ x, const float *__restrict__ gamma,
                                                       float eps, float *__restrict__ xn, int n, uint16_t *xnb)
{
    __shared__ float wsum[4];
    const int n4 = n / 4;
    const float4 *xt = reinterpret_cast<const float4 *>(x + (int64_t)blockIdx.x * n);
    const float4 *gt = reinterpret_cast<const float4 *>(gamma);
    float4 v[P], gm[P];
#pragma unroll
    for (int k = 0; k < P; k++) {
        const int j = (int)threadIdx.x + k * 256;
        const int jc = j < n4 ? j : n4 - 1;   // a valid piece; not counted, not stored
        v[k] = xt[jc];
        gm[k] = gt[jc];
    }
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < P; k++) {
        const float4 a = (int)threadIdx.x + k * 256 < n4 ? v[k] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        ss = __builtin_fmaf(a.x, a.x, ss);
        ss = __builtin_fmaf(a.y, a.y, ss);
        ss = __builtin_fmaf(a.z, a.z, ss);
        ss = __builtin_fmaf(a.w, a.w, ss);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
    const float sc = 1.0f / sqrtf(tot / (float)n + eps);
    float4 *o = reinterpret_cast<float4 *>(xn + (int64_t)blockIdx.x * n);
    uint2 *ob = xnb ? reinterpret_cast<uint2 *>(xnb + (int64_t)blockIdx.x * n) : nullptr;
#pragma unroll
    for (int k = 0; k < P; k++) {
        const int j = (int)threadIdx.x + k * 256;
        if (j < n4) {
            const float4 r = make_float4(v[k].x * sc * gm[k].x, v[k].y * sc * gm[k].y, v[k].z * sc * gm[k].z,
                                         v[k].w * sc * gm[k].w);
            o[j] = r;
            if (ob) ob[j] = make_uint2(pack_bf16(r.x, r.y), pack_bf16(r.z, r.w));
        }
    }
}

// x -> bf16 (nearest even, the kernel's own rounding of x), 4 values per thread
__global__ void to_bf16_kernel(const float4 *__restrict__ x, uint2 *__restrict__ xb, int64_t n4)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    const float4 a = x[i];
    xb[i] = make_uint2(pack_bf16(a.x, a.y), pack_bf16(a.z, a.w));
}

} // namespace

hipError_t launch_prefill_reduce(int nmat, const float *part, float *y, int64_t n, int ksplit, const float *resid,
                                 hipStream_t s, hipEvent_t stop, uint16_t *yb)
{
    const uintptr_t al = reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(part) |
                         reinterpret_cast<uintptr_t>(resid) | reinterpret_cast<uintptr_t>(yb);
    const bool v4 = n % 4 == 0 && (al & 15) == 0;
    const void *red;
    if (nmat == 2) red = v4 ? (const void *)prefill_reduce_kernel<2, 4> : (const void *)prefill_reduce_kernel<2, 1>;
    else red = v4 ? (const void *)prefill_reduce_kernel<1, 4> : (const void *)prefill_reduce_kernel<1, 1>;
    const int64_t blocks = ((v4 ? n / 4 : n) + 255) / 256;
    void *rargs[] = {&part, &y, &n, &ksplit, &resid, &yb};
    if (stop) return hipExtLaunchKernel(red, dim3((unsigned)blocks), dim3(256), rargs, 0, s, nullptr, stop, 0);
    return hipLaunchKernel(red, dim3((unsigned)blocks), dim3(256), rargs, 0, s);
}

namespace {

// tuning override of the calling thread (qgemv_set_prefill_override)
thread_local PrefillCfg g_pf_override = {0, 0, 0, 0, 0};

// The built-in tile choice (from kernel-trace sweeps of every built shape on
// the 27B-class FFN at 8 to 128 tokens and the SmolLM2-1.7B-shaped FFN and
// head at 128 tokens, all five formats): one 16-row tile per matrix and wave;
// one token tile: 4 waves, runs of two steps; 8 token tiles (128 tokens
// sharing each decoded weight): 8 waves for the fused gate/up pair, 16 for a
// single matrix (256 rows share each staged x tile); 4 token tiles: 4 waves
// for the pair, 8 for a single matrix (a per-kernel trace of the down
// products at 128 tokens: [2048][8192] 21.7 to 15.1 us against 16 waves,
// [5120][17408] 62.0 to 60.0); 2: 4 waves for the pair, and for a
// single matrix 4 waves with runs of two steps; then K ranges until the grid
// has about four workgroups per CU (if the caller gave room for the
// partials), as long as the partial sums (written, then read back) stay
// within half the weight bytes or 16 MB, whichever is more.  A matrix too
// small for its shape (even with the K split that budget and the caller's
// room allow: fewer workgroups than half the CUs, or fewer waves than one per
// SIMD) takes the shape for fewer token tiles, i.e. more token groups.
static void default_tile(PrefillCfg &c, int nmat, int64_t n_tiles)
{
    c.mtr = 1;
    c.ksplit = 0;
    if (n_tiles == 1) {
        c.ntw = 1, c.waves = 4, c.run = 2;
    } else if (n_tiles >= 8) {
        c.ntw = 8, c.waves = nmat == 2 ? 8 : 16, c.run = 1;
    } else if (n_tiles >= 4) {
        c.ntw = 4, c.waves = nmat == 2 ? 4 : 8, c.run = 1;
    } else {
        c.ntw = 2, c.waves = 4, c.run = nmat == 2 ? 1 : 2;
    }
}

// Most K ranges the shape may take: a few ring turns each, at most 16, and
// the partial-sum traffic budget above.
static int64_t max_ksplit(const PrefillCfg &c, int nmat, int64_t rows, int64_t cols, int64_t n_tok)
{
    const int64_t ssteps = (cols / 32 + 4 * c.run - 1) / (4 * c.run);
    int64_t ks = ssteps / 4 > 1 ? ssteps / 4 : 1;
    ks = ks < 16 ? ks : 16;
    // 8 bytes per partial (written, read back) against 18 bytes per 32 weights
    const int64_t per_range = 8 * (int64_t)nmat * n_tok * rows;
    const int64_t weights = (int64_t)nmat * rows * (cols / 32) * 18;
    const int64_t budget = weights / 2 > (int64_t(16) << 20) ? weights / 2 : (int64_t(16) << 20);
    const int64_t by_traffic = budget / per_range;
    return ks < by_traffic ? ks : (by_traffic > 1 ? by_traffic : 1);
}

PrefillCfg choose(int fmt, int nmat, int64_t rows, int64_t cols, int64_t n_tok, int64_t part_elems, int64_t cus)
{
    PrefillCfg c = g_pf_override;
    const int64_t n_tiles = (n_tok + 15) / 16;
    if (c.mtr <= 0) {
        // K ranges the caller's room for partial sums allows (1: none)
        const int64_t room = part_elems / ((int64_t)nmat * n_tok * rows);
        int64_t eff = n_tiles;
        default_tile(c, nmat, eff);
        while (eff > 1) {
            const int64_t grid = ((rows + c.waves * 16 - 1) / (c.waves * 16)) * ((n_tok + c.ntw * 16 - 1) / (c.ntw * 16));
            int64_t ks = max_ksplit(c, nmat, rows, cols, n_tok);
            ks = ks < room ? ks : (room > 1 ? room : 1);
            if (2 * grid * ks >= cus && grid * ks * c.waves >= 4 * cus) break;
            eff = eff >= 8 ? 4 : (eff >= 4 ? 2 : 1);
            default_tile(c, nmat, eff);
        }
        // several token tiles stepped down to one (few rows, no K split):
        // long rows take runs of four steps (sweeps at 128 tokens: Q6_K
        // [2048][5632] 31.3 to 27.8 us, Q4_0 [2048][8192] 30.6 to 29.9; rows of
        // 2048 or fewer columns keep runs of two)
        if (n_tiles > 1 && eff == 1 && cols >= 4096) c.run = 4;
    }
    // a shape that is not built falls back to the nearest one that is: fewer
    // token tiles last, then one row tile per matrix, the other wave count,
    // shorter runs (every nmat has 1, 1, 4, 1)
    if (!pf_fits(fmt, nmat, c.mtr, c.ntw, c.waves, c.run)) {
        bool found = false;
        for (int nt = c.ntw; nt >= 1 && !found; nt /= 2)
            for (int mr : {c.mtr, 1})
                for (int wv : {c.waves, c.waves == 8 ? 4 : 8})
                    for (int rn = c.run; rn >= 1 && !found; rn /= 2)
                        if (pf_fits(fmt, nmat, mr, nt, wv, rn)) {
                            c.mtr = mr, c.ntw = nt, c.waves = wv, c.run = rn;
                            found = true;
                        }
    }
    const int64_t ssteps = (cols / 32 + 4 * c.run - 1) / (4 * c.run);
    const int64_t row_groups = (rows + c.waves * c.mtr * 16 - 1) / (c.waves * c.mtr * 16);
    const int64_t tok_groups = (n_tok + c.ntw * 16 - 1) / (c.ntw * 16);
    int64_t ks = c.ksplit;
    if (ks <= 0) {
        const int64_t want = 4 * cus;
        const int64_t base = row_groups * tok_groups;
        ks = base >= want ? 1 : (want + base - 1) / base;
        const int64_t most = max_ksplit(c, nmat, rows, cols, n_tok);
        ks = ks < most ? ks : most;
    }
    ks = ks < ssteps ? ks : ssteps;
    while (ks > 1 && ks * nmat * n_tok * rows > part_elems) ks--;
    const int64_t spk = (ssteps + ks - 1) / ks;
    c.ksplit = (int)((ssteps + spk - 1) / spk);   // every range non-empty
    return c;
}

} // namespace

extern "C" int qgemv_set_prefill_override(int mtr, int ntw, int waves, int run, int ksplit)
{
    if (mtr == 0 || mtr == -1) {
        g_pf_override = {mtr, 0, 0, 0, 0};
        return QG_OK;
    }
    if ((mtr != 1 && mtr != 2) || (ntw != 1 && ntw != 2 && ntw != 4 && ntw != 8) || (waves != 4 && waves != 8 && waves != 16) ||
        (run != 1 && run != 2 && run != 4) || ksplit < 0 || ksplit > 64)
        return QG_ERR_SHAPE;
    g_pf_override = {mtr, ntw, waves, run, ksplit};
    return QG_OK;
}

extern "C" int qgemv_prefill_plan(int fmt, int nmat, int64_t rows, int64_t cols, int64_t n_tok, int64_t part_elems,
                                  int cus, int *plan)
{
    if (!plan) return QG_ERR_NULL;
    if (!prefill_format(fmt)) return QG_ERR_FORMAT;
    Layout L;
    if ((nmat != 1 && nmat != 2) || n_tok < 2 || n_tok >= (int64_t(1) << 31) || part_elems < 0 || cus < 1 ||
        !layout_for(fmt, rows, cols, &L))
        return QG_ERR_SHAPE;
    const PrefillCfg c = choose(fmt, nmat, rows, cols, n_tok, part_elems, cus);
    plan[0] = c.mtr;
    plan[1] = c.ntw;
    plan[2] = c.waves;
    plan[3] = c.run;
    plan[4] = c.ksplit;
    return QG_OK;
}

bool prefill_enabled() { return g_pf_override.mtr >= 0; }
PrefillCfg prefill_override() { return g_pf_override; }

bool prefill_format(int fmt)
{
    return fmt == QG_Q4_0 || fmt == QG_Q4_K || fmt == QG_Q6_K || fmt == QG_Q8_0 || fmt == QG_I8ROW;
}

int64_t prefill_part_elems(int fmt, int nmat, int64_t rows, int64_t cols, int64_t n_tok)
{
    const PrefillCfg c = choose(fmt, nmat, rows, cols, n_tok, INT64_MAX, cu_count());
    return c.ksplit > 1 ? (int64_t)c.ksplit * nmat * n_tok * rows : 0;
}

hipError_t launch_rmsnorm(const float *x, const float *gamma, float eps, float *xn, int64_t n, int64_t n_tok,
                          hipStream_t s, uint16_t *xnb)
{
    if (n < 1 || n_tok < 1 || n_tok >= (int64_t(1) << 31) || n >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    const uintptr_t al = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(gamma) |
                         reinterpret_cast<uintptr_t>(xn) | reinterpret_cast<uintptr_t>(xnb);
    const int64_t per = (n / 4 + 255) / 256;   // 16-byte pieces per thread
    const dim3 grid((unsigned)n_tok), block(256);
    if (n % 4 == 0 && (al & 15) == 0 && per <= 8) {
        if (per <= 1) hipLaunchKernelGGL(rmsnorm4_kernel<1>, grid, block, 0, s, x, gamma, eps, xn, (int)n, xnb);
        else if (per <= 2) hipLaunchKernelGGL(rmsnorm4_kernel<2>, grid, block, 0, s, x, gamma, eps, xn, (int)n, xnb);
        else if (per <= 4) hipLaunchKernelGGL(rmsnorm4_kernel<4>, grid, block, 0, s, x, gamma, eps, xn, (int)n, xnb);
        else if (per <= 6) hipLaunchKernelGGL(rmsnorm4_kernel<6>, grid, block, 0, s, x, gamma, eps, xn, (int)n, xnb);
        else hipLaunchKernelGGL(rmsnorm4_kernel<8>, grid, block, 0, s, x, gamma, eps, xn, (int)n, xnb);
    } else {
        hipLaunchKernelGGL(rmsnorm_kernel, grid, block, 0, s, x, gamma, eps, xn, (int)n, xnb);
    }
    return hipGetLastError();
}

hipError_t launch_to_bf16(const float *x, uint16_t *xb, int64_t n, hipStream_t s)
{
    if (n < 4 || n % 4 || n / 4 >= (int64_t(1) << 38)) return hipErrorInvalidValue;
    const int64_t n4 = n / 4;
    hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<const float4 *>(x), reinterpret_cast<uint2 *>(xb), n4);
    return hipGetLastError();
}

hipError_t launch_prefill(int fmt, int nmat, const uint8_t *w0, const uint8_t *w1, const float *x, float *y,
                          int64_t rows, int64_t cols, int64_t n_tok, float *part, int64_t part_elems, hipStream_t s,
                          const float *resid, const uint16_t *xb, uint16_t *yb)
{
    Layout L;
    if (!prefill_format(fmt) || !layout_for(fmt, rows, cols, &L) || n_tok < 1 || n_tok >= (int64_t(1) << 31))
        return hipErrorInvalidValue;
    const PrefillCfg c = choose(fmt, nmat, rows, cols, n_tok, part ? part_elems : 0, cu_count());
    PrefillParams p;
    p.q[0] = w0;
    p.q[1] = w1 ? w1 : w0;
    p.x = x;
    p.y = c.ksplit > 1 ? part : y;
    p.rows = rows;
    p.row_qbytes = L.row_qbytes;
    p.soff = L.splane_off;
    p.nb = (int)(cols / 32);
    p.cols = (int)cols;
    p.ssteps = (int)((p.nb + 4 * c.run - 1) / (4 * c.run));
    p.n_tok = (int)n_tok;
    p.row_groups = (rows + c.waves * c.mtr * 16 - 1) / (c.waves * c.mtr * 16);
    p.tok_groups = (int)((n_tok + c.ntw * 16 - 1) / (c.ntw * 16));
    p.ksplit = c.ksplit;
    p.spk = (p.ssteps + c.ksplit - 1) / c.ksplit;
    p.resid = nmat == 1 ? resid : nullptr;
    p.hoff = L.hplane_off;
    p.doff = L.dplane_off;
    p.xb = xb;
    p.yb = nmat == 2 ? yb : nullptr;
    switch (fmt) {
    case QG_Q4_0: return prefill_dispatch_q4_0(c, nmat, p, y, s);
    case QG_Q4_K: return prefill_dispatch_q4_k(c, nmat, p, y, s);
    case QG_Q6_K: return prefill_dispatch_q6_k(c, nmat, p, y, s);
    case QG_Q8_0: return prefill_dispatch_q8_0(c, nmat, p, y, s);
    case QG_I8ROW: return prefill_dispatch_i8row(c, nmat, p, y, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace qg

