// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qgemv.h"

namespace qg {

constexpr int kChunk = 32;           // weights per lane work item (a Q4_0/Q8_0 block, a Q4_K sub-block,
                                     // two Q6_K sub-blocks)
constexpr int kXStride = 36;         // LDS floats per staged x chunk: 32 values + chunk sum + 3 pad
constexpr int64_t kPlaneAlign = 256; // packed plane alignment
constexpr int kLayoutVersion = 1;
// Added to a format code (Q4_0, Q8_0) inside the library: the GEMV quantizes
// its activation row to Q8_0 while staging it and takes integer dot products.
constexpr int kQ8Act = 8;

inline int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Packed layout v1: a quant plane [rows][row_qbytes] followed (at a 256-byte
// boundary) by a scale plane.
//   Q4_0  quant row = cols/2 bytes, 16 B per block, nibble order of the raw
//         block; scale plane f16 [rows][cols/32].
//   Q8_0  quant row = cols bytes (int8, column order); scale plane f16 [rows][cols/32].
//   Q4_K  quant row = cols/2 bytes, 16 B per 32-wide sub-block, re-ordered so
//         byte l holds element l (low nibble) and l+16 (high nibble) of that
//         sub-block; scale plane = the raw 16-byte super-block headers
//         (d, dmin, scales[12]) [rows][cols/256].
//   I8ROW quant row = cols bytes; scale plane fp32 [rows].
//   Q6_K  quant row = cols/2 bytes of low nibbles, 16 B per 32 columns in the
//         Q4_0 nibble order; then a high-bit plane [rows][cols/4] (8 B per 32
//         columns, each 32-bit word holding the top two bits of the codes of
//         two quant words, placed for the kernel's masks); a scale plane of
//         int8 [rows][cols/16]; a d plane of f16 [rows][cols/256].
struct Layout {
    int64_t row_qbytes;   // bytes per row in the quant plane
    int64_t qplane_bytes; // rows * row_qbytes
    int64_t splane_off;   // offset of the scale plane
    int64_t splane_bytes;
    int64_t hplane_off;   // Q6_K: offset of the high-bit plane (0 otherwise)
    int64_t dplane_off;   // Q6_K: offset of the d plane (0 otherwise)
    int64_t total;
};

bool layout_for(int fmt, int64_t rows, int64_t cols, Layout *L);

// Launch configuration of the GEMV kernels.
struct GemvCfg {
    int lpr;    // lanes cooperating on one row (8, 16, 32, 64)
    int r;      // rows per lane group sharing each staged x chunk (1, 2, 4)
    int waves;  // waves per workgroup
    int depth;  // prefetch ring depth per lane (2, 4)
    int max_wg; // cap on workgroups (grid-stride over row batches); 0 = one batch per wave
    int cpl;    // adjacent chunks per lane per pass (1, 2, 4)
};

GemvCfg choose_cfg(int fmt, int64_t rows, int64_t cols, int nmat);

// Measurement hook (qgemv_time_next_launch): true, with the calling thread's
// oldest queued start/stop events, which it dequeues; the launcher then
// launches with them.
bool take_launch_timing(hipEvent_t *start, hipEvent_t *stop);

// Compute units of the current device (cached per device; 256 if the query fails).
int cu_count();

// Optional override of the heuristic (tuning sweeps); lpr == 0 clears it.
extern "C" int qgemv_set_launch_override(int lpr, int r, int waves, int depth, int max_wg, int cpl);
bool launch_override(GemvCfg *c);

// Greedy sampling fused into a one-token product: every workgroup's
// candidate, counters of finished workgroups (a top counter and group
// counters, each on its own 128-byte line; zero before the launch, left zero
// by it) and the token.
// The product's candidates for greedy sampling (EPI 3): one (value bits,
// index) per workgroup, and the number of them, which workgroup 0 stores;
// launch_am_combine then reduces them to the token.
struct ArgmaxOut {
    uint2 *cand;        // max_cand entries
    int64_t max_cand;   // the launch fails if it would take more workgroups
    uint32_t *count;    // the number of candidates (written by the product)
    int64_t *grid_out;  // host memory: the launcher records its number of workgroups there
};
// One wave: the token from the n candidates a product launch wrote (the
// first index of the largest value; 0 if a candidate flags row 0 as NaN).
hipError_t launch_am_combine(const uint2 *cand, int64_t n, int32_t *token, hipStream_t s);

// One-token Q8_0 products with short rows (gemv_rows.hip): a lane per block
// position, rows packed across the lanes.  rows_choose: false when the kernel
// does not take the shape (or the row-streaming kernels are switched off).
struct RowsCfg {
    int threads, rps, nrs, grid, depth;
};
bool rows_choose(int fmt, int64_t rows, int64_t cols, RowsCfg *c);
// resid (may be null) is added to y; am (may be null): greedy sampling fused in.
hipError_t launch_rows(int fmt, const uint8_t *packed, const float *x, float *y, int64_t rows, int64_t cols,
                       const RowsCfg &c, hipStream_t s, const float *resid, const ArgmaxOut *am);
// The row-streaming tuning mode of the calling thread (qgemv_set_xs_override):
// -1 = off, 0 = built-in, 1 = forced shape.
int xs_mode();


// Kernel launchers (enqueue only; arguments already validated).
// resid (may equal y): y = resid + W x.  gamma: the input is RMS-normalized
// with that gain and eps before the gate/up products.  am: also the index of
// the largest y (plain product, no resid).
hipError_t launch_gemv(int fmt, const uint8_t *packed, const float *x, float *y, int64_t rows,
                       int64_t cols, hipStream_t s, const GemvCfg &cfg, const float *resid = nullptr,
                       const ArgmaxOut *am = nullptr);
// zero (row-streaming gate/up only, else an error): nzero floats set to zero
// after the products, for a K-halves down product.
hipError_t launch_gate_up(int fmt, const uint8_t *wg, const uint8_t *wu, const float *x, float *h,
                          int64_t ffn, int64_t d_model, hipStream_t s, const GemvCfg &cfg,
                          const float *gamma = nullptr, float eps = 0.0f, float *zero = nullptr,
                          int64_t nzero = 0);
// Whether the one-token FFN of this shape (norm: with the RMSNorm in) runs
// its down product in K halves: both products on the row-streaming kernel,
// the gate/up launch clearing out (qgemv_set_ffn_khalf of the calling thread;
// off under a launch override).
bool ffn_down_khalf(int fmt, int64_t d_model, int64_t ffn, bool norm = false);
// out [d_model] += Wd h (+ resid, may be null, disjoint from out) over the two
// column halves of Wd, one atomic add each (out holds zeros before: then the
// result does not depend on their order).
hipError_t launch_down_khalf(int fmt, const uint8_t *wd, const float *h, float *out, int64_t d_model, int64_t ffn,
                             hipStream_t s, const float *resid = nullptr);
hipError_t launch_repack(int fmt, const void *raw, const float *row_scale, uint8_t *packed,
                         int64_t rows, int64_t cols, hipStream_t s);
hipError_t launch_dequant(int fmt, const uint8_t *packed, float *w, int64_t rows, int64_t cols,
                          hipStream_t s);

size_t gemv_lds_bytes(int64_t cols);

// Batched-token path on the matrix cores (every format, n_tok > 1).
struct PrefillCfg {
    int mtr;     // 16-row tiles per wave and matrix (1, 2); 0 = built-in choice, -1 = path off
    int ntw;     // 16-token tiles per workgroup (1, 2, 4, 8)
    int waves;   // waves per workgroup (4, 8)
    int run;     // consecutive Q4_0 blocks a lane reads per row and super-step (1, 2, 4)
    int ksplit;  // K ranges per (row group, token group); 0 = built-in choice
};
extern "C" int qgemv_set_prefill_override(int mtr, int ntw, int waves, int run, int ksplit);
bool prefill_enabled();   // false after qgemv_set_prefill_override(-1, ...): per-token GEMV loop instead
PrefillCfg prefill_override();   // the calling thread's tuning override (mtr 0: none)
bool prefill_format(int fmt);   // formats the matrix-core path takes
// Floats of partial sums the built-in choice splits K into (0: no split).
int64_t prefill_part_elems(int fmt, int nmat, int64_t rows, int64_t cols, int64_t n_tok);
// nmat == 1: y = W0 x (+ resid, which may equal y).  nmat == 2: y = silu(W0 x) * (W1 x).
// x fp32 [n_tok][cols].  part (part_elems floats, may be null) lets the K
// dimension split over workgroups; the partial sums are then added in a
// second, small launch.
// xb (may be null): x already rounded to bf16 (nearest even, as the kernel
// rounds it), 16-byte aligned; the kernel then reads it instead of x
// (half the bytes, the same result).  yb (nmat == 2, may be null): y is also
// written there rounded to bf16 (16-byte aligned), the next product's xb.
hipError_t launch_prefill(int fmt, int nmat, const uint8_t *w0, const uint8_t *w1, const float *x, float *y,
                          int64_t rows, int64_t cols, int64_t n_tok, float *part, int64_t part_elems,
                          hipStream_t s, const float *resid = nullptr, const uint16_t *xb = nullptr,
                          uint16_t *yb = nullptr);
// Q8_0 activations with several tokens (q8act_mfma.hip).  First every x row
// is quantized once into a workspace (q8act_x_bytes of it: the blocks' codes
// as binary16 operand slots, then their scales); then the product multiplies
// the codes on the matrix cores.  nmat == 1: y = W0 xq; nmat == 2:
// y = silu(W0 xq) * (W1 xq).  Q4_0 or Q8_0 weights.  part (part_elems
// floats, may be null) lets K split over workgroups, the partial sums added
// by a second launch in range order.
struct Q8mPlan {
    int mtr, ntw, ksplit, spk;
};
Q8mPlan q8act_mfma_plan(int nmat, int64_t rows, int64_t cols, int64_t n_tok, int64_t part_elems);
int64_t q8act_x_bytes(int64_t cols, int64_t n_tok);
hipError_t launch_q8act_quantize(const float *x, uint8_t *ws, int64_t cols, int64_t n_tok, hipStream_t s);
hipError_t launch_q8act_mfma(int fmt, int nmat, const uint8_t *w0, const uint8_t *w1, const uint8_t *xws, float *y,
                             int64_t rows, int64_t cols, int64_t n_tok, float *part, int64_t part_elems,
                             hipStream_t s);
// xb[i] = bf16(x[i]) (nearest even), n % 4 == 0, both 16-byte aligned.
hipError_t launch_to_bf16(const float *x, uint16_t *xb, int64_t n, hipStream_t s);
// Raw Q8_0 blocks (f16 d, 32 int8) of activation rows x [n_tok][n], n a multiple of 32.
hipError_t launch_quantize_q8_0(const float *x, uint8_t *blocks, int64_t n, int64_t n_tok, hipStream_t s);
// token[t] = first index of the largest of logits[t][0..n) (NaN never chosen, unless at index 0).
hipError_t launch_argmax(const float *logits, int32_t *token, int64_t n, int64_t n_tok, hipStream_t s);
// xn[t][j] = x[t][j] * gamma[j] / sqrt(mean_j x[t][j]^2 + eps), fp32, one workgroup per token.
// xnb (may be null): xn also written rounded to bf16 (nearest even).
hipError_t launch_rmsnorm(const float *x, const float *gamma, float eps, float *xn, int64_t n, int64_t n_tok,
                          hipStream_t s, uint16_t *xnb = nullptr);

} // namespace qg
