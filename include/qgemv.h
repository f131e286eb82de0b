/*
 * qgemv: block-quantized matrix-vector product for single-token LLM decode on
 * MI355X (gfx950), with dequantization fused into the dot product, and the
 * SwiGLU feed-forward block built from it.
 *
 * C ABI.  Every pointer argument except `stream` is DEVICE memory owned by the
 * caller; the library allocates nothing and keeps no mutable global state
 * beyond a lazily read per-device property cache.  The tuning and measurement
 * hooks (qgemv_set_launch_override, qgemv_set_xs_override,
 * qgemv_set_prefill_override, qgemv_set_ffn_khalf, qgemv_time_next_launch)
 * keep their setting per calling thread and affect only that thread's later
 * calls.  `stream` is a hipStream_t passed as void*
 * (NULL = the legacy null stream).
 *
 * Errors are returned, never thrown: every entry point validates its arguments
 * synchronously and, on any error, returns a negative qg_status and enqueues
 * nothing.  On success the work is enqueued on `stream` and the call returns
 * immediately; device-side faults surface at the caller's next synchronization.
 * A kernel launch that the runtime rejects returns QG_ERR_LAUNCH.
 * Calls on different streams are independent and thread-safe.
 *
 * Definitions the operations follow (pages cited by title and section):
 *  - y = W x with W stored one row per output: "Running an LLM, then forgetting
 *    it" (the llmoxide blog), section 1 "A neuron is a dot product"; the matmul
 *    of dasLLAMA-00, section 8.7.1.4 "Five small functions".
 *  - Batched tokens: x is [n_tok][cols], y is [n_tok][rows], row-major (llmoxide
 *    blog, section 11 "Prefill and decode").
 *  - Each dot product decodes its row's blocks on the fly (llmoxide blog,
 *    section 10 "Loading weights"; "Building llamini.cpp", section "Optimizing
 *    for CPU, and finding out what was actually true").
 *  - Block formats: Q8_0 (llmoxide blog section 10: f16 scale + 32 int8, 34 B);
 *    Q4_0 (Go "llm" package README, Design points: 18-byte blocks; w=(q-8)*d);
 *    Q4_K (llamini.cpp post, "What I reimplemented": 256-weight super-blocks,
 *    six-bit scale/min pairs unpacked by get_scale_min_k4, 144 B); Q6_K
 *    (llmoxide blog section 10: the other k-quant, 256-weight super-blocks
 *    with their own scales at about 6.6 bits per weight; the llamini.cpp post
 *    names it the second format of a Q4_K_M file; 210 B); per-row symmetric
 *    INT8 (minillm-cpp README, Quantization paragraph: one scale per output
 *    row).  The byte layouts of the raw blocks are spelled out below.
 *  - SwiGLU: gate = Wg x, up = Wu x, h = silu(gate) * up, out = Wd h (llmoxide
 *    blog, section 2 "Layers, and the bend between them"; dasLLAMA-00, section
 *    8.7.1.6.3); no residual add and no normalization inside.
 *  - Load-time repack of raw blocks into aligned planes: Go "llm" package
 *    README, Design points (its Q4_0 blocks become aligned u32 quants and f32
 *    scales; here the f16 scales are kept, so the bytes streamed per weight are
 *    exactly the raw format's).
 *
 * Raw block layouts (little-endian; a tensor is [rows][cols/B] blocks,
 * row-major; block b of a row covers columns [B*b, B*b+B)):
 *   Q4_0  B=32, 18 bytes: f16 d; 16 code bytes, byte l holding column l in its
 *         low nibble and column l+16 in its high nibble; w = (q - 8) * d.
 *   Q8_0  B=32, 34 bytes: f16 d; 32 int8 codes in column order; w = d * q.
 *   Q4_K  B=256, 144 bytes: f16 d; f16 dmin; 12 bytes of six-bit (sc, m)
 *         pairs for the eight 32-wide sub-blocks (get_scale_min_k4 packing);
 *         128 code bytes, byte 32c+l holding element l of sub-block 2c (low
 *         nibble) and of sub-block 2c+1 (high nibble); w = d*sc*q - dmin*m.
 *   Q6_K  B=256, 210 bytes (the GGUF layout of the files the pages load; the
 *         pages give only the size): ql[128], qh[64], 16 int8 scales (one per
 *         16 columns), f16 d.  The 6-bit code of column c = 128h + 32j + l
 *         (h < 2, j < 4, l < 32) has its low four bits in ql[64h + 32(j%2) + l]
 *         (low nibble for j < 2, high nibble for j >= 2) and its top two bits
 *         at bits 2j..2j+1 of qh[32h + l]; w = d * scales[c/16] * (q - 32).
 *   I8ROW int8 codes [rows][cols] plus fp32 scales [rows]; w = s_row * q.
 *
 * Shape rules: rows, cols, n_tok >= 1; cols a multiple of 32 (Q4_0, Q8_0,
 * I8ROW) or of 256 (Q4_K, Q6_K); cols <= qgemv_max_cols(); rows, cols < 2^31.
 * Alignment: packed buffers 256 bytes; x, y, h, out and w_out 16 bytes.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QG_OK = 0,
    QG_ERR_NULL = -1,    /* a required pointer is NULL */
    QG_ERR_SHAPE = -2,   /* rows/cols/n_tok out of range or not a block multiple */
    QG_ERR_ALIGN = -3,   /* a pointer breaks the alignment rule */
    QG_ERR_FORMAT = -4,  /* unknown format code */
    QG_ERR_ALIAS = -5,   /* an output overlaps an input or another output */
    QG_ERR_SCRATCH = -6, /* the caller's scratch buffer is too small */
    QG_ERR_LAUNCH = -7,  /* the HIP runtime rejected a launch */
    QG_ERR_DEVICE = -8   /* no usable HIP device / device query failed */
} qg_status;

typedef enum { QG_Q4_0 = 0, QG_Q8_0 = 1, QG_Q4_K = 2, QG_I8ROW = 3, QG_Q6_K = 4 } qg_format;

/* Version of the packed (repacked) layout; packed buffers are only valid for
 * the library that wrote them. */
int qgemv_layout_version(void);

/* Human-readable text for a qg_status (static storage, never NULL). */
const char *qgemv_status_string(int status);

/* Largest supported cols for the current device (bounded by the LDS that
 * stages one activation row per workgroup), or a negative qg_status. */
int64_t qgemv_max_cols(void);

/* Bytes of the packed buffer for a [rows][cols] tensor of format fmt, or a
 * negative qg_status if the shape or format is invalid.  The packed buffer
 * holds exactly the raw format's bytes (quant plane + scale plane; Q6_K:
 * low-nibble, high-bit, scale and d planes), plus padding to 256-byte plane
 * boundaries. */
int64_t qgemv_packed_bytes(int fmt, int64_t rows, int64_t cols);

/* Load-time repack: raw blocks (device, layout above) -> packed planes
 * (device, qgemv_packed_bytes bytes, 256-byte aligned).  raw must not
 * overlap packed.  For I8ROW, q is the int8 code matrix and row_scale the fp32
 * per-row scales. */
int qgemv_repack_q4_0(const void *raw, void *packed, int64_t rows, int64_t cols, void *stream);
int qgemv_repack_q8_0(const void *raw, void *packed, int64_t rows, int64_t cols, void *stream);
int qgemv_repack_q4_k(const void *raw, void *packed, int64_t rows, int64_t cols, void *stream);
int qgemv_repack_q6_k(const void *raw, void *packed, int64_t rows, int64_t cols, void *stream);
int qgemv_repack_i8row(const int8_t *q, const float *row_scale, void *packed, int64_t rows,
                       int64_t cols, void *stream);

/* y[t][i] = sum_j Wdeq[i][j] * x[t][j] for t < n_tok, i < rows.
 * packed: made by the matching qgemv_repack_*; x: fp32 [n_tok][cols];
 * y: fp32 [n_tok][rows], overwritten.  x must not overlap y.
 * n_tok == 1 runs the fused dequant-dot GEMV kernels: exact weights, fp32 x,
 * fp32 accumulation.  n_tok > 1:
 *  every format runs on the matrix cores (llmoxide blog, section 11 "Prefill
 *  and decode": with several tokens the product is a real GEMM, each weight
 *  tile dequantized once for all tokens).  Weights and x are rounded to bf16
 *  (nearest even; per-row INT8 codes are exact in bf16 and their row scale
 *  multiplies the fp32 sums) and multiplied by v_mfma_f32_16x16x32_bf16 with
 *  fp32 accumulation: |y - exact| <= 8e-3 * sum_j |w_ij x_tj| + 1e-7.  One
 *  launch, no workspace.  qgemv_set_prefill_override(-1, ...) turns this off:
 *  the GEMV then loops over the tokens (fp32 accuracy). */
int qgemv_q4_0(const void *packed, const float *x, float *y, int64_t rows, int64_t cols,
               int64_t n_tok, void *stream);
int qgemv_q8_0(const void *packed, const float *x, float *y, int64_t rows, int64_t cols,
               int64_t n_tok, void *stream);
int qgemv_q4_k(const void *packed, const float *x, float *y, int64_t rows, int64_t cols,
               int64_t n_tok, void *stream);
int qgemv_i8row(const void *packed, const float *x, float *y, int64_t rows, int64_t cols,
                int64_t n_tok, void *stream);
int qgemv_q6_k(const void *packed, const float *x, float *y, int64_t rows, int64_t cols,
               int64_t n_tok, void *stream);

/* Format-generic form of the five calls above. */
int qgemv(int fmt, const void *packed, const float *x, float *y, int64_t rows, int64_t cols,
          int64_t n_tok, void *stream);

/* First half of the SwiGLU block: h[t][i] = silu(Wg x)[t][i] * (Wu x)[t][i],
 * silu(g) = g / (1 + exp(-g)).  wg, wu: packed [ffn][d_model] of format fmt;
 * x: fp32 [n_tok][d_model]; h: fp32 [n_tok][ffn], overwritten, must not
 * overlap x.  With n_tok > 1 the products run on the matrix cores as qgemv's
 * do, with silu(g) * u applied in the same kernel. */
int swiglu_gate_up(int fmt, const void *wg, const void *wu, const float *x, float *h,
                   int64_t d_model, int64_t ffn, int64_t n_tok, void *stream);

/* Whole SwiGLU block: out = Wd (silu(Wg x) * (Wu x)).
 * wd: packed [d_model][ffn]; x: fp32 [n_tok][d_model]; out: fp32
 * [n_tok][d_model], overwritten; h_scratch: caller-owned fp32 scratch of
 * h_scratch_elems >= n_tok*ffn elements, whose first n_tok*ffn elements hold
 * h ([n_tok][ffn]) on return (so the caller can inspect the intermediate).
 * On the matrix-core path (n_tok > 1) a scratch of
 * swiglu_ffn_scratch_elems() elements (16-byte aligned) also holds the partial
 * sums that let both products split their K dimension over more workgroups
 * (deterministic: fixed summation order) and, from 8 tokens on with
 * d_model * ffn >= 2^24, bf16 copies of x and h (rounded to nearest even as the matrix cores take them, so the
 * results are bit-identical; the products then read half the bytes of x and
 * h, for one short conversion launch each); with less, the products run
 * unsplit and on fp32 x and h, with the same accuracy bound.  One token, Q4_0
 * with ffn >= 8192: the down product runs in K halves (qgemv_set_ffn_khalf),
 * out cleared by the gate/up launch and each output the sum of its two
 * half-rows, added atomically (deterministic: two additions onto zero
 * commute).  x, out and the whole declared
 * scratch must be pairwise disjoint.  Two launches on `stream` for n_tok == 1,
 * up to six on the matrix-core path, else two per token; no host
 * synchronization. */
int swiglu_ffn(int fmt, const void *wg, const void *wu, const void *wd, const float *x,
               float *out, float *h_scratch, int64_t h_scratch_elems, int64_t d_model,
               int64_t ffn, int64_t n_tok, void *stream);

/* swiglu_ffn for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same products and results as swiglu_ffn given min(swiglu_ffn_scratch_elems(),
 * QG_NOALLOC_SCRATCH_ELEMS) floats of scratch, with that scratch in an array
 * of QG_NOALLOC_SCRATCH_ELEMS floats (32 MiB) that the library keeps on each
 * device it runs on until the process ends; the call itself allocates
 * nothing.  Arguments as swiglu_ffn without the scratch (h is not returned).
 * QG_ERR_SCRATCH when n_tok * ffn > QG_NOALLOC_SCRATCH_ELEMS; QG_ERR_DEVICE if
 * the array's device address cannot be found.  Every call on one device uses
 * the same array: calls that overlap in time on one device (other streams,
 * other threads) race and must be serialized by the caller. */
#define QG_NOALLOC_SCRATCH_ELEMS (1 << 23)
int swiglu_ffn_noalloc(int fmt, const void *wg, const void *wu, const void *wd, const float *x, float *out,
                       int64_t d_model, int64_t ffn, int64_t n_tok, void *stream);

/* The FFN block of the residual stream: out = x + Wd (silu(Wg xn) * (Wu xn)),
 * xn = x * gamma / sqrt(mean(x^2) + eps) per token row -- RMSNorm before the
 * block (llmoxide blog, section 4 "Keeping the numbers in range"; the rmsnorm
 * of dasLLAMA-00, which uses eps = 1e-5) and the residual add after it (same
 * blog, section 7 "The block, and the residual stream").
 * gamma: fp32 [d_model] (16-byte aligned); eps >= 0 and finite; x, out: fp32
 * [n_tok][d_model]; out may be x itself (the stream updated in place) or must
 * not overlap it.  h_scratch: >= swiglu_ffn_block_scratch_elems() floats
 * (QG_ERR_SCRATCH below the minimum that query's comment states), first
 * n_tok*ffn of them hold h on return.  With n_tok == 1, or with the
 * matrix-core path turned off, the norm is fused into the gate/up GEMV (the per-token scale factors
 * out of every dot product; the workgroup sums x^2 while staging x*gamma) and
 * the residual into the down GEMV's epilogue: two launches per token.  Out of
 * place (out != x), Q4_0 with ffn >= 8192: the down product runs in K halves
 * as in swiglu_ffn, the first half adding the residual with its half-row sums
 * (deterministic); in place, on whole rows.  With
 * n_tok > 1 the matrix-core path runs a small RMSNorm launch into the scratch, then the
 * matrix-core products (residual added in the down product's epilogue or in
 * its split-K reduce). */
int swiglu_ffn_block(int fmt, const void *wg, const void *wu, const void *wd, const float *gamma,
                     float eps, const float *x, float *out, float *h_scratch, int64_t h_scratch_elems,
                     int64_t d_model, int64_t ffn, int64_t n_tok, void *stream);

/* Scratch elements (fp32) for which swiglu_ffn_block runs its fastest form:
 * n_tok*ffn on the GEMV path; on the matrix-core path (n_tok > 1) h,
 * the normalized input (required: together the minimum), room for split-K
 * partial sums and, from 8 tokens on with d_model * ffn >= 2^24, bf16 copies
 * of the normalized input and h as swiglu_ffn keeps them (both optional; the
 * results are bit-identical with or without the copies).  Negative qg_status for an invalid shape
 * or format. */
int64_t swiglu_ffn_block_scratch_elems(int fmt, int64_t d_model, int64_t ffn, int64_t n_tok);

/* Scratch elements (fp32) for which swiglu_ffn runs its fastest form on the
 * current device: n_tok*ffn, plus room for partial sums on the matrix-core
 * path.  Negative qg_status for an invalid shape or format. */
int64_t swiglu_ffn_scratch_elems(int fmt, int64_t d_model, int64_t ffn, int64_t n_tok);

/* Greedy sampling on the device: token[t] = index of the largest of
 * logits[t][0..n), the first on ties (the Go "llm" package's Argmax;
 * dasLLAMA-00's most_likely moves only on a strictly greater logit, so -0
 * equals +0, a NaN is never chosen, and a NaN at index 0 keeps index 0).
 * logits: fp32 [n_tok][n]; token: int32 [n_tok].  One launch, deterministic. */
int qgemv_argmax(const float *logits, int32_t *token, int64_t n, int64_t n_tok, void *stream);

/* The vocab head then greedy sampling (llmoxide blog section 7: the output
 * head is one more matrix multiply; Go "llm" package: sampling runs on the
 * GPU and only the 4-byte token is read back): logits = W x as qgemv (the
 * same paths and bounds), then qgemv_argmax over each token's logits.
 * logits: fp32 [n_tok][rows] (kept for the caller); token: int32 [n_tok]. */
int qgemv_head_argmax(int fmt, const void *packed, const float *x, float *logits, int32_t *token,
                      int64_t rows, int64_t cols, int64_t n_tok, void *stream);

/* The same head with the argmax fused into the product (Go "llm" package,
 * Design points: greedy sampling on the GPU, the token the only readback;
 * func Argmax: the first index of the largest logit): for n_tok == 1 the
 * product's workgroups each reduce the rows they wrote to one (value, index)
 * candidate in the workspace (workgroup 0 also writes their number), and a
 * one-workgroup launch combines the candidates into the token, by the rule
 * of qgemv_argmax (first index on ties, NaN never chosen unless logits[0] is
 * NaN, then 0): two launches, the second reading 8 bytes per workgroup
 * instead of the logits.  logits are written as by qgemv.  For n_tok > 1 the
 * call is qgemv_head_argmax (workspace unused).  workspace (device, 16-byte
 * aligned, caller-owned, no initialization needed): at least
 * qgemv_head_argmax_workspace_bytes bytes.  Calls that share a workspace
 * must not overlap (order them on one stream).
 * Errors as qgemv, plus QG_ERR_NULL (token, workspace), QG_ERR_ALIGN,
 * QG_ERR_SCRATCH (workspace too small) and QG_ERR_ALIAS (token or workspace
 * overlapping each other or an input). */
int qgemv_head_argmax_ws(int fmt, const void *packed, const float *x, float *logits, int32_t *token,
                         int64_t rows, int64_t cols, int64_t n_tok, void *workspace, int64_t workspace_bytes,
                         void *stream);
/* Bytes of workspace qgemv_head_argmax_ws needs for a head of this shape
 * (a 256-byte header, then 8 * rows of candidates, the same layout for
 * every shape, so one workspace of the largest size serves several heads;
 * host only), or QG_ERR_FORMAT / QG_ERR_SHAPE. */
int64_t qgemv_head_argmax_workspace_bytes(int fmt, int64_t rows, int64_t cols);

/* Q8_0 activations: the products as the Go "llm" package's ExactGGML mode
 * computes them (its CPU type: activations are quantised to Q8_0 before every
 * quantised matrix product).  Each 32-element block of the activation row is
 * quantized -- d = max|x|/127, q = round(x * (1/d)) with halves away from
 * zero (q = 0 when d = 0), binary32 with correctly rounded divisions, d kept
 * as binary16 nearest even -- and y is the product with x replaced by
 * f16(d) * q: per block an exact integer dot product (Q4_0 codes minus 8, or
 * Q8_0 codes, times the activation codes) scaled by d_w * d_x, accumulated in
 * fp32 (|y - exact| <= 2e-5 * sum_j |w_ij xq_j| + 1e-7 for xq the quantized
 * activations).  Q4_0 and Q8_0 weights only (QG_ERR_FORMAT otherwise); same
 * arguments, layouts and checks as qgemv and swiglu_ffn.  swiglu_ffn_q8act
 * quantizes x before the gate/up pair and h before the down product (h,
 * fp32, is left in the scratch as in swiglu_ffn).  qgemv_q8act: one launch
 * per token.  swiglu_ffn_q8act: with n_tok * ffn floats of scratch, two
 * launches per token (Q4_0 with ffn >= 8192: the down product in K halves,
 * as in swiglu_ffn); with n_tok > 1 and at least
 * swiglu_ffn_q8act_scratch_elems() floats, the batched path of
 * qgemv_q8act_ws for both products (the quantized activations, then any
 * partial sums, live in the scratch behind h, which starts the scratch
 * aligned up to 64 floats); between the two, the batched path without a K
 * split when the quantized activations fit. */
int qgemv_q8act(int fmt, const void *packed, const float *x, float *y, int64_t rows, int64_t cols,
                int64_t n_tok, void *stream);
int swiglu_ffn_q8act(int fmt, const void *wg, const void *wu, const void *wd, const float *x,
                     float *out, float *h_scratch, int64_t h_scratch_elems, int64_t d_model,
                     int64_t ffn, int64_t n_tok, void *stream);
/* Floats of scratch for the batched path of swiglu_ffn_q8act (n_tok * ffn
 * when n_tok == 1), or a negative status (QG_ERR_FORMAT, QG_ERR_SHAPE). */
int64_t swiglu_ffn_q8act_scratch_elems(int fmt, int64_t d_model, int64_t ffn, int64_t n_tok);

/* The same product for several tokens in a fixed number of launches (the
 * Go "llm" package's ExactGGML mode quantizes the prompt's activations too):
 * one launch quantizes every token's blocks into `workspace` (device,
 * 256-byte aligned, not overlapping packed, x or y), one multiplies on the
 * matrix cores -- the 32-term block sums of 16 rows by 16 tokens as one
 * binary16 matrix-core product of the codes (small integers: exact products
 * and sums in fp32), each scaled by d_w * d_x and added in fp32, the bound
 * above unchanged -- and, when the workspace also holds partial sums of a K
 * split, a third adds them in a fixed order (deterministic).  workspace_bytes
 * >= qgemv_q8act_workspace_bytes() allows the built-in K split; less (down to
 * the quantized activations alone) narrows it; less than that: QG_ERR_SCRATCH
 * (QG_ERR_NULL without a workspace).  n_tok == 1, or the matrix-core path
 * turned off by qgemv_set_prefill_override(-1, ...): qgemv_q8act, the
 * workspace unused.  The workspace's contents are scratch (nothing carries
 * over between calls).  Calls that share a workspace must not overlap. */
int qgemv_q8act_ws(int fmt, const void *packed, const float *x, float *y, int64_t rows, int64_t cols,
                   int64_t n_tok, void *workspace, int64_t workspace_bytes, void *stream);
/* Bytes of workspace for qgemv_q8act_ws with the built-in K split (0 when
 * n_tok == 1), or a negative status (QG_ERR_FORMAT, QG_ERR_SHAPE). */
int64_t qgemv_q8act_workspace_bytes(int fmt, int64_t rows, int64_t cols, int64_t n_tok);

/* Test export: the activation quantizer above on its own.  x: fp32
 * [n_tok][n] (16-byte aligned), n a multiple of 32; blocks: n_tok * n/32 raw
 * Q8_0 blocks of 34 bytes (f16 d, then 32 int8 codes in column order), any
 * alignment, not overlapping x.  Not used on the hot path. */
int qquantize_q8_0(const float *x, void *blocks, int64_t n, int64_t n_tok, void *stream);

/* Test export: the packed tensor decoded to fp32 [rows][cols] (each weight its
 * exact value rounded once to binary32).  Not used on the hot path. */
int qdequant(int fmt, const void *packed, float *w_out, int64_t rows, int64_t cols, void *stream);

/* Tuning hook for launch-shape sweeps: force the GEMV kernels' lanes per row
 * (8, 16, 32 or 64), rows per lane group (1 or 2), waves per workgroup (1..8),
 * prefetch depth per lane (2 or 4), a cap on the number of workgroups (0 =
 * none; with a cap, workgroups loop over row batches) and adjacent 32-weight
 * chunks per lane per pass (1, 2 or 4) for the calling thread's subsequent
 * calls; lpr == 0 restores the built-in choice.  Results depend on the shape only
 * through summation order (every choice stays within the fp32 bound).
 * Per calling thread: it applies to that thread's later calls only.  Returns
 * QG_ERR_SHAPE for values outside these sets. */
int qgemv_set_launch_override(int lpr, int r, int waves, int depth, int max_wg, int cpl);

/* Tuning hook for the one-token products of Q4_0 matrices whose rows have at
 * most 1024 blocks: by default these run on a row-streaming kernel in which
 * each lane keeps one block's activations in registers and streams that
 * block of consecutive rows.  (Q8_0 matrices whose rows have at most 64
 * blocks run on a row-packed kernel: one lane per block position, the rows
 * laid across the lanes without gaps.)  mode -1 keeps both on the lane-group
 * kernels (also the effect of any qgemv_set_launch_override shape); mode 1
 * forces the
 * row-streaming kernel's rows per row-step (rs 1, 2, 4 or 8), 32-lane
 * segments per row (seg: 32 * seg >= blocks per row, rs * seg even,
 * rs * seg / 2 <= 16 waves), row-steps in flight per lane (depth 2 or 4; 8
 * for a single matrix), row-steps per workgroup (nrs >= 1), the order in
 * which row-steps are dealt to workgroups (order 1: round robin, 0:
 * consecutive, -1: built-in) and wg_per_cu (1..8: exactly that many
 * workgroups per CU, nrs following, and no more resident per CU; 0: off; -1:
 * built-in); a 0 field keeps the built-in value, and a combination outside
 * these rules falls back to the lane-group kernels (the row-packed Q8_0
 * kernel takes depth 2, 4 or 8, nrs and wg_per_cu from the same fields, and
 * falls back when its row-steps would not fit 64 KB of LDS).  mode 0
 * restores the built-in choice.  Results depend on the choice only through summation
 * order.  Per calling thread.  Returns QG_ERR_SHAPE for other modes or
 * fields out of range. */
int qgemv_set_xs_override(int mode, int rs, int seg, int depth, int nrs, int order, int wg_per_cu);

/* Tuning hook for the one-token SwiGLU block (swiglu_ffn, swiglu_ffn_noalloc,
 * swiglu_ffn_q8act and swiglu_ffn_block out of place, with n_tok == 1 or any
 * n_tok on the per-token loop) of Q4_0 matrices whose
 * products both run on the row-streaming kernel: its down product can run in
 * K halves -- each workgroup takes one half of the columns of its rows,
 * staging half of h, and adds its half-row sums into out with an atomic add,
 * after the gate/up launch has set out to zero.  Each output then receives
 * exactly two additions onto an exact zero, so it does not depend on their
 * order (runs are bit-identical); the summation order differs from the whole-row
 * product's.  mode 0: built in (from ffn >= 8192 on); 1: off; 2: on wherever
 * the kernel takes the shape (any ffn >= 64).  Off under
 * qgemv_set_launch_override; qgemv_set_xs_override's fields apply to both
 * forms.  Per calling thread.  Returns QG_ERR_SHAPE for other modes. */
int qgemv_set_ffn_khalf(int mode);

/* Measurement export (not the hot path): read `bytes` of device memory at
 * `buf` (16-byte aligned, a multiple of 16) as 16-byte words with a plain
 * grid-stride kernel -- wg_per_cu (1..64) workgroups of 256 threads per CU,
 * `unroll` (2, 4 or 8) loads in flight per thread -- so that bytes / its
 * device time is the streaming-read rate the products' weight streams are
 * compared against (the llmoxide blog, section 11, measures its decode
 * against a kernel that only reads the bytes).  `out` (device, 4-byte
 * aligned, cu_count * wg_per_cu words) is written only if the XOR of all the
 * words read hits one fixed value.  One launch. */
int qgemv_read_probe(const void *buf, int64_t bytes, int wg_per_cu, int unroll, uint32_t *out, void *stream);

/* Measurement hook: the next product kernel that the calling thread
 * launches (a GEMV kernel of any call, or a matrix-core product with its
 * split-K reduce) is launched with hipExtLaunchKernel and these two events
 * (hipEvent_t passed as void*), which then hold that dispatch's own start and
 * end (a matrix-core product: the start of its main kernel, the end of its
 * reduce when K is split): hipEventElapsedTime gives the device time with no
 * marker packets between launches (a hipEventRecord pair costs a pipeline
 * drain of a few microseconds on each side).  Each call queues one pair, up
 * to 4, for the thread's next product launches in order (a swiglu_ffn call
 * with two pairs queued: its gate/up kernel, then its down kernel); each
 * pair is consumed by one product.  Both events or neither (NULL, NULL clears
 * the queue); thread-local.  Returns QG_ERR_NULL if only one event is given,
 * QG_ERR_SHAPE when 4 pairs are already queued. */
int qgemv_time_next_launch(void *start_event, void *stop_event);

/* Tuning hook for the matrix-core path (n_tok > 1): force 16-row tiles
 * per wave and matrix (mtr 1 or 2), 16-token tiles per workgroup (ntw 1, 2, 4
 * or 8), waves per workgroup (4, 8 or 16), consecutive 32-weight blocks a lane
 * reads from a row per pass (run 1, 2 or 4) and the number of K ranges
 * (ksplit 1..64, 0 = built-in; honoured as far as the caller's scratch holds
 * the partial sums, and never more than the passes over K).  A shape the
 * library does not build (it would spill registers or overflow the LDS) runs
 * as the nearest built one.  mtr == 0 restores the built-in choice; mtr == -1
 * turns the matrix-core path off, so that n_tok > 1 loops the GEMV over the
 * tokens (fp32 accuracy), for comparisons.  The batched Q8_0-activation
 * products (qgemv_q8act_ws, swiglu_ffn_q8act) take mtr, ntw (8 as 4) and
 * ksplit from it, and loop over the tokens after mtr == -1.  Per calling
 * thread, as qgemv_set_launch_override.  Returns QG_ERR_SHAPE for other
 * values. */
int qgemv_set_prefill_override(int mtr, int ntw, int waves, int run, int ksplit);

/* The tile and K split the matrix-core path picks for one product (tuning and
 * tests; host only, no device call): nmat 1 (a qgemv product, or the down
 * product) or 2 (the gate/up pair); n_tok >= 2; part_elems the floats of
 * room for partial sums the call gives (0 for qgemv and swiglu_gate_up; the
 * partial-sum share of the swiglu_ffn scratch otherwise); cus the compute
 * units to plan for (256 on MI355X).  plan (5 ints, caller-owned) receives
 * the 16-row tiles per wave and matrix, 16-token tiles per workgroup, waves
 * per workgroup, 32-weight blocks a lane reads per row and pass, and K
 * ranges, as the product would launch them (the current
 * qgemv_set_prefill_override applies).  Returns QG_OK, QG_ERR_NULL (plan),
 * QG_ERR_FORMAT or QG_ERR_SHAPE; plan is untouched on an error. */
int qgemv_prefill_plan(int fmt, int nmat, int64_t rows, int64_t cols, int64_t n_tok, int64_t part_elems,
                       int cus, int *plan);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
