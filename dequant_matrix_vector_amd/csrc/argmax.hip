// Greedy sampling on the GPU: the index of the largest logit of each token
// row, the first one on ties (the Go "llm" package's Argmax; dasLLAMA-00's
// most_likely scans in order and moves only on a strictly greater logit), so
// that only 4 bytes per token leave the device instead of the logits.
//
// The in-order scan's result has a closed description that any order of
// comparisons reaches: if element 0 is NaN the answer is 0 (nothing compares
// greater than it); otherwise NaN elements never win, and the answer is the
// smallest index whose value equals the maximum of the others (-0 equal to
// +0).  So each thread scans a strided slice keeping (value, index) under the
// rule "greater value, or equal value and smaller index", and the slices
// combine by the same rule through a fixed xor-shuffle tree and the waves'
// results in order: deterministic, no atomics.
#include "qg_internal.h"

namespace qg {

namespace {

constexpr int kArgmaxThreads = 1024;
constexpr int kArgmaxUnroll = 16;   // independent float4 loads in flight per thread: 64K logits per round trip

__device__ __forceinline__ void take_better(float &bv, int &bi, float v, int i)
{
    // NaN v: both comparisons false, never taken
    if (v > bv || (v == bv && i < bi)) {
        bv = v;
        bi = i;
    }
}

// V = 4: rows of whole 16-byte pieces (n % 4 == 0, 16-byte aligned); V = 1: any n
template <int V>
__global__ __launch_bounds__(kArgmaxThreads) void argmax_kernel(const float *__restrict__ logits,
                                                                int32_t *__restrict__ token, int n)
{
    typedef float fv __attribute__((ext_vector_type(V)));
    __shared__ float wv[kArgmaxThreads / 64];
    __shared__ int wi[kArgmaxThreads / 64];
    const float *row = logits + (int64_t)blockIdx.x * n;
    const fv *rv = reinterpret_cast<const fv *>(row);
    const int nv = n / V;
    float bv = -__builtin_inff();
    int bi = 0x7FFFFFFF;   // loses to every element, -inf included
    // piece p = base + k * threads + tid: all kArgmaxUnroll loads issued before any compare
    constexpr int STEP = kArgmaxThreads * kArgmaxUnroll;
    for (int base = 0; base < nv; base += STEP) {
        fv v[kArgmaxUnroll];
#pragma unroll
        for (int k = 0; k < kArgmaxUnroll; k++) {
            const int pc = base + k * kArgmaxThreads + (int)threadIdx.x;
            v[k] = rv[pc < nv ? pc : nv - 1];
        }
#pragma unroll
        for (int k = 0; k < kArgmaxUnroll; k++) {
            const int pc = base + k * kArgmaxThreads + (int)threadIdx.x;
            if (pc < nv) {
#pragma unroll
                for (int e = 0; e < V; e++) take_better(bv, bi, v[k][e], pc * V + e);
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        take_better(bv, bi, ov, oi);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        wv[wave] = bv;
        wi[wave] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float v = wv[0];
        int i = wi[0];
#pragma unroll
        for (int w = 1; w < kArgmaxThreads / 64; w++) take_better(v, i, wv[w], wi[w]);
        const float first = row[0];
        token[blockIdx.x] = (first != first) ? 0 : i;   // a NaN at index 0 is never replaced
    }
}

// Rows of whole 16-byte pieces that fit U pieces per thread (n % 4 == 0,
// 16-byte aligned, n <= 4096 U): all loads in one round trip, values kept in
// registers.  First the maximum M of the non-NaN values (fmaxf drops NaN;
// -0 and +0 compare equal below, whichever fmaxf returns), agreed by the
// whole workgroup; then the threads holding M scan their values in index
// order for the first equal one, and the smallest such index wins.  The
// result is the closed description above, with a few VALU operations per
// element instead of a (value, index) update.
template <int U>
__global__ __launch_bounds__(kArgmaxThreads) void argmax4_kernel(const float *__restrict__ logits,
                                                                 int32_t *__restrict__ token, int n)
{
    __shared__ float wmax[kArgmaxThreads / 64];
    __shared__ int widx[kArgmaxThreads / 64];
    const float *row = logits + (int64_t)blockIdx.x * n;
    const float4 *rv = reinterpret_cast<const float4 *>(row);
    const int nv = n / 4;
    float4 v[U];
#pragma unroll
    for (int k = 0; k < U; k++) {
        const int pc = k * kArgmaxThreads + (int)threadIdx.x;
        v[k] = rv[pc < nv ? pc : nv - 1];
    }
    float tm = -__builtin_inff();   // this thread's maximum
#pragma unroll
    for (int k = 0; k < U; k++) {
        const float m4 = fmaxf(fmaxf(v[k].x, v[k].y), fmaxf(v[k].z, v[k].w));
        tm = fmaxf(tm, k * kArgmaxThreads + (int)threadIdx.x < nv ? m4 : -__builtin_inff());
    }
    float m = tm;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) wmax[wave] = m;
    __syncthreads();
    float M = wmax[0];
#pragma unroll
    for (int w = 1; w < kArgmaxThreads / 64; w++) M = fmaxf(M, wmax[w]);
    int bi = 0x7FFFFFFF;
    if (tm == M) {   // the few threads holding the maximum
#pragma unroll
        for (int k = U - 1; k >= 0; k--) {   // downwards: the last match written is the first index
            const int pc = k * kArgmaxThreads + (int)threadIdx.x;
            if (pc < nv) {
                if (v[k].w == M) bi = pc * 4 + 3;
                if (v[k].z == M) bi = pc * 4 + 2;
                if (v[k].y == M) bi = pc * 4 + 1;
                if (v[k].x == M) bi = pc * 4;
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) bi = min(bi, __shfl_xor(bi, off, 64));
    if ((threadIdx.x & 63) == 0) widx[wave] = bi;
    __syncthreads();
    if (threadIdx.x == 0) {
        int i = widx[0];
#pragma unroll
        for (int w = 1; w < kArgmaxThreads / 64; w++) i = min(i, widx[w]);
        const float first = row[0];
        token[blockIdx.x] = (first != first) ? 0 : i;   // a NaN at index 0 is never replaced
    }
}

// The token from a product's workgroup candidates (the fused head), in one
// wave: each lane scans a strided slice of the n (value bits, index) pairs
// under the same rule, an index of 0xFFFFFFFF flagging a NaN at row 0 (then
// the token is 0); the lanes combine through the xor tree.  n comes from the
// host, so all of a lane's loads go out at once.
constexpr int kCombineUnroll = 8;

__global__ __launch_bounds__(64) void am_combine_kernel(const uint2 *__restrict__ cand, int n,
                                                        int32_t *__restrict__ token)
{
    float bv = -__builtin_inff();
    int bi = 0x7FFFFFFF;
    int nan0 = 0;
    for (int base = 0; base < n; base += 64 * kCombineUnroll) {
        uint2 c[kCombineUnroll];
#pragma unroll
        for (int k = 0; k < kCombineUnroll; k++) {
            const int j = base + k * 64 + (int)threadIdx.x;
            c[k] = cand[j < n ? j : n - 1];
        }
#pragma unroll
        for (int k = 0; k < kCombineUnroll; k++) {
            if (base + k * 64 + (int)threadIdx.x < n) {
                if (c[k].y == 0xFFFFFFFFu) nan0 = 1;
                else take_better(bv, bi, __builtin_bit_cast(float, c[k].x), (int)c[k].y);
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        nan0 |= __shfl_xor(nan0, off, 64);
        take_better(bv, bi, ov, oi);
    }
    if (threadIdx.x == 0) *token = nan0 ? 0 : bi;
}

} // namespace

hipError_t launch_am_combine(const uint2 *cand, int64_t n, int32_t *token, hipStream_t s)
{
    if (n < 1 || n >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(am_combine_kernel, dim3(1), dim3(64), 0, s, cand, (int)n, token);
    return hipGetLastError();
}

hipError_t launch_argmax(const float *logits, int32_t *token, int64_t n, int64_t n_tok, hipStream_t s)
{
    if (n < 1 || n >= (int64_t(1) << 31) || n_tok < 1 || n_tok >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    const bool v4 = n % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
    const int64_t per = (n / 4 + kArgmaxThreads - 1) / kArgmaxThreads;   // pieces per thread
    const dim3 grid((unsigned)n_tok), block(kArgmaxThreads);
    if (v4 && per <= 1)
        hipLaunchKernelGGL(argmax4_kernel<1>, grid, block, 0, s, logits, token, (int)n);
    else if (v4 && per <= 2)
        hipLaunchKernelGGL(argmax4_kernel<2>, grid, block, 0, s, logits, token, (int)n);
    else if (v4 && per <= 4)
        hipLaunchKernelGGL(argmax4_kernel<4>, grid, block, 0, s, logits, token, (int)n);
    else if (v4 && per <= 8)
        hipLaunchKernelGGL(argmax4_kernel<8>, grid, block, 0, s, logits, token, (int)n);
    else if (v4 && per <= 12)
        hipLaunchKernelGGL(argmax4_kernel<12>, grid, block, 0, s, logits, token, (int)n);
    else if (v4 && per <= 16)
        hipLaunchKernelGGL(argmax4_kernel<16>, grid, block, 0, s, logits, token, (int)n);
    else if (v4)
        hipLaunchKernelGGL(argmax_kernel<4>, dim3((unsigned)n_tok), dim3(kArgmaxThreads), 0, s, logits, token, (int)n);
    else
        hipLaunchKernelGGL(argmax_kernel<1>, dim3((unsigned)n_tok), dim3(kArgmaxThreads), 0, s, logits, token, (int)n);
    return hipGetLastError();
}

} // namespace qg
