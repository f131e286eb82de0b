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

} // namespace

hipError_t launch_argmax(const float *logits, int32_t *token, int64_t n, int64_t n_tok, hipStream_t s)
{
    if (n < 1 || n >= (int64_t(1) << 31) || n_tok < 1 || n_tok >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    if (n % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0)
        hipLaunchKernelGGL(argmax_kernel<4>, dim3((unsigned)n_tok), dim3(kArgmaxThreads), 0, s, logits, token, (int)n);
    else
        hipLaunchKernelGGL(argmax_kernel<1>, dim3((unsigned)n_tok), dim3(kArgmaxThreads), 0, s, logits, token, (int)n);
    return hipGetLastError();
}

} // namespace qg
