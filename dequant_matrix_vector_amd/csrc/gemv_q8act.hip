// GEMV kernel instantiations with Q8_0 activations (Q4_0 and Q8_0 weights;
// see gemv_impl.h and q8act.h), and the test export of the activation
// quantizer itself.
#include "gemv_impl.h"

namespace qg {

template <>
hipError_t gemv_dispatch<QG_Q4_0 | kQ8Act, 1, 0>(const gemv_detail::GemvParams &p, const GemvCfg &c, hipStream_t s)
{
    return gemv_detail::dispatch<QG_Q4_0 | kQ8Act, 1, gemv_detail::kEpiPlain>(p, c, s);
}

template <>
hipError_t gemv_dispatch<QG_Q4_0 | kQ8Act, 2, 0>(const gemv_detail::GemvParams &p, const GemvCfg &c, hipStream_t s)
{
    return gemv_detail::dispatch<QG_Q4_0 | kQ8Act, 2, gemv_detail::kEpiPlain>(p, c, s);
}

template <>
hipError_t gemv_dispatch<QG_Q8_0 | kQ8Act, 1, 0>(const gemv_detail::GemvParams &p, const GemvCfg &c, hipStream_t s)
{
    return gemv_detail::dispatch<QG_Q8_0 | kQ8Act, 1, gemv_detail::kEpiPlain>(p, c, s);
}

template <>
hipError_t gemv_dispatch<QG_Q8_0 | kQ8Act, 2, 0>(const gemv_detail::GemvParams &p, const GemvCfg &c, hipStream_t s)
{
    return gemv_detail::dispatch<QG_Q8_0 | kQ8Act, 2, gemv_detail::kEpiPlain>(p, c, s);
}

namespace {

// One thread per 32-element block: the same quantizer the GEMV staging runs,
// written out as a raw Q8_0 block (f16 d, then 32 int8 codes).
__global__ void quantize_q8_0_kernel(const float *__restrict__ x, uint8_t *__restrict__ blocks, int64_t nblocks)
{
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblocks) return;
    const float4 *src = reinterpret_cast<const float4 *>(x + b * 32);
    float4 v[8];
#pragma unroll
    for (int k = 0; k < 8; k++) v[k] = src[k];
    Q8Chunk qc;
    quantize_chunk_q8_0(v, qc);
    uint8_t *o = blocks + b * 34;
    o[0] = (uint8_t)(qc.d_bits & 0xFFu);
    o[1] = (uint8_t)(qc.d_bits >> 8);
#pragma unroll
    for (int k = 0; k < 8; k++) {
#pragma unroll
        for (int i = 0; i < 4; i++) o[2 + 4 * k + i] = (uint8_t)(qc.q[k] >> (8 * i));
    }
}

} // namespace

hipError_t launch_quantize_q8_0(const float *x, uint8_t *blocks, int64_t n, int64_t n_tok, hipStream_t s)
{
    const int64_t nb = n_tok * (n / 32);
    const int bs = 256;
    quantize_q8_0_kernel<<<(unsigned)((nb + bs - 1) / bs), bs, 0, s>>>(x, blocks, nb);
    return hipGetLastError();
}

} // namespace qg
