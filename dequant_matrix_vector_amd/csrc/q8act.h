// Q8_0 quantization of activations, for the mode in which every quantized
// product sees its activation row as Q8_0 blocks (the Go "llm" package's
// ExactGGML mode, which quantises activations to Q8_0 before each quantised
// matrix product).  Per 32-element chunk: d = max|x| / 127, q = round(x * (1/d))
// with halves away from zero (q = 0 when d = 0), in binary32 with correctly
// rounded divisions; the chunk keeps d rounded to binary16 (nearest even), so
// it stands for f16(d) * q.  Codes are packed four per 32-bit word in column
// order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

struct Q8Chunk {
    uint32_t q[8];    // codes of columns 4k..4k+3 in word k, low byte first
    float d;          // the binary16 scale, as binary32
    int qsum;         // sum of the 32 codes
    uint16_t d_bits;  // the binary16 scale
};

__device__ __forceinline__ uint32_t q8_pack4(int a, int b, int c, int d)
{
    return ((uint32_t)a & 0xFFu) | (((uint32_t)b & 0xFFu) << 8) | (((uint32_t)c & 0xFFu) << 16) |
           ((uint32_t)d << 24);
}

__device__ __forceinline__ void quantize_chunk_q8_0(const float4 (&v)[8], Q8Chunk &o)
{
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; k++) {
        amax = fmaxf(amax, fabsf(v[k].x));
        amax = fmaxf(amax, fabsf(v[k].y));
        amax = fmaxf(amax, fabsf(v[k].z));
        amax = fmaxf(amax, fabsf(v[k].w));
    }
    const float d = amax / 127.0f;
    const float id = d != 0.0f ? 1.0f / d : 0.0f;
    int qs = 0;
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const int a = (int)__builtin_roundf(v[k].x * id);
        const int b = (int)__builtin_roundf(v[k].y * id);
        const int c = (int)__builtin_roundf(v[k].z * id);
        const int e = (int)__builtin_roundf(v[k].w * id);
        qs += a + b + c + e;
        o.q[k] = q8_pack4(a, b, c, e);
    }
    const _Float16 dh = (_Float16)d;
    o.d = (float)dh;
    o.d_bits = __builtin_bit_cast(uint16_t, dh);
    o.qsum = qs;
}

} // namespace qg
