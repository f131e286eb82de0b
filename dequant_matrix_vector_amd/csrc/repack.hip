// Load-time repack of raw quantized blocks into the packed planes, and the
// test-only dequantization of packed planes back to fp32.
//
// The repack follows the Go "llm" package's Design points (raw 18-byte Q4_0
// blocks become aligned quant words plus scales), kept byte-exact: the f16
// scales stay f16, so the packed buffer streams the same bytes per weight as
// the raw format.
#include "qg_internal.h"

namespace qg {

bool layout_for(int fmt, int64_t rows, int64_t cols, Layout *L)
{
    if (rows < 1 || cols < 1 || rows >= (int64_t(1) << 31) || cols >= (int64_t(1) << 31))
        return false;
    switch (fmt) {
    case QG_Q4_0:
        if (cols % 32) return false;
        L->row_qbytes = cols / 2;
        L->splane_bytes = rows * (cols / 32) * 2;
        break;
    case QG_Q8_0:
        if (cols % 32) return false;
        L->row_qbytes = cols;
        L->splane_bytes = rows * (cols / 32) * 2;
        break;
    case QG_Q4_K:
        if (cols % 256) return false;
        L->row_qbytes = cols / 2;
        L->splane_bytes = rows * (cols / 256) * 16;
        break;
    case QG_I8ROW:
        if (cols % 32) return false;
        L->row_qbytes = cols;
        L->splane_bytes = rows * 4;
        break;
    default:
        return false;
    }
    L->qplane_bytes = rows * L->row_qbytes;
    L->splane_off = align_up(L->qplane_bytes, kPlaneAlign);
    L->total = align_up(L->splane_off + L->splane_bytes, kPlaneAlign);
    return true;
}

namespace {

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

// ---------------------------------------------------------------- repack --
// One thread per 32-weight block (Q4_0, Q8_0).
__global__ void repack_q4_0_kernel(const uint8_t *__restrict__ raw, uint8_t *__restrict__ packed,
                                   int64_t nblocks, int64_t nb, int64_t row_qbytes, int64_t soff)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nblocks) return;
    int64_t r = i / nb, b = i % nb;
    const uint8_t *src = raw + i * 18;
    uint8_t *q = packed + r * row_qbytes + b * 16;
#pragma unroll
    for (int l = 0; l < 16; l++) q[l] = src[2 + l];
    uint8_t *s = packed + soff + i * 2;
    s[0] = src[0];
    s[1] = src[1];
}

__global__ void repack_q8_0_kernel(const uint8_t *__restrict__ raw, uint8_t *__restrict__ packed,
                                   int64_t nblocks, int64_t nb, int64_t row_qbytes, int64_t soff)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nblocks) return;
    int64_t r = i / nb, b = i % nb;
    const uint8_t *src = raw + i * 34;
    uint8_t *q = packed + r * row_qbytes + b * 32;
#pragma unroll
    for (int l = 0; l < 32; l++) q[l] = src[2 + l];
    uint8_t *s = packed + soff + i * 2;
    s[0] = src[0];
    s[1] = src[1];
}

// One thread per 256-weight super-block.  The 128 code bytes are regrouped
// so that each 16-byte run holds one 32-wide sub-block in the Q4_0 nibble
// order (element l low, element l+16 high).
__global__ void repack_q4_k_kernel(const uint8_t *__restrict__ raw, uint8_t *__restrict__ packed,
                                   int64_t nsbs, int64_t nsb, int64_t row_qbytes, int64_t soff)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nsbs) return;
    int64_t r = i / nsb, sb = i % nsb;
    const uint8_t *src = raw + i * 144;
    uint8_t *h = packed + soff + i * 16;
#pragma unroll
    for (int l = 0; l < 16; l++) h[l] = src[l];
    const uint8_t *qs = src + 16;
    uint8_t *q = packed + r * row_qbytes + sb * 128;
    for (int s = 0; s < 8; s++) {
        const uint8_t *pair = qs + 32 * (s >> 1);
        const int shift = (s & 1) ? 4 : 0;
        for (int l = 0; l < 16; l++) {
            uint32_t lo = (pair[l] >> shift) & 0xFu;
            uint32_t hi = (pair[l + 16] >> shift) & 0xFu;
            q[s * 16 + l] = (uint8_t)(lo | (hi << 4));
        }
    }
}

__global__ void repack_i8row_kernel(const uint8_t *__restrict__ q, const float *__restrict__ scale,
                                    uint8_t *__restrict__ packed, int64_t rows, int64_t cols,
                                    int64_t soff)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // one thread per 16 bytes
    int64_t n16 = rows * cols / 16;
    if (i < n16) {
        reinterpret_cast<uint4 *>(packed)[i] = reinterpret_cast<const uint4 *>(q)[i];
    }
    if (i < rows) reinterpret_cast<float *>(packed + soff)[i] = scale[i];
}

// --------------------------------------------------------------- dequant --
// Each weight's exact value rounded once to binary32 (the products below are
// exact; the Q4_K fma rounds only at the final subtraction).
__global__ void dequant_q4_0_kernel(const uint8_t *__restrict__ packed, float *__restrict__ w,
                                    int64_t nblocks, int64_t nb, int64_t row_qbytes, int64_t soff)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nblocks) return;
    int64_t r = i / nb, b = i % nb;
    const uint8_t *q = packed + r * row_qbytes + b * 16;
    const uint16_t *s = reinterpret_cast<const uint16_t *>(packed + soff);
    float d = f16_bits_to_f32(s[i]);
    float *o = w + r * nb * 32 + b * 32;
    for (int l = 0; l < 16; l++) {
        o[l] = (float)((int)(q[l] & 0xF) - 8) * d;
        o[l + 16] = (float)((int)(q[l] >> 4) - 8) * d;
    }
}

__global__ void dequant_q8_0_kernel(const uint8_t *__restrict__ packed, float *__restrict__ w,
                                    int64_t nblocks, int64_t nb, int64_t row_qbytes, int64_t soff)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nblocks) return;
    int64_t r = i / nb, b = i % nb;
    const int8_t *q = reinterpret_cast<const int8_t *>(packed + r * row_qbytes + b * 32);
    const uint16_t *s = reinterpret_cast<const uint16_t *>(packed + soff);
    float d = f16_bits_to_f32(s[i]);
    float *o = w + r * nb * 32 + b * 32;
    for (int l = 0; l < 32; l++) o[l] = (float)q[l] * d;
}

// One thread per 32-wide sub-block.
__global__ void dequant_q4_k_kernel(const uint8_t *__restrict__ packed, float *__restrict__ w,
                                    int64_t nsubs, int64_t nsub, int64_t row_qbytes, int64_t soff)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nsubs) return;
    int64_t r = i / nsub, c = i % nsub;
    int s = (int)(c & 7);
    const uint8_t *h = packed + soff + (r * (nsub / 8) + c / 8) * 16;
    float d = f16_bits_to_f32(h[0] | (h[1] << 8));
    float dmin = f16_bits_to_f32(h[2] | (h[3] << 8));
    const uint8_t *sc12 = h + 4;
    int sc, m;
    if (s < 4) {
        sc = sc12[s] & 63;
        m = sc12[s + 4] & 63;
    } else {
        sc = (sc12[s + 4] & 0xF) | ((sc12[s - 4] >> 6) << 4);
        m = (sc12[s + 4] >> 4) | ((sc12[s] >> 6) << 4);
    }
    float D = d * (float)sc;    // exact: 11-bit x 6-bit significands
    float M = dmin * (float)m;  // exact
    const uint8_t *q = packed + r * row_qbytes + c * 16;
    float *o = w + r * nsub * 32 + c * 32;
    for (int l = 0; l < 16; l++) {
        o[l] = __builtin_fmaf(D, (float)(q[l] & 0xF), -M);
        o[l + 16] = __builtin_fmaf(D, (float)(q[l] >> 4), -M);
    }
}

__global__ void dequant_i8row_kernel(const uint8_t *__restrict__ packed, float *__restrict__ w,
                                     int64_t rows, int64_t cols, int64_t soff)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= rows * cols) return;
    int64_t r = i / cols;
    float s = reinterpret_cast<const float *>(packed + soff)[r];
    w[i] = s * (float)reinterpret_cast<const int8_t *>(packed)[i];
}

inline unsigned grid_for(int64_t n, int bs) { return (unsigned)((n + bs - 1) / bs); }

} // namespace

hipError_t launch_repack(int fmt, const void *raw, const float *row_scale, uint8_t *packed,
                         int64_t rows, int64_t cols, hipStream_t st)
{
    Layout L;
    if (!layout_for(fmt, rows, cols, &L)) return hipErrorInvalidValue;
    const int bs = 256;
    const uint8_t *src = static_cast<const uint8_t *>(raw);
    switch (fmt) {
    case QG_Q4_0: {
        int64_t n = rows * (cols / 32);
        repack_q4_0_kernel<<<grid_for(n, bs), bs, 0, st>>>(src, packed, n, cols / 32, L.row_qbytes, L.splane_off);
        break;
    }
    case QG_Q8_0: {
        int64_t n = rows * (cols / 32);
        repack_q8_0_kernel<<<grid_for(n, bs), bs, 0, st>>>(src, packed, n, cols / 32, L.row_qbytes, L.splane_off);
        break;
    }
    case QG_Q4_K: {
        int64_t n = rows * (cols / 256);
        repack_q4_k_kernel<<<grid_for(n, bs), bs, 0, st>>>(src, packed, n, cols / 256, L.row_qbytes, L.splane_off);
        break;
    }
    case QG_I8ROW: {
        int64_t n = rows * cols / 16;
        if (rows > n) n = rows;
        repack_i8row_kernel<<<grid_for(n, bs), bs, 0, st>>>(src, row_scale, packed, rows, cols, L.splane_off);
        break;
    }
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_dequant(int fmt, const uint8_t *packed, float *w, int64_t rows, int64_t cols,
                          hipStream_t st)
{
    Layout L;
    if (!layout_for(fmt, rows, cols, &L)) return hipErrorInvalidValue;
    const int bs = 256;
    switch (fmt) {
    case QG_Q4_0: {
        int64_t n = rows * (cols / 32);
        dequant_q4_0_kernel<<<grid_for(n, bs), bs, 0, st>>>(packed, w, n, cols / 32, L.row_qbytes, L.splane_off);
        break;
    }
    case QG_Q8_0: {
        int64_t n = rows * (cols / 32);
        dequant_q8_0_kernel<<<grid_for(n, bs), bs, 0, st>>>(packed, w, n, cols / 32, L.row_qbytes, L.splane_off);
        break;
    }
    case QG_Q4_K: {
        int64_t n = rows * (cols / 32);
        dequant_q4_k_kernel<<<grid_for(n, bs), bs, 0, st>>>(packed, w, n, cols / 32, L.row_qbytes, L.splane_off);
        break;
    }
    case QG_I8ROW: {
        int64_t n = rows * cols;
        dequant_i8row_kernel<<<grid_for(n, bs), bs, 0, st>>>(packed, w, rows, cols, L.splane_off);
        break;
    }
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace qg
