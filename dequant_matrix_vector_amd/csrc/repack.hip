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
    case QG_Q6_K:
        if (cols % 256) return false;
        L->row_qbytes = cols / 2;
        L->splane_bytes = rows * (cols / 16);
        break;
    default:
        return false;
    }
    L->qplane_bytes = rows * L->row_qbytes;
    L->hplane_off = 0;
    L->dplane_off = 0;
    if (fmt == QG_Q6_K) {
        // quant, high-bit, scale and d planes, each at a 256-byte boundary
        L->hplane_off = align_up(L->qplane_bytes, kPlaneAlign);
        L->splane_off = align_up(L->hplane_off + rows * (cols / 4), kPlaneAlign);
        L->dplane_off = align_up(L->splane_off + L->splane_bytes, kPlaneAlign);
        L->total = align_up(L->dplane_off + rows * (cols / 256) * 2, kPlaneAlign);
        return true;
    }
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

// Q6_K, one thread per 256-weight super-block.  Raw: ql[128], qh[64],
// scales[16] (int8), d (f16); column c = 128h + 32j + l has its low four bits
// in ql[64h + 32(j mod 2) + l] (high nibble when j >= 2) and its top two bits
// at bit 2j of qh[32h + l].
__device__ __forceinline__ uint32_t q6_code(const uint8_t *blk, int c)
{
    const int h = c >> 7, j = (c >> 5) & 3, l = c & 31;
    const uint32_t lo = (blk[64 * h + 32 * (j & 1) + l] >> (j >= 2 ? 4 : 0)) & 0xFu;
    const uint32_t hi = (blk[128 + 32 * h + l] >> (2 * j)) & 3u;
    return lo | (hi << 4);
}

// Bit position, in the high-bit word of a packed quant word, of the top two
// bits of the code at nibble position n (0..7) of that quant word: the
// kernel's masks 0x000F000F | 0x00300030, 0x00F000F0 | 0x03000300 and the same
// after a byte shift (high bits shifted by 8 the same way; the last mask takes
// them shifted left by 8) read nibbles 0,4 / 1,5 / 2,6 / 3,7 with high bits at
// 4,20 / 8,24 / 12,28 / 0,16.
__device__ __forceinline__ int q6_hbit(int n)
{
    const int pos[8] = {4, 8, 12, 0, 20, 24, 28, 16};
    return pos[n];
}

__global__ void repack_q6_k_kernel(const uint8_t *__restrict__ raw, uint8_t *__restrict__ packed,
                                   int64_t nsbs, int64_t nsb, int64_t row_qbytes, int64_t hoff, int64_t soff,
                                   int64_t doff)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nsbs) return;
    int64_t r = i / nsb, sb = i % nsb;
    const uint8_t *blk = raw + i * 210;
    uint8_t *q = packed + r * row_qbytes + sb * 128;
    uint32_t *hw = reinterpret_cast<uint32_t *>(packed + hoff + (r * nsb + sb) * 64);
    for (int ch = 0; ch < 8; ch++) {
        // quant word k of the chunk holds columns 4k..4k+3 (low nibbles) and
        // 16+4k..16+4k+3 (high nibbles) of the chunk, byte by byte
        for (int l = 0; l < 16; l++) {
            const uint32_t a = q6_code(blk, 32 * ch + l) & 0xFu;
            const uint32_t b = q6_code(blk, 32 * ch + 16 + l) & 0xFu;
            q[16 * ch + l] = (uint8_t)(a | (b << 4));
        }
        // high-bit word m covers quant words 2m (shift 0) and 2m+1 (shift 2)
        for (int m = 0; m < 2; m++) {
            uint32_t v = 0;
            for (int kk = 0; kk < 2; kk++) {
                const int k = 2 * m + kk;
                for (int n = 0; n < 8; n++) {
                    // nibble n of quant word k: byte n/2, low (n even) or high nibble
                    const int col = (n & 1) ? 16 + 4 * k + (n >> 1) : 4 * k + (n >> 1);
                    const uint32_t hi = q6_code(blk, 32 * ch + col) >> 4;
                    v |= hi << (q6_hbit(n) + 2 * kk);
                }
            }
            hw[2 * ch + m] = v;
        }
    }
    uint8_t *sc = packed + soff + (r * nsb + sb) * 16;
    for (int l = 0; l < 16; l++) sc[l] = blk[192 + l];
    uint8_t *d = packed + doff + (r * nsb + sb) * 2;
    d[0] = blk[208];
    d[1] = blk[209];
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

// Q6_K, one thread per 32-wide chunk, through the same masks as the GEMV
// kernel; d*sc (11 x 8 significant bits) times q-32 is exact in binary32.
__global__ void dequant_q6_k_kernel(const uint8_t *__restrict__ packed, float *__restrict__ w, int64_t nchunks,
                                    int64_t nch, int64_t row_qbytes, int64_t hoff, int64_t soff, int64_t doff)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nchunks) return;
    int64_t r = i / nch, c = i % nch;
    const uint32_t *qw = reinterpret_cast<const uint32_t *>(packed + r * row_qbytes + c * 16);
    const uint32_t *hw = reinterpret_cast<const uint32_t *>(packed + hoff + i * 8);
    const int8_t *sc = reinterpret_cast<const int8_t *>(packed + soff + i * 2);
    const float d = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(packed + doff)[r * (nch / 8) + c / 8]);
    const float da = d * (float)sc[0], db = d * (float)sc[1];
    float *o = w + i * 32;
    for (int k = 0; k < 4; k++) {
        const uint32_t H = hw[k >> 1] >> (2 * (k & 1));
        const uint32_t pa = (qw[k] & 0x000F000Fu) | (H & 0x00300030u);
        const uint32_t pb = (qw[k] & 0x00F000F0u) | (H & 0x03000300u);
        const uint32_t sh = qw[k] >> 8;
        const uint32_t pc = (sh & 0x000F000Fu) | ((H >> 8) & 0x00300030u);
        const uint32_t pd = (sh & 0x00F000F0u) | ((H << 8) & 0x03000300u);
        o[4 * k] = da * (float)((int)(pa & 0x3Fu) - 32);
        o[4 * k + 2] = da * (float)((int)((pa >> 16) & 0x3Fu) - 32);
        o[4 * k + 1] = da * (float)((int)(pc & 0x3Fu) - 32);
        o[4 * k + 3] = da * (float)((int)((pc >> 16) & 0x3Fu) - 32);
        o[16 + 4 * k] = db * (float)((int)((pb >> 4) & 0x3Fu) - 32);
        o[16 + 4 * k + 2] = db * (float)((int)((pb >> 20) & 0x3Fu) - 32);
        o[16 + 4 * k + 1] = db * (float)((int)((pd >> 4) & 0x3Fu) - 32);
        o[16 + 4 * k + 3] = db * (float)((int)((pd >> 20) & 0x3Fu) - 32);
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
    case QG_Q6_K: {
        int64_t n = rows * (cols / 256);
        repack_q6_k_kernel<<<grid_for(n, bs), bs, 0, st>>>(src, packed, n, cols / 256, L.row_qbytes, L.hplane_off,
                                                           L.splane_off, L.dplane_off);
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
    case QG_Q6_K: {
        int64_t n = rows * (cols / 32);
        dequant_q6_k_kernel<<<grid_for(n, bs), bs, 0, st>>>(packed, w, n, cols / 32, L.row_qbytes, L.hplane_off,
                                                            L.splane_off, L.dplane_off);
        break;
    }
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace qg
