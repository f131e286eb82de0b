// Batched-token products with Q8_0 activations, on the matrix cores.
//
// The Go "llm" package's ExactGGML mode (type CPU) quantizes every activation
// row to Q8_0 before each quantized product, the prompt's tokens included.  A
// block's product is then an exact integer sum of code products, scaled by
// the weight block's and the activation block's binary16 scales.  For n_tok >
// 1 the integer sums of 16 rows x 16 tokens x one 32-weight block are one
// v_mfma_f32_16x16x32_f16: the weight codes (Q4_0: q - 8, Q8_0: q) and the
// activation codes are small integers, exact in binary16, and their products
// and 32-term sums are exact in the fp32 result.  Each block's 16 x 16 sums
// are then scaled by d_w * d_x (exact in binary32) and added to the fp32
// accumulators with one fma each, as in the one-token kernels.
//
// Work decomposition
//   * A first launch quantizes every token's x blocks once (the one-token
//     path's rule, q8act.h) into the caller's workspace: the 32 codes of a
//     block as binary16 operand slots (64 bytes), and its scale as fp32.
//   * The product: W waves per workgroup, each with MTR 16-row tiles of each
//     of the NMAT matrices (the gate/up pair shares the tokens); the
//     workgroup covers NTW 16-token tiles and one range of K.  K advances by
//     super-steps of kSB blocks: the workgroup copies the operand slots and
//     scales of its tokens into LDS, each wave the code bytes and scales of
//     its own rows into its own LDS area.  Two super-steps of loads are in
//     flight while one is multiplied.
//   * Codes become binary16 operands by placing a byte (Q8_0 and activation
//     codes, xor 0x80: q + 128) or a nibble (Q4_0: q) in the mantissa of 1024
//     (0x6400) and subtracting the bias with one packed binary16 subtract, two
//     codes at a time.  Those pairs hold bytes 0 and 2, then 1 and 3, of a
//     code word, so a lane's eight k slots of a block take its columns in the
//     order 0 2 1 3 4 6 5 7 (plus 8 times its k group); weights and
//     activations use the same order, which leaves every block sum unchanged.
//   * Epilogue: y, or silu(g) * u for the pair; with K split over
//     workgroups, raw partial sums that a second launch adds in range order.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "q8act.h"
#include "qg_internal.h"

namespace qg {
namespace {

typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSB = 4;   // blocks per super-step

}  // namespace

// split-K sum of partials [ksplit][nmat][n] in range order (prefill.hip)
hipError_t launch_prefill_reduce(int nmat, const float *part, float *y, int64_t n, int ksplit, const float *resid,
                                 hipStream_t s, hipEvent_t stop, uint16_t *yb);

namespace {

struct Q8mParams {
    const uint8_t *q[2];  // packed tensors (quant plane at offset 0)
    const uint16_t *xq;   // activation operand slots [n_tok][nchunk][32] (binary16)
    const float *xd;      // activation block scales [n_tok][nchunk]
    float *y;             // [n_tok][rows], or partials [ksplit][NMAT][n_tok][rows]
    int64_t row_qbytes;   // quant-plane bytes per row
    int64_t soff;         // scale-plane offset (f16 per row and block)
    int rows;
    int nchunk;           // blocks per row (cols / 32)
    int n_tok;
    int tok_groups;
    int ssteps;           // super-steps covering a row
    int ksplit;           // K ranges (workgroups per row group and token group)
    int spk;              // super-steps per K range
};

template <int N, typename F>
__device__ __forceinline__ void sfor(F &&f)
{
    if constexpr (N > 0) {
        sfor<N - 1>(f);
        f(std::integral_constant<int, N - 1>{});
    }
}

// Two binary16 integers from bytes 0 and 2 of w under mask (0x00FF00FF for a
// byte, 0x000F000F for a nibble): the masked value in the mantissa of 1024
// (0x6400), minus bias.
__device__ __forceinline__ uint32_t f16_pair(uint32_t w, uint32_t mask, _Float16 bias)
{
    const uint32_t v = (w & mask) | 0x64006400u;
    const h16x2 h = __builtin_bit_cast(h16x2, v) - h16x2{bias, bias};
    return __builtin_bit_cast(uint32_t, h);
}

// Eight codes of two code words (wa: slots 0-3, wb: slots 4-7) as binary16
// operand slots in the order bytes 0 2 1 3 of each word.
__device__ __forceinline__ h16x8 f16_slots(uint32_t wa, uint32_t wb, uint32_t mask, _Float16 bias)
{
    u32x4 u;
    u.x = f16_pair(wa, mask, bias);
    u.y = f16_pair(wa >> 8, mask, bias);
    u.z = f16_pair(wb, mask, bias);
    u.w = f16_pair(wb >> 8, mask, bias);
    return __builtin_bit_cast(h16x8, u);
}

// The same slots from code bytes (each byte one code, 0..255 after any
// offset), one byte permute per pair: v_perm_b32 takes bytes 0 and 2 (or 1
// and 3) of the code word and a 0x64 byte from c64 (0x64646464) above each.
__device__ __forceinline__ h16x8 f16_slots_bytes(uint32_t wa, uint32_t wb, uint32_t c64, _Float16 bias)
{
    const h16x2 bb{bias, bias};
    u32x4 u;
    u.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h16x2, __builtin_amdgcn_perm(c64, wa, 0x04020400u)) - bb);
    u.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h16x2, __builtin_amdgcn_perm(c64, wa, 0x04030401u)) - bb);
    u.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h16x2, __builtin_amdgcn_perm(c64, wb, 0x04020400u)) - bb);
    u.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h16x2, __builtin_amdgcn_perm(c64, wb, 0x04030401u)) - bb);
    return __builtin_bit_cast(h16x8, u);
}

__device__ __forceinline__ float silu_times(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// x [n_tok][nchunk * 32] -> operand slots and scales, one thread per block.
__global__ void q8act_quantize_kernel(const float *__restrict__ x, uint16_t *__restrict__ xq, float *__restrict__ xd,
                                      int64_t blocks)
{
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= blocks) return;
    const float4 *src = reinterpret_cast<const float4 *>(x) + b * 8;
    float4 v[8];
#pragma unroll
    for (int k = 0; k < 8; k++) v[k] = src[k];
    Q8Chunk o;
    quantize_chunk_q8_0(v, o);
    u32x4 *dst = reinterpret_cast<u32x4 *>(xq + b * 32);
#pragma unroll
    for (int g = 0; g < 4; g++)
        dst[g] = __builtin_bit_cast(u32x4, f16_slots(o.q[2 * g] ^ 0x80808080u, o.q[2 * g + 1] ^ 0x80808080u,
                                                     0x00FF00FFu, (_Float16)1152.0f));
    xd[b] = o.d;
}

template <int FMT, int NMAT, int MTR, int NTW, int W>
__global__ __launch_bounds__(W * 64) void q8act_mfma_kernel(Q8mParams p)
{
    static_assert(FMT == QG_Q4_0 || FMT == QG_Q8_0, "Q8_0 activations: Q4_0 or Q8_0 weights");
    constexpr bool K8 = FMT == QG_Q8_0;
    constexpr int BB = K8 ? 32 : 16;           // code bytes per block
    constexpr int MT = MTR * NMAT;             // 16-row tiles per wave
    constexpr int NTOK = NTW * 16;             // tokens per workgroup
    constexpr int NT = W * 64;                 // threads
    constexpr int XP = NTOK * kSB * 4;         // 16-byte pieces of operand slots per super-step
    constexpr int XPT = XP / NT;               // per thread
    static_assert(XP % NT == 0 && NTOK * kSB <= NT, "x pieces and scales split over the threads");
    constexpr int XROW = kSB * 64 + 16;        // LDS bytes per token: kSB blocks of 32 slots, padded
    constexpr int XBUF = NTOK * XROW + kSB * NTOK * 4;   // slots, then d_x [block][token]
    constexpr int AROW = kSB * BB + 16;        // LDS bytes per weight row, padded
    constexpr int AWAVE = MT * 16 * AROW + MT * kSB * 16 * 4;   // codes, then d_w [tile][block][row]
    constexpr int LPI = K8 ? 2 : 1;            // 16-byte loads per tile and super-step (per lane)
    extern __shared__ float4 q8m_lds[];
    uint8_t *lds = reinterpret_cast<uint8_t *>(q8m_lds);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    uint8_t *aw = lds + 2 * XBUF + wave * AWAVE;
    float *dws = reinterpret_cast<float *>(aw + MT * 16 * AROW);

    // work item (row group, K range, token group), token group fastest:
    // consecutive workgroups share the weights of one row group and range
    const int tg = (int)(blockIdx.x % (unsigned)p.tok_groups);
    const int rest = (int)(blockIdx.x / (unsigned)p.tok_groups);
    const int ks = rest % p.ksplit;
    const int rg = rest / p.ksplit;
    const int row_base = (rg * W + wave) * (MTR * 16);
    const int tok_base = tg * NTOK;
    const int k0 = ks * p.spk;
    const int k1 = k0 + p.spk < p.ssteps ? k0 + p.spk : p.ssteps;

    // weight loads: Q4_0 lane -> (row lane / 4, block lane % 4), 16 bytes;
    // Q8_0 load h: row 8h + lane / 8, block (lane % 8) / 2, half lane % 2
    const int lrow0 = K8 ? (lane >> 3) : (lane >> 2);
    const int lblk = K8 ? ((lane & 7) >> 1) : (lane & 3);
    const int lhalf = K8 ? (lane & 1) : 0;

    // the ring: two super-steps of weight codes, scales, operand slots and
    // activation scales (bit 0 of live: the lane's block inside the row; bit
    // 1 + k: x piece k live; bit 31: the thread's activation scale live)
    u32x4 wq[2][MT][LPI];
    uint32_t wd[2][MT][LPI];
    u32x4 xr[2][XPT];
    float dxr[2];
    uint32_t live[2];

    auto issue = [&](auto jc, int ss) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        int blk = ss * kSB + lblk;
        const bool bl = blk < p.nchunk;
        blk = bl ? blk : p.nchunk - 1;   // past the row: a valid block, scaled by 0
        uint32_t lv = bl ? 1u : 0u;
        sfor<MT>([&](auto mc) __attribute__((always_inline)) {
            constexpr int m = decltype(mc)::value;
            const uint8_t *base = p.q[m / MTR];
            sfor<LPI>([&](auto hc) __attribute__((always_inline)) {
                constexpr int h = decltype(hc)::value;
                int row = row_base + (m % MTR) * 16 + h * 8 + lrow0;
                row = row < p.rows ? row : p.rows - 1;   // rows past the end read a valid row; never stored
                wq[J][m][h] = *reinterpret_cast<const u32x4 *>(base + (int64_t)row * p.row_qbytes +
                                                               (int64_t)blk * BB + lhalf * 16);
                // the (row, block) scale; for Q8_0 the lanes of both halves load it
                wd[J][m][h] = *reinterpret_cast<const uint16_t *>(base + p.soff + ((int64_t)row * p.nchunk + blk) * 2);
            });
        });
        // operand slots: piece -> (token, block of the super-step, quarter)
        sfor<XPT>([&](auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            const int piece = tid + k * NT;
            const int t = piece / (kSB * 4), c = (piece >> 2) % kSB, qq = piece & 3;
            const int tok = tok_base + t, b = ss * kSB + c;
            const bool alive = (tok < p.n_tok) & (b < p.nchunk);   // no branch: the loads stay in flight
            lv |= alive ? (2u << k) : 0u;
            const int64_t off = alive ? ((int64_t)tok * p.nchunk + b) * 32 + qq * 8 : 0;
            xr[J][k] = *reinterpret_cast<const u32x4 *>(p.xq + off);
        });
        {
            const int t = tid / kSB, c = tid % kSB;
            const int tok = tok_base + t, b = ss * kSB + c;
            const bool alive = (tid < NTOK * kSB) & (tok < p.n_tok) & (b < p.nchunk);
            lv |= alive ? 0x80000000u : 0u;
            dxr[J] = p.xd[alive ? (int64_t)tok * p.nchunk + b : 0];
        }
        live[J] = lv;
    };

    f32x4 acc[MT][NTW];
    sfor<MT>([&](auto mc) __attribute__((always_inline)) {
        sfor<NTW>([&](auto nc) __attribute__((always_inline)) {
            acc[decltype(mc)::value][decltype(nc)::value] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        });
    });

    // ring slot J -> LDS buffer J (activations) and this wave's weight area;
    // then, after the barrier, the products of the super-step's kSB blocks
    auto step = [&](auto jc, int nxt, bool refill) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        uint8_t *xt = lds + J * XBUF;
        float *dxs = reinterpret_cast<float *>(xt + NTOK * XROW);
        const uint32_t lv = live[J];
        sfor<XPT>([&](auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            const int piece = tid + k * NT;
            const int t = piece / (kSB * 4), c = (piece >> 2) % kSB, qq = piece & 3;
            // dead pieces (tokens past n_tok, blocks past the row) are zero codes
            const u32x4 v = ((lv >> (1 + k)) & 1u) ? xr[J][k] : u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4 *>(xt + t * XROW + c * 64 + qq * 16) = v;
        });
        if (tid < NTOK * kSB) {
            const int t = tid / kSB, c = tid % kSB;
            dxs[c * NTOK + t] = (lv >> 31) ? dxr[J] : 0.0f;
        }
        const bool bl = lv & 1u;
        sfor<MT>([&](auto mc) __attribute__((always_inline)) {
            constexpr int m = decltype(mc)::value;
            sfor<LPI>([&](auto hc) __attribute__((always_inline)) {
                constexpr int h = decltype(hc)::value;
                const int r = h * 8 + lrow0;
                *reinterpret_cast<u32x4 *>(aw + (m * 16 + r) * AROW + lblk * BB + lhalf * 16) = wq[J][m][h];
                if (lhalf == 0) {
                    const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd[J][m][h] & 0xFFFFu));
                    dws[(m * kSB + lblk) * 16 + r] = bl ? d : 0.0f;
                }
            });
        });
        __syncthreads();
        if (refill) issue(jc, nxt);
        sfor<kSB>([&](auto cc) __attribute__((always_inline)) {
            constexpr int c = decltype(cc)::value;
            h16x8 af[MT];
            f32x4 dw[MT];
            sfor<MT>([&](auto mc) __attribute__((always_inline)) {
                constexpr int m = decltype(mc)::value;
                const uint8_t *ap = aw + (m * 16 + r16) * AROW + c * BB;
                if constexpr (K8) {
                    const uint2 w = *reinterpret_cast<const uint2 *>(ap + 8 * g);
                    af[m] = f16_slots_bytes(w.x ^ 0x80808080u, w.y ^ 0x80808080u, 0x64646464u, (_Float16)1152.0f);
                } else {
                    // k group g: bytes 8(g & 1) .. +7, low nibbles (g < 2) or high,
                    // as bytes
                    const uint2 w = *reinterpret_cast<const uint2 *>(ap + 8 * (g & 1));
                    const uint32_t sh = 4u * (uint32_t)(g >> 1);
                    af[m] = f16_slots_bytes((w.x >> sh) & 0x0F0F0F0Fu, (w.y >> sh) & 0x0F0F0F0Fu, 0x64646464u,
                                            (_Float16)1032.0f);
                }
                dw[m] = *reinterpret_cast<const f32x4 *>(dws + (m * kSB + c) * 16 + 4 * g);
            });
            sfor<NTW>([&](auto nc) __attribute__((always_inline)) {
                constexpr int n = decltype(nc)::value;
                const h16x8 bf = *reinterpret_cast<const h16x8 *>(xt + (n * 16 + r16) * XROW + c * 64 + 16 * g);
                const float dx = dxs[c * NTOK + n * 16 + r16];
                f32x4 cs[MT];
                sfor<MT>([&](auto mc) __attribute__((always_inline)) {
                    constexpr int m = decltype(mc)::value;
                    cs[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[m], bf, f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                });
                sfor<MT>([&](auto mc) __attribute__((always_inline)) {
                    constexpr int m = decltype(mc)::value;
                    sfor<4>([&](auto ic) __attribute__((always_inline)) {
                        constexpr int i = decltype(ic)::value;
                        acc[m][n][i] = __builtin_fmaf(cs[m][i], dw[m][i] * dx, acc[m][n][i]);
                    });
                });
            });
        });
    };

    // prologue: super-steps k0, k0 + 1 (past k1: the last one again, never used)
    issue(std::integral_constant<int, 0>{}, k0);
    issue(std::integral_constant<int, 1>{}, k0 + 1 < k1 ? k0 + 1 : k1 - 1);
    int k = k0;
    // every refill in the loop is unconditional (past k1: the last super-step
    // again, never used): a conditional one would make the loop wait for it
    for (; k + 2 <= k1; k += 2) {
        step(std::integral_constant<int, 0>{}, k + 2 < k1 ? k + 2 : k1 - 1, true);
        step(std::integral_constant<int, 1>{}, k + 3 < k1 ? k + 3 : k1 - 1, true);
    }
    if (k < k1) step(std::integral_constant<int, 0>{}, 0, false);   // uniform branch

    // epilogue: the lane holds rows 4g + i of each tile for token r16
    const bool partial = p.ksplit > 1;
    sfor<NTW>([&](auto nc) __attribute__((always_inline)) {
        constexpr int n = decltype(nc)::value;
        const int tok = tok_base + n * 16 + r16;
        if (tok < p.n_tok) {
            sfor<MTR>([&](auto rc) __attribute__((always_inline)) {
                constexpr int mr = decltype(rc)::value;
                const int row = row_base + mr * 16 + 4 * g;
                auto store4 = [&](float *dst, const float (&v)[4]) __attribute__((always_inline)) {
                    if ((p.rows & 3) == 0 && row + 3 < p.rows) {
                        *reinterpret_cast<float4 *>(dst) = make_float4(v[0], v[1], v[2], v[3]);
                    } else {
                        for (int i = 0; i < 4; i++)
                            if (row + i < p.rows) dst[i] = v[i];
                    }
                };
                if (partial) {
                    // raw sums of this K range: [ks][matrix][token][row]
                    sfor<NMAT>([&](auto oc) __attribute__((always_inline)) {
                        constexpr int mo = decltype(oc)::value;
                        float v[4];
                        sfor<4>([&](auto ic) __attribute__((always_inline)) {
                            v[decltype(ic)::value] = acc[mo * MTR + mr][n][decltype(ic)::value];
                        });
                        store4(p.y + (((int64_t)(ks * NMAT + mo) * p.n_tok + tok) * p.rows + row), v);
                    });
                } else {
                    float v[4];
                    sfor<4>([&](auto ic) __attribute__((always_inline)) {
                        constexpr int i = decltype(ic)::value;
                        if constexpr (NMAT == 1) v[i] = acc[mr][n][i];
                        else v[i] = silu_times(acc[mr][n][i], acc[MTR + mr][n][i]);
                    });
                    store4(p.y + (int64_t)tok * p.rows + row, v);
                }
            });
        }
    });
}

// LDS of a workgroup: two x buffers (binary16 codes of kSB blocks per token,
// padded rows, then the per-block scales) and one weight area per wave
// (codes in padded rows, then the scales as fp32 [tile][block][row]).
constexpr size_t q8m_lds_bytes(int fmt, int nmat, int mtr, int ntw, int waves)
{
    const size_t ntok = (size_t)ntw * 16, bb = fmt == QG_Q8_0 ? 32 : 16, mt = (size_t)mtr * nmat;
    const size_t xbuf = ntok * (kSB * 64 + 16) + kSB * ntok * 4;
    const size_t awave = mt * 16 * (kSB * bb + 16) + mt * kSB * 16 * 4;
    return 2 * xbuf + (size_t)waves * awave;
}

constexpr int kQ8mWaves = 4;

template <int FMT, int NMAT, int MTR, int NTW>
hipError_t q8m_go(const Q8mParams &p, int64_t grid, hipStream_t s, hipEvent_t t0, hipEvent_t t1)
{
    constexpr int W = kQ8mWaves;
    constexpr size_t lds = q8m_lds_bytes(FMT, NMAT, MTR, NTW, W);
    static_assert(lds <= 160 * 1024, "LDS of one CU");
    auto kern = q8act_mfma_kernel<FMT, NMAT, MTR, NTW, W>;
    if constexpr (lds > 65536) {
        static std::atomic<bool> configured[64];
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
        if (!configured[dev].load(std::memory_order_relaxed)) {
            hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            configured[dev].store(true, std::memory_order_relaxed);
        }
    }
    if (t0 || t1) {
        Q8mParams arg = p;
        void *args[] = {&arg};
        return hipExtLaunchKernel((const void *)kern, dim3((unsigned)grid), dim3(64 * W), args, lds, s, t0, t1, 0);
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * W), lds, s, p);
    return hipGetLastError();
}

template <int FMT, int NMAT>
hipError_t q8m_tile(int mtr, int ntw, const Q8mParams &p, int64_t grid, hipStream_t s, hipEvent_t t0, hipEvent_t t1)
{
    if (mtr == 1) {
        if (ntw == 1) return q8m_go<FMT, NMAT, 1, 1>(p, grid, s, t0, t1);
        if (ntw == 2) return q8m_go<FMT, NMAT, 1, 2>(p, grid, s, t0, t1);
        return q8m_go<FMT, NMAT, 1, 4>(p, grid, s, t0, t1);
    }
    if (ntw == 1) return q8m_go<FMT, NMAT, 2, 1>(p, grid, s, t0, t1);
    if (ntw == 2) return q8m_go<FMT, NMAT, 2, 2>(p, grid, s, t0, t1);
    return q8m_go<FMT, NMAT, 2, 4>(p, grid, s, t0, t1);
}

}  // namespace

// The tile: 16, 32 or 64 tokens per workgroup by the batch; two 16-row tiles
// per wave and matrix while that still leaves two workgroups per CU before
// any K split.  The matrix-core tuning hook's mtr and ntw (ntw 8 taken as 4)
// and its ksplit override the choice.
Q8mPlan q8act_mfma_plan(int nmat, int64_t rows, int64_t cols, int64_t n_tok, int64_t part_elems)
{
    const PrefillCfg o = prefill_override();
    Q8mPlan c;
    c.ntw = n_tok <= 16 ? 1 : (n_tok <= 32 ? 2 : 4);
    const int64_t tg = (n_tok + c.ntw * 16 - 1) / (c.ntw * 16);
    const int64_t rg2 = (rows + kQ8mWaves * 32 - 1) / (kQ8mWaves * 32);
    c.mtr = rg2 * tg >= 2 * (int64_t)cu_count() ? 2 : 1;
    if (o.mtr > 0) {
        c.mtr = o.mtr;
        c.ntw = o.ntw > 4 ? 4 : o.ntw;
    }
    const int64_t ssteps = (cols / 32 + kSB - 1) / kSB;
    const int64_t base = ((rows + kQ8mWaves * c.mtr * 16 - 1) / (kQ8mWaves * c.mtr * 16)) *
                         ((n_tok + c.ntw * 16 - 1) / (c.ntw * 16));
    // K ranges for about four workgroups per CU, at least four super-steps
    // each, as far as the room for the partial sums goes
    int64_t ks = o.mtr > 0 && o.ksplit > 0 ? o.ksplit : (4 * (int64_t)cu_count() + base - 1) / base;
    const int64_t most = ssteps / 4 > 1 ? ssteps / 4 : 1;
    if (!(o.mtr > 0 && o.ksplit > 0) && ks > most) ks = most;
    if (ks > ssteps) ks = ssteps;
    while (ks > 1 && ks * nmat * n_tok * rows > part_elems) ks--;
    if (ks < 1) ks = 1;
    const int64_t spk = (ssteps + ks - 1) / ks;
    c.ksplit = (int)((ssteps + spk - 1) / spk);   // every range non-empty
    c.spk = (int)spk;
    return c;
}

int64_t q8act_x_bytes(int64_t cols, int64_t n_tok)
{
    // operand slots (64 bytes per block), then the scales (4 bytes per block)
    const int64_t blocks = n_tok * (cols / 32);
    return align_up(blocks * 64, kPlaneAlign) + align_up(blocks * 4, kPlaneAlign);
}

hipError_t launch_q8act_quantize(const float *x, uint8_t *ws, int64_t cols, int64_t n_tok, hipStream_t s)
{
    const int64_t blocks = n_tok * (cols / 32);
    uint16_t *xq = reinterpret_cast<uint16_t *>(ws);
    float *xd = reinterpret_cast<float *>(ws + align_up(blocks * 64, kPlaneAlign));
    hipLaunchKernelGGL(q8act_quantize_kernel, dim3((unsigned)((blocks + 255) / 256)), dim3(256), 0, s, x, xq, xd,
                       blocks);
    return hipGetLastError();
}

hipError_t launch_q8act_mfma(int fmt, int nmat, const uint8_t *w0, const uint8_t *w1, const uint8_t *xws, float *y,
                             int64_t rows, int64_t cols, int64_t n_tok, float *part, int64_t part_elems,
                             hipStream_t s)
{
    Layout L;
    if ((fmt != QG_Q4_0 && fmt != QG_Q8_0) || (nmat != 1 && nmat != 2) || n_tok < 1 ||
        n_tok >= (int64_t(1) << 31) || !layout_for(fmt, rows, cols, &L))
        return hipErrorInvalidValue;
    const Q8mPlan c = q8act_mfma_plan(nmat, rows, cols, n_tok, part ? part_elems : 0);
    const int64_t blocks = n_tok * (cols / 32);
    Q8mParams p;
    p.q[0] = w0;
    p.q[1] = nmat == 2 ? w1 : w0;
    p.xq = reinterpret_cast<const uint16_t *>(xws);
    p.xd = reinterpret_cast<const float *>(xws + align_up(blocks * 64, kPlaneAlign));
    p.y = c.ksplit > 1 ? part : y;
    p.row_qbytes = L.row_qbytes;
    p.soff = L.splane_off;
    p.rows = (int)rows;
    p.nchunk = (int)(cols / 32);
    p.n_tok = (int)n_tok;
    p.tok_groups = (int)((n_tok + c.ntw * 16 - 1) / (c.ntw * 16));
    p.ssteps = (p.nchunk + kSB - 1) / kSB;
    p.ksplit = c.ksplit;
    p.spk = c.spk;
    const int64_t row_groups = (rows + kQ8mWaves * c.mtr * 16 - 1) / (kQ8mWaves * c.mtr * 16);
    const int64_t grid = row_groups * p.tok_groups * c.ksplit;
    if (grid >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    hipEvent_t t0 = nullptr, t1 = nullptr;
    const bool timed = take_launch_timing(&t0, &t1);
    hipError_t e;
    if (fmt == QG_Q4_0)
        e = nmat == 1 ? q8m_tile<QG_Q4_0, 1>(c.mtr, c.ntw, p, grid, s, t0, c.ksplit == 1 ? t1 : nullptr)
                      : q8m_tile<QG_Q4_0, 2>(c.mtr, c.ntw, p, grid, s, t0, c.ksplit == 1 ? t1 : nullptr);
    else
        e = nmat == 1 ? q8m_tile<QG_Q8_0, 1>(c.mtr, c.ntw, p, grid, s, t0, c.ksplit == 1 ? t1 : nullptr)
                      : q8m_tile<QG_Q8_0, 2>(c.mtr, c.ntw, p, grid, s, t0, c.ksplit == 1 ? t1 : nullptr);
    if (e != hipSuccess || c.ksplit == 1) return e;
    return launch_prefill_reduce(nmat, part, y, n_tok * rows, c.ksplit, nullptr, s, timed ? t1 : nullptr, nullptr);
}

}  // namespace qg
