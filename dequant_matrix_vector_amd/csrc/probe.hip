// Measurement export: the streaming-read rate the memory system gives a plain
// kernel, the ceiling the products' weight streams are compared against (the
// llmoxide blog, section 11 "Prefill and decode", measures its decode against
// a kernel that only reads the bytes).
#include "qg_internal.h"

namespace {

// Grid-stride read of 16-byte words, U loads in flight per thread, folded
// into one word per thread so that no load can be dropped; one word per
// workgroup is written only if the fold hits a value it cannot reach for the
// inputs used (so nothing is written in practice).
template <int U>
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4 *__restrict__ p, int64_t n16, uint32_t *out)
{
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; u++) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u) out[blockIdx.x] = acc;
}

} // namespace

extern "C" int qgemv_read_probe(const void *buf, int64_t bytes, int wg_per_cu, int unroll, uint32_t *out, void *stream)
{
    if (!buf || !out) return QG_ERR_NULL;
    if (bytes < 16 || bytes % 16 || wg_per_cu < 1 || wg_per_cu > 64 || (unroll != 2 && unroll != 4 && unroll != 8))
        return QG_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(buf) & 15) || (reinterpret_cast<uintptr_t>(out) & 3)) return QG_ERR_ALIGN;
    const int nwg = qg::cu_count() * wg_per_cu;
    hipStream_t s = (hipStream_t)stream;
    switch (unroll) {
    case 2: hipLaunchKernelGGL(read_probe_kernel<2>, dim3(nwg), dim3(256), 0, s, (const uint4 *)buf, bytes / 16, out); break;
    case 4: hipLaunchKernelGGL(read_probe_kernel<4>, dim3(nwg), dim3(256), 0, s, (const uint4 *)buf, bytes / 16, out); break;
    default: hipLaunchKernelGGL(read_probe_kernel<8>, dim3(nwg), dim3(256), 0, s, (const uint4 *)buf, bytes / 16, out); break;
    }
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}
