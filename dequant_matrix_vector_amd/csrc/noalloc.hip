// swiglu_ffn for callers that cannot allocate: the same products, with the
// scratch (h, split-K partial sums, bf16 copies of x and h) in a fixed array
// that the library's code object carries on each device.
#include <mutex>

#include "qg_internal.h"

namespace {

// QG_NOALLOC_SCRATCH_ELEMS floats, 256-byte aligned, one copy per device (held
// until the process ends).  Host code never uses this name as an address: the
// device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) float scratch[QG_NOALLOC_SCRATCH_ELEMS];

constexpr int kMaxDevices = 64;
float *g_scratch_ptr[kMaxDevices];
int g_scratch_status[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// The device address of this device's copy of `scratch` (looked up once per
// device, with that device current), or nullptr with *status set.
float *scratch_for_current_device(int *status)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *status = QG_ERR_DEVICE;
        return nullptr;
    }
    std::call_once(g_scratch_once[dev], [dev]() {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            g_scratch_status[dev] = QG_ERR_DEVICE;
            return;
        }
        g_scratch_ptr[dev] = static_cast<float *>(p);
        g_scratch_status[dev] = QG_OK;
    });
    *status = g_scratch_status[dev];
    return g_scratch_ptr[dev];
}

} // namespace

extern "C" int swiglu_ffn_noalloc(int fmt, const void *wg, const void *wu, const void *wd, const float *x, float *out,
                                  int64_t d_model, int64_t ffn, int64_t n_tok, void *stream)
{
    // the scratch swiglu_ffn would use at its fastest, as far as the array
    // holds it; h itself (n_tok * ffn floats) must fit
    const int64_t want = swiglu_ffn_scratch_elems(fmt, d_model, ffn, n_tok);
    if (want < 0) return (int)want;
    if (n_tok * ffn > QG_NOALLOC_SCRATCH_ELEMS) return QG_ERR_SCRATCH;
    int st = QG_OK;
    float *s = scratch_for_current_device(&st);
    if (!s) return st;
    const int64_t elems = want < QG_NOALLOC_SCRATCH_ELEMS ? want : QG_NOALLOC_SCRATCH_ELEMS;
    return swiglu_ffn(fmt, wg, wu, wd, x, out, s, elems, d_model, ffn, n_tok, stream);
}
