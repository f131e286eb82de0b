// Matrix-core product instantiated for per-row INT8 weights (prefill_impl.h).
#include "prefill_impl.h"

namespace qg {

hipError_t prefill_dispatch_i8row(const PrefillCfg &c, int nmat, const PrefillParams &p, float *y, hipStream_t s)
{
    return prefill_dispatch<QG_I8ROW>(c, nmat, p, y, s);
}

} // namespace qg
