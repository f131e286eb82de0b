// Matrix-core product instantiated for Q8_0 weights (prefill_impl.h).
#include "prefill_impl.h"

namespace qg {

hipError_t prefill_dispatch_q8_0(const PrefillCfg &c, int nmat, const PrefillParams &p, float *y, hipStream_t s)
{
    return prefill_dispatch<QG_Q8_0>(c, nmat, p, y, s);
}

} // namespace qg
