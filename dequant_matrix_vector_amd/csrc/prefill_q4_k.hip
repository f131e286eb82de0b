// Matrix-core product instantiated for Q4_K weights (prefill_impl.h).
#include "prefill_impl.h"

namespace qg {

hipError_t prefill_dispatch_q4_k(const PrefillCfg &c, int nmat, const PrefillParams &p, float *y, hipStream_t s)
{
    return prefill_dispatch<QG_Q4_K>(c, nmat, p, y, s);
}

} // namespace qg
