// GEMV kernel instantiations for one weight format (see gemv_impl.h).
#include "gemv_impl.h"

namespace qg {

template <>
hipError_t gemv_dispatch<QG_Q4_K, 1, 0>(const gemv_detail::GemvParams &p, const GemvCfg &c, hipStream_t s)
{
    return gemv_detail::dispatch<QG_Q4_K, 1, gemv_detail::kEpiPlain>(p, c, s);
}

template <>
hipError_t gemv_dispatch<QG_Q4_K, 2, 0>(const gemv_detail::GemvParams &p, const GemvCfg &c, hipStream_t s)
{
    return gemv_detail::dispatch<QG_Q4_K, 2, gemv_detail::kEpiPlain>(p, c, s);
}

template <>
hipError_t gemv_dispatch<QG_Q4_K, 2, 1>(const gemv_detail::GemvParams &p, const GemvCfg &c, hipStream_t s)
{
    return gemv_detail::dispatch<QG_Q4_K, 2, gemv_detail::kEpiNorm>(p, c, s);
}

template <>
hipError_t gemv_dispatch<QG_Q4_K, 1, 2>(const gemv_detail::GemvParams &p, const GemvCfg &c, hipStream_t s)
{
    return gemv_detail::dispatch<QG_Q4_K, 1, gemv_detail::kEpiResid>(p, c, s);
}

template <>
hipError_t gemv_dispatch<QG_Q4_K, 1, 3>(const gemv_detail::GemvParams &p, const GemvCfg &c, hipStream_t s)
{
    return gemv_detail::dispatch<QG_Q4_K, 1, gemv_detail::kEpiArgmax>(p, c, s);
}

} // namespace qg
