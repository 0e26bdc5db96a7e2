// mxq_nvfp4_quant_sr_aout.hip -- the grouped NVFP4 quant kernels with stochastic rounding and measured maxima out (supplied maxima)
// (one translation unit per variant family, so that the variants compile in parallel).
#include "mxq_nvfp4_impl.hpp"

namespace mxq {

hipError_t launch_quant_sr_aout(const Nvfp4Group& g, uint32_t flags, hipStream_t stream) {
    return launch_quant_variant<true, true>(g, flags, stream);
}

}  // namespace mxq
