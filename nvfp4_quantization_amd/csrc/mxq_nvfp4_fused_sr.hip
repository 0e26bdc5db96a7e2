// mxq_nvfp4_fused_sr.hip -- the single-read grouped NVFP4 kernels with stochastic
// rounding (one translation unit per rounding mode, so that the variants compile in
// parallel).
#include "mxq_nvfp4_fused.hpp"

namespace mxq {

hipError_t launch_fused_sr(const Nvfp4Group& g, const Nvfp4Fused& f, uint32_t flags, hipStream_t stream) {
    return launch_fused_variant<true>(g, f, flags, stream);
}

hipError_t fused_blocks_per_cu_sr(uint32_t flags, int* blocks) { return fused_occupancy<true>(flags, blocks); }

}  // namespace mxq
