// mxq_nvfp4_fused_rne.hip -- the single-read grouped NVFP4 kernels with nearest-even
// rounding (one translation unit per rounding mode, so that the variants compile in
// parallel).
#include "mxq_nvfp4_fused.hpp"

namespace mxq {

hipError_t launch_fused_rne(const Nvfp4Group& g, const Nvfp4Fused& f, uint32_t flags, hipStream_t stream) {
    return launch_fused_variant<false>(g, f, flags, stream);
}

hipError_t fused_blocks_per_cu_rne(uint32_t flags, int* blocks) { return fused_occupancy<false>(flags, blocks); }

}  // namespace mxq
