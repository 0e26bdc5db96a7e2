// mxq_nvfp4.hip -- grouped NVFP4 quantization with a 16-point RHT on the
// column-wise operand (gfx950): the amax, supplied-amax and empty-group kernels and
// the launch plan; the quant kernel variants are instantiated in
// mxq_nvfp4_quant_*.hip.  The method and the kernels' design are described in
// mxq_nvfp4_impl.hpp.
#include "mxq_nvfp4_impl.hpp"

namespace mxq {

// A group without rows: only the floor tensor scales of its (empty) sections.
template <bool ROW, bool COL>
__global__ __launch_bounds__(64) void k_nvfp4_empty(const Nvfp4Group G) {
    for (int i = threadIdx.x; i < G.num_sections; i += 64) {
        if (ROW) G.row_global[i] = tensor_scale(0.0f);
        if (COL) G.col_global[i] = tensor_scale(0.0f);
        if (ROW && G.amax_out_row) G.amax_out_row[i] = 0.0f;
        if (COL && G.amax_out_col) G.amax_out_col[i] = 0.0f;
    }
}

namespace {
template <bool ROW, bool COL, bool FP8>
hipError_t launch_sel(const Nvfp4Group& g, hipStream_t stream) {
    const bool given = g.amax_in_row || g.amax_in_col;
    if (hipError_t m = launch_mark(0, stream); m != hipSuccess) return m;
    if (given) {
        hipLaunchKernelGGL((k_nvfp4_given<ROW, COL>), dim3(g.num_sections), dim3(64), 0, stream, g);
    } else if (g.total_tiles == 0) {
        hipLaunchKernelGGL((k_nvfp4_empty<ROW, COL>), dim3(1), dim3(64), 0, stream, g);
        return hipGetLastError();
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.total_tiles == 0) return e;
    if (!given) {
        if (g.total_tiles % 4 == 0)
            hipLaunchKernelGGL((k_nvfp4_amax<ROW, COL, 4>), dim3((unsigned)(g.total_tiles / 4)), dim3(256), 0, stream, g);
        else
            hipLaunchKernelGGL((k_nvfp4_amax<ROW, COL, 1>), dim3((unsigned)g.total_tiles), dim3(64), 0, stream, g);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    if ((e = launch_mark(1, stream)) != hipSuccess) return e;
    const uint32_t flags = (ROW ? 1u : 0u) | (COL ? 2u : 0u) | (FP8 ? 4u : 0u);
    const bool sr = g.sr_row || g.sr_col, aout = given && (g.amax_out_row || g.amax_out_col);
    e = sr ? (aout ? launch_quant_sr_aout(g, flags, stream) : launch_quant_sr(g, flags, stream))
           : (aout ? launch_quant_rne_aout(g, flags, stream) : launch_quant_rne(g, flags, stream));
    if (e != hipSuccess) return e;
    return launch_mark(2, stream);
}
}  // namespace

hipError_t launch_nvfp4_group(const Nvfp4Group& g, uint32_t flags, hipStream_t stream) {
    const bool row = flags & 1u, col = flags & 2u, fp8 = flags & 4u;
    switch ((row ? 1 : 0) | (col ? 2 : 0) | (fp8 ? 4 : 0)) {
        case 1: return launch_sel<true, false, false>(g, stream);
        case 2: return launch_sel<false, true, false>(g, stream);
        case 3: return launch_sel<true, true, false>(g, stream);
        case 5: return launch_sel<true, false, true>(g, stream);
        case 6: return launch_sel<false, true, true>(g, stream);
        case 7: return launch_sel<true, true, true>(g, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mxq

