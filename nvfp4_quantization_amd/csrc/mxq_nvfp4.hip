// mxq_nvfp4.hip -- grouped NVFP4 quantization with a 16-point RHT on the
// column-wise operand (gfx950): the amax, scales and empty-group kernels and the
// launch plan; the quant kernel variants are instantiated in
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
    if (!given && g.total_tiles == 0) {
        hipLaunchKernelGGL((k_nvfp4_empty<ROW, COL>), dim3(1), dim3(64), 0, stream, g);
        return hipGetLastError();
    }
    hipError_t e = hipSuccess;
    if (given) {
        hipLaunchKernelGGL((k_nvfp4_scales<ROW, COL, true>), dim3(g.num_sections), dim3(kScalesThreads), 0, stream,
                           g, 1);
    } else {
        const int n_chunks = (int)((g.k + kAmaxCols - 1) / kAmaxCols);
        const int bands = g.tt_start[g.num_sections] * (kTileRows / kAmaxRows);
        hipLaunchKernelGGL((k_nvfp4_amax<ROW, COL>), dim3((unsigned)(bands * n_chunks)), dim3(256), 0, stream, g,
                           n_chunks);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((k_nvfp4_scales<ROW, COL, false>), dim3(g.num_sections), dim3(kScalesThreads), 0, stream,
                           g, (kTileRows / kAmaxRows) * n_chunks);
    }
    if ((e = hipGetLastError()) != hipSuccess || g.total_tiles == 0) return e;
    const uint32_t flags = (ROW ? 1u : 0u) | (COL ? 2u : 0u) | (FP8 ? 4u : 0u);
    const bool sr = g.sr_row || g.sr_col, aout = given && (g.amax_out_row || g.amax_out_col);
    return sr ? (aout ? launch_quant_sr_aout(g, flags, stream) : launch_quant_sr(g, flags, stream))
              : (aout ? launch_quant_rne_aout(g, flags, stream) : launch_quant_rne(g, flags, stream));
}
}  // namespace

// Processing order of the single-read form: the non-empty sections in index order
// (work-group b takes item b).
static void fused_plan(const Nvfp4Group& g, Nvfp4Fused& f) {
    const int per_tile_row = g.n_ctiles / 4;
    f.n_cgroups = per_tile_row;
    f.n_order = 0;
    int32_t items = 0;
    for (int s = 0; s < g.num_sections; ++s) {
        const int n = (g.tt_start[s + 1] - g.tt_start[s]) * per_tile_row;
        if (n == 0) continue;
        f.order[f.n_order] = (uint8_t)s;
        f.istart[f.n_order] = items;
        ++f.n_order;
        items += n;
    }
    f.istart[f.n_order] = items;
    f.n_items = items;
}

// The single-read form applies when the measured maxima are wanted, the column tiles
// come in fours, and every item of the group fits the resident grid at once.  Then
// the whole input is read in one burst and each section is quantized as soon as its
// last tile has arrived.  Larger groups would run as two or more batches in which
// the loads of one batch and the quantizing of the previous one barely overlap; the
// three-kernel form (whose second read comes partly from the Infinity Cache and
// overlaps its arithmetic) is faster for them (measured on MI355X: 40.1 against
// 46.6 us for 8192 x 4096 in 8 sections, 512 items; 78.9 against 74.0 us for 16384 x
// 4096, 1024 items).
static bool fused_eligible(const Nvfp4Group& g, uint32_t flags, hipStream_t stream, hipError_t* err) {
    *err = hipSuccess;
    if (g.amax_in_row || g.amax_in_col || g.total_tiles == 0 || g.n_ctiles % 4 != 0) return false;
    int blocks = 0, dev = 0, cus = 0;
    *err = (g.sr_row || g.sr_col) ? fused_blocks_per_cu_sr(flags, &blocks) : fused_blocks_per_cu_rne(flags, &blocks);
    if (*err != hipSuccess) return false;
    if ((*err = hipStreamGetDevice(stream, &dev)) != hipSuccess) return false;
    if ((*err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return false;
    const int64_t items = (int64_t)g.total_tiles / 4;
    return items <= (int64_t)blocks * cus && items <= kFusedMaxItems;
}

hipError_t launch_nvfp4_group(const Nvfp4Group& g, uint32_t flags, uint32_t* slots, uint32_t* status,
                              hipStream_t stream) {
    hipError_t e = hipSuccess;
    const bool fused = slots && fused_eligible(g, flags, stream, &e);
    if (e != hipSuccess) return e;
    if (fused) {
        Nvfp4Fused f{};
        f.slots = slots;
        f.err = status;
        fused_plan(g, f);
        return (g.sr_row || g.sr_col) ? launch_fused_sr(g, f, flags, stream) : launch_fused_rne(g, f, flags, stream);
    }
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

