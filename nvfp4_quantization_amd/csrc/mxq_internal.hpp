// mxq_internal.hpp -- launch descriptors shared by the host entry points
// (mxq_api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

// ---------------------------------------------------------------- FP8 1x128
struct Fp8Args {
    const uint16_t* x;
    uint8_t* q;
    float* scales;
    int64_t m, k, ldx, ldq, srow, sgroup;
};
hipError_t launch_quant_fp8_1x128(const Fp8Args& a, hipStream_t stream);

// ---------------------------------------------------------------- DSA rotate + FP8
struct DsaArgs {
    const uint16_t* pe;
    const uint16_t* nope;
    uint8_t* q;
    float* scales;
    int64_t ld_pe, ld_nope, m;
    int32_t d_pe;
};
hipError_t launch_hadamard_quant_fp8(const DsaArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- grouped NVFP4
// Sections are processed in launch groups of at most kGroupSections so that the
// per-section tables travel in the kernel arguments.
constexpr int kGroupSections = 64;
constexpr int kTileRows = 128;        // token tile (rows) of both phases
constexpr int kTileCols = 128;        // column tile
constexpr int kChunkTiles = 4;        // token tiles per phase-A work-group

struct Nvfp4Group {
    const uint16_t* x;                // first row of the group
    int64_t k;
    uint8_t* row_codes;               // at the group's first row
    uint8_t* row_scales;
    uint8_t* fp8_codes;
    float* fp8_scales;
    uint8_t* col_codes;               // at the group's first section
    uint8_t* col_scales;
    float* row_global;                // at the group's first section
    float* col_global;
    float* partials;                  // workspace: 2 floats per phase-A work-group
    uint64_t seed;
    uint32_t flags;
    uint32_t sign_mask;
    uint32_t sr_row, sr_col;
    int32_t num_sections;
    int32_t n_ctiles;                 // k / 128
    int32_t total_tiles;              // phase-B tiles (token tiles x column tiles)
    int32_t total_chunks;             // phase-A work-groups
    int32_t tt_start[kGroupSections + 1];    // first token tile of each section (group-relative)
    int32_t chunk_start[kGroupSections + 1]; // first phase-A work-group of each section
    uint64_t row_off[kGroupSections];
    uint64_t col_off[kGroupSections];
};
hipError_t launch_nvfp4_group(const Nvfp4Group& g, hipStream_t stream);

}  // namespace mxq
