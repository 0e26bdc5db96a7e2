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
// One launch group per at most kGroupSections sections (their tables travel in the
// kernel arguments).  A group runs two kernels on the caller's stream:
//   reset   one work-group: clears the group's control words and writes the floor
//           tensor scales of empty sections;
//   fused   one wave per work-group, work items in blockIdx order:
//     A item  (section, 128-row tile, up to kATiles 128-column tiles): max |x| and
//             max |H16 D x| of the block, stored as a partial; the section's last A
//             item (a counter tells which) reduces the partials, publishes the two
//             tensor scales and raises the section's ready flag;
//     B item  (section, 128 x 128 tile): waits for the ready flag, then writes all
//             outputs of its tile.
// Items are listed round by round; the host puts every A item of a section before
// all of its B items (all A items first, then all B items).
constexpr int kGroupSections = 32;
constexpr int kTileRows = 128;        // token tile
constexpr int kTileCols = 128;        // column tile (one wave)
constexpr int kATiles = 1;            // column tiles per A item

struct Nvfp4Round {
    int32_t sec_b, sec_a;             // section of the B / A items (-1: none)
    int32_t n_b, n_a;                 // item counts
    int32_t start;                    // first blockIdx of the round
};

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
    uint32_t* ctrl;                   // workspace: control words
    uint64_t* partials;               // workspace: one (row, column) amax pair per A item
    uint64_t seed;
    uint32_t flags;
    uint32_t sign_mask;
    uint32_t sr_row, sr_col;
    int32_t num_sections;
    int32_t n_ctiles;                 // k / 128
    int32_t n_agroups;                // ceil(n_ctiles / kATiles)
    int32_t num_rounds;
    int32_t total_items;
    int32_t tt_start[kGroupSections + 1];    // first token tile of each section (group-relative)
    int32_t a_start[kGroupSections + 1];     // first partial of each section
    Nvfp4Round rounds[2 * kGroupSections];
    uint64_t row_off[kGroupSections];
    uint64_t col_off[kGroupSections];
};
hipError_t launch_nvfp4_group(const Nvfp4Group& g, hipStream_t stream);

// Workspace layout: control words of section s at word kCtrlStride * s
// ([0] A items done, [1] ready flag, [2] row tensor scale bits, [3] column tensor
// scale bits), each section in its own 256-byte line; the error word after them
// (a wait that timed out sets it); then the partials.
constexpr int kCtrlStride = 64;
constexpr int kCtrlErrorWord = kGroupSections * kCtrlStride;
constexpr int64_t kCtrlBytes = (int64_t)(kGroupSections + 1) * kCtrlStride * 4;

}  // namespace mxq
