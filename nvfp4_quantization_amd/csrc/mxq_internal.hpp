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
hipError_t launch_quant_fp8_1x128(const Fp8Args& a, hipStream_t stream, bool ue8m0 = false);

// ---------------------------------------------------------------- FP8 block variants
// Row-wise 1x128 and/or column-wise 128x1 (codes of x^T) from one read of x, 128 x 128
// tiles staged in LDS; ue8m0: scales rounded up to powers of two.
struct Fp8BlockArgs {
    const uint16_t* x;
    int64_t m, k, ldx;
    uint8_t* rq;                      // row-wise codes [m][rld] (null: not wanted)
    int64_t rld;
    float* rs;                        // scale of (row r, group g) at r * rsr + g * rsg
    int64_t rsr, rsg;
    uint8_t* cq;                      // column-wise codes [k][cld] (null: not wanted)
    int64_t cld;
    float* cs;                        // scale of (column c, row block b) at c * csc + b * csb
    int64_t csc, csb;
};
hipError_t launch_quant_fp8_blockwise(const Fp8BlockArgs& a, bool ue8m0, hipStream_t stream);

// ---------------------------------------------------------------- SwiGLU -> FP8 1x128
struct SwigluFp8Args {
    const uint16_t* gate;
    const uint16_t* up;
    uint8_t* q;
    float* scales;
    int64_t m, n, ld_gate, ld_up, ldq, srow, sgroup;
};
hipError_t launch_swiglu_quant_fp8(const SwigluFp8Args& a, hipStream_t stream);

// ---------------------------------------------------------------- DSA rotate + FP8
struct DsaArgs {
    const uint16_t* pe;
    const uint16_t* nope;
    uint8_t* q;
    float* scales;                    // scale of row r = (token r / heads, head r % heads)
    int64_t ld_pe, ld_nope, m;
    int32_t d_pe;
    int64_t heads, stride_token, stride_head;
};
hipError_t launch_hadamard_quant_fp8(const DsaArgs& a, hipStream_t stream, bool ue8m0 = false);

// ---------------------------------------------------------------- DSA rotate + NVFP4
// Two kernels: the first rotates 64 rows per 256-thread work-group and stores the
// work-group's max |y| as a partial; the work-group that finishes last (two levels
// of counters tell which) folds the partials into the tensor scale, writes the
// scale table and resets the counters; the second rotates again and encodes.  With
// a supplied amax a one-work-group kernel forms the scale and the table instead.
struct DsaNvfp4Args {
    const uint16_t* pe;
    const uint16_t* nope;
    int64_t ld_pe, ld_nope, m;
    int32_t d_pe;
    int32_t n_wg;                     // work-groups of the row kernels
    uint8_t* codes;                   // [m][64]
    uint8_t* scales;                  // [m][8]
    float* global_scale;              // [1]
    const float* amax_in;             // [1] or null: measure
    float* amax_out;                  // [1] or null
    uint32_t* ctrl;                   // workspace: kDsaGroups group counters and the top counter
    float4* table;                    // workspace: 128 scale-table entries
    float* partials;                  // workspace: one max per work-group
};
hipError_t launch_hadamard_quant_nvfp4(const DsaNvfp4Args& a, hipStream_t stream);
// Workspace layout of the DSA NVFP4 call (byte offsets): counters (each on its own
// 256-byte line: group counter g at word g * kDsaCtrlStride, the top counter after
// them), the scale table, one partial per work-group.
constexpr int kDsaGroups = 64;
constexpr int kDsaCtrlStride = 64;
constexpr int64_t kDsaCtrlOffset = 0;
constexpr int64_t kDsaTableOffset = (int64_t)(kDsaGroups + 1) * kDsaCtrlStride * 4;
constexpr int64_t kDsaPartialsOffset = kDsaTableOffset + 128 * 16;

// ---------------------------------------------------------------- grouped NVFP4
// One launch group per at most kGroupSections sections.  A group runs two kernels
// on the caller's stream, one wave per 128 x 128 tile in each (with a caller-supplied
// amax, a small per-section kernel that builds the tables replaces the first):
//   amax    max |x| and max |H16 D x| of the tile into a per-tile partial; the
//           section's last tile (a counter tells which) folds the partials into
//           the two tensor scales, writes the section's (d, 1/d) tables and resets
//           the counter for the next call;
//   quant   every output of the tile.
constexpr int kGroupSections = 32;
constexpr int kTileRows = 128;        // token tile
constexpr int kTileCols = 128;        // column tile

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
    uint32_t* ctrl;                   // workspace: per-section counters
    float4* tables;                   // workspace: per-section scale tables
    uint64_t* partials;               // workspace: one (row, column) amax pair per tile
    uint64_t seed;
    uint32_t sign_mask;
    uint32_t sr_row, sr_col;
    int32_t num_sections;
    int32_t n_ctiles;                 // k / 128
    int32_t total_tiles;
    int32_t tt_start[kGroupSections + 1];    // first token tile of each section (group-relative)
    uint64_t row_off[kGroupSections];
    uint64_t col_off[kGroupSections];
    // caller-supplied section maxima (at the group's first section; both null: measure)
    const float* amax_in_row;
    const float* amax_in_col;
    // measured section maxima out (at the group's first section; null: not wanted)
    float* amax_out_row;
    float* amax_out_col;
};
hipError_t launch_nvfp4_group(const Nvfp4Group& g, uint32_t flags, hipStream_t stream);
// Launch marks of the calling thread (mxq_set_launch_marks): records mark i
// (0 before the first kernel, 1 between the scale and quantize kernels, 2 after)
// on the stream when marks are set; hipSuccess otherwise.
hipError_t launch_mark(int i, hipStream_t stream);
// The quant kernel's variant families (one translation unit each): nearest-even or
// stochastic rounding, with or without measured maxima out (supplied maxima).
hipError_t launch_quant_rne(const Nvfp4Group& g, uint32_t flags, hipStream_t stream);
hipError_t launch_quant_sr(const Nvfp4Group& g, uint32_t flags, hipStream_t stream);
hipError_t launch_quant_rne_aout(const Nvfp4Group& g, uint32_t flags, hipStream_t stream);
hipError_t launch_quant_sr_aout(const Nvfp4Group& g, uint32_t flags, hipStream_t stream);

// Workspace layout (byte offsets):
//   kCtrlOffset    section s: kCtrlGroups group counters and a top counter, each on
//                  its own 256-byte line, at words kCtrlStride * ((kCtrlGroups + 1) * s + i)
//   kTablesOffset  section s, direction dir (0 row, 1 column), scale code c:
//                  float4 at index (s * 2 + dir) * 128 + c = (d, 1/d, multiplier, 0)
//   kPartialsOffset  one 8-byte partial per 128 x 128 tile
constexpr int kCtrlStride = 64;
constexpr int kCtrlGroups = 16;
constexpr int64_t kCtrlOffset = 0;
constexpr int64_t kTablesOffset = (int64_t)kGroupSections * (kCtrlGroups + 1) * kCtrlStride * 4;
constexpr int64_t kTablesBytes = (int64_t)kGroupSections * 2 * 128 * 16;
constexpr int64_t kPartialsOffset = kTablesOffset + kTablesBytes;

}  // namespace mxq
