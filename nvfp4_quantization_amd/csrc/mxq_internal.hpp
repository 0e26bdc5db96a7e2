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
// Three kernels on the caller's stream: the first rotates 64 rows per 256-thread
// work-group and stores the work-group's max |y| as a partial; a one-work-group
// kernel folds the partials into the tensor scale and writes the scale table; the
// third rotates again and encodes.  With a supplied amax the first is skipped and
// the second takes the supplied value.  The kernels meet only through the stream
// order, so the workspace holds no state between calls.
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
    float4* table;                    // workspace: 128 scale-table entries
    float* partials;                  // workspace: one max per work-group
};
hipError_t launch_hadamard_quant_nvfp4(const DsaNvfp4Args& a, hipStream_t stream);
// Workspace layout of the DSA NVFP4 call (byte offsets): the scale table, then one
// partial per work-group.
constexpr int64_t kDsaTableOffset = 0;
constexpr int64_t kDsaPartialsOffset = kDsaTableOffset + 128 * 16;

// ---------------------------------------------------------------- grouped NVFP4
// One launch group per at most kGroupSections sections.  A group runs three kernels
// on the caller's stream (with caller-supplied maxima, the last two):
//   amax    one work-group per band of 16 rows x 1024 columns: max |x| and
//           max |H16 D x| of the band, one partial each;
//   scales  one work-group per section: folds the section's partials (or takes
//           the supplied maxima) into the two tensor scales and writes the
//           section's (d, 1/d, multiplier) tables;
//   quant   one wave per tile: every output of the tile.
// They meet only through the stream order, so the workspace holds no state between
// calls of this form.  The single-read form (one kernel) replaces all three when
// the whole group is resident on the chip at once.
constexpr int kGroupSections = 32;
constexpr int kTileRows = 128;        // token tile
constexpr int kTileCols = 128;        // column tile
constexpr int kAmaxRows = 16;         // amax pass: a work-group's band of rows
constexpr int kAmaxCols = 1024;       //   and of columns (256 threads x kAmaxWords BF16 pairs)
constexpr int kAmaxWords = kAmaxCols / 512;
static_assert(kAmaxWords == 2 || kAmaxWords == 4, "a thread loads 8 or 16 bytes of each row");

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
    float4* tables;                   // workspace: per-section scale tables
    uint64_t* partials;               // workspace: one (row, column) amax pair per amax work-group
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
// slots: the single-read form's partial words (zero between calls); status: its error word.
hipError_t launch_nvfp4_group(const Nvfp4Group& g, uint32_t flags, uint32_t* slots, uint32_t* status, hipStream_t stream);
}  // namespace mxq
#include "mxq.h"
namespace mxq {
// The grouped call's argument checks without the workspace (mxq_api.cpp): MXQ_OK and
// the total rows, or the first error; nothing is enqueued.
mxq_status grouped_check(const uint16_t* x_bf16, int64_t k, const int64_t* split_sections, int64_t num_sections,
                         uint32_t flags, const mxq_nvfp4_out* rowwise, const mxq_nvfp4_out* columnwise,
                         const mxq_fp8_out* fp8_rowwise, const mxq_amax* amax, int64_t* total_rows);
// The quant kernel's variant families (one translation unit each): nearest-even or
// stochastic rounding, with or without measured maxima out (supplied maxima).
hipError_t launch_quant_rne(const Nvfp4Group& g, uint32_t flags, hipStream_t stream);
hipError_t launch_quant_sr(const Nvfp4Group& g, uint32_t flags, hipStream_t stream);
hipError_t launch_quant_rne_aout(const Nvfp4Group& g, uint32_t flags, hipStream_t stream);
hipError_t launch_quant_sr_aout(const Nvfp4Group& g, uint32_t flags, hipStream_t stream);

// The single-read form of a launch group (mxq_nvfp4_fused.hpp): one 4-wave
// work-group per item (4 adjacent column tiles of one token tile).  Sections are
// processed in the order `order`, the items of position i being istart[i] ..
// istart[i + 1] - 1.
constexpr int kFusedMaxItems = 1024;           // items of a launch group (partial words, deferred lists)
struct Nvfp4Fused {
    uint32_t* slots;                  // workspace: one partial word per item, zero between calls
    uint32_t* err;                    // workspace: set to 1 when a wait gave up
    int32_t n_items;
    int32_t n_cgroups;                // items per token tile: k / 512
    int32_t n_order;                  // non-empty sections of the group
    int32_t istart[kGroupSections + 1];
    uint8_t order[kGroupSections];
};
// A partial word: bit 31 present, bits 16..30 the BF16 bits of the item's column
// maximum / 4, bits 0..14 those of its row maximum, bit 15 deferred.
constexpr uint32_t kSlotPresent = 0x80000000u;
constexpr uint32_t kSlotDeferred = 0x00008000u;
// Waits of the single-read kernel, in ticks of the 100 MHz constant clock: an item
// defers after kDeferTicks (about 0.66 ms; a call takes tens of microseconds), and
// the last item's wait for its section's partials (which always ends) gives up
// after kWaitTicks (about 21 ms) and sets the error word.
#ifndef MXQ_FUSED_DEFER_TICKS
#define MXQ_FUSED_DEFER_TICKS (1ull << 16)
#endif
constexpr uint64_t kDeferTicks = MXQ_FUSED_DEFER_TICKS;   // 0 in the deferral test build only
constexpr uint64_t kWaitTicks = 1ull << 21;
hipError_t launch_fused_rne(const Nvfp4Group& g, const Nvfp4Fused& f, uint32_t flags, hipStream_t stream);
hipError_t launch_fused_sr(const Nvfp4Group& g, const Nvfp4Fused& f, uint32_t flags, hipStream_t stream);
// Resident work-groups per CU of the single-read kernel for these flags.
hipError_t fused_blocks_per_cu_rne(uint32_t flags, int* blocks);
hipError_t fused_blocks_per_cu_sr(uint32_t flags, int* blocks);

// Workspace layout (byte offsets):
//   kStatusOffset  two 256-byte lines; word 0 is the single-read form's error word
//   kTablesOffset  section s, direction dir (0 row, 1 column), scale code c:
//                  float4 at index (s * 2 + dir) * 128 + c = (d, 1/d, multiplier, 0)
//   kSlotsOffset   the single-read form's partial words, one per item (at most
//                  kFusedMaxItems), zero between calls; the three-kernel form never
//                  touches them, so calls of either form can share a workspace
//   kPartialsOffset  one 8-byte partial per amax work-group: per 16 rows and
//                  kAmaxCols = 1024 columns (or part) of the largest launch group
constexpr int64_t kStatusOffset = 0;
constexpr int64_t kTablesOffset = kStatusOffset + 512;
constexpr int64_t kTablesBytes = (int64_t)kGroupSections * 2 * 128 * 16;
constexpr int64_t kSlotsOffset = kTablesOffset + kTablesBytes;
constexpr int64_t kPartialsOffset = kSlotsOffset + 4 * (int64_t)kFusedMaxItems;

}  // namespace mxq
