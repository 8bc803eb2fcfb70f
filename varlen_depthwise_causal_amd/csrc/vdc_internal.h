// Internal interface between the host entry points (vdc_api.cpp) and the
// HIP kernels (vdc_kernels.hip).  Not installed; include/vdc.h is the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace vdc {

// Waves per SIMD each kernel is built for (register budget) and planned
// for: one, with a deep double-buffered load pipeline per wave.
#ifndef VDC_FWD_WAVES
#define VDC_FWD_WAVES 1
#endif
#ifndef VDC_BWD_WAVES
#define VDC_BWD_WAVES 1
#endif
constexpr int kFwdWaves = VDC_FWD_WAVES;
constexpr int kBwdWaves = VDC_BWD_WAVES;
// Channels one lane owns: 4 BF16 values, one 8-byte vector per row.
constexpr int kFwdVec = 4;
constexpr int kBwdVec = 4;
// Threads per workgroup of the main kernels (four wave64).
constexpr int kBlock = 256;
// Rows per load group (two groups are in flight per lane).
#ifndef VDC_FWD_GROUP
#define VDC_FWD_GROUP 16
#endif
#ifndef VDC_BWD_GROUP
#define VDC_BWD_GROUP 8
#endif
constexpr int kFwdGroup = VDC_FWD_GROUP;
constexpr int kBwdGroup = VDC_BWD_GROUP;
// The forward's row group for rows that are not a multiple of 128 bytes
// with C < 1024 (Stress's C = 520): shorter groups there.
#ifndef VDC_FWD_GROUP_SHORT
#define VDC_FWD_GROUP_SHORT 8
#endif
constexpr int kFwdGroupShort = VDC_FWD_GROUP_SHORT;
inline int fwd_group(int64_t C) { return ((C * 2) % 128 != 0 && C < 1024) ? kFwdGroupShort : kFwdGroup; }
// Document-start bitmask of one workgroup, in 32-bit LDS words: the rows a
// workgroup touches (its bands and three halo rows on each side) must span
// fewer than 32 * (kDocMaskWords - 1) rows.
constexpr int kDocMaskWords = 1024;

// Workgroup placement: 1 = neighbouring workgroups of the lane order on one
// XCD (grid padded to a multiple of 8), 0 = hardware order.
#ifndef VDC_XCD_REMAP
#define VDC_XCD_REMAP 1
#endif
constexpr int kXcds = 8;

inline int64_t padded_grid(int64_t blocks) {
  return VDC_XCD_REMAP ? (blocks + kXcds - 1) / kXcds * kXcds : blocks;
}

// Reduce kernels: outputs per workgroup and row chunks (one wave each).
constexpr int kRedOut = 64;
constexpr int kRedChunks = 8;
// Partial rows one first-stage reduce workgroup sums.  With more rows than
// this the reduce runs in two stages: workgroups of kRedBlockRows rows
// each, then one pass over their sums; with fewer, one pass.
constexpr int kRedBlockRows = 2048;
// Backward lanes in column blocks (C / V a multiple of 64 and at least
// kBlock, bands shorter than kCbMaxRows): a workgroup holds 64 channel
// vectors of kCbBands consecutive bands, one band per wave, and writes one
// partial row for them.  Its rows, kCbBands * rows + 6 < 4103, always fit
// the document-start bitmask.
constexpr int kCbBands = 4;
constexpr int kCbMaxRows = 1024;
inline bool bwd_column_blocks(int64_t nvec, int64_t rows) {
  return nvec >= kBlock && nvec % 64 == 0 && rows < kCbMaxRows;
}
static_assert(kCbBands * kCbMaxRows + 6 < 32 * (kDocMaskWords - 1),
              "column-block workgroups must fit the document-start bitmask");

// Everything a launch needs, decided on the host from (direction, S, C,
// policy) alone - never from tensor contents.
struct Plan {
  int32_t vec;         // channels per lane (V)
  int32_t rows;        // tokens per band (T)
  int32_t bands;       // ceil(S / T)
  int64_t lanes;       // bands * C / V
  int32_t blocks;      // main-kernel workgroups
  int32_t acc_bytes;   // backward partial element: 4 (FP32) or 8 (FP64)
  int32_t red_blocks;  // reduce workgroups per row range (kRedOut outputs each)
  int32_t red_stage1;  // first-stage row ranges (0: the reduce is one pass)
  int32_t wg_rows;     // backward: 1 = one partial row per workgroup, 0 = per band
  int32_t cb;          // backward: 1 = lanes in column blocks of kCbBands bands
  int32_t prows;       // backward partial rows: blocks (wg_rows), band groups (cb) or bands
};

struct FwdArgs {
  const uint16_t* x;
  uint16_t* y;
  const void* w;
  const void* b;
  const int32_t* cu;
  int32_t num_docs;
  int32_t w_bf16;
  int32_t b_bf16;
  int32_t S;
  int32_t C;
  int32_t nvec;        // C / V
  int32_t rows;        // T
  int32_t bands;
  int32_t blocks;      // workgroups with lanes (the grid may be padded)
};

struct BwdArgs {
  const uint16_t* x;
  const uint16_t* dy;
  uint16_t* dx;
  const void* w;
  const void* b;
  const int32_t* cu;
  void* part;          // [P][5][C] of FP32 or FP64 (P = Plan::prows)
  int32_t num_docs;
  int32_t w_bf16;
  int32_t b_bf16;
  int32_t S;
  int32_t C;
  int32_t nvec;
  int32_t rows;
  int32_t bands;
  int32_t blocks;      // workgroups with lanes (the grid may be padded)
  int32_t wg_rows;     // 1: one partial row per workgroup (see Plan)
  int32_t cb;          // 1: column-block lanes, one partial row per band group
};

struct ReduceArgs {
  const void* part;    // [P][5][C] rows to sum
  void* inter;         // stage 1 output: [ceil(P / kRedBlockRows)][5][C] binary64
  void* dw;            // [C][4]
  void* db;            // [C] or null
  int32_t P;
  int32_t C;
  int32_t dw_bf16;
  int32_t db_bf16;
};

// Bytes of the library's own device array that conv1d_bwd_noalloc uses as
// its workspace (one copy per GPU, held until the process ends).  Every
// backward whose launch plan keeps at most one band per lane of a full
// machine (bands * C <= 2^18) needs at most 10.5 MB of partial rows; 16 MiB
// covers those with the reduce's first-stage sums on top.
constexpr size_t kScratchBytes = size_t(16) << 20;

// Device address of that array on `device` (looked up once per device,
// with the device current, then cached).
hipError_t scratch_pointer(int device, void** out);

// Launchers (return the hipError_t of the launch).
hipError_t launch_fwd(const Plan& plan, const FwdArgs& a, bool has_bias, hipStream_t s);
hipError_t launch_bwd_main(const Plan& plan, const BwdArgs& a, bool has_bias, bool fp32_policy,
                           hipStream_t s);
hipError_t launch_bwd_reduce(const Plan& plan, const ReduceArgs& a, bool part_f64, hipStream_t s);
// First stage of a two-stage reduce: part rows -> inter (binary64).
hipError_t launch_bwd_reduce_rows(const Plan& plan, const ReduceArgs& a, bool part_f64,
                                  hipStream_t s);

}  // namespace vdc
