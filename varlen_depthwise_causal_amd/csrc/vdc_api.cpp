// Host side of libvdc.so: argument validation, launch planning and the
// C entry points declared in include/vdc.h.
//
// Nothing here allocates device memory, synchronizes, or reads device
// memory: cu_seqlens is only passed through to the kernels (documentation
// of flashinfer.cake_causal_conv1d_train_forward, Parameters cu_seqlens).

#include "vdc.h"

#include <algorithm>
#include <climits>
#include <atomic>
#include <stdint.h>

#include "vdc_internal.h"

namespace vdc {
namespace {

std::atomic<uint64_t> g_launches{0};

constexpr int64_t kMaxC = int64_t(1) << 20;
constexpr int64_t kMaxS = (int64_t(1) << 31) - 1;
// Smallest lane vector and largest row group: the size checks below are
// made for them.
constexpr int64_t kMinVec = 4;
constexpr int64_t kMaxGroup = kFwdGroup > kBwdGroup ? kFwdGroup : kBwdGroup;
// Compute units of the MI355X; plans are made for it.
constexpr int64_t kCUs = 256;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

bool valid_dtype(int d) { return d == VDC_F32 || d == VDC_BF16; }
size_t dtype_bytes(int d) { return d == VDC_BF16 ? 2 : 4; }

// Largest span, in rows, one wave can touch: the bands of its 64 lanes
// plus the halos.  Offsets inside that span must stay below 2^31 bytes.
int64_t wave_span_rows(int64_t nvec, int64_t rows) {
  return (ceil_div(64, nvec) + 1) * rows + 8;
}

// Largest span, in rows, of one workgroup: the bands of its kBlock lanes
// plus three halo rows on each side.  Its document starts must fit the
// workgroup's LDS bitmask.  (Column-block workgroups span kCbBands bands of
// fewer than kCbMaxRows rows, which always fit.)
int64_t block_span_rows(int64_t nvec, int64_t rows) {
  return (ceil_div(kBlock, nvec) + 1) * rows + 6;
}
bool block_fits(int64_t nvec, int64_t rows) {
  return block_span_rows(nvec, rows) < 32 * (int64_t)(kDocMaskWords - 1);
}

// Tokens per band T.  A band is covered by C/V lanes (V channels each), and
// the kernels are built to run one wave per SIMD with a deep load pipeline,
// so T is the smallest multiple of 2G for which all bands x C/V lanes fit
// one wave per SIMD of the MI355X (256 CUs x 4 SIMDs x 64 lanes): all waves
// start together and finish together.  Lowered if one wave's span of rows
// would not fit 32-bit offsets (C in the hundreds of thousands) or one
// workgroup's rows would not fit its document-start bitmask (small C with
// very long S); then there are more bands than SIMDs.
// A function of (direction, S, C) only.
int32_t pick_vec(int dir) { return dir == VDC_FWD ? kFwdVec : kBwdVec; }

int64_t pick_rows(int dir, int64_t S, int64_t C) {
  const int64_t nvec = C / pick_vec(dir);
  const int64_t step = 2 * (dir == VDC_FWD ? fwd_group(C) : kBwdGroup);
  const int64_t lanes_cap = kCUs * 4 * (dir == VDC_FWD ? kFwdWaves : kBwdWaves) * 64;
  const int64_t bands_cap = std::max<int64_t>(1, lanes_cap / nvec);
  int64_t rows = std::max<int64_t>(step, ceil_div(ceil_div(std::max<int64_t>(S, 1), bands_cap), step) * step);
  while (rows > step && (wave_span_rows(nvec, rows) * C * 2 >= (int64_t(1) << 31) ||
                         !block_fits(nvec, rows)))
    rows -= step;
  return rows;
}

Plan make_plan(int dir, int64_t S, int64_t C, int policy) {
  Plan p{};
  p.vec = pick_vec(dir);
  p.rows = (int32_t)pick_rows(dir, S, C);
  p.bands = (int32_t)ceil_div(S, p.rows);
  p.lanes = (int64_t)p.bands * (C / p.vec);
  p.blocks = (int32_t)ceil_div(p.lanes, kBlock);
  p.acc_bytes = dir == VDC_FWD ? 0 : (policy == VDC_SILU_GRAD_FP32 ? 8 : 4);
  p.red_blocks = dir == VDC_FWD ? 0 : (int32_t)ceil_div(5 * C, kRedOut);
  // Backward partial rows.  With 64 <= C/V < kBlock, a workgroup's lanes
  // cover every channel (one or two bands' worth, some channels twice), so
  // the workgroup sums its lanes' band totals in a fixed order and writes
  // one row: fewer rows than bands where bands are short.  With C/V a
  // multiple of 64 and at least kBlock, and bands shorter than kCbMaxRows,
  // lanes go in column blocks: a workgroup holds 64 vectors of kCbBands
  // consecutive bands (one per wave) and sums their totals into one row
  // segment, so a row stands for a group of kCbBands bands.  (With longer
  // bands the partials are small anyway, and the linear map keeps a
  // workgroup's waves on one band's rows, which measured faster where
  // documents are dense.)
  const int64_t nvec = C / p.vec;
  p.wg_rows = (dir == VDC_BWD && nvec >= 64 && nvec < kBlock) ? 1 : 0;
  p.cb = (dir == VDC_BWD && bwd_column_blocks(nvec, p.rows)) ? 1 : 0;
  if (p.cb) p.blocks = (int32_t)(ceil_div(p.bands, kCbBands) * (nvec / 64));
  p.prows = dir == VDC_FWD ? 0
            : p.wg_rows    ? p.blocks
            : p.cb         ? (int32_t)ceil_div(p.bands, kCbBands)
                           : p.bands;
  p.red_stage1 = (dir == VDC_FWD || p.prows <= kRedBlockRows)
                     ? 0
                     : (int32_t)ceil_div(p.prows, kRedBlockRows);
  return p;
}

// Lane and workgroup indices are 32-bit in the kernels.
bool plan_fits(const Plan& p) {
  return p.lanes <= (int64_t)INT32_MAX - kXcds * kBlock && padded_grid(p.blocks) <= INT32_MAX;
}

int check_sizes(int64_t S, int64_t C, int64_t num_docs) {
  if (C <= 0 || C % 8 != 0 || C > kMaxC) return VDC_EINVAL;
  if (S < 0 || S > kMaxS) return VDC_EINVAL;
  if (num_docs < 0 || num_docs > kMaxS - 1) return VDC_EINVAL;
  if (S > 0 && num_docs < 1) return VDC_EINVAL;
  // The planner must find a band size whose wave span fits 32-bit offsets.
  if (wave_span_rows(C / kMinVec, 2 * kMaxGroup) * C * 2 >= (int64_t(1) << 31)) return VDC_EINVAL;
  static_assert((kBlock / 2 + 2) * 2 * kMaxGroup + 6 < 32 * (kDocMaskWords - 1),
                "the smallest band must fit the document-start bitmask at C = 8");
  return VDC_OK;
}

}  // namespace
}  // namespace vdc

using namespace vdc;

extern "C" size_t workspace_bytes(int direction, int64_t S, int64_t C) {
  if (direction != VDC_FWD && direction != VDC_BWD) return 0;
  if (check_sizes(S, C, S > 0 ? 1 : 0) != VDC_OK) return 0;
  if (direction == VDC_FWD || S == 0) return 0;
  // Largest partial element over the policies (FP64 under the fp32 policy),
  // then the binary64 sums of the reduce's first stage when it has one.
  const Plan p = make_plan(VDC_BWD, S, C, VDC_SILU_GRAD_FP32);
  if (!plan_fits(p)) return 0;
  return ((size_t)p.prows + (size_t)p.red_stage1) * 5 * (size_t)C * 8;
}

extern "C" int conv1d_plan(int direction, int64_t S, int64_t C, int policy, int64_t out[11]) {
  if (!out) return VDC_EINVAL;
  if (direction != VDC_FWD && direction != VDC_BWD) return VDC_EINVAL;
  if (direction == VDC_BWD && policy != VDC_SILU_GRAD_BF16 && policy != VDC_SILU_GRAD_FP32)
    return VDC_EDTYPE;
  int rc = check_sizes(S, C, S > 0 ? 1 : 0);
  if (rc) return rc;
  const Plan p = make_plan(direction, S, C, policy);
  if (!plan_fits(p)) return VDC_EINVAL;
  out[0] = p.rows;
  out[1] = p.bands;
  out[2] = p.lanes;
  out[3] = p.blocks;
  out[4] = kBlock;
  out[5] = p.acc_bytes;
  out[6] = p.red_blocks;
  out[7] = kRedChunks;
  out[8] = p.vec;
  out[9] = p.red_stage1;
  out[10] = p.prows;
  return VDC_OK;
}

extern "C" int conv1d_fwd(const void* x, const void* weight, int w_dtype, const void* bias,
                          int b_dtype, const int32_t* cu_seqlens, int64_t num_docs, int64_t S,
                          int64_t C, void* y, void* workspace, size_t ws_bytes,
                          hipStream_t stream) {
  (void)workspace;
  (void)ws_bytes;
  int rc = check_sizes(S, C, num_docs);
  if (rc) return rc;
  if (!valid_dtype(w_dtype)) return VDC_EDTYPE;
  if (bias && !valid_dtype(b_dtype)) return VDC_EDTYPE;
  if (S == 0) return VDC_OK;  // nothing to compute, nothing enqueued
  if (!x || !weight || !cu_seqlens || !y) return VDC_EINVAL;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(weight, 16) || (bias && !aligned(bias, 16)))
    return VDC_EALIGN;
  const size_t act = (size_t)S * (size_t)C * 2;
  if (overlaps(x, act, y, act)) return VDC_EINVAL;
  if (overlaps(y, act, weight, (size_t)C * 4 * dtype_bytes(w_dtype))) return VDC_EINVAL;
  if (bias && overlaps(y, act, bias, (size_t)C * dtype_bytes(b_dtype))) return VDC_EINVAL;
  if (overlaps(y, act, cu_seqlens, (size_t)(num_docs + 1) * 4)) return VDC_EINVAL;

  const Plan plan = make_plan(VDC_FWD, S, C, 0);
  if (!plan_fits(plan)) return VDC_EINVAL;
  FwdArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.y = static_cast<uint16_t*>(y);
  a.w = weight;
  a.b = bias;
  a.cu = cu_seqlens;
  a.num_docs = (int32_t)num_docs;
  a.w_bf16 = w_dtype == VDC_BF16;
  a.b_bf16 = b_dtype == VDC_BF16;
  a.S = (int32_t)S;
  a.C = (int32_t)C;
  a.nvec = (int32_t)(C / plan.vec);
  a.rows = plan.rows;
  a.bands = plan.bands;
  a.blocks = plan.blocks;
  g_launches.fetch_add(1, std::memory_order_relaxed);
  return launch_fwd(plan, a, bias != nullptr, stream) == hipSuccess ? VDC_OK : VDC_EHIP;
}

namespace vdc {
namespace {

// The arguments of one backward call (conv1d_bwd and conv1d_bwd_noalloc
// share their validation and their launches).
struct BwdCall {
  const void* x;
  const void* weight;
  int w_dtype;
  const void* bias;
  int b_dtype;
  const int32_t* cu_seqlens;
  int64_t num_docs;
  const void* dy;
  int64_t S;
  int64_t C;
  int policy;
  void* dx;
  void* dweight;
  int dw_dtype;
  void* dbias;
  int db_dtype;
};

// Every check that does not involve the workspace.
int bwd_check(const BwdCall& c) {
  int rc = check_sizes(c.S, c.C, c.num_docs);
  if (rc) return rc;
  if (!valid_dtype(c.w_dtype) || !valid_dtype(c.dw_dtype)) return VDC_EDTYPE;
  if (c.bias && !valid_dtype(c.b_dtype)) return VDC_EDTYPE;
  if (c.dbias && !valid_dtype(c.db_dtype)) return VDC_EDTYPE;
  if (c.policy != VDC_SILU_GRAD_BF16 && c.policy != VDC_SILU_GRAD_FP32) return VDC_EDTYPE;
  if (c.dbias && !c.bias) return VDC_ENOBIAS;
  if (!c.dweight) return VDC_EINVAL;
  if (!aligned(c.dweight, dtype_bytes(c.dw_dtype)) ||
      (c.dbias && !aligned(c.dbias, dtype_bytes(c.db_dtype))))
    return VDC_EALIGN;
  const size_t dw_n = (size_t)c.C * 4 * dtype_bytes(c.dw_dtype);
  const size_t db_n = c.dbias ? (size_t)c.C * dtype_bytes(c.db_dtype) : 0;
  if (overlaps(c.dweight, dw_n, c.dbias, db_n)) return VDC_EINVAL;
  if (c.S == 0) return VDC_OK;
  if (!c.x || !c.weight || !c.cu_seqlens || !c.dy || !c.dx) return VDC_EINVAL;
  if (!aligned(c.x, 16) || !aligned(c.dy, 16) || !aligned(c.dx, 16) || !aligned(c.weight, 16) ||
      (c.bias && !aligned(c.bias, 16)))
    return VDC_EALIGN;
  const size_t act = (size_t)c.S * (size_t)c.C * 2;
  const size_t w_n = (size_t)c.C * 4 * dtype_bytes(c.w_dtype);
  const size_t b_n = c.bias ? (size_t)c.C * dtype_bytes(c.b_dtype) : 0;
  const size_t cu_n = (size_t)(c.num_docs + 1) * 4;
  const void* ins[5] = {c.x, c.dy, c.weight, c.bias, c.cu_seqlens};
  const size_t in_n[5] = {act, act, w_n, b_n, cu_n};
  void* outs[3] = {c.dx, c.dweight, c.dbias};
  const size_t out_n[3] = {act, dw_n, db_n};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 5; ++i)
      if (overlaps(outs[o], out_n[o], ins[i], in_n[i])) return VDC_EINVAL;
    for (int q = o + 1; q < 3; ++q)
      if (overlaps(outs[o], out_n[o], outs[q], out_n[q])) return VDC_EINVAL;
  }
  return plan_fits(make_plan(VDC_BWD, c.S, c.C, c.policy)) ? VDC_OK : VDC_EINVAL;
}

// The workspace must not overlap any tensor argument.
bool workspace_overlaps(const BwdCall& c, const void* ws, size_t need) {
  const size_t act = (size_t)c.S * (size_t)c.C * 2;
  const void* p[8] = {c.x, c.dy, c.weight, c.bias, c.cu_seqlens, c.dx, c.dweight, c.dbias};
  const size_t n[8] = {act, act, (size_t)c.C * 4 * dtype_bytes(c.w_dtype),
                       c.bias ? (size_t)c.C * dtype_bytes(c.b_dtype) : 0,
                       (size_t)(c.num_docs + 1) * 4, act,
                       (size_t)c.C * 4 * dtype_bytes(c.dw_dtype),
                       c.dbias ? (size_t)c.C * dtype_bytes(c.db_dtype) : 0};
  for (int i = 0; i < 8; ++i)
    if (overlaps(ws, need, p[i], n[i])) return true;
  return false;
}

// S == 0: no token, dx is empty and both gradients are zero.  No main or
// reduce kernel runs; under graph capture the zeros come from the reduce
// kernel run over zero partial rows instead of a memset node.
int bwd_zero(const BwdCall& c, hipStream_t stream) {
  const size_t dw_n = (size_t)c.C * 4 * dtype_bytes(c.dw_dtype);
  const size_t db_n = c.dbias ? (size_t)c.C * dtype_bytes(c.db_dtype) : 0;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return VDC_EHIP;
  if (cap == hipStreamCaptureStatusNone) {
    if (hipMemsetAsync(c.dweight, 0, dw_n, stream) != hipSuccess) return VDC_EHIP;
    if (c.dbias && hipMemsetAsync(c.dbias, 0, db_n, stream) != hipSuccess) return VDC_EHIP;
    return VDC_OK;
  }
  Plan plan{};
  plan.red_blocks = (int32_t)ceil_div(5 * c.C, kRedOut);
  ReduceArgs r{};
  r.part = nullptr;
  r.dw = c.dweight;
  r.db = c.dbias;
  r.P = 0;
  r.C = (int32_t)c.C;
  r.dw_bf16 = c.dw_dtype == VDC_BF16;
  r.db_bf16 = c.db_dtype == VDC_BF16;
  g_launches.fetch_add(1, std::memory_order_relaxed);
  return launch_bwd_reduce(plan, r, false, stream) == hipSuccess ? VDC_OK : VDC_EHIP;
}

// The main kernel, then the fixed-order reduce, on a checked call (S > 0)
// with a workspace of at least workspace_bytes(VDC_BWD, S, C) bytes.
int bwd_enqueue(const BwdCall& c, void* workspace, hipStream_t stream) {
  const bool fp32_policy = c.policy == VDC_SILU_GRAD_FP32;
  const Plan plan = make_plan(VDC_BWD, c.S, c.C, c.policy);
  BwdArgs a{};
  a.x = static_cast<const uint16_t*>(c.x);
  a.dy = static_cast<const uint16_t*>(c.dy);
  a.dx = static_cast<uint16_t*>(c.dx);
  a.w = c.weight;
  a.b = c.bias;
  a.cu = c.cu_seqlens;
  a.part = workspace;
  a.num_docs = (int32_t)c.num_docs;
  a.w_bf16 = c.w_dtype == VDC_BF16;
  a.b_bf16 = c.b_dtype == VDC_BF16;
  a.S = (int32_t)c.S;
  a.C = (int32_t)c.C;
  a.nvec = (int32_t)(c.C / plan.vec);
  a.rows = plan.rows;
  a.bands = plan.bands;
  a.blocks = plan.blocks;
  a.wg_rows = plan.wg_rows;
  a.cb = plan.cb;
  g_launches.fetch_add(1, std::memory_order_relaxed);
  if (launch_bwd_main(plan, a, c.bias != nullptr, fp32_policy, stream) != hipSuccess)
    return VDC_EHIP;

  ReduceArgs r{};
  r.part = workspace;
  r.dw = c.dweight;
  r.db = c.dbias;
  r.P = plan.prows;
  r.C = (int32_t)c.C;
  r.dw_bf16 = c.dw_dtype == VDC_BF16;
  r.db_bf16 = c.db_dtype == VDC_BF16;
  bool part_f64 = fp32_policy;
  if (plan.red_stage1 > 0) {
    // Many partial rows: sums of kRedBlockRows-row ranges first, into the
    // workspace after the largest partial-row area, then one pass over them.
    r.inter = static_cast<char*>(workspace) + (size_t)plan.prows * 5 * (size_t)c.C * 8;
    g_launches.fetch_add(1, std::memory_order_relaxed);
    if (launch_bwd_reduce_rows(plan, r, part_f64, stream) != hipSuccess) return VDC_EHIP;
    r.part = r.inter;
    r.P = plan.red_stage1;
    part_f64 = true;
  }
  g_launches.fetch_add(1, std::memory_order_relaxed);
  return launch_bwd_reduce(plan, r, part_f64, stream) == hipSuccess ? VDC_OK : VDC_EHIP;
}

}  // namespace
}  // namespace vdc

extern "C" int conv1d_bwd(const void* x, const void* weight, int w_dtype, const void* bias,
                          int b_dtype, const int32_t* cu_seqlens, int64_t num_docs,
                          const void* dy, int64_t S, int64_t C, int policy, void* dx,
                          void* dweight, int dw_dtype, void* dbias, int db_dtype,
                          void* workspace, size_t ws_bytes, hipStream_t stream) {
  const BwdCall c{x, weight, w_dtype, bias, b_dtype, cu_seqlens, num_docs, dy, S, C, policy,
                  dx, dweight, dw_dtype, dbias, db_dtype};
  int rc = bwd_check(c);
  if (rc) return rc;
  if (S == 0) return bwd_zero(c, stream);
  const size_t need = workspace_bytes(VDC_BWD, S, C);
  if (!workspace || ws_bytes < need) return VDC_EWORKSPACE;
  if (!aligned(workspace, 16)) return VDC_EALIGN;
  if (workspace_overlaps(c, workspace, need)) return VDC_EINVAL;
  return bwd_enqueue(c, workspace, stream);
}

extern "C" size_t conv1d_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" int conv1d_bwd_noalloc(const void* x, const void* weight, int w_dtype,
                                  const void* bias, int b_dtype, const int32_t* cu_seqlens,
                                  int64_t num_docs, const void* dy, int64_t S, int64_t C,
                                  int policy, void* dx, void* dweight, int dw_dtype, void* dbias,
                                  int db_dtype, hipStream_t stream) {
  const BwdCall c{x, weight, w_dtype, bias, b_dtype, cu_seqlens, num_docs, dy, S, C, policy,
                  dx, dweight, dw_dtype, dbias, db_dtype};
  int rc = bwd_check(c);
  if (rc) return rc;
  if (S == 0) return bwd_zero(c, stream);
  // The same workspace layout as conv1d_bwd, in the library's own device
  // array: refused before anything is enqueued when it does not fit.
  if (workspace_bytes(VDC_BWD, S, C) > kScratchBytes) return VDC_ESCRATCH;
  // The stream's device holds the kernels' copy of the array.
  int dev = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess) return VDC_EHIP;
  void* scratch = nullptr;
  if (scratch_pointer(dev, &scratch) != hipSuccess || !scratch) return VDC_EHIP;
  return bwd_enqueue(c, scratch, stream);
}

extern "C" const char* conv1d_status_string(int status) {
  switch (status) {
    case VDC_OK: return "ok";
    case VDC_EINVAL: return "invalid argument (size, missing pointer or overlapping buffers)";
    case VDC_EDTYPE: return "unknown dtype or SiLU-derivative policy";
    case VDC_EALIGN: return "misaligned tensor pointer";
    case VDC_EWORKSPACE: return "workspace missing or too small";
    case VDC_ENOBIAS: return "dbias requested without a bias";
    case VDC_EHIP: return "HIP runtime error";
    case VDC_ESCRATCH:
      return "the call needs more scratch than conv1d_bwd_noalloc holds "
             "(see conv1d_noalloc_scratch_bytes); use conv1d_bwd with a workspace";
    default: return "unknown status";
  }
}

extern "C" uint64_t conv1d_launch_count(void) {
  return g_launches.load(std::memory_order_relaxed);
}
