// HIP kernels for gfx950: packed variable-length width-4 depthwise causal
// convolution + SiLU, training forward and backward.
//
// The operation is the one documented on the pages of
// flashinfer.cake_causal_conv1d_train (cake_causal_conv1d_train_forward:
// Returns; cake_causal_conv1d_train_backward: Description, Returns).  It is
// a 4-tap stencil along the token axis followed by an elementwise SiLU, so
// it is bound by HBM traffic and VALU issue, not by matrix throughput: no
// MFMA here.
//
// Work decomposition (same for both main kernels):
//  * A lane owns V = 4 consecutive BF16 channels (one 8-byte vector) and a
//    band of T consecutive tokens, and walks the band row by row.  Lanes are
//    numbered (band, vector) -> band * (C/4) + vector, so the 64 lanes of a
//    wave read 64 consecutive vectors of a row (fully coalesced) and, when
//    C/4 is not a multiple of 64, simply continue into the next band.  The
//    backward of short bands with C a multiple of 256 numbers them in
//    column blocks instead (lane_coords_cb): the same 64 vectors per wave,
//    four bands per workgroup, so that one partial row covers four bands.
//  * The kernels run one wave per SIMD and the host picks T so that all
//    waves fit the machine at once; each wave double-buffers groups of
//    rows in registers and stores a group's outputs after its last row; the
//    forward and the "bf16" backward pace themselves once per pair of
//    groups (wait_vm).
//  * A lane keeps the previous three rows of x in registers; at a document
//    start the window is cleared, which is exactly the zero history the
//    forward prescribes, so no tap needs a mask.  Each workgroup marks the
//    document starts of its rows in an LDS bitmask; a wave whose lanes have
//    no start near a group takes a plain path without any check.
//  * Tensors are addressed through buffer resources based at the wave's
//    first row, with 32-bit per-lane offsets: rows outside [0, S) and
//    negative offsets read as zero and their stores are dropped by the
//    hardware range check.
//  * Arithmetic is FP32 with one fixed evaluation order for the
//    preactivation, shared by the forward and the backward recompute, so
//    both see the same bits of p.

#include <hip/hip_runtime.h>

#include <climits>
#include <mutex>
#include <stdint.h>

#include "vdc_internal.h"
#include "vdc_lines.h"
#include "vdc_search.h"

namespace vdc {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr float kLog2e = 1.4426950408889634f;
// Below this preactivation sigmoid() leaves the binary32 normal range on
// the fast path (exp overflow, or a flushed reciprocal); such values take
// the scaled evaluation instead.
constexpr float kDeep = -80.0f;
// Word 3 of a raw (untyped, unswizzled) gfx9 buffer resource.
constexpr int kRsrcWord3 = 0x00020000;
// Cache-policy bits of the activation accesses.  Every activation byte is
// used once per call, so where a wave's 512-byte row pieces cover whole
// 128-byte cache lines (rows a multiple of 128 bytes, C a multiple of 64)
// they stream with "nt" (non-temporal).  Otherwise two neighbouring waves
// share the lines at their boundary, and plain accesses, which let the
// line stay in L2 for the second wave, move about 25% fewer bytes; the
// forward's stores still stream the lines inside a wave's piece
// (whole_line_bits).
constexpr int kStream = 2;
constexpr int kPlain = 0;

// ---------------------------------------------------------------- BF16 --

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Two FP32 -> packed BF16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2 h = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// FP32 -> BF16 bits, round to nearest even, by integer arithmetic; exact for
// subnormal inputs too (used on the rare deep-negative path).
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// FP64 -> BF16 bits, round to nearest even with a single rounding: round to
// binary32 with round-to-odd (the sticky bit kept in the last place), then
// to BF16 with round-to-nearest-even.
__device__ __forceinline__ uint16_t bf16_bits_from_f64(double d) {
  float f = (float)d;
  double back = (double)f;
  uint32_t u = __float_as_uint(f);
  if (back != d) {
    if (__builtin_fabs(back) > __builtin_fabs(d)) u -= 1u;  // toward zero
    u |= 1u;
  }
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// ------------------------------------------------------ lane vectors --

template <int V> struct Vec;
template <> struct Vec<4> {
  typedef u32x2 raw;
  __device__ static __forceinline__ raw zero() { return (raw){0u, 0u}; }
};

// Activation rows of one lane (8 bytes) with cache policy kAux.
template <int kAux> struct Io {
  __device__ static __forceinline__ u32x2 load(rsrc_t r, int32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kAux);
  }
  __device__ static __forceinline__ void store(rsrc_t r, int32_t off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kAux);
  }
};

template <int V>
__device__ __forceinline__ void unpack(typename Vec<V>::raw v, float (&f)[V]) {
#pragma unroll
  for (int d = 0; d < V / 2; ++d) {
    f[2 * d] = bf_lo(v[d]);
    f[2 * d + 1] = bf_hi(v[d]);
  }
}

template <int V>
__device__ __forceinline__ typename Vec<V>::raw pack(const float (&f)[V]) {
  typename Vec<V>::raw r = Vec<V>::zero();
#pragma unroll
  for (int d = 0; d < V / 2; ++d) r[d] = pack2(f[2 * d], f[2 * d + 1]);
  return r;
}

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

// Bytes from row `row` to the end of an [S][C] BF16 tensor, clamped below
// 2^31.  The clamp keeps every negative 32-bit offset out of range, so a
// load there reads zero and a store there is dropped, without a memory
// access; the host keeps a wave's whole span below 2^31 bytes, so the clamp
// never cuts a row the wave uses.
__device__ __forceinline__ uint32_t span_bytes(int32_t S, int32_t C, int32_t row) {
  uint64_t rem = (uint64_t)(int64_t)(S - row) * (uint64_t)C * 2u;
  return rem > 0x7fffffffull ? 0x7fffffffu : (uint32_t)rem;
}

// Offset of "no row": loads there read zero, stores are dropped (see
// span_bytes); kNoRow + g * row_bytes stays negative for every row group.
// The main loops issue the same memory instructions on every path and send
// the accesses they do not need here.  The compiler counts outstanding
// accesses per path to place its waits, and takes the smallest count where
// paths meet: an access skipped on one path would make every later wait
// also wait for younger accesses that are still in flight.
constexpr int32_t kNoRow = INT32_MIN;

// Wait until at most N vector memory accesses of this wave are in flight
// (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt at their
// maxima, so they are not waited for).
//
// The forward and the "bf16" backward use it to pace themselves: once per
// pair of row groups a wave waits until everything but the next group's
// loads has retired, stores included.  Without that wait each wave runs at
// its own pace, the rows in flight across the machine drift apart, and the
// memory side loses efficiency: at 8 KiB rows the L2's read latency to
// memory grows by about a quarter, its DRAM credit stalls grow four- to
// fivefold, and the kernels lose 5-11%.  Issuing the next group's loads before the stores of the
// group just computed (more accesses in flight per wave) is slower still.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// ------------------------------------------------------- parameters --

// Parameters of the lane's channels c0 .. c0+V-1, loaded raw and unpacked
// later, so that the loads can be issued first without their values being
// waited for: weight [C][4] (FP32: one 16-byte vector per channel; BF16:
// 8 bytes per channel, two channels per 16-byte vector) and bias [C] (FP32:
// 16 bytes per 4 channels; BF16: 8 bytes).
template <int V>
struct ParamRaw {
  u32x4 w[V];
  u32x4 b[V / 4];
};

template <int V>
__device__ __forceinline__ void load_params(const void* w, int w_bf16, const void* b, int b_bf16,
                                            bool has_bias, uint32_t c0, ParamRaw<V>& raw) {
  static_assert(V == 4, "four channels per lane");
  // The same loads for either dtype, at offsets chosen without a branch:
  // a branch here makes the compiler copy loaded registers at its join, and
  // each copy waits for its load.  BF16 weights take 32 bytes (two 16-byte
  // loads, each issued twice); a BF16 bias 8 bytes (issued twice).
  const char* pw = reinterpret_cast<const char*>(w);
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const uint32_t off = w_bf16 ? c0 * 8u + 16u * (uint32_t)(i & 1) : c0 * 16u + 16u * (uint32_t)i;
    raw.w[i] = *reinterpret_cast<const u32x4*>(pw + off);
  }
  if (has_bias) {
    const char* pb = reinterpret_cast<const char*>(b);
    const uint32_t off0 = b_bf16 ? c0 * 2u : c0 * 4u;
    const uint32_t off1 = b_bf16 ? c0 * 2u : c0 * 4u + 8u;
    const u32x2 lo = *reinterpret_cast<const u32x2*>(pb + off0);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(pb + off1);
    raw.b[0] = (u32x4){lo.x, lo.y, hi.x, hi.y};
  } else {
    raw.b[0] = (u32x4){0u, 0u, 0u, 0u};
  }
}

template <int V>
__device__ __forceinline__ void unpack_params(const ParamRaw<V>& raw, int w_bf16, int b_bf16,
                                              float (&wk)[4][V], float (&bv)[V]) {
#pragma unroll
  for (int i = 0; i < V; ++i) {
    if (!w_bf16) {
      wk[0][i] = __uint_as_float(raw.w[i].x);
      wk[1][i] = __uint_as_float(raw.w[i].y);
      wk[2][i] = __uint_as_float(raw.w[i].z);
      wk[3][i] = __uint_as_float(raw.w[i].w);
    } else {
      const u32x4 v = raw.w[(i / 2) & 1];
      const uint32_t lo = (i & 1) ? v.z : v.x, hi = (i & 1) ? v.w : v.y;
      wk[0][i] = bf_lo(lo);
      wk[1][i] = bf_hi(lo);
      wk[2][i] = bf_lo(hi);
      wk[3][i] = bf_hi(hi);
    }
  }
#pragma unroll
  for (int q = 0; q < V / 4; ++q) {
    const u32x4 v = raw.b[q];
    if (!b_bf16) {
      bv[4 * q + 0] = __uint_as_float(v.x);
      bv[4 * q + 1] = __uint_as_float(v.y);
      bv[4 * q + 2] = __uint_as_float(v.z);
      bv[4 * q + 3] = __uint_as_float(v.w);
    } else {
      bv[4 * q + 0] = bf_lo(v.x);
      bv[4 * q + 1] = bf_hi(v.x);
      bv[4 * q + 2] = bf_lo(v.y);
      bv[4 * q + 3] = bf_hi(v.y);
    }
  }
}

// ------------------------------------------------- document starts --
//
// A row t is a document start when t equals a value of cu_seqlens below S
// (an empty document repeats its successor's start).  Each workgroup marks
// the starts among the rows its lanes touch in an LDS bitmask.  With fewer
// documents than threads every thread reads one entry of cu_seqlens; with
// more, the first wave finds the range of entries that fall in the rows
// with two 64-ary searches, and the whole workgroup reads that range.  A
// lane then reads the starts of a group of rows with two LDS loads,
// however many documents it holds.  The host sizes bands so that a
// workgroup's rows fit the bitmask.

// First index i in [0, n) with cu[i] >= v (n if none), by a whole wave:
// each round probes 64 evenly spaced entries and keeps the bracket, so the
// range shrinks 64-fold per dependent load.  Terminates for any contents;
// the bracket arithmetic is 64-bit (vdc_search.h), so every probe lies in
// [0, n) up to n = 2^31 - 1.
__device__ __forceinline__ int32_t wave_lower_bound(const int32_t* cu, int32_t n, int32_t v) {
  const int lane = (int)(threadIdx.x & 63);
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t step = search_step(lo, hi);
    const int64_t idx = search_probe(lo, hi, step, lane);
    const bool less = idx >= 0 && cu[idx] < v;
    const uint64_t ball = __ballot(less);
    const int c = ~ball == 0 ? 64 : (int)__builtin_ctzll(~ball);
    search_narrow(lo, hi, step, c);
  }
  return (int32_t)lo;
}

struct DocMask {
  uint32_t bits[kDocMaskWords + 1];  // bit j: row row_lo + j starts a document
  int32_t row_lo;
  int32_t idx_lo, idx_hi;            // cu_seqlens entries that fall in the rows
};

// With fewer documents than threads, each thread reads one entry of
// cu_seqlens up front (issued before the activation loads, so waiting for
// it waits for nothing else); with more, the entries are found by search.
__device__ __forceinline__ int32_t doc_mask_prefetch(const int32_t* cu, int32_t num_docs) {
  return (num_docs < kBlock && (int32_t)threadIdx.x <= num_docs) ? cu[threadIdx.x] : -1;
}

// Every thread of the workgroup must call this (two barriers).  The rows
// touched are the workgroup's bands (first_band .. last_band, clamped to the
// last band by the caller) plus three halo rows on each side; the
// last band's rows may run past S (and past 2^31 - 1), where no start
// matters, so only starts below S are marked.
__device__ __forceinline__ void build_doc_mask(DocMask& m, int32_t first_band, int32_t last_band,
                                               int32_t t_pre, const int32_t* cu, int32_t num_docs,
                                               int32_t S, int32_t rows) {
  const int32_t row_lo = first_band * rows - 3;
  const int64_t row_end = (int64_t)(last_band + 1) * rows + 3;
  // At most kDocMaskWords + 1 words by the host's choice of rows.
  const int32_t nwords = (int32_t)((row_end - row_lo) >> 5) + 2;
  const int32_t row_hi = (int32_t)min(row_end, (int64_t)S);
  const int32_t first_row = max(row_lo, 0);
  if (num_docs < kBlock) {
    // Few documents: the entry this thread read up front, no search.
    const int32_t t = t_pre;
    for (int32_t i = threadIdx.x; i < nwords; i += kBlock) m.bits[i] = 0u;
    if (threadIdx.x == 0) m.row_lo = row_lo;
    __syncthreads();
    if (t >= first_row && t < row_hi)
      atomicOr(&m.bits[(t - row_lo) >> 5], 1u << ((t - row_lo) & 31));
    __syncthreads();
    return;
  }
  for (int32_t i = threadIdx.x; i < nwords; i += kBlock) m.bits[i] = 0u;
  if (threadIdx.x < 64) {
    const int32_t lo = wave_lower_bound(cu, num_docs + 1, max(row_lo, 0));
    const int32_t hi = wave_lower_bound(cu, num_docs + 1, row_hi);
    if (threadIdx.x == 0) {
      m.row_lo = row_lo;
      m.idx_lo = lo;
      m.idx_hi = hi;
    }
  }
  __syncthreads();
  for (int32_t i = m.idx_lo + (int32_t)threadIdx.x; i < m.idx_hi; i += kBlock) {
    const int32_t t = cu[i];
    if (t >= first_row && t < row_hi)
      atomicOr(&m.bits[(t - row_lo) >> 5], 1u << ((t - row_lo) & 31));
  }
  __syncthreads();
}

// True when `c` holds for no lane of the wave.  The row loops choose
// between their plain and their masked path with it: a wave-uniform branch
// runs one path, where a per-lane one would run both under lane masks and
// keep every value of the first alive through the second (registers the
// plain path needs).  Lanes without a start are correct on the masked path.
__device__ __forceinline__ bool wave_none(bool c) { return __builtin_amdgcn_ballot_w64(c) == 0; }

// Bit g set: row row_lo + j + g starts a document, for a row index j
// relative to the workgroup's first row (1 <= n <= 32).
__device__ __forceinline__ uint32_t doc_starts(const DocMask& m, int32_t j, int n) {
  const uint32_t bits =
      __builtin_amdgcn_alignbit(m.bits[(j >> 5) + 1], m.bits[j >> 5], (uint32_t)j & 31u);
  return n >= 32 ? bits : bits & ((1u << n) - 1u);
}

// ------------------------------------------------------ SiLU pieces --

__device__ __forceinline__ float sigmoid_fast(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// 2^64 * sigmoid(z), for z far below zero where sigmoid(z) itself is below
// the binary32 normal range.
__device__ __forceinline__ float sigmoid_scaled64(float z) {
  return __builtin_amdgcn_rcpf(0x1p-64f +
                               __builtin_amdgcn_exp2f(__builtin_fmaf(z, -kLog2e, -64.0f)));
}

// SiLU'(z) for z < kDeep: there 1 - s == 1 in binary32, so s * (1 + z).
__device__ __forceinline__ float silu_grad_deep(float z) {
  return (sigmoid_scaled64(z) * (1.0f + z)) * 0x1p-64f;
}

// ---------------------------------- SiLU' of every BF16 value (table) --
//
// Under the "bf16" policy SiLU' is only ever evaluated at BF16 values, so it
// is read from a table of its binary32 roundings, computed here at compile
// time in double precision.  The table covers the BF16 magnitudes with
// biased exponents kLutExpLo .. kLutExpHi (2^-25 <= |z| < 256), both signs.
// Smaller magnitudes clamp to the smallest entry (SiLU' rounds to 1/2
// there), larger ones to the largest (SiLU' rounds to 1 for z > 0 and to
// 0 for z < 0).

constexpr int kLutExpLo = 102;
constexpr int kLutExpHi = 134;
constexpr uint32_t kLutLo = uint32_t(kLutExpLo) << 7;
constexpr uint32_t kLutHi = (uint32_t(kLutExpHi + 1) << 7) - 1;
constexpr int kLutN = int(kLutHi - kLutLo + 1);  // entries per sign

constexpr double cx_pow2(int e) {
  double r = 1.0, b = e >= 0 ? 2.0 : 0.5;
  int n = e >= 0 ? e : -e;
  while (n) {
    if (n & 1) r *= b;
    b *= b;
    n >>= 1;
  }
  return r;
}

// exp(x) for |x| < 700: x = k ln 2 + r with |r| <= ln 2 / 2, then a Taylor
// series for exp(r) (terms beyond r^27/27! are below 2^-100) times 2^k.
constexpr double cx_exp(double x) {
  constexpr double kLn2 = 0.6931471805599453;
  double kd = x / kLn2;
  long long k = (long long)(kd >= 0 ? kd + 0.5 : kd - 0.5);
  double r = x - double(k) * kLn2;
  double term = 1.0, sum = 1.0;
  for (int n = 1; n <= 27; ++n) {
    term = term * r / double(n);
    sum += term;
  }
  return sum * cx_pow2(int(k));
}

constexpr float cx_silu_grad(double z) {
  double e = cx_exp(-z);
  double s = 1.0 / (1.0 + e);
  double one_minus_s = e / (1.0 + e);
  return float(s * (1.0 + z * one_minus_s));
}

// SiLU' near its zero.  SiLU'(z) = s (1 + z (1 - s)) vanishes at z0 ~ -1.2785,
// where any binary32 evaluation of the bracket cancels: its absolute error
// stays near 2^-24 while its value goes to zero.  There the "fp32" policy
// takes the Taylor series of SiLU' about z0 instead, in d = z - z0 formed
// from a two-float split of z0 (z - z0_hi is exact near z0).
struct NearZero {
  float z0_hi, z0_lo;
  float c1, c2, c3;  // second, third / 2 and fourth / 6 derivative of SiLU at z0
};

constexpr NearZero make_near_zero() {
  // z0 solves 1 + z / (1 + e^z) = 0 (the bracket of SiLU'), by Newton's method.
  double z = -1.28;
  for (int it = 0; it < 40; ++it) {
    const double ez = cx_exp(z);
    const double g = 1.0 + z / (1.0 + ez);
    const double dg = 1.0 / (1.0 + ez) - z * ez / ((1.0 + ez) * (1.0 + ez));
    z -= g / dg;
  }
  const double s = 1.0 / (1.0 + cx_exp(-z));
  const double s1 = s * (1.0 - s);                         // sigmoid, first derivative
  const double s2 = s1 * (1.0 - 2.0 * s);                  // second
  const double s3 = s2 * (1.0 - 2.0 * s) - 2.0 * s1 * s1;  // third
  const double s4 = s3 * (1.0 - 2.0 * s) - 6.0 * s1 * s2;  // fourth
  NearZero n{};
  n.z0_hi = float(z);
  n.z0_lo = float(z - double(n.z0_hi));
  // Derivatives of SiLU(z) = z s: the (k+1)-th is (k+1) s^(k) + z s^(k+1).
  n.c1 = float(2.0 * s1 + z * s2);
  n.c2 = float((3.0 * s2 + z * s3) / 2.0);
  n.c3 = float((4.0 * s3 + z * s4) / 6.0);
  return n;
}

constexpr NearZero kNearZero = make_near_zero();
// |1 + z (1 - s)| below this selects the series: the bracket's derivative
// at z0 is 1, so this is |z - z0| < ~2^-12.  The bracket's absolute error
// is a few 2^-24 (from exp, the reciprocal and the products), so outside
// the window its relative error stays near 2^-10, a quarter of a BF16 ulp;
// inside, the series' first omitted term is below 2^-40 |SiLU'|.
constexpr float kNearZeroU = 0x1p-12f;

__device__ __forceinline__ float silu_grad_series(float z) {
  const float d = (z - kNearZero.z0_hi) - kNearZero.z0_lo;
  float t = __builtin_fmaf(d, kNearZero.c3, kNearZero.c2);
  t = __builtin_fmaf(d, t, kNearZero.c1);
  return d * t;
}

struct alignas(16) SiluGradTable {
  float v[2 * kLutN];  // [0, N): +z, [N, 2N): -z, index = magnitude pattern - kLutLo
};

constexpr SiluGradTable make_silu_grad_table() {
  SiluGradTable t{};
  for (int i = 0; i < kLutN; ++i) {
    const uint32_t a = kLutLo + uint32_t(i);
    const int e = int(a >> 7);
    const double m = 1.0 + double(a & 127u) / 128.0;
    const double z = m * cx_pow2(e - 127);
    t.v[i] = cx_silu_grad(z);
    t.v[kLutN + i] = cx_silu_grad(-z);
  }
  return t;
}

__constant__ SiluGradTable kSiluGradTable = make_silu_grad_table();

// Staging of the table into LDS by a whole workgroup: 16-byte loads, all
// issued before any is waited for (a loop of one load and one store per
// element would wait out a memory round trip per element).
constexpr int kLutQuads = 2 * kLutN / 4;
constexpr int kLutStageIters = (kLutQuads + kBlock - 1) / kBlock;
static_assert(2 * kLutN % 4 == 0, "the table is staged in 16-byte pieces");

struct LutStage {
  u32x4 q[kLutStageIters];
};

__device__ __forceinline__ void lut_stage_load(LutStage& st) {
  const u32x4* src = reinterpret_cast<const u32x4*>(kSiluGradTable.v);
#pragma unroll
  for (int k = 0; k < kLutStageIters; ++k) {
    const int i = (int)threadIdx.x + k * kBlock;
    if (i < kLutQuads) st.q[k] = src[i];
  }
}

__device__ __forceinline__ void lut_stage_store(const LutStage& st, float* lds) {
  u32x4* dst = reinterpret_cast<u32x4*>(lds);
#pragma unroll
  for (int k = 0; k < kLutStageIters; ++k) {
    const int i = (int)threadIdx.x + k * kBlock;
    if (i < kLutQuads) dst[i] = st.q[k];
  }
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Byte offsets in the table of the two BF16 values packed in h (low half,
// high half): 4 (clamp(magnitude) - kLutLo) + 4 kLutN sign.  Both halves
// are formed in one 32-bit word: each half's offset stays below 2^16, so
// the word's 32-bit sums carry nothing between the halves.
static_assert(4 * 2 * kLutN < 65536, "table offsets must fit 16 bits");
__device__ __forceinline__ void lut_offsets2(uint32_t h, uint32_t& off_lo, uint32_t& off_hi) {
  constexpr uint32_t kLo2 = kLutLo * 0x10001u, kHi2 = kLutHi * 0x10001u;
  u16x2 m = __builtin_bit_cast(u16x2, h & 0x7fff7fffu);
  m = __builtin_elementwise_min(__builtin_elementwise_max(m, __builtin_bit_cast(u16x2, kLo2)),
                                __builtin_bit_cast(u16x2, kHi2));
  const uint32_t sign2 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, h) >> (u16x2)(15));
  const uint32_t o = (__builtin_bit_cast(uint32_t, m) << 2) +
                     (sign2 * uint32_t(4 * kLutN) - 4u * kLo2);
  off_lo = o & 0xffffu;
  off_hi = o >> 16;
}

// ------------------------------------------------- the preactivation --

// One fixed order used by both directions:
// ((w0 x[t-3] + w1 x[t-2]) + w2 x[t-1]) + w3 x[t], then + bias.
template <bool kBias, int V>
__device__ __forceinline__ float preact(const float (&w)[4][V], const float (&bv)[V], int i,
                                        float xm3, float xm2, float xm1, float x0) {
  float p = w[0][i] * xm3;
  p = __builtin_fmaf(w[1][i], xm2, p);
  p = __builtin_fmaf(w[2][i], xm1, p);
  p = __builtin_fmaf(w[3][i], x0, p);
  if (kBias) p = p + bv[i];
  return p;
}

// Lane coordinates shared by the main kernels.
struct Lane {
  uint32_t band, vec;
  int32_t t0;        // first token of the band
  int32_t base_row;  // row of the wave's buffer base
  int32_t off;       // byte offset of (t0 - 3, vec) from the base
};

// The workgroup's place in the lane order.  Workgroups are dispatched to
// the XCDs round-robin (workgroup i to XCD i mod 8), and each XCD has its
// own L2.  With the grid padded to a multiple of 8, workgroup i takes place
// (i mod 8) (grid / 8) + i / 8, so that neighbouring places sit on one XCD:
// they share the cache lines at their boundary whenever a row is not a
// multiple of 128 bytes, and one L2 then fetches each such line once.
__device__ __forceinline__ uint32_t block_place() {
  if (!VDC_XCD_REMAP) return blockIdx.x;
  const uint32_t per = gridDim.x / kXcds;
  return (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
}

template <int V>
__device__ __forceinline__ bool lane_coords(uint32_t place, int32_t nvec, int32_t rows,
                                            int32_t bands, int32_t C, Lane& L) {
  const uint32_t g = place * (uint32_t)kBlock + threadIdx.x;
  const uint32_t band = g / (uint32_t)nvec;
  const bool active = band < (uint32_t)bands;
  // Lanes past the last band keep the last band's coordinates (they load
  // and store nothing) so that every address below stays meaningful.
  L.band = active ? band : (uint32_t)bands - 1u;
  L.vec = active ? g - band * (uint32_t)nvec : 0u;
  L.t0 = (int32_t)L.band * rows;
  // The wave's base row comes from its first lane, which has the smallest
  // band of the wave.
  const int32_t first_band = __builtin_amdgcn_readfirstlane((int32_t)L.band);
  L.base_row = max(first_band * rows - 3, 0);
  L.off = (L.t0 - 3 - L.base_row) * (C * 2) + (int32_t)L.vec * (V * 2);
  return active;
}

// Bands of the linear lane map's workgroup `place`: its kBlock lanes.
__device__ __forceinline__ void linear_bands(uint32_t place, int32_t nvec, int32_t bands,
                                             int32_t& first, int32_t& last) {
  const int32_t g0 = (int32_t)place * kBlock;
  first = g0 / nvec;
  last = min((g0 + kBlock - 1) / nvec, bands - 1);
}

// Column-block lanes of the backward (C / V a multiple of 64, at least
// kBlock): workgroup `place` holds vectors [64 b, 64 b + 64) of bands
// kCbBands q .. kCbBands q + kCbBands - 1, one band per wave, with
// q = place / (C / (64 V)) and b the remainder.  A wave reads the same
// 512 contiguous bytes of each row as under the linear map; the workgroup
// can then add its bands' totals before writing them.
template <int V>
__device__ __forceinline__ bool lane_coords_cb(uint32_t place, int32_t nvec, int32_t rows,
                                               int32_t bands, int32_t C, Lane& L) {
  const uint32_t nblk = (uint32_t)nvec / 64u;
  const uint32_t q = place / nblk;
  // The wave's band, the same for all its lanes.
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x) / 64u;
  const uint32_t band = q * (uint32_t)kCbBands + wave;
  const bool active = band < (uint32_t)bands;
  // Waves past the last band keep the last band's coordinates (they load
  // and store nothing), as under the linear map.
  L.band = active ? band : (uint32_t)bands - 1u;
  L.vec = active ? (place - q * nblk) * 64u + (threadIdx.x & 63u) : 0u;
  L.t0 = (int32_t)L.band * rows;
  L.base_row = max(L.t0 - 3, 0);
  L.off = (L.t0 - 3 - L.base_row) * (C * 2) + (int32_t)L.vec * (V * 2);
  return active;
}

// ===================================================== forward kernel ==

template <bool kBias, int V>
__device__ __forceinline__ typename Vec<V>::raw fwd_row(const float (&w)[4][V],
                                                        const float (&bv)[V],
                                                        const float (&h3)[V], const float (&h2)[V],
                                                        const float (&h1)[V],
                                                        const float (&xc)[V]) {
  float p[V], yv[V];
  float pmin = 0.0f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    p[i] = preact<kBias, V>(w, bv, i, h3[i], h2[i], h1[i], xc[i]);
    pmin = __builtin_fminf(pmin, p[i]);
    yv[i] = p[i] * sigmoid_fast(p[i]);
  }
  typename Vec<V>::raw out = pack<V>(yv);
  if (pmin < kDeep) {
    // Rare: some p is so negative that sigmoid(p) underflows on the fast
    // path; redo those values in scaled form and round them exactly.
#pragma unroll
    for (int d = 0; d < V / 2; ++d) {
      uint32_t h[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int i = 2 * d + q;
        const float yd = (p[i] * sigmoid_scaled64(p[i])) * 0x1p-64f;
        h[q] = p[i] < kDeep ? bf16_bits_rne(yd) : bf16_bits_rne(yv[i]);
      }
      out[d] = h[0] | (h[1] << 16);
    }
  }
  return out;
}

template <bool kBias, bool kNt, int V, int kFwdGroup>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(kFwdWaves)))
void fwd_kernel(FwdArgs a) {
  typedef Vec<V> VT;
  typedef Io<kNt ? kStream : kPlain> IO;
  typedef typename VT::raw Raw;
  __shared__ DocMask dmask;
  Lane L;
  const uint32_t place = block_place();
  if (place >= (uint32_t)a.blocks) return;  // padding workgroup: no lane
  const bool active = lane_coords<V>(place, a.nvec, a.rows, a.bands, a.C, L);
  // Parameters and the document starts are requested before the
  // activations: loads complete in issue order, so waiting for these waits
  // for no activation row.
  ParamRaw<V> praw;
  load_params<V>(a.w, a.w_bf16, a.b, a.b_bf16, kBias, L.vec * V, praw);
  const int32_t cu_pre = doc_mask_prefetch(a.cu, a.num_docs);
  const int32_t row_bytes = a.C * 2;
  const uint32_t nrec = span_bytes(a.S, a.C, L.base_row);  // wave-uniform
  const rsrc_t rx = make_rsrc(a.x + (int64_t)L.base_row * a.C, nrec);
  const rsrc_t ry = make_rsrc(a.y + (int64_t)L.base_row * a.C, nrec);

  // The halo rows t0-3 .. t0-1 and the first group are requested before the
  // workgroup resolves its document starts.
  int32_t off = L.off;
  Raw halo[3], A[kFwdGroup], B[kFwdGroup];
#pragma unroll
  for (int q = 0; q < 3; ++q) halo[q] = VT::zero();
  off += 3 * row_bytes;
  // Unconditional, so that no wait on the document-start loads issued later
  // has to cover a path without them: rows before row 0 have negative
  // offsets, which read as zero, and lanes past the last band read rows of
  // the last band, then leave.  The loads are issued in row order (kept by
  // scheduling barriers), and dropped stores stand for the previous group's
  // y rows: the loop is then entered with the same accesses in flight, in
  // the same order, as from its own back edge.
#pragma unroll
  for (int q = 0; q < 3; ++q) halo[q] = IO::load(rx, off + (q - 3) * row_bytes);
#pragma unroll
  for (int g = 0; g < kFwdGroup; ++g) {
    __builtin_amdgcn_sched_barrier(0);
    A[g] = IO::load(rx, off + g * row_bytes);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int g = 0; g < kFwdGroup; ++g) {
    IO::store(ry, kNoRow + g * row_bytes, VT::zero());
    if (!kNt) IO::store(ry, kNoRow + g * row_bytes, VT::zero());
  }
  // Unaligned rows: the y stores of row g of every group stream where bit
  // g & 7 is set, for the lines a wave writes alone (whole_line_bits); the
  // lines at the ends of its piece, which another wave writes too, stay
  // plain so that the two halves can meet in L2.
  const uint32_t whole =
      kNt ? 0u
          : whole_line_bits((int64_t)(uintptr_t)(a.y + (int64_t)L.base_row * a.C) + L.off +
                                3 * (int64_t)row_bytes,
                            row_bytes, threadIdx.x & 63u, L.vec, a.nvec, V * 2);

  {
    int32_t first, last;
    linear_bands(place, a.nvec, a.bands, first, last);
    build_doc_mask(dmask, first, last, cu_pre, a.cu, a.num_docs, a.S, a.rows);
  }
  if (!active) return;
  float w[4][V], bv[V];
  unpack_params<V>(praw, a.w_bf16, a.b_bf16, w, bv);

  // Window of the three previous rows: h1 = x[r-1], h2 = x[r-2], h3 = x[r-3].
  float h1[V], h2[V], h3[V];
#pragma unroll
  for (int i = 0; i < V; ++i) h1[i] = h2[i] = h3[i] = 0.0f;
  // Row index relative to the workgroup's first row (no overflow near 2^31).
  int32_t r = L.t0 - 3 - dmask.row_lo;
  const uint32_t hs = doc_starts(dmask, r, 3);
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    if ((hs >> q) & 1u) {
#pragma unroll
      for (int i = 0; i < V; ++i) h1[i] = h2[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < V; ++i) h3[i] = h2[i], h2[i] = h1[i];
    unpack<V>(halo[q], h1);
  }
  r += 3;

  // Groups of G rows, two register buffers: the loads of group k+1 are in
  // flight while group k is computed, and a group's y rows are stored
  // together after its last row (loads and stores share one wait counter on
  // this architecture, so a store between loads would stall the next wait).
  auto load = [&](Raw (&buf)[kFwdGroup], int32_t at) {
#pragma unroll
    for (int g = 0; g < kFwdGroup; ++g) buf[g] = IO::load(rx, at + g * row_bytes);
  };
  auto compute = [&](const Raw (&buf)[kFwdGroup], Raw (&out)[kFwdGroup]) {
    const uint32_t starts = doc_starts(dmask, r, kFwdGroup);
    if (wave_none(starts != 0u)) {
      // No document starts in this group, for any lane of the wave.
#pragma unroll
      for (int g = 0; g < kFwdGroup; ++g) {
        float xc[V];
        unpack<V>(buf[g], xc);
        out[g] = fwd_row<kBias, V>(w, bv, h3, h2, h1, xc);
#pragma unroll
        for (int i = 0; i < V; ++i) h3[i] = h2[i], h2[i] = h1[i], h1[i] = xc[i];
      }
    } else {
#pragma unroll
      for (int g = 0; g < kFwdGroup; ++g) {
        if ((starts >> g) & 1u) {
#pragma unroll
          for (int i = 0; i < V; ++i) h1[i] = h2[i] = h3[i] = 0.0f;
        }
        float xc[V];
        unpack<V>(buf[g], xc);
        out[g] = fwd_row<kBias, V>(w, bv, h3, h2, h1, xc);
#pragma unroll
        for (int i = 0; i < V; ++i) h3[i] = h2[i], h2[i] = h1[i], h1[i] = xc[i];
      }
    }
    r += kFwdGroup;
  };
  // On unaligned rows each row is two stores, one streaming and one plain,
  // each lane's bytes in one of them (the other takes kNoRow): both are
  // issued on every row, so every path keeps the same accesses in flight.
  auto store = [&](const Raw (&out)[kFwdGroup]) {
#pragma unroll
    for (int g = 0; g < kFwdGroup; ++g) {
      const int32_t o = off + g * row_bytes;
      if (kNt) {
        IO::store(ry, o, out[g]);
      } else {
        const bool stream = (whole >> (g & 7)) & 1u;
        Io<kStream>::store(ry, stream ? o : kNoRow, out[g]);
        Io<kPlain>::store(ry, stream ? kNoRow : o, out[g]);
      }
    }
    off += kFwdGroup * row_bytes;
  };
  // T is a multiple of 2G (host rule).  The last pair's reload of A reads
  // nothing (kNoRow).  y goes to its own registers: the loaded rows stay
  // read-only.
  Raw out[kFwdGroup];
  for (int32_t done = 0; done < a.rows; done += 2 * kFwdGroup) {
    load(B, off + kFwdGroup * row_bytes);
    wait_vm<kFwdGroup>();  // pace: only B's loads remain in flight
    compute(A, out);
    store(out);
    load(A, done + 2 * kFwdGroup < a.rows ? off + kFwdGroup * row_bytes : kNoRow);
    compute(B, out);
    store(out);
  }
}

// ================================================ backward main kernel ==

// A lane's gradient partials: taps k = 0..3, then the bias term.  The rows
// of one row group (G rows) are summed in binary32 in `run`, and each
// group's sum is added into the band totals: binary64 under the "fp32"
// policy (Acc = double), binary32 under "bf16" (Acc = float).  A run of G
// products rounds within a few units in the last place of its own
// magnitude; the totals then take T/G additions instead of T, which bounds
// the binary32 error of a band by about (G + T/G) units in the last place
// of its sum of magnitudes instead of T.  Under "fp32" this costs an eighth
// of the binary64 operations of a per-row binary64 sum.
template <typename Acc, int V>
struct Partials {
  float run[5][V];
  Acc v[5][V];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int k = 0; k < 5; ++k)
#pragma unroll
      for (int i = 0; i < V; ++i) run[k][i] = 0.0f, v[k][i] = (Acc)0;
  }
  __device__ __forceinline__ void fold() {
#pragma unroll
    for (int k = 0; k < 5; ++k)
#pragma unroll
      for (int i = 0; i < V; ++i) {
        v[k][i] += (Acc)run[k][i];
        run[k][i] = 0.0f;
      }
  }
  __device__ __forceinline__ Acc total(int k, int i) const { return v[k][i]; }
};

// dpre = dy * SiLU'(z) for the lane's V channels of one row.
template <bool kBf16Policy, int V>
__device__ __forceinline__ void dpre_row(const float (&p)[V], const float (&dyv)[V],
                                         const float* lut, float (&dp)[V]) {
  if (kBf16Policy) {
    // z = bf16(p); SiLU'(z) from the table.
#pragma unroll
    for (int d = 0; d < V / 2; ++d) {
      const uint32_t h = pack2(p[2 * d], p[2 * d + 1]);
      uint32_t o0, o1;
      lut_offsets2(h, o0, o1);
      const char* base = reinterpret_cast<const char*>(lut);
      dp[2 * d] = dyv[2 * d] * *reinterpret_cast<const float*>(base + o0);
      dp[2 * d + 1] = dyv[2 * d + 1] * *reinterpret_cast<const float*>(base + o1);
    }
  } else {
    // SiLU'(z) = s u, s = 1 / (1 + e), e = exp(-z), u = 1 + z (1 - s) as
    // one fused multiply-add.  1 - s is formed as e s, which keeps its
    // relative accuracy where s is close to 1 (1 - s itself would leave an
    // absolute error of about z 2^-24 in SiLU' for large positive z).  Two
    // rare cases take a wave-uniform branch: z below kDeep (s leaves the
    // binary32 normal range) and |u| below kNearZeroU (the bracket cancels
    // near SiLU's zero; the series about the zero is exact there).
    float zmin = 0.0f, umin = 1.0f, r[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const float z = p[i];
      const float e = __builtin_amdgcn_exp2f(-z * kLog2e);
      const float sg = __builtin_amdgcn_rcpf(1.0f + e);
      const float u = __builtin_fmaf(z, e * sg, 1.0f);
      zmin = __builtin_fminf(zmin, z);
      umin = __builtin_fminf(umin, __builtin_fabsf(u));
      r[i] = sg * u;
    }
    if (!wave_none(zmin < kDeep || umin < kNearZeroU)) {
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const float z = p[i];
        const float e = __builtin_amdgcn_exp2f(-z * kLog2e);
        const float u = __builtin_fmaf(z, e * __builtin_amdgcn_rcpf(1.0f + e), 1.0f);
        if (__builtin_fabsf(u) < kNearZeroU) r[i] = silu_grad_series(z);
        if (z < kDeep) r[i] = silu_grad_deep(z);
      }
    }
#pragma unroll
    for (int i = 0; i < V; ++i) dp[i] = dyv[i] * r[i];
  }
}

// One row v of the backward: recompute p, form dpre, accumulate partials
// (rows of the band) and emit dx of row v-3 (from the band's fourth row on).
// kMasked: a document starts within rows v-2 .. v (bits of `hist`: bit 0 =
// row v, bit 1 = row v-1, bit 2 = row v-2); then later rows count toward
// dx[v-3] only if no start lies between.
template <bool kBias, bool kBf16Policy, bool kMasked, typename Acc, int V>
__device__ __forceinline__ void bwd_row(const float (&w)[4][V], const float (&bv)[V],
                                        const float* lut, const float (&xc)[V],
                                        typename Vec<V>::raw dyraw, float (&h1)[V],
                                        float (&h2)[V], float (&h3)[V], float (&d1)[V],
                                        float (&d2)[V], float (&d3)[V], Partials<Acc, V>& acc,
                                        bool accumulate, bool emit, uint32_t hist,
                                        typename Vec<V>::raw& dx_out) {
  float dyv[V], p[V], dp[V];
  unpack<V>(dyraw, dyv);
#pragma unroll
  for (int i = 0; i < V; ++i) p[i] = preact<kBias, V>(w, bv, i, h3[i], h2[i], h1[i], xc[i]);
  dpre_row<kBf16Policy, V>(p, dyv, lut, dp);
  if (accumulate) {
    // acc_k += dpre * x[v-3+k] as one fused multiply-add; acc_4 += dpre.
    float(&dst)[5][V] = acc.run;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      dst[0][i] = __builtin_fmaf(dp[i], h3[i], dst[0][i]);
      dst[1][i] = __builtin_fmaf(dp[i], h2[i], dst[1][i]);
      dst[2][i] = __builtin_fmaf(dp[i], h1[i], dst[2][i]);
      dst[3][i] = __builtin_fmaf(dp[i], xc[i], dst[3][i]);
      dst[4][i] += dp[i];
    }
  }
  if (emit) {
    // dx[v-3] = w3 d[v-3] + w2 d[v-2] + w1 d[v-1] + w0 d[v].
    const bool m1 = !kMasked || !(hist & 4u);
    const bool m2 = !kMasked || !(hist & 6u);
    const bool m3 = !kMasked || !(hist & 7u);
    float dxv[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      float s = w[3][i] * d3[i];
      s = __builtin_fmaf(w[2][i], m1 ? d2[i] : 0.0f, s);
      s = __builtin_fmaf(w[1][i], m2 ? d1[i] : 0.0f, s);
      s = __builtin_fmaf(w[0][i], m3 ? dp[i] : 0.0f, s);
      dxv[i] = s;
    }
    dx_out = pack<V>(dxv);
  }
#pragma unroll
  for (int i = 0; i < V; ++i) {
    h3[i] = h2[i]; h2[i] = h1[i]; h1[i] = xc[i];
    d3[i] = d2[i]; d2[i] = d1[i]; d1[i] = dp[i];
  }
}

template <bool kBias, bool kBf16Policy, bool kNt, bool kCb, typename Acc, int V>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(kBwdWaves)))
void bwd_main_kernel(BwdArgs a) {
  typedef Vec<V> VT;
  typedef Io<kNt ? kStream : kPlain> IO;
  typedef typename VT::raw Raw;
  __shared__ __attribute__((aligned(16))) float lut_lds[kBf16Policy ? 2 * kLutN : 4];
  __shared__ DocMask dmask;
  // Rows of a masked group, [row][thread]: x in words 0-1, dy in 2-3; at
  // the end, each thread's band totals, [total][thread].
  constexpr int kStageRows = kBwdGroup > 5 * (int)sizeof(Acc) / 4 ? kBwdGroup
                                                                   : 5 * (int)sizeof(Acc) / 4;
  __shared__ u32x4 stage[kStageRows * kBlock];
  Lane L;
  const uint32_t place = block_place();
  if (place >= (uint32_t)a.blocks) return;  // padding workgroup: no lane
  const bool active = kCb ? lane_coords_cb<V>(place, a.nvec, a.rows, a.bands, a.C, L)
                           : lane_coords<V>(place, a.nvec, a.rows, a.bands, a.C, L);
  // Parameters, the SiLU' table and the document starts are requested
  // before the activations: loads complete in issue order, so waiting for
  // these waits for no activation row.
  ParamRaw<V> praw;
  load_params<V>(a.w, a.w_bf16, a.b, a.b_bf16, kBias, L.vec * V, praw);
  LutStage lut_stage;
  if (kBf16Policy) lut_stage_load(lut_stage);
  const int32_t cu_pre = doc_mask_prefetch(a.cu, a.num_docs);
  const int32_t row_bytes = a.C * 2;
  const uint32_t nrec = span_bytes(a.S, a.C, L.base_row);  // wave-uniform
  const int64_t base_elt = (int64_t)L.base_row * a.C;
  const rsrc_t rx = make_rsrc(a.x + base_elt, nrec);
  const rsrc_t rdy = make_rsrc(a.dy + base_elt, nrec);
  const rsrc_t rdx = make_rsrc(a.dx + base_elt, nrec);

  // The halo rows t0-3 .. t0-1 (x only) and the first group are requested
  // before the workgroup stages its tables.
  int32_t off = L.off;
  Raw halo[3], xa[kBwdGroup], da[kBwdGroup], xb[kBwdGroup], db[kBwdGroup];
#pragma unroll
  for (int q = 0; q < 3; ++q) halo[q] = VT::zero();
  off += 3 * row_bytes;
  // Unconditional, so that no wait on the table or mask loads issued later
  // has to cover a path without them: rows before row 0 have negative
  // offsets, which read as zero, and lanes past the last band read rows of
  // the last band, then leave.  The loads are issued in row order (kept by
  // scheduling barriers), and dropped stores stand for the previous group's
  // dx rows: the loop is then entered with the same accesses in flight, in
  // the same order, as from its own back edge.
#pragma unroll
  for (int q = 0; q < 3; ++q) halo[q] = IO::load(rx, off + (q - 3) * row_bytes);
#pragma unroll
  for (int g = 0; g < kBwdGroup; ++g) {
    __builtin_amdgcn_sched_barrier(0);
    xa[g] = IO::load(rx, off + g * row_bytes);
    da[g] = IO::load(rdy, off + g * row_bytes);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int g = 0; g < kBwdGroup; ++g) IO::store(rdx, kNoRow + g * row_bytes, VT::zero());

  // Every thread stages its part of the SiLU' table (the mask builder's
  // barriers make it visible).
  if (kBf16Policy) lut_stage_store(lut_stage, lut_lds);
  {
    int32_t first, last;
    if (kCb) {
      first = (int32_t)(place / ((uint32_t)a.nvec / 64u)) * kCbBands;
      last = min(first + kCbBands - 1, a.bands - 1);
    } else {
      linear_bands(place, a.nvec, a.bands, first, last);
    }
    build_doc_mask(dmask, first, last, cu_pre, a.cu, a.num_docs, a.S, a.rows);
  }
  // Lanes past the last band have nothing to compute; with one partial row
  // per workgroup (or band group) they still join its final sum (one
  // barrier).
  if (!active && !a.wg_rows && !kCb) return;
  // Band total j of lane l in LDS: in the lane's own 16-byte column of
  // `stage` (the masked path uses only the thread's own column too, so a
  // thread writing its totals disturbs no thread still in its loop).
  constexpr int kPerSlot = 16 / (int)sizeof(Acc);
  auto slot = [&](int j, uint32_t l) -> Acc* {
    return reinterpret_cast<Acc*>(stage + (j / kPerSlot) * kBlock + l) + j % kPerSlot;
  };
  if (active) {
  float w[4][V], bv[V];
  unpack_params<V>(praw, a.w_bf16, a.b_bf16, w, bv);

  Partials<Acc, V> acc;
  acc.init();

  float h1[V], h2[V], h3[V], d1[V], d2[V], d3[V];
#pragma unroll
  for (int i = 0; i < V; ++i) h1[i] = h2[i] = h3[i] = d1[i] = d2[i] = d3[i] = 0.0f;
  // hist: bit 0 = row r-1 starts a document, bit 1 = row r-2.
  // Row index relative to the workgroup's first row (no overflow near 2^31).
  int32_t r = L.t0 - 3 - dmask.row_lo;
  const uint32_t hs = doc_starts(dmask, r, 3);
  uint32_t hist = 0;
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const uint32_t start = (hs >> q) & 1u;
    if (start) {
#pragma unroll
      for (int i = 0; i < V; ++i) h1[i] = h2[i] = 0.0f;
    }
    hist = ((hist << 1) | start) & 3u;
#pragma unroll
    for (int i = 0; i < V; ++i) h3[i] = h2[i], h2[i] = h1[i];
    unpack<V>(halo[q], h1);
  }
  r += 3;

  // Band rows t0 .. t0+T-1 (partials) in groups of G with two register
  // buffers: the loads of group k+1 are in flight while group k is
  // computed, and a group's dx rows are stored together after its last row
  // (loads and stores share one wait counter on this architecture).  Row
  // t0+idx emits dx of row t0+idx-3, so the band's first three rows emit
  // nothing and three look-ahead rows, loaded during the last pair, finish
  // the band.
  //
  // Rows 0..2 of a group load from `at`, rows 3.. from `at_rest`: `at`
  // again for a whole group, kNoRow for the band's three look-ahead rows.
  auto load = [&](Raw (&xr)[kBwdGroup], Raw (&dr)[kBwdGroup], int32_t at, int32_t at_rest) {
#pragma unroll
    for (int g = 0; g < kBwdGroup; ++g) {
      const int32_t o = (g < 3 ? at : at_rest) + g * row_bytes;
      xr[g] = IO::load(rx, o);
      dr[g] = IO::load(rdy, o);
    }
  };
  auto run = [&](const Raw (&xr)[kBwdGroup], const Raw (&dr)[kBwdGroup], int32_t done, int nrows,
                 bool accumulate) {
    // dx goes to its own registers: the loaded rows stay read-only.
    Raw dxr[kBwdGroup];
#pragma unroll
    for (int g = 0; g < kBwdGroup; ++g) dxr[g] = VT::zero();
    const uint32_t starts = doc_starts(dmask, r, nrows);
    if (wave_none(hist != 0u || starts != 0u)) {
      // No document starts in rows r-2 .. r+nrows-1, for any lane of the
      // wave: no resets, no masks.
#pragma unroll
      for (int g = 0; g < kBwdGroup; ++g) {
        if (g >= nrows) break;
        float xc[V];
        unpack<V>(xr[g], xc);
        bwd_row<kBias, kBf16Policy, false, Acc, V>(w, bv, lut_lds, xc, dr[g], h1, h2, h3, d1, d2,
                                                   d3, acc, accumulate, done + g >= 3, 0u,
                                                   dxr[g]);
      }
    } else {
      // A document start within reach: the group's rows go through this
      // thread's LDS slots and a loop takes them in turn, each dx row back
      // into its slot.  Unrolled like the plain path, this path needed more
      // registers than the kernel has, and the allocation for it (parked
      // values, register copies) slowed the plain path too.  Four rows per
      // pass under "bf16" hide the table reads; under "fp32", with more
      // registers per row, one.
      u32x4* slot = stage + threadIdx.x;
#pragma unroll
      for (int g = 0; g < kBwdGroup; ++g)
        if (g < nrows) slot[g * kBlock] = (u32x4){xr[g].x, xr[g].y, dr[g].x, dr[g].y};
      constexpr int kMaskedUnroll = kBf16Policy ? 4 : 1;
#pragma unroll kMaskedUnroll
      for (int g = 0; g < nrows; ++g) {
        const u32x4 row = slot[g * kBlock];
        const uint32_t start = (starts >> g) & 1u;
        if (start) {
#pragma unroll
          for (int i = 0; i < V; ++i) h1[i] = h2[i] = h3[i] = 0.0f;
        }
        const uint32_t h3bits = (hist << 1) | start;
        hist = h3bits & 3u;
        float xc[V];
        unpack<V>((Raw){row.x, row.y}, xc);
        Raw dxg = VT::zero();
        bwd_row<kBias, kBf16Policy, true, Acc, V>(w, bv, lut_lds, xc, (Raw){row.z, row.w}, h1,
                                                  h2, h3, d1, d2, d3, acc, accumulate,
                                                  done + g >= 3, h3bits, dxg);
        slot[g * kBlock] = (u32x4){dxg.x, dxg.y, 0u, 0u};
      }
#pragma unroll
      for (int g = 0; g < kBwdGroup; ++g)
        if (g < nrows) {
          const u32x4 v = slot[g * kBlock];
          dxr[g] = (Raw){v.x, v.y};
        }
    }
    // dxr[g] holds the packed dx of row r+g-3; the band's first three rows
    // have no dx to store (kNoRow).
#pragma unroll
    for (int g = 0; g < kBwdGroup; ++g)
      if (g < nrows)
        IO::store(rdx, done + g >= 3 ? off + (g - 3) * row_bytes : kNoRow, dxr[g]);
    if (accumulate) acc.fold();
    r += nrows;
    off += nrows * row_bytes;
  };
  // T is a multiple of 2G (host rule).  In the last pair the reload of the
  // first buffer takes the look-ahead rows.  Under "bf16" the loop paces
  // itself once per pair (see wait_vm); under "fp32", with more arithmetic
  // per row, the wait costs more than it saves (about 3%), so there is none.
  for (int32_t done = 0; done < a.rows; done += 2 * kBwdGroup) {
    const int32_t nb = off + kBwdGroup * row_bytes;
    load(xb, db, nb, nb);
    run(xa, da, done, kBwdGroup, true);
    const int32_t na = off + kBwdGroup * row_bytes;
    load(xa, da, na, done + 2 * kBwdGroup < a.rows ? na : kNoRow);
    if (kBf16Policy) wait_vm<2 * kBwdGroup>();  // pace: only the reload remains in flight
    run(xb, db, done + kBwdGroup, kBwdGroup, true);
  }
  run(xa, da, a.rows, 3, false);

  if (!a.wg_rows && !kCb) {
    // One partial row per band: part[band][k][c].
    Acc* part = reinterpret_cast<Acc*>(a.part) + (int64_t)L.band * 5 * a.C + L.vec * V;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      Acc* dst = part + (int64_t)k * a.C;
#pragma unroll
      for (int i = 0; i < V; ++i) dst[i] = acc.total(k, i);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 5; ++k)
#pragma unroll
      for (int i = 0; i < V; ++i) *slot(k * V + i, threadIdx.x) = acc.total(k, i);
  }
  }  // active
  else {
#pragma unroll
    for (int j = 0; j < 5 * V; ++j) *slot(j, threadIdx.x) = (Acc)0;
  }
  if (!a.wg_rows && !kCb) return;
  __syncthreads();

  if (kCb) {
    // One partial row per band group: part[q][k][c] for the workgroup's 64
    // vectors.  Thread t sums lane t of each wave, that is vector t of
    // bands kCbBands q, kCbBands q + 1, ... in that order, in binary64, and
    // rounds once to the partial element type (waves past the last band
    // left zeros).
    if (threadIdx.x < 64u) {
      const uint32_t nblk = (uint32_t)a.nvec / 64u;
      const uint32_t q = place / nblk;
      const uint32_t vec = (place - q * nblk) * 64u + threadIdx.x;
      double s[5 * V];
#pragma unroll
      for (int j = 0; j < 5 * V; ++j) s[j] = 0.0;
#pragma unroll
      for (int w = 0; w < kCbBands; ++w)
#pragma unroll
        for (int j = 0; j < 5 * V; ++j) s[j] += (double)*slot(j, threadIdx.x + 64u * w);
      Acc* part = reinterpret_cast<Acc*>(a.part) + (int64_t)q * 5 * a.C + (int64_t)vec * V;
#pragma unroll
      for (int k = 0; k < 5; ++k)
#pragma unroll
        for (int i = 0; i < V; ++i) part[(int64_t)k * a.C + i] = (Acc)s[k * V + i];
    }
    return;
  }

  // One partial row per workgroup: part[place][k][c].  The workgroup's lanes
  // cover every vector of channels (C/V < kBlock), some twice; thread t sums
  // vector t's lanes in increasing lane order, that is in increasing band
  // order, in binary64, and rounds once to the partial element type.
  if ((int32_t)threadIdx.x < a.nvec) {
    const uint32_t nvec = (uint32_t)a.nvec;
    const uint32_t first = (threadIdx.x + nvec - (place * (uint32_t)kBlock) % nvec) % nvec;
    double s[5 * V];
#pragma unroll
    for (int j = 0; j < 5 * V; ++j) s[j] = 0.0;
    for (uint32_t l = first; l < (uint32_t)kBlock; l += nvec)
#pragma unroll
      for (int j = 0; j < 5 * V; ++j) s[j] += (double)*slot(j, l);
    Acc* part = reinterpret_cast<Acc*>(a.part) + (int64_t)place * 5 * a.C + threadIdx.x * V;
#pragma unroll
    for (int k = 0; k < 5; ++k)
#pragma unroll
      for (int i = 0; i < V; ++i) part[(int64_t)k * a.C + i] = (Acc)s[k * V + i];
  }
}

// =================================================== backward reduce ==

// Sum over rows [r0, r1) of column o of a row-major [rows][n_out] matrix,
// in a fixed order: the kRedChunks threads of output o take chunk q = rows
// [r0 + q R, r0 + q R + R), R = ceil((r1 - r0) / kRedChunks), each in
// increasing row order, and the chunk sums are added in increasing q.  The
// sums are binary64 whatever the element type (binary32 partial rows under
// "bf16", binary64 under "fp32"): a binary32 running sum over many rows
// would lose digits in proportion to their count.  Every thread of the
// workgroup calls this (one barrier); the result is valid in chunk 0.
template <typename Part>
__device__ __forceinline__ double sum_rows(const Part* m, int64_t n_out, int64_t o, int32_t r0,
                                           int32_t r1, double (&red)[kRedChunks][kRedOut]) {
  const int lane = threadIdx.x % kRedOut;
  const int chunk = threadIdx.x / kRedOut;
  const int32_t len = (r1 - r0 + kRedChunks - 1) / kRedChunks;
  double s = 0.0;
  if (o < n_out) {
    const int32_t b0 = min(r0 + chunk * len, r1);
    const int32_t b1 = min(b0 + len, r1);
    const Part* p = m + (int64_t)b0 * n_out + o;
#pragma unroll 8
    for (int32_t b = b0; b < b1; ++b, p += n_out) s += (double)*p;
  }
  red[chunk][lane] = s;
  __syncthreads();
  double t = red[0][lane];
#pragma unroll
  for (int q = 1; q < kRedChunks; ++q) t += red[q][lane];
  return t;
}

// A gradient element: binary64 sum -> binary32 (round to nearest even) or
// BF16 (rounded once, from the binary64 value).
__device__ __forceinline__ void store_grad(void* dst, int64_t i, double v, int bf16) {
  if (bf16) reinterpret_cast<uint16_t*>(dst)[i] = bf16_bits_from_f64(v);
  else reinterpret_cast<float*>(dst)[i] = (float)v;
}

// First stage (more than kRedBlockRows partial rows): workgroup (x, y) sums
// rows [y kRedBlockRows, (y + 1) kRedBlockRows) of outputs
// [x kRedOut, (x + 1) kRedOut) into inter[y][o].
template <typename Part>
__global__ __launch_bounds__(kRedOut * kRedChunks) void bwd_reduce_rows_kernel(ReduceArgs a) {
  __shared__ double red[kRedChunks][kRedOut];
  const int64_t n_out = 5 * (int64_t)a.C;
  const int64_t o = (int64_t)blockIdx.x * kRedOut + threadIdx.x % kRedOut;
  const int32_t r0 = (int32_t)blockIdx.y * kRedBlockRows;
  const int32_t r1 = min(r0 + kRedBlockRows, a.P);
  const double t = sum_rows(reinterpret_cast<const Part*>(a.part), n_out, o, r0, r1, red);
  if (threadIdx.x < kRedOut && o < n_out)
    reinterpret_cast<double*>(a.inter)[(int64_t)blockIdx.y * n_out + o] = t;
}

// Final pass: out[o] = sum_{b=0..P-1} part[b][o] for o = k*C + c, rounded
// once to the output dtype.  The order depends on (P, C) only.
template <typename Part>
__global__ __launch_bounds__(kRedOut * kRedChunks) void bwd_reduce_kernel(ReduceArgs a) {
  __shared__ double red[kRedChunks][kRedOut];
  const int64_t n_out = 5 * (int64_t)a.C;
  const int64_t o = (int64_t)blockIdx.x * kRedOut + threadIdx.x % kRedOut;
  const double t = sum_rows(reinterpret_cast<const Part*>(a.part), n_out, o, 0, a.P, red);
  if (threadIdx.x < kRedOut && o < n_out) {
    const int64_t k = o / a.C;
    const int64_t c = o - k * a.C;
    if (k < 4) store_grad(a.dw, c * 4 + k, t, a.dw_bf16);
    else if (a.db) store_grad(a.db, c, t, a.db_bf16);
  }
}

// Rows of a multiple of 128 bytes stream non-temporally (see kStream).
inline bool rows_line_aligned(int32_t C) { return (C * 2) % 128 == 0; }

template <int V>
hipError_t launch_fwd_v(const Plan& plan, const FwdArgs& a, bool has_bias, hipStream_t s) {
  dim3 grid((uint32_t)padded_grid(plan.blocks)), block(kBlock);
  const bool nt = rows_line_aligned(a.C);
  const int group = fwd_group(a.C);
  if (plan.rows % (2 * group)) return hipErrorInvalidValue;
  if (group == kFwdGroupShort) {
    if (has_bias) hipLaunchKernelGGL((fwd_kernel<true, false, V, kFwdGroupShort>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fwd_kernel<false, false, V, kFwdGroupShort>), grid, block, 0, s, a);
  } else if (has_bias) {
    if (nt) hipLaunchKernelGGL((fwd_kernel<true, true, V, kFwdGroup>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fwd_kernel<true, false, V, kFwdGroup>), grid, block, 0, s, a);
  } else {
    if (nt) hipLaunchKernelGGL((fwd_kernel<false, true, V, kFwdGroup>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fwd_kernel<false, false, V, kFwdGroup>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <bool kBias, bool kBf16Policy, typename Acc, int V>
void launch_bwd_main_t(dim3 grid, dim3 block, hipStream_t s, const BwdArgs& a) {
  // Column blocks (C a multiple of 256) imply rows of a multiple of 128 bytes.
  if (a.cb)
    hipLaunchKernelGGL((bwd_main_kernel<kBias, kBf16Policy, true, true, Acc, V>), grid, block, 0,
                       s, a);
  else if (rows_line_aligned(a.C))
    hipLaunchKernelGGL((bwd_main_kernel<kBias, kBf16Policy, true, false, Acc, V>), grid, block, 0,
                       s, a);
  else
    hipLaunchKernelGGL((bwd_main_kernel<kBias, kBf16Policy, false, false, Acc, V>), grid, block, 0,
                       s, a);
}

template <int V>
hipError_t launch_bwd_main_v(const Plan& plan, const BwdArgs& a, bool has_bias, bool fp32_policy,
                             hipStream_t s) {
  dim3 grid((uint32_t)padded_grid(plan.blocks)), block(kBlock);
  if (fp32_policy) {
    if (has_bias) launch_bwd_main_t<true, false, double, V>(grid, block, s, a);
    else launch_bwd_main_t<false, false, double, V>(grid, block, s, a);
  } else {
    if (has_bias) launch_bwd_main_t<true, true, float, V>(grid, block, s, a);
    else launch_bwd_main_t<false, true, float, V>(grid, block, s, a);
  }
  return hipGetLastError();
}

}  // namespace

// ======================================================== scratch array ==
//
// The workspace of conv1d_bwd_noalloc: a file-scope device array, one copy
// per GPU.  In host code its name stands for a host-side shadow, not a
// device address, so the kernels only ever receive the address that
// hipGetSymbolAddress returns for the device.  The lookup is made once per
// device, with that device current, and cached.  Calls on one GPU share
// the array: two such calls that may overlap in time race.  Nothing in it
// needs to start at zero (the backward writes every byte it reads).

namespace {
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_pointer(int device, void** out) {
  *out = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int current = 0;
    hipError_t e = hipGetDevice(&current);
    if (e != hipSuccess) return e;
    if (current != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (current != device) {
      const hipError_t r = hipSetDevice(current);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

// ============================================================ launchers ==

hipError_t launch_fwd(const Plan& plan, const FwdArgs& a, bool has_bias, hipStream_t s) {
  if (plan.vec != kFwdVec) return hipErrorInvalidValue;
  return launch_fwd_v<kFwdVec>(plan, a, has_bias, s);
}

hipError_t launch_bwd_main(const Plan& plan, const BwdArgs& a, bool has_bias, bool fp32_policy,
                           hipStream_t s) {
  if (plan.vec != kBwdVec) return hipErrorInvalidValue;
  return launch_bwd_main_v<kBwdVec>(plan, a, has_bias, fp32_policy, s);
}

hipError_t launch_bwd_reduce_rows(const Plan& plan, const ReduceArgs& a, bool part_f64,
                                  hipStream_t s) {
  dim3 grid(plan.red_blocks, plan.red_stage1), block(kRedOut * kRedChunks);
  if (part_f64) hipLaunchKernelGGL(bwd_reduce_rows_kernel<double>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(bwd_reduce_rows_kernel<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_reduce(const Plan& plan, const ReduceArgs& a, bool part_f64, hipStream_t s) {
  dim3 grid(plan.red_blocks), block(kRedOut * kRedChunks);
  if (part_f64) hipLaunchKernelGGL(bwd_reduce_kernel<double>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(bwd_reduce_kernel<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace vdc
