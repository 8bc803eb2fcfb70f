// HIP kernels for gfx950: packed variable-length width-4 depthwise causal
// convolution + SiLU, training forward and backward.
//
// The operation is the one documented on the pages of
// flashinfer.cake_causal_conv1d_train (cake_causal_conv1d_train_forward:
// Returns; cake_causal_conv1d_train_backward: Description, Returns).  It is
// a 4-tap stencil along the token axis followed by an elementwise SiLU, so
// it is bound by HBM traffic, not by matrix throughput: no MFMA here.
//
// Work decomposition (same for every kernel of the main path):
//  * A lane owns one 16-byte vector of 8 consecutive BF16 channels and a
//    band of T consecutive tokens, and walks the band row by row.  Lanes are
//    numbered (band, vector) -> band * (C/8) + vector, so the 64 lanes of a
//    wave read 64 consecutive vectors of a row (1 KiB, fully coalesced) and,
//    when C/8 is not a multiple of 64, simply continue into the next band.
//  * A lane keeps the previous three rows of x in registers; at a document
//    start the window is cleared, which is exactly the zero history the
//    forward prescribes, so no tap needs a mask.  The document starts are
//    found by one binary search of cu_seqlens per lane and a forward walk.
//  * Tensors are addressed through buffer resources based at the wave's
//    first row, with 32-bit per-lane offsets: rows past S read as zero and
//    their stores are dropped by the hardware range check.
//  * Arithmetic is FP32 with one fixed evaluation order for the
//    preactivation, shared by the forward and the backward recompute, so
//    both see the same bits of p.

#include <hip/hip_runtime.h>

#include <climits>
#include <stdint.h>

#include "vdc_internal.h"

namespace vdc {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
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

// ---------------------------------------------------------------- BF16 --

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ void unpack8(u32x4 v, float (&f)[8]) {
  f[0] = bf_lo(v.x); f[1] = bf_hi(v.x);
  f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
  f[4] = bf_lo(v.z); f[5] = bf_hi(v.z);
  f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
}

// Two FP32 -> packed BF16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2 h = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  u32x4 r;
  r.x = pack2(f[0], f[1]);
  r.y = pack2(f[2], f[3]);
  r.z = pack2(f[4], f[5]);
  r.w = pack2(f[6], f[7]);
  return r;
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

// ------------------------------------------------------ buffer access --

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}
__device__ __forceinline__ u32x4 ld16(rsrc_t r, int32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ void st16(rsrc_t r, int32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

// Bytes from row `row` to the end of an [S][C] BF16 tensor, clamped to what
// a buffer resource can describe.  The host keeps a wave's whole span far
// below 2^31 bytes, so the clamp only ever applies far from the end.
__device__ __forceinline__ uint32_t span_bytes(int32_t S, int32_t C, int32_t row) {
  uint64_t rem = (uint64_t)(int64_t)(S - row) * (uint64_t)C * 2u;
  return rem > 0xffffffffull ? 0xffffffffu : (uint32_t)rem;
}

// ------------------------------------------------------- parameters --

// weight [C][4] (FP32: one 16-byte vector per channel; BF16: two channels
// per 16-byte vector) -> w[k][i] for the lane's channels c0 .. c0+7.
__device__ __forceinline__ void load_weights(const void* w, int bf16, uint32_t c0,
                                             float (&wk)[4][8]) {
  if (!bf16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(w) + c0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4 v = p[i];
      wk[0][i] = __uint_as_float(v.x);
      wk[1][i] = __uint_as_float(v.y);
      wk[2][i] = __uint_as_float(v.z);
      wk[3][i] = __uint_as_float(v.w);
    }
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(w) + c0 / 2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4 v = p[q];
      wk[0][2 * q] = bf_lo(v.x);
      wk[1][2 * q] = bf_hi(v.x);
      wk[2][2 * q] = bf_lo(v.y);
      wk[3][2 * q] = bf_hi(v.y);
      wk[0][2 * q + 1] = bf_lo(v.z);
      wk[1][2 * q + 1] = bf_hi(v.z);
      wk[2][2 * q + 1] = bf_lo(v.w);
      wk[3][2 * q + 1] = bf_hi(v.w);
    }
  }
}

__device__ __forceinline__ void load_bias(const void* b, int bf16, uint32_t c0, float (&bv)[8]) {
  if (!bf16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(b) + c0 / 4;
    u32x4 v0 = p[0], v1 = p[1];
    bv[0] = __uint_as_float(v0.x); bv[1] = __uint_as_float(v0.y);
    bv[2] = __uint_as_float(v0.z); bv[3] = __uint_as_float(v0.w);
    bv[4] = __uint_as_float(v1.x); bv[5] = __uint_as_float(v1.y);
    bv[6] = __uint_as_float(v1.z); bv[7] = __uint_as_float(v1.w);
  } else {
    unpack8(reinterpret_cast<const u32x4*>(b)[c0 / 8], bv);
  }
}

// ------------------------------------------------- document starts --

// The document starts are the values of cu_seqlens below S (an empty
// document repeats its successor's start).  A lane finds the first start at
// or after its first row with a binary search and then walks forward.
struct DocWalk {
  const int32_t* cu;
  int32_t last;  // index of the last entry (num_docs)
  int32_t idx;
  int32_t next;  // smallest start >= the current row (INT_MAX if none)

  __device__ __forceinline__ void init(const int32_t* cu_, int32_t num_docs, int32_t row) {
    cu = cu_;
    last = num_docs;
    int32_t lo = 0, hi = num_docs + 1;
    while (lo < hi) {
      int32_t mid = (lo + hi) >> 1;
      if (cu[mid] < row) lo = mid + 1; else hi = mid;
    }
    idx = lo;
    next = lo <= last ? cu[lo] : INT_MAX;
  }
  // Called on the row that equals `next`: move past every start <= row.
  __device__ __forceinline__ void advance(int32_t row) {
    do {
      ++idx;
      next = idx <= last ? cu[idx] : INT_MAX;
    } while (next <= row);
  }
};

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

// SiLU'(z) = s * (1 + z * (1 - s)), evaluated as fma(z - z*s, s, s).
__device__ __forceinline__ float silu_grad_fast(float z) {
  float s = sigmoid_fast(z);
  float t = __builtin_fmaf(-z, s, z);
  return __builtin_fmaf(t, s, s);
}

// SiLU'(z) for z < kDeep: there 1 - s == 1 in binary32, so s * (1 + z).
__device__ __forceinline__ float silu_grad_deep(float z) {
  return (sigmoid_scaled64(z) * (1.0f + z)) * 0x1p-64f;
}

// The preactivation, in the one fixed order used by both directions:
// ((w0 x[t-3] + w1 x[t-2]) + w2 x[t-1]) + w3 x[t], then + bias.
template <bool kBias>
__device__ __forceinline__ float preact(const float (&w)[4][8], const float (&bv)[8], int i,
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

__device__ __forceinline__ bool lane_coords(int32_t nvec, int32_t rows, int32_t bands, int32_t C,
                                            Lane& L) {
  const uint32_t g = blockIdx.x * (uint32_t)kBlock + threadIdx.x;
  L.band = g / (uint32_t)nvec;
  if (L.band >= (uint32_t)bands) return false;
  L.vec = g - L.band * (uint32_t)nvec;
  L.t0 = (int32_t)L.band * rows;
  const int32_t first_band = __builtin_amdgcn_readfirstlane((int32_t)L.band);
  L.base_row = max(first_band * rows - 3, 0);
  L.off = (L.t0 - 3 - L.base_row) * (C * 2) + (int32_t)L.vec * 16;
  return true;
}

// ===================================================== forward kernel ==

template <bool kBias>
__global__ __launch_bounds__(kBlock) void fwd_kernel(FwdArgs a) {
  Lane L;
  if (!lane_coords(a.nvec, a.rows, a.bands, a.C, L)) return;
  const int32_t row_bytes = a.C * 2;
  const uint32_t nrec = span_bytes(a.S, a.C, L.base_row);
  const rsrc_t rx = make_rsrc(a.x + (int64_t)L.base_row * a.C, nrec);
  const rsrc_t ry = make_rsrc(a.y + (int64_t)L.base_row * a.C, nrec);

  float w[4][8], bv[8];
  load_weights(a.w, a.w_bf16, L.vec * kVec, w);
  if (kBias) load_bias(a.b, a.b_bf16, L.vec * kVec, bv);

  int32_t r = L.t0 - 3;
  int32_t off = L.off;
  DocWalk walk;
  walk.init(a.cu, a.num_docs, max(r, 0));

  // Window of the three previous rows: h1 = x[r-1], h2 = x[r-2], h3 = x[r-3].
  float h1[8], h2[8], h3[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h1[i] = h2[i] = h3[i] = 0.0f;

  // Halo rows t0-3 .. t0-1 (before the first token nothing is read).
#pragma unroll
  for (int q = 0; q < 3; ++q, ++r, off += row_bytes) {
    u32x4 v = (u32x4){0u, 0u, 0u, 0u};
    if (r >= 0) v = ld16(rx, off);
    if (r == walk.next) {
#pragma unroll
      for (int i = 0; i < 8; ++i) h1[i] = h2[i] = 0.0f;
      walk.advance(r);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) h3[i] = h2[i], h2[i] = h1[i];
    unpack8(v, h1);
  }

  for (int32_t done = 0; done < a.rows; done += kFwdGroup) {
    u32x4 raw[kFwdGroup];
#pragma unroll
    for (int g = 0; g < kFwdGroup; ++g) raw[g] = ld16(rx, off + g * row_bytes);
    const bool quiet = walk.next > r + (kFwdGroup - 1);
#pragma unroll
    for (int g = 0; g < kFwdGroup; ++g) {
      if (!quiet && r + g == walk.next) {
#pragma unroll
        for (int i = 0; i < 8; ++i) h1[i] = h2[i] = h3[i] = 0.0f;
        walk.advance(r + g);
      }
      float xc[8], p[8], yv[8];
      unpack8(raw[g], xc);
      float pmin = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = preact<kBias>(w, bv, i, h3[i], h2[i], h1[i], xc[i]);
        pmin = __builtin_fminf(pmin, p[i]);
        yv[i] = p[i] * sigmoid_fast(p[i]);
      }
      u32x4 out = pack8(yv);
      if (pmin < kDeep) {
        // Rare: some p is so negative that sigmoid(p) underflows on the fast
        // path; redo those values in scaled form and round them exactly.
        uint32_t hbits[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float yd = (p[i] * sigmoid_scaled64(p[i])) * 0x1p-64f;
          hbits[i] = p[i] < kDeep ? bf16_bits_rne(yd) : bf16_bits_rne(yv[i]);
        }
        out.x = hbits[0] | (hbits[1] << 16);
        out.y = hbits[2] | (hbits[3] << 16);
        out.z = hbits[4] | (hbits[5] << 16);
        out.w = hbits[6] | (hbits[7] << 16);
      }
      st16(ry, off + g * row_bytes, out);
#pragma unroll
      for (int i = 0; i < 8; ++i) h3[i] = h2[i], h2[i] = h1[i], h1[i] = xc[i];
    }
    r += kFwdGroup;
    off += kFwdGroup * row_bytes;
  }
}

// ================================================ backward main kernel ==

template <typename Acc>
struct Partials {
  Acc v[5][8];  // taps k = 0..3, then the bias term
};

// One row of the backward: recompute p, form dpre, accumulate partials and
// emit dx of the row three tokens back.
//  hist: bit 0 = row v is a document start, bit 1 = row v-1, bit 2 = row v-2.
template <bool kBias, bool kBf16Policy, typename Acc>
__device__ __forceinline__ void bwd_row(const float (&w)[4][8], const float (&bv)[8],
                                        const float (&xc)[8], u32x4 dyraw,
                                        float (&h1)[8], float (&h2)[8], float (&h3)[8],
                                        float (&d1)[8], float (&d2)[8], float (&d3)[8],
                                        Partials<Acc>& acc, bool accumulate, bool emit,
                                        uint32_t hist, bool masked, rsrc_t rdx, int32_t dx_off) {
  float dyv[8], p[8], dp[8];
  unpack8(dyraw, dyv);
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = preact<kBias>(w, bv, i, h3[i], h2[i], h1[i], xc[i]);
  float z[8];
  if (kBf16Policy) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      uint32_t h = pack2(p[i], p[i + 1]);
      z[i] = bf_lo(h);
      z[i + 1] = bf_hi(h);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = p[i];
  }
  float zmin = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    zmin = __builtin_fminf(zmin, z[i]);
    dp[i] = dyv[i] * silu_grad_fast(z[i]);
  }
  if (zmin < kDeep) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (z[i] < kDeep) dp[i] = dyv[i] * silu_grad_deep(z[i]);
  }
  if (accumulate) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const Acc g = (Acc)dp[i];
      acc.v[0][i] += g * (Acc)h3[i];
      acc.v[1][i] += g * (Acc)h2[i];
      acc.v[2][i] += g * (Acc)h1[i];
      acc.v[3][i] += g * (Acc)xc[i];
      acc.v[4][i] += g;
    }
  }
  if (emit) {
    // dx[v-3] = w3 d[v-3] + w2 d[v-2] + w1 d[v-1] + w0 d[v], each later
    // token counted only if no document starts between v-3 and it.
    const bool m1 = !masked || !(hist & 4u);
    const bool m2 = !masked || !(hist & 6u);
    const bool m3 = !masked || !(hist & 7u);
    float dxv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float s = w[3][i] * d3[i];
      s = __builtin_fmaf(w[2][i], m1 ? d2[i] : 0.0f, s);
      s = __builtin_fmaf(w[1][i], m2 ? d1[i] : 0.0f, s);
      s = __builtin_fmaf(w[0][i], m3 ? dp[i] : 0.0f, s);
      dxv[i] = s;
    }
    st16(rdx, dx_off, pack8(dxv));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h3[i] = h2[i]; h2[i] = h1[i]; h1[i] = xc[i];
    d3[i] = d2[i]; d2[i] = d1[i]; d1[i] = dp[i];
  }
}

template <bool kBias, bool kBf16Policy, typename Acc>
__global__ __launch_bounds__(kBlock) void bwd_main_kernel(BwdArgs a) {
  Lane L;
  if (!lane_coords(a.nvec, a.rows, a.bands, a.C, L)) return;
  const int32_t row_bytes = a.C * 2;
  const uint32_t nrec = span_bytes(a.S, a.C, L.base_row);
  const int64_t base_elt = (int64_t)L.base_row * a.C;
  const rsrc_t rx = make_rsrc(a.x + base_elt, nrec);
  const rsrc_t rdy = make_rsrc(a.dy + base_elt, nrec);
  const rsrc_t rdx = make_rsrc(a.dx + base_elt, nrec);

  float w[4][8], bv[8];
  load_weights(a.w, a.w_bf16, L.vec * kVec, w);
  if (kBias) load_bias(a.b, a.b_bf16, L.vec * kVec, bv);

  Partials<Acc> acc;
#pragma unroll
  for (int k = 0; k < 5; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc.v[k][i] = (Acc)0;

  int32_t r = L.t0 - 3;
  int32_t off = L.off;
  DocWalk walk;
  walk.init(a.cu, a.num_docs, max(r, 0));
  uint32_t hist = 0;  // bit 0 = row r-1 starts a document, bit 1 = row r-2

  float h1[8], h2[8], h3[8], d1[8], d2[8], d3[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h1[i] = h2[i] = h3[i] = d1[i] = d2[i] = d3[i] = 0.0f;

  // Halo rows t0-3 .. t0-1: x only.
#pragma unroll
  for (int q = 0; q < 3; ++q, ++r, off += row_bytes) {
    u32x4 v = (u32x4){0u, 0u, 0u, 0u};
    if (r >= 0) v = ld16(rx, off);
    uint32_t start = 0;
    if (r == walk.next) {
#pragma unroll
      for (int i = 0; i < 8; ++i) h1[i] = h2[i] = 0.0f;
      walk.advance(r);
      start = 1;
    }
    hist = ((hist << 1) | start) & 3u;
#pragma unroll
    for (int i = 0; i < 8; ++i) h3[i] = h2[i], h2[i] = h1[i];
    unpack8(v, h1);
  }

  // Band rows t0 .. t0+T-1 (partials), then three look-ahead rows (dx only).
  const int32_t total = a.rows + 3;
  for (int32_t done = 0; done < total; done += kBwdGroup) {
    u32x4 xr[kBwdGroup], dr[kBwdGroup];
#pragma unroll
    for (int g = 0; g < kBwdGroup; ++g) {
      xr[g] = ld16(rx, off + g * row_bytes);
      dr[g] = ld16(rdy, off + g * row_bytes);
    }
    const bool quiet = hist == 0 && walk.next > r + (kBwdGroup - 1);
#pragma unroll
    for (int g = 0; g < kBwdGroup; ++g) {
      const int32_t idx = done + g;        // row t0 + idx
      if (idx >= total) break;
      uint32_t h3bits = 0;
      if (!quiet) {
        uint32_t start = 0;
        if (r + g == walk.next) {
#pragma unroll
          for (int i = 0; i < 8; ++i) h1[i] = h2[i] = h3[i] = 0.0f;
          walk.advance(r + g);
          start = 1;
        }
        h3bits = (hist << 1) | start;
        hist = h3bits & 3u;
      }
      float xc[8];
      unpack8(xr[g], xc);
      bwd_row<kBias, kBf16Policy, Acc>(w, bv, xc, dr[g], h1, h2, h3, d1, d2, d3, acc,
                                       idx < a.rows, idx >= 3, h3bits, !quiet, rdx,
                                       off + (g - 3) * row_bytes);
    }
    r += kBwdGroup;
    off += kBwdGroup * row_bytes;
  }

  // One partial row per band: part[band][k][c].
  Acc* part = reinterpret_cast<Acc*>(a.part) + (int64_t)L.band * 5 * a.C + L.vec * kVec;
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    Acc* dst = part + (int64_t)k * a.C;
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = acc.v[k][i];
  }
}

// =================================================== backward reduce ==

template <typename Acc>
__device__ __forceinline__ void store_grad(void* dst, int64_t i, Acc v, int bf16);

template <>
__device__ __forceinline__ void store_grad<float>(void* dst, int64_t i, float v, int bf16) {
  if (bf16) reinterpret_cast<uint16_t*>(dst)[i] = (uint16_t)bf16_bits_rne(v);
  else reinterpret_cast<float*>(dst)[i] = v;
}

template <>
__device__ __forceinline__ void store_grad<double>(void* dst, int64_t i, double v, int bf16) {
  if (bf16) reinterpret_cast<uint16_t*>(dst)[i] = bf16_bits_from_f64(v);
  else reinterpret_cast<float*>(dst)[i] = (float)v;
}

// out[o] = sum_{b=0..P-1} part[b][o] for o = k*C + c, in a fixed order:
// chunk q sums rows [q*R, q*R+R) in increasing b, then the kRedChunks chunk
// sums are added in increasing q.  The order depends on (P, C) only.
template <typename Acc>
__global__ __launch_bounds__(kRedOut * kRedChunks) void bwd_reduce_kernel(ReduceArgs a) {
  __shared__ Acc red[kRedChunks][kRedOut];
  const int lane = threadIdx.x % kRedOut;
  const int chunk = threadIdx.x / kRedOut;
  const int64_t n_out = 5 * (int64_t)a.C;
  const int64_t o = (int64_t)blockIdx.x * kRedOut + lane;
  Acc s = (Acc)0;
  if (o < n_out) {
    const int32_t b0 = chunk * a.rows_per_chunk;
    const int32_t b1 = min(b0 + a.rows_per_chunk, a.P);
    const Acc* p = reinterpret_cast<const Acc*>(a.part) + (int64_t)b0 * n_out + o;
#pragma unroll 8
    for (int32_t b = b0; b < b1; ++b, p += n_out) s += *p;
  }
  red[chunk][lane] = s;
  __syncthreads();
  if (chunk == 0 && o < n_out) {
    Acc t = red[0][lane];
#pragma unroll
    for (int q = 1; q < kRedChunks; ++q) t += red[q][lane];
    const int64_t k = o / a.C;
    const int64_t c = o - k * a.C;
    if (k < 4) store_grad<Acc>(a.dw, c * 4 + k, t, a.dw_bf16);
    else if (a.db) store_grad<Acc>(a.db, c, t, a.db_bf16);
  }
}

}  // namespace

// ============================================================ launchers ==

hipError_t launch_fwd(const Plan& plan, const FwdArgs& a, bool has_bias, hipStream_t s) {
  dim3 grid(plan.blocks), block(kBlock);
  if (has_bias) hipLaunchKernelGGL(fwd_kernel<true>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(fwd_kernel<false>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_main(const Plan& plan, const BwdArgs& a, bool has_bias, bool fp32_policy,
                           hipStream_t s) {
  dim3 grid(plan.blocks), block(kBlock);
  if (fp32_policy) {
    if (has_bias) hipLaunchKernelGGL((bwd_main_kernel<true, false, double>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((bwd_main_kernel<false, false, double>), grid, block, 0, s, a);
  } else {
    if (has_bias) hipLaunchKernelGGL((bwd_main_kernel<true, true, float>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((bwd_main_kernel<false, true, float>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_reduce(const Plan& plan, const ReduceArgs& a, bool fp64, hipStream_t s) {
  dim3 grid(plan.red_blocks), block(kRedOut * kRedChunks);
  if (fp64) hipLaunchKernelGGL(bwd_reduce_kernel<double>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(bwd_reduce_kernel<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace vdc
