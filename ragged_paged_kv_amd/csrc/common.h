// Device-side helpers shared by the kernels: element types, MFMA operand
// vectors, conversions, wave reductions.  gfx950 (CDNA4) only, wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nk.h"

#define NK_DEVICE __device__ __forceinline__

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kFp8Max = 448.0f;

// ---------------------------------------------------------------- bf16
NK_DEVICE float bf16_to_f32(bf16_t x) { return (float)x; }
NK_DEVICE bf16_t f32_to_bf16(float x) { return (bf16_t)x; }  // round to nearest even

NK_DEVICE float bits_bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// ---------------------------------------------------------------- e4m3 (OCP e4m3fn)
// Eight codes (two dwords) to an MFMA bf16x8 operand.  Exact: a code has at
// most four significant bits and its exponent range lies inside bf16's; the
// scaled convert with scale 1.0 applies no scaling.
NK_DEVICE bf16x8_t fp8x8_to_bf16x8(u32x2_t w) {
  bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
  bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
  bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
  bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Round two floats to e4m3 codes (nearest even), packed into bytes 0,1 of the
// result.  Inputs are clamped to +-448 first so that the conversion never
// sees an out-of-range value (the quantiser's inputs are within a rounding
// step of that range by construction).
NK_DEVICE uint32_t f32x2_to_fp8x2(float a, float b) {
  a = fminf(fmaxf(a, -kFp8Max), kFp8Max);
  b = fminf(fmaxf(b, -kFp8Max), kFp8Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// ---------------------------------------------------------------- wave helpers
NK_DEVICE float shfl_xor_f32(float v, int mask) { return __shfl_xor(v, mask, kWave); }

NK_DEVICE float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor_f32(v, m));
  return v;
}

NK_DEVICE float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f32(v, m);
  return v;
}

NK_DEVICE float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
NK_DEVICE float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Last key visible to a query at position p of a segment with L keys:
// min(p + window_right, L - 1), or L - 1 when the right side is unbounded
// (-1).  p may be negative (a row placed before the segment's first key);
// the comparison is made without forming p + window_right, which could
// overflow.
NK_DEVICE int band_hi(int p, int L, int window_right) {
  if (window_right < 0 || p >= L - 1 - window_right) return L - 1;
  return p + window_right;
}

// First key visible at position p: max(0, p - window_left), or 0 when the
// left side is unbounded (-1); p - window_left is formed only when positive.
NK_DEVICE int band_lo(int p, int window_left) {
  return (window_left < 0 || p <= window_left) ? 0 : p - window_left;
}

// Split-KV chunks of a single-token row with L keys (its position L - 1):
// the band [lo, L-1] cut into chunks of `split` keys from c0 (lo rounded
// down to 32), then, when sink keys lie before lo, one chunk of the keys
// [0, sink_end).  At most max_chunks chunks (a key count above the batch's
// bound violates the precondition and loses the rest).
struct DecodeChunks {
  int lo, c0, n_band, n, sink_end;
};
NK_DEVICE DecodeChunks decode_chunks(int L, int window_left, int sink_keys, int split, int max_chunks) {
  DecodeChunks d;
  const int hi = L - 1;
  d.lo = band_lo(hi, window_left);
  d.c0 = (d.lo / 32) * 32;
  d.sink_end = min(sink_keys, d.lo);
  d.n_band = L > 0 ? min((hi + 1 - d.c0 + split - 1) / split, max_chunks) : 1;
  d.n = min(d.n_band + (L > 0 && d.sink_end > 0 ? 1 : 0), max_chunks);
  return d;
}

// Index of the first segment s with q_offsets[s+1] > t (binary search).
NK_DEVICE int find_segment(const int32_t *__restrict__ q_offsets, int num_seqs, int t) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (q_offsets[mid + 1] > t) hi = mid; else lo = mid + 1;
  }
  return lo;
}
