// Fused RoPE on Q and K + append of K/V into the paged cache.
//
// What it computes: Mojo docs, generic_fused_qk_rope_bshd_paged_ragged_
// kernel_api (rotate Q and K by the freqs_cis row of each token's position,
// write rotated Q to the output, update the keys of the paged cache in
// place), with V appended unrotated to the same slot; pair layouts of the
// aria_kernel crate (`rope`: interleaved, `rope_half`: rotate-half,
// `rope_half_partial`: only the first rotary_dim dims).  float8 caches store
// one scale per (token, kv head), absmax / 448.
//
// Design: a streaming pass, HBM-bound.  One thread owns a "unit" of 16
// elements of one head of one token: for the rotate-half layout the 8
// elements [8j, 8j+8) and their partners [R/2+8j, R/2+8j+8); for the
// interleaved layout and for pass-through dims, 16 consecutive elements.
// Consecutive threads own consecutive units of a head, so every load and
// K-store is a coalesced 16/32-byte vector access.  The D/16 units of a head
// are consecutive lanes of one wave, so the float8 absmax is a lane-group
// reduction.  V is stored dimension-major inside a page: its stores are
// per-element (stride page_size).

#include "common.h"
#include "internal.h"

namespace nk {
namespace {

enum CacheKind { kCacheF32 = 0, kCacheBF16 = 1, kCacheE4M3 = 2 };

template <typename T> struct InTraits;
template <> struct InTraits<float> {
  static NK_DEVICE void load8(const float *p, float *x) {
    f32x4_t a = *(const f32x4_t *)p, b = *(const f32x4_t *)(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
  }
  static NK_DEVICE void store8(float *p, const float *x) {
    f32x4_t a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = x[i]; b[i] = x[4 + i]; }
    *(f32x4_t *)p = a;
    *(f32x4_t *)(p + 4) = b;
  }
};
template <> struct InTraits<bf16_t> {
  static NK_DEVICE void load8(const bf16_t *p, float *x) {
    bf16x8_t a = *(const bf16x8_t *)p;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)a[i];
  }
  static NK_DEVICE void store8(bf16_t *p, const float *x) {
    bf16x8_t a;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (bf16_t)x[i];
    *(bf16x8_t *)p = a;
  }
};

// Store 8 consecutive K elements of a cache row (same element order).
template <int CACHE> NK_DEVICE void store_k8(void *row, int d0, const float *x, float inv_scale);
template <> NK_DEVICE void store_k8<kCacheF32>(void *row, int d0, const float *x, float) {
  InTraits<float>::store8((float *)row + d0, x);
}
template <> NK_DEVICE void store_k8<kCacheBF16>(void *row, int d0, const float *x, float) {
  InTraits<bf16_t>::store8((bf16_t *)row + d0, x);
}
template <> NK_DEVICE void store_k8<kCacheE4M3>(void *row, int d0, const float *x, float inv) {
  u32x2_t w;
  w[0] = f32x2_to_fp8x2(x[0] * inv, x[1] * inv) | (f32x2_to_fp8x2(x[2] * inv, x[3] * inv) << 16);
  w[1] = f32x2_to_fp8x2(x[4] * inv, x[5] * inv) | (f32x2_to_fp8x2(x[6] * inv, x[7] * inv) << 16);
  *(u32x2_t *)((uint8_t *)row + d0) = w;
}

// Store 8 V elements d0..d0+7 into a dimension-major page (stride P).
template <int CACHE> NK_DEVICE void store_v8(void *col, int d0, int P, const float *x, float inv);
template <> NK_DEVICE void store_v8<kCacheF32>(void *col, int d0, int P, const float *x, float) {
#pragma unroll
  for (int e = 0; e < 8; ++e) ((float *)col)[(size_t)(d0 + e) * P] = x[e];
}
template <> NK_DEVICE void store_v8<kCacheBF16>(void *col, int d0, int P, const float *x, float) {
#pragma unroll
  for (int e = 0; e < 8; ++e) ((bf16_t *)col)[(size_t)(d0 + e) * P] = (bf16_t)x[e];
}
template <> NK_DEVICE void store_v8<kCacheE4M3>(void *col, int d0, int P, const float *x, float inv) {
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    uint32_t c = f32x2_to_fp8x2(x[e] * inv, x[e + 1] * inv);
    ((uint8_t *)col)[(size_t)(d0 + e) * P] = (uint8_t)(c & 0xff);
    ((uint8_t *)col)[(size_t)(d0 + e + 1) * P] = (uint8_t)(c >> 8);
  }
}

// x / scale for the float8 quantiser, returned so that rounding it to e4m3
// (nearest, ties to even) gives the rounding of the EXACT quotient.  The
// float32 quotient is correctly rounded, so it can only be on the wrong side
// of an e4m3 rounding midpoint by landing exactly on that midpoint; then the
// sign of the exact remainder x - q*scale (one fma, exactly signed) says which
// way the exact quotient lies, and q moves one float32 step that way.  With
// bf16 inputs such near-ties are common (x*448/absmax is often a midpoint).
NK_DEVICE float fp8_quotient(float x, float scale) {
  float q = x / scale;
  const float aq = fabsf(q);
  if (!(aq < kFp8Max) || aq == 0.f) return q;
  const int e = (int)((__float_as_uint(aq) >> 23) & 0xff) - 127;   // aq in [2^e, 2^(e+1))
  if (e < -126) return q;
  const int step = max(e, -6) - 3;                  // e4m3 spacing 2^step around aq
  const float t = ldexpf(aq, 1 - step);             // exact: power-of-two scaling
  if (t == truncf(t) && (((int)t) & 1)) {           // aq is a midpoint
    const float r = fmaf(-q, scale, x);
    if (r != 0.f) q = nextafterf(q, r > 0.f ? INFINITY : -INFINITY);
  }
  return q;
}

struct Fp8Div {
  float scale;
  NK_DEVICE void apply(float *x) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = scale > 0.f ? fp8_quotient(x[e], scale) : 0.f;
  }
};

// a*d - b*c to within 1.5 float32 ulps of the exact value (Kahan's 2x2
// determinant: the product b*c is split into its float32 value and its exact
// rounding error by an fma).  A plain float32 x*c - y*s can lose every digit
// to cancellation; this keeps the stored rotation within one storage
// rounding of the exact one.
NK_DEVICE float det2(float a, float d, float b, float c) {
#pragma clang fp contract(off)
  const float w = b * c;
  const float e = fmaf(-b, c, w);       // w - b*c, exactly
  const float f = fmaf(a, d, -w);
  return f + e;
}

template <typename TIn, int CACHE, bool INTERLEAVED>
__global__ void __launch_bounds__(256) rope_write_kernel(RopeArgs a) {
  const int D = a.cache.head_dim;
  const int R = a.rotary_dim;
  const int P = a.cache.page_size;
  const int hkv = a.cache.num_kv_heads;
  const int units_per_head = D >> 4;
  const int heads_per_token = a.hq + 2 * hkv;
  const long long units = (long long)a.total_tokens * heads_per_token * units_per_head;
  const long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= units) return;

  const int j = (int)(u % units_per_head);
  const long long th = u / units_per_head;
  const int hh = (int)(th % heads_per_token);
  const int t = (int)(th / heads_per_token);

  const int kind = hh < a.hq ? 0 : (hh < a.hq + hkv ? 1 : 2);   // q, k, v
  const int head = kind == 0 ? hh : (kind == 1 ? hh - a.hq : hh - a.hq - hkv);
  const int hn = kind == 0 ? a.hq : hkv;
  const TIn *src = (const TIn *)(kind == 0 ? a.q : (kind == 1 ? a.k : a.v)) +
                   ((size_t)t * hn + head) * D;

  // run A / run B of this unit and whether it rotates
  const bool rotates = kind != 2 && (INTERLEAVED ? 16 * j < R : j < (R >> 4));
  int a0, b0;
  if (INTERLEAVED || kind == 2) {
    a0 = 16 * j; b0 = a0 + 8;
  } else if (rotates) {
    a0 = 8 * j; b0 = (R >> 1) + 8 * j;
  } else {
    a0 = R + 16 * (j - (R >> 4)); b0 = a0 + 8;
  }
  float xa[8], xb[8];
  InTraits<TIn>::load8(src + a0, xa);
  InTraits<TIn>::load8(src + b0, xb);

  const int s = find_segment(a.q_offsets, a.num_seqs, t);
  const int q0 = a.q_offsets[s];
  const int q_len = a.q_offsets[s + 1] - q0;
  const int slot = a.kv_lens[s] - q_len + (t - q0);

  if (rotates) {
    // out-of-range positions (a precondition violation) are clamped so that
    // the table read stays inside the table
    const int pos = min(max(a.position_ids ? a.position_ids[t] : slot, 0), a.max_pos - 1);
    const f32x4_t *cs = (const f32x4_t *)(a.freqs + ((size_t)pos * (R >> 1) + 8 * j) * 2);
    float c[8], sn[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4_t v = cs[i];
      c[2 * i] = v[0]; sn[2 * i] = v[1]; c[2 * i + 1] = v[2]; sn[2 * i + 1] = v[3];
    }
    if (INTERLEAVED) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = xa[2 * e], y = xa[2 * e + 1];
        xa[2 * e] = det2(x, c[e], y, sn[e]);
        xa[2 * e + 1] = det2(x, sn[e], -y, c[e]);
        x = xb[2 * e]; y = xb[2 * e + 1];
        xb[2 * e] = det2(x, c[4 + e], y, sn[4 + e]);
        xb[2 * e + 1] = det2(x, sn[4 + e], -y, c[4 + e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = xa[e], y = xb[e];
        xa[e] = det2(x, c[e], y, sn[e]);
        xb[e] = det2(x, sn[e], -y, c[e]);
      }
    }
  }

  if (kind == 0) {
    TIn *dst = (TIn *)a.q_out + ((size_t)t * a.hq + head) * D;
    InTraits<TIn>::store8(dst + a0, xa);
    InTraits<TIn>::store8(dst + b0, xb);
    return;
  }

  if (slot < 0) return;      // q_len > kv_len violates the precondition: no slot to write
  const int page = a.cache.page_table[(size_t)s * a.cache.page_table_stride + slot / P];
  const int off = slot % P;
  const size_t ph = (size_t)page * hkv + head;

  float inv = 1.f;
  if (CACHE == kCacheE4M3) {
    // absmax over the head: the D/16 units of a head are consecutive lanes
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fmaxf(fabsf(xa[e]), fabsf(xb[e])));
    for (int mask = 1; mask < units_per_head; mask <<= 1) m = fmaxf(m, shfl_xor_f32(m, mask));
    const float scale = m / kFp8Max;
    Fp8Div{scale}.apply(xa);
    Fp8Div{scale}.apply(xb);
    if (j == 0) (kind == 1 ? a.cache.k_scales : a.cache.v_scales)[ph * P + off] = scale;
  }

  constexpr int esz = CACHE == kCacheF32 ? 4 : (CACHE == kCacheBF16 ? 2 : 1);
  if (kind == 1) {
    void *row = (uint8_t *)a.cache.k_pages + (ph * P + off) * (size_t)D * esz;
    store_k8<CACHE>(row, a0, xa, inv);
    store_k8<CACHE>(row, b0, xb, inv);
  } else {
    void *col = (uint8_t *)a.cache.v_pages + (ph * D * P + off) * (size_t)esz;
    store_v8<CACHE>(col, a0, P, xa, inv);
    store_v8<CACHE>(col, b0, P, xb, inv);
  }
}

template <typename TIn, int CACHE>
hipError_t launch_layout(const RopeArgs &a, hipStream_t stream) {
  const int hkv = a.cache.num_kv_heads;
  const long long units = (long long)a.total_tokens * (a.hq + 2 * hkv) * (a.cache.head_dim / 16);
  const int block = 256;
  const long long grid = (units + block - 1) / block;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.layout == NK_ROPE_INTERLEAVED)
    rope_write_kernel<TIn, CACHE, true><<<(unsigned)grid, block, 0, stream>>>(a);
  else
    rope_write_kernel<TIn, CACHE, false><<<(unsigned)grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_write(const RopeArgs &a, hipStream_t stream) {
  if (a.total_tokens == 0) return hipSuccess;
  ProfileScope prof("rope_write", stream);
  if (a.in_dtype == NK_F32 && a.cache.dtype == NK_F32) return launch_layout<float, kCacheF32>(a, stream);
  if (a.in_dtype == NK_BF16 && a.cache.dtype == NK_BF16) return launch_layout<bf16_t, kCacheBF16>(a, stream);
  if (a.in_dtype == NK_BF16 && a.cache.dtype == NK_E4M3) return launch_layout<bf16_t, kCacheE4M3>(a, stream);
  if (a.in_dtype == NK_F32 && a.cache.dtype == NK_E4M3) return launch_layout<float, kCacheE4M3>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace nk
