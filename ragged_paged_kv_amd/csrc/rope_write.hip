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
// Rounding: the rotation runs in float64 and every stored element is rounded
// once from it (see round_odd_f32), so q_out and the appended cache rows are
// exactly the float64 definition rounded to the storage type.
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

// ---------------------------------------------------------------- rounding
// The rotation is computed in float64: an input (bf16 or float32) times a
// float32 table entry is exact in float64, so x*c - y*s is the float64
// nearest to the exact value, as the float64 definition computes it.  Each
// stored element is then rounded ONCE from that float64: to float32 directly,
// to bf16 / e4m3 through a float32 rounded to odd (truncate, then set the last
// bit if anything was dropped) -- with at least two spare bits, the final
// round-to-nearest-even of a round-to-odd intermediate equals the direct
// rounding of the float64.

NK_DEVICE float round_odd_f32(double d) {
  float f = __double2float_rz(d);
  if ((double)f != d) f = __uint_as_float(__float_as_uint(f) | 1u);
  return f;
}

template <typename T> struct InTraits;
template <> struct InTraits<float> {
  static NK_DEVICE void load8(const float *p, double *x) {
    f32x4_t a = *(const f32x4_t *)p, b = *(const f32x4_t *)(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
  }
  static NK_DEVICE void store8(float *p, const double *x) {
    f32x4_t a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = (float)x[i]; b[i] = (float)x[4 + i]; }
    *(f32x4_t *)p = a;
    *(f32x4_t *)(p + 4) = b;
  }
};
template <> struct InTraits<bf16_t> {
  static NK_DEVICE void load8(const bf16_t *p, double *x) {
    bf16x8_t a = *(const bf16x8_t *)p;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (double)(float)a[i];
  }
  static NK_DEVICE void store8(bf16_t *p, const double *x) {
    bf16x8_t a;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (bf16_t)round_odd_f32(x[i]);
    *(bf16x8_t *)p = a;
  }
};

// e4m3 code pair from two float64 quotients x/scale (already in range or
// saturated at +-448 here).
NK_DEVICE uint32_t fp8x2(double a, double b) {
  return f32x2_to_fp8x2(round_odd_f32(fmin(fmax(a, -448.0), 448.0)),
                        round_odd_f32(fmin(fmax(b, -448.0), 448.0)));
}

// Store 8 consecutive K elements (within one 32-dim block of a token).
template <int CACHE> NK_DEVICE void store_k8(void *row, int d0, const double *x);
template <> NK_DEVICE void store_k8<kCacheF32>(void *row, int d0, const double *x) {
  InTraits<float>::store8((float *)row + d0, x);
}
template <> NK_DEVICE void store_k8<kCacheBF16>(void *row, int d0, const double *x) {
  InTraits<bf16_t>::store8((bf16_t *)row + d0, x);
}
template <> NK_DEVICE void store_k8<kCacheE4M3>(void *row, int d0, const double *x) {
  u32x2_t w;
  w[0] = fp8x2(x[0], x[1]) | (fp8x2(x[2], x[3]) << 16);
  w[1] = fp8x2(x[4], x[5]) | (fp8x2(x[6], x[7]) << 16);
  *(u32x2_t *)((uint8_t *)row + d0) = w;
}

// K page-head block (include/nk.h): blocks of 32*NK dims (NK 2 for e4m3,
// else 1), slot after slot; a slot's row of a block is 4 runs of NK*8
// elements, run g holding dims 8g..8g+7 of each 32-dim half.  Offset of
// (dim d, slot t), d a multiple of 8: the 8 dims d..d+7 are contiguous.
template <int CACHE> NK_DEVICE size_t k_index(int d, int t, int P) {
  constexpr int NK = CACHE == kCacheE4M3 ? 2 : 1;
  return ((size_t)(d / (32 * NK)) * P + t) * (32 * NK) + ((d & 31) >> 3) * (NK * 8) + ((d >> 5) % NK) * 8;
}

// V page-head block in MFMA operand order (include/nk.h): element (dim d,
// slot t) sits at v_index(d, t); for 8 consecutive dims of one 16-dim tile
// the offsets step by 4*NV elements, NV = 4 / element bytes.
template <int CACHE> constexpr int v_nv() { return CACHE == kCacheF32 ? 1 : (CACHE == kCacheBF16 ? 2 : 4); }
template <int CACHE> NK_DEVICE size_t v_index(int d, int t, int D) {
  constexpr int NV = v_nv<CACHE>();
  const int c = (d >> 4) / NV;
  return ((size_t)(t >> 4) * (D / (16 * NV)) + c) * (64 * 4 * NV) +
         (size_t)(16 * ((t & 15) >> 2) + (d & 15)) * (4 * NV) + ((d >> 4) % NV) * 4 + (t & 3);
}

// Store 8 V elements d0..d0+7 (d0 a multiple of 8) of slot t.
template <int CACHE> NK_DEVICE void store_v8(void *blk, int d0, int t, int D, const double *x);
template <> NK_DEVICE void store_v8<kCacheF32>(void *blk, int d0, int t, int D, const double *x) {
  float *p = (float *)blk + v_index<kCacheF32>(d0, t, D);
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e * 4] = (float)x[e];
}
template <> NK_DEVICE void store_v8<kCacheBF16>(void *blk, int d0, int t, int D, const double *x) {
  bf16_t *p = (bf16_t *)blk + v_index<kCacheBF16>(d0, t, D);
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e * 8] = (bf16_t)round_odd_f32(x[e]);
}
template <> NK_DEVICE void store_v8<kCacheE4M3>(void *blk, int d0, int t, int D, const double *x) {
  uint8_t *p = (uint8_t *)blk + v_index<kCacheE4M3>(d0, t, D);
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    uint32_t c = fp8x2(x[e], x[e + 1]);
    p[e * 16] = (uint8_t)(c & 0xff);
    p[(e + 1) * 16] = (uint8_t)(c >> 8);
  }
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
  double xa[8], xb[8];
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
    double c[8], sn[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4_t v = cs[i];
      c[2 * i] = v[0]; sn[2 * i] = v[1]; c[2 * i + 1] = v[2]; sn[2 * i + 1] = v[3];
    }
    if (INTERLEAVED) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        double x = xa[2 * e], y = xa[2 * e + 1];
        xa[2 * e] = x * c[e] - y * sn[e];
        xa[2 * e + 1] = x * sn[e] + y * c[e];
        x = xb[2 * e]; y = xb[2 * e + 1];
        xb[2 * e] = x * c[4 + e] - y * sn[4 + e];
        xb[2 * e + 1] = x * sn[4 + e] + y * c[4 + e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        double x = xa[e], y = xb[e];
        xa[e] = x * c[e] - y * sn[e];
        xb[e] = x * sn[e] + y * c[e];
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

  if (CACHE == kCacheE4M3) {
    // absmax over the head: the D/16 units of a head are consecutive lanes
    double m = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmax(m, fmax(fabs(xa[e]), fabs(xb[e])));
    for (int mask = 1; mask < units_per_head; mask <<= 1) m = fmax(m, __shfl_xor(m, mask, kWave));
    const float scale = (float)(m / 448.0);            // float32 nearest to absmax / 448
    const double sd = scale;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      xa[e] = scale > 0.f ? xa[e] / sd : 0.0;
      xb[e] = scale > 0.f ? xb[e] / sd : 0.0;
    }
    if (j == 0) (kind == 1 ? a.cache.k_scales : a.cache.v_scales)[ph * P + off] = scale;
  }

  constexpr int esz = CACHE == kCacheF32 ? 4 : (CACHE == kCacheBF16 ? 2 : 1);
  if (kind == 1) {
    // K page: blocks of 32*NK dims, see k_index
    uint8_t *kph = (uint8_t *)a.cache.k_pages + ph * P * (size_t)D * esz;
    store_k8<CACHE>(kph + k_index<CACHE>(a0, off, P) * esz, 0, xa);
    store_k8<CACHE>(kph + k_index<CACHE>(b0, off, P) * esz, 0, xb);
  } else {
    // V page: MFMA operand order, see v_index
    void *blk = (uint8_t *)a.cache.v_pages + ph * D * (size_t)P * esz;
    store_v8<CACHE>(blk, a0, off, D, xa);
    store_v8<CACHE>(blk, b0, off, D, xb);
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
