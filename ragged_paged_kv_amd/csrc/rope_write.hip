// Fused RoPE on Q and K + append of K/V into the paged cache.
//
// What it computes: Mojo docs, generic_fused_qk_rope_bshd_paged_ragged_
// kernel_api (rotate Q and K by the freqs_cis row of each token's position,
// write rotated Q to the output, update the keys of the paged cache in
// place), with V appended unrotated to the same slot; pair layouts of the
// aria_kernel crate (`rope`: interleaved, `rope_half`: rotate-half,
// `rope_half_partial`: only the first rotary_dim dims, `rope_half_proportional`:
// rotate-half pairs over the whole head, only the first rotary_dim/2
// rotated).  float8 caches store one scale per (token, kv head), absmax / 448.
//
// Rounding: the rotation runs in float64 and every stored element is rounded
// once from it (see round_odd_f32), so q_out and the appended cache rows are
// exactly the float64 definition rounded to the storage type.
//
// Design: a streaming pass, HBM-bound.  One work-group per token (more if its
// units exceed 1024 threads).  One thread owns a "unit" of 16
// elements of one head of one token: for the rotate-half layout the 8
// elements [8j, 8j+8) and their partners [R/2+8j, R/2+8j+8); for the
// proportional layout [8j, 8j+8) and [D/2+8j, D/2+8j+8); for the interleaved
// layout and for pass-through dims, 16 consecutive elements.
// Consecutive threads own consecutive units of a head, so every load and
// K-store is a coalesced 16/32-byte vector access.  The D/16 units of a head
// are consecutive lanes of one wave, so the float8 absmax is a lane-group
// reduction.  V goes to the page's 16-byte runs of 4 consecutive slots:
// whole runs from LDS where a run's 4 slots are all new, single elements
// where a segment's new slots start or end inside one (append_v_quads).

#include <type_traits>

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
  // nearest float32 first (one conversion instruction); where that rounded
  // away from zero, step one unit back toward zero (the truncation), then
  // mark any inexact result by setting the last bit
  const float f = (float)d;
  const double fd = f;
  uint32_t u = __float_as_uint(f);
  if (fd != d) u = (u - (fabs(fd) > fabs(d) ? 1u : 0u)) | 1u;
  return __uint_as_float(u);
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

// Segment of token t with its row range and key count.  In a batch of
// single-token rows (decode steps) token t is segment t: that guess is read
// first, with no lookup before it, and kept when its rows hold t (then it
// is the segment a search would find); otherwise the offsets are searched.
struct Seg { int s, q0, q_end, kv; };
NK_DEVICE Seg segment_of(const RopeArgs &a, int t) {
  const int g = min(t, a.num_seqs - 1);
  const int g0 = a.q_offsets[g], g1 = a.q_offsets[g + 1], gk = a.kv_lens[g];
  if (g0 <= t && t < g1) return Seg{g, g0, g1, gk};
  const int s = find_segment(a.q_offsets, a.num_seqs, t);
  return Seg{s, a.q_offsets[s], a.q_offsets[s + 1], a.kv_lens[s]};
}

// V append, one wave per (group of consecutive tokens, kv head).  A 16-byte
// run of a V page holds 4 consecutive slots (a "quad") of NV dims (v_index):
// one token alone can only fill esz bytes of each run.  The wave therefore
// writes every quad whose first new slot belongs to one of its tokens,
// reading the quad's other new rows itself (they may belong to the next
// group): rows go to LDS in run order, and a full quad leaves as whole
// 16-byte runs; quads cut by the start or end of a segment's new slots are
// written element by element.
template <typename TIn, int CACHE, int D>
NK_DEVICE void append_v_quads(const RopeArgs &a, int t0, int ntok, int head, uint8_t *stage) {
  constexpr int esz = CACHE == kCacheF32 ? 4 : (CACHE == kCacheBF16 ? 2 : 1);
  constexpr int NV = v_nv<CACHE>();
  constexpr int E = D / 16;        // elements of a row per lane, 16 lanes per row
  constexpr int NR = D / NV;       // 16-byte runs per quad and head
  const int P = a.cache.page_size, hkv = a.cache.num_kv_heads;
  const int lane = threadIdx.x & 63, b = lane >> 4, chunk = lane & 15;
  Seg sg = segment_of(a, t0);
  int s = sg.s, q0 = sg.q0, q_end = sg.q_end, kv = sg.kv;
  for (int t = t0; t < t0 + ntok; ++t) {
    if (t >= q_end) {        // next non-empty segment
      sg = segment_of(a, t);
      s = sg.s; q0 = sg.q0; q_end = sg.q_end; kv = sg.kv;
    }
    const int slot = kv - (q_end - q0) + (t - q0);
    // only the first new slot of a quad starts one; slot < 0 violates the
    // precondition and has nowhere to go
    if (slot < 0 || ((slot & 3) != 0 && t != q0)) continue;
    const int a0 = slot & 3, n = min(4 - a0, q_end - t);
    const int page = a.cache.page_table[(size_t)s * a.cache.page_table_stride + slot / P];
    const size_t ph = (size_t)page * hkv + head;

    // row b of the quad (slot slot - a0 + b) is token t + b - a0
    if (b >= a0 && b < a0 + n) {
      const TIn *src = (const TIn *)a.v + ((size_t)(t + b - a0) * hkv + head) * D + chunk * E;
      TIn x[E];
      constexpr int W = (int)(16 / sizeof(TIn)) < E ? (int)(16 / sizeof(TIn)) : E;   // per vector load
      typedef TIn vec_t __attribute__((__vector_size__(W * sizeof(TIn))));
#pragma unroll
      for (int e = 0; e < E; e += W) {
        const vec_t v = *(const vec_t *)(src + e);
#pragma unroll
        for (int k = 0; k < W; ++k) x[e + k] = v[k];
      }
      if (CACHE == kCacheE4M3) {
        double xd[E], m = 0.0;
#pragma unroll
        for (int e = 0; e < E; ++e) { xd[e] = (double)(float)x[e]; m = fmax(m, fabs(xd[e])); }
#pragma unroll
        for (int mask = 1; mask < 16; mask <<= 1) m = fmax(m, __shfl_xor(m, mask, kWave));
        const float scale = (float)(m / 448.0);
        const double sd = scale;
#pragma unroll
        for (int e = 0; e < E; e += 2) {
          const uint32_t c2 = scale > 0.f ? fp8x2(xd[e] / sd, xd[e + 1] / sd) : 0u;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int d = chunk * E + e + h;
            stage[((((d >> 4) / NV) * 16 + (d & 15)) * 4 * NV + ((d >> 4) % NV) * 4 + b) * esz] =
                (uint8_t)(c2 >> (8 * h));
          }
        }
        if (chunk == 0) a.cache.v_scales[ph * P + (slot % P - a0 + b)] = scale;   // slot within the page
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int d = chunk * E + e;
          *(TIn *)(stage + ((((d >> 4) / NV) * 16 + (d & 15)) * 4 * NV + ((d >> 4) % NV) * 4 + b) * esz) = x[e];
        }
      }
    }   // (a row's 16 lanes are all in or all out, so the absmax shuffles stay in active lanes)
    // LDS operations of one wave are performed in order; the barrier keeps
    // the compiler from moving the reads above the writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const int qs = slot - a0;                    // first slot of the quad
    uint8_t *blk = (uint8_t *)a.cache.v_pages + ph * (size_t)P * D * esz;
#pragma unroll
    for (int r = lane; r < NR; r += 64) {
      const int c = r >> 4, r16 = r & 15;
      const size_t off = ((size_t)((qs % P) >> 4) * (D / (16 * NV)) + c) * (64 * 4 * NV) +
                         (size_t)(16 * ((qs & 15) >> 2) + r16) * (4 * NV);
      const u32x4_t run = *(const u32x4_t *)(stage + r * 16);
      if (a0 == 0 && n == 4) {
        *(u32x4_t *)(blk + off * esz) = run;
      } else {
#pragma unroll
        for (int j = 0; j < 4 * NV; ++j) {
          if ((j & 3) < a0 || (j & 3) >= a0 + n) continue;
          const uint8_t *e8 = (const uint8_t *)&run + j * esz;
          if (esz == 4) *(uint32_t *)(blk + (off + j) * esz) = *(const uint32_t *)e8;
          else if (esz == 2) *(uint16_t *)(blk + (off + j) * esz) = *(const uint16_t *)e8;
          else blk[off + j] = *e8;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// LAYOUT: NK_ROPE_HALF, NK_ROPE_INTERLEAVED or NK_ROPE_HALF_PROPORTIONAL;
// MROPE: position streams per section of pairs (a separate instantiation,
// so the one-stream kernel carries none of its lookup)
template <typename TIn, int CACHE, int LAYOUT, bool MROPE>
__global__ void __launch_bounds__(1024) rope_write_kernel(RopeArgs a, int units_per_token, int blocks_per_token,
                                                          int v_blocks, int v_group) {
  extern __shared__ __attribute__((aligned(16))) uint8_t v_stage[];
  const int D = a.cache.head_dim;
  const int hkv = a.cache.num_kv_heads;
  if ((int)blockIdx.x < v_blocks) {
    // V append first (its waves are latency-bound; the streaming Q/K blocks
    // dispatched behind them overlap that latency): one wave per (group of
    // v_group tokens, kv head), 4*D elements of LDS each
    const int item = (int)blockIdx.x * (int)(blockDim.x >> 6) + (int)(threadIdx.x >> 6);
    const int g = item / hkv, head = item - g * hkv;
    const int t0 = g * v_group;
    if (t0 >= a.total_tokens) return;
    const int ntok = min(v_group, a.total_tokens - t0);
    constexpr int esz = CACHE == kCacheF32 ? 4 : (CACHE == kCacheBF16 ? 2 : 1);
    uint8_t *stage = v_stage + (threadIdx.x >> 6) * (size_t)(4 * D * esz);
    if (D == 64) append_v_quads<TIn, CACHE, 64>(a, t0, ntok, head, stage);
    else if (D == 128) append_v_quads<TIn, CACHE, 128>(a, t0, ntok, head, stage);
    else append_v_quads<TIn, CACHE, 256>(a, t0, ntok, head, stage);
    return;
  }
  const unsigned qb = blockIdx.x - (unsigned)v_blocks;
  const int R = a.rotary_dim;
  const int P = a.cache.page_size;
  const int units_per_head = D >> 4;
  // Q and K: one token per work-group (blocks_per_token of them when its
  // units do not fit one), so the token and its segment are wave-uniform
  const int t = (int)(qb / (unsigned)blocks_per_token);
  const int lu = (int)(qb - (unsigned)t * blocks_per_token) * blockDim.x + threadIdx.x;
  if (lu >= units_per_token) return;
  const int hh = lu / units_per_head;
  const int j = lu - hh * units_per_head;

  const int kind = hh < a.hq ? 0 : 1;   // q, k
  const int head = kind == 0 ? hh : hh - a.hq;
  const int hn = kind == 0 ? a.hq : hkv;
  const TIn *src = (const TIn *)(kind == 0 ? a.q : a.k) + ((size_t)t * hn + head) * D;

  // run A / run B of this unit and whether it rotates
  constexpr bool INTERLEAVED = LAYOUT == NK_ROPE_INTERLEAVED;
  const bool rotates = INTERLEAVED ? 16 * j < R : j < (R >> 4);
  int a0, b0;
  if (INTERLEAVED) {
    a0 = 16 * j; b0 = a0 + 8;
  } else if (LAYOUT == NK_ROPE_HALF_PROPORTIONAL) {
    // pairs span the whole head: unit j holds dims 8j.. and D/2 + 8j..,
    // rotated when its pairs are among the first R/2
    a0 = 8 * j; b0 = (D >> 1) + 8 * j;
  } else if (rotates) {
    a0 = 8 * j; b0 = (R >> 1) + 8 * j;
  } else {
    a0 = R + 16 * (j - (R >> 4)); b0 = a0 + 8;
  }
  double xa[8], xb[8];
  InTraits<TIn>::load8(src + a0, xa);
  InTraits<TIn>::load8(src + b0, xb);

  const Seg sg = segment_of(a, t);
  const int s = sg.s, q0 = sg.q0;
  const int slot = sg.kv - (sg.q_end - q0) + (t - q0);

  if (rotates) {
    // out-of-range positions (a precondition violation) are clamped so that
    // the table read stays inside the table
    int p = slot;
    if (MROPE) {
      // the unit's 8 pairs (8j..8j+7) lie in one section (sections are
      // multiples of 8 pairs); that section's position stream
      int sec = 0;
      while (sec + 1 < a.mrope_sections && 8 * j >= a.mrope_end[sec]) ++sec;
      p = a.position_ids[(size_t)sec * a.total_tokens + t];
    } else if (a.position_ids) {
      p = a.position_ids[t];
    }
    const int pos = min(max(p, 0), a.max_pos - 1);
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
    if (j == 0) a.cache.k_scales[ph * P + off] = scale;
  }

  // K page: blocks of 32*NK dims, see k_index
  constexpr int esz = CACHE == kCacheF32 ? 4 : (CACHE == kCacheBF16 ? 2 : 1);
  uint8_t *kph = (uint8_t *)a.cache.k_pages + ph * P * (size_t)D * esz;
  store_k8<CACHE>(kph + k_index<CACHE>(a0, off, P) * esz, 0, xa);
  store_k8<CACHE>(kph + k_index<CACHE>(b0, off, P) * esz, 0, xb);
}

template <typename TIn, int CACHE>
hipError_t launch_layout(const RopeArgs &a, hipStream_t stream) {
  constexpr int esz = CACHE == kCacheF32 ? 4 : (CACHE == kCacheBF16 ? 2 : 1);
  const int hkv = a.cache.num_kv_heads, D = a.cache.head_dim;
  const int upt = (a.hq + hkv) * (D / 16);          // Q and K units of a token
  const int bpt = (upt + 1023) / 1024;
  const int block = ((upt + bpt - 1) / bpt + 63) / 64 * 64;
  const long long qk_blocks = (long long)a.total_tokens * bpt;
  // V groups: 4 tokens per wave when segments are long enough for whole
  // quads to be common, else one (decode steps: every token its own quad)
  const int v_group = a.total_tokens >= 4 * a.num_seqs ? 4 : 1;
  const long long v_items = (long long)((a.total_tokens + v_group - 1) / v_group) * hkv;
  const long long v_blocks = (v_items + block / 64 - 1) / (block / 64);
  if (qk_blocks + v_blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const unsigned grid = (unsigned)(qk_blocks + v_blocks);
  const size_t lds = (size_t)(block / 64) * 4 * D * esz;
  auto pick = [&](auto mrope) {
    constexpr bool M = decltype(mrope)::value;
    return a.layout == NK_ROPE_INTERLEAVED ? rope_write_kernel<TIn, CACHE, NK_ROPE_INTERLEAVED, M>
           : a.layout == NK_ROPE_HALF_PROPORTIONAL ? rope_write_kernel<TIn, CACHE, NK_ROPE_HALF_PROPORTIONAL, M>
                                                  : rope_write_kernel<TIn, CACHE, NK_ROPE_HALF, M>;
  };
  auto k = a.mrope_sections > 0 ? pick(std::true_type{}) : pick(std::false_type{});
  return launch(k, dim3(grid), dim3(block), lds, stream, a, upt, bpt, (int)v_blocks, v_group);
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

// ------------------------------------------------------------------ packing
// NumKong matrix-kernels page, "Attention with a Pre-Packed KV-Cache" and
// attention_pack.  Segment s's input slot is rows key_offsets[s] ..
// key_offsets[s+1]-1, of which the first kept_s enter the pack (kept_s =
// key_lengths[s], or the slot's size without lengths).  The pack here is
// this library's paged cache: segment s
// takes the next ceil(kept/P) pages after those of segments 0..s-1, its
// table row lists them, and kv_lens_out[s] = kept.  The keys are stored as
// they come (no rotation), rounded once to the cache type; e4m3 rows take
// one scale per (token, kv head), absmax / 448, as the append step does.
namespace {

// kept keys of segment s: key_lengths[s] clamped to [0, slot] and to the
// stated maximum (a larger value violates the precondition; clamping keeps
// every access inside the table row and the grid)
NK_DEVICE int pack_len(const PackArgs &a, int s) {
  const int slot = a.key_offsets[s + 1] - a.key_offsets[s];
  const int n = a.key_lengths ? a.key_lengths[s] : slot;
  return max(0, min(min(n, slot), a.max_key_len));
}

constexpr int kPackPlanThreads = 1024;

// One work-group: kept lengths, then an exclusive scan of the page counts in
// blocks of kPackPlanThreads segments, then the table rows.  Page ids are
// clamped to the cache (a cache smaller than the pack violates the
// precondition; nothing is then read or written out of bounds).
__global__ void __launch_bounds__(kPackPlanThreads) pack_plan_kernel(PackArgs a) {
  __shared__ int part[kPackPlanThreads / 64];
  __shared__ int first[kPackPlanThreads], count[kPackPlanThreads];
  __shared__ int carry;
  const int P = a.cache.page_size;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int s0 = 0; s0 < a.num_seqs; s0 += kPackPlanThreads) {
    const int s = s0 + tid;
    const int len = s < a.num_seqs ? pack_len(a, s) : 0;
    const int np = (len + P - 1) / P;
    int x = np;                                   // inclusive scan within the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d, kWave);
      if (lane >= d) x += y;
    }
    if (lane == 63) part[w] = x;
    __syncthreads();
    int before = carry;
    for (int i = 0; i < w; ++i) before += part[i];
    first[tid] = before + x - np;
    count[tid] = np;
    if (s < a.num_seqs) a.kv_lens_out[s] = len;
    __syncthreads();                              // every read of carry and part is done
    if (tid == kPackPlanThreads - 1) carry = first[tid] + np;
    const int nseg = min(kPackPlanThreads, a.num_seqs - s0);
    for (int k = 0; k < nseg; ++k) {
      int32_t *row = const_cast<int32_t *>(a.cache.page_table) + (size_t)(s0 + k) * a.cache.page_table_stride;
      for (int i = tid; i < count[k]; i += kPackPlanThreads) row[i] = min(first[k] + i, a.cache.num_pages - 1);
    }
    __syncthreads();
  }
}

template <int CACHE> NK_DEVICE void store_v1(uint8_t *p, double x);
template <> NK_DEVICE void store_v1<kCacheF32>(uint8_t *p, double x) { *(float *)p = (float)x; }
template <> NK_DEVICE void store_v1<kCacheBF16>(uint8_t *p, double x) { *(bf16_t *)p = (bf16_t)round_odd_f32(x); }
template <> NK_DEVICE void store_v1<kCacheE4M3>(uint8_t *p, double x) { *p = (uint8_t)(fp8x2(x, 0.0) & 0xffu); }

// One work-group per (segment, page of its pack, kv head): every 8-dim unit
// of the page's kept tokens, K and V (V through LDS, stored as whole runs).  A token's D/8 units are consecutive
// lanes (D/8 divides 64), so the e4m3 absmax is a lane-group reduction.
template <typename TIn, int CACHE>
__global__ void __launch_bounds__(256) pack_kernel(PackArgs a, int pages_per_seq) {
  constexpr int esz = CACHE == kCacheF32 ? 4 : (CACHE == kCacheBF16 ? 2 : 1);
  const int s = blockIdx.x / pages_per_seq, i = blockIdx.x % pages_per_seq, g = blockIdx.y;
  const int P = a.cache.page_size, D = a.cache.head_dim, hkv = a.cache.num_kv_heads;
  const int len = pack_len(a, s);
  if (i * P >= len) return;
  const int page = a.cache.page_table[(size_t)s * a.cache.page_table_stride + i];
  const size_t ph = (size_t)page * hkv + g;
  uint8_t *kph = (uint8_t *)a.cache.k_pages + ph * P * (size_t)D * esz;
  uint8_t *vph = (uint8_t *)a.cache.v_pages + ph * P * (size_t)D * esz;
  // V is assembled in LDS in its page-block order, then leaves as 16-byte runs
  __shared__ __attribute__((aligned(16))) uint8_t vtile[32 * 256 * esz];
  const int upt = D / 8;
  const int row0 = a.key_offsets[s] + i * P;
  for (int u0 = 0; u0 < P * upt; u0 += 256) {          // uniform trip count: shuffles see every lane
    const int u = u0 + (int)threadIdx.x;
    const int t = u / upt, c = u % upt;
    const bool valid = u < P * upt && i * P + t < len;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      double x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (valid) {
        const TIn *src = (const TIn *)(kv == 0 ? a.k : a.v) + ((size_t)(row0 + t) * hkv + g) * D + 8 * c;
        InTraits<TIn>::load8(src, x);
      }
      if (CACHE == kCacheE4M3) {
        double m = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmax(m, fabs(x[e]));
        for (int mask = 1; mask < upt; mask <<= 1) m = fmax(m, __shfl_xor(m, mask, kWave));
        const float scale = (float)(m / 448.0);          // float32 nearest to absmax / 448
        const double sd = scale;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = scale > 0.f ? x[e] / sd : 0.0;
        if (valid && c == 0) (kv == 0 ? a.cache.k_scales : a.cache.v_scales)[ph * P + t] = scale;
      }
      if (!valid) continue;
      if (kv == 0) {
        store_k8<CACHE>(kph + k_index<CACHE>(8 * c, t, P) * esz, 0, x);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) store_v1<CACHE>(vtile + v_index<CACHE>(8 * c + e, t, D) * esz, x[e]);
      }
    }
  }
  __syncthreads();
  // a run holds 4 consecutive slots (t0 .. t0+3) of 4*NV elements: whole
  // runs of kept slots leave as one store; a run cut by the segment's last
  // kept key (the last page only) is written element by element
  constexpr int NV = v_nv<CACHE>();
  const int kept = min(P, len - i * P);
  const int runs = P * D / (4 * NV);
  for (int r = (int)threadIdx.x; r < runs; r += 256) {
    const int t0 = 16 * ((r / 64) / (D / (16 * NV))) + 4 * ((r % 64) / 16);
    if (t0 >= kept) continue;
    if (t0 + 3 < kept) {
      *(u32x4_t *)(vph + (size_t)r * 16) = *(const u32x4_t *)(vtile + r * 16);
    } else {
      for (int k = 0; k < 4 * NV; ++k)
        if (t0 + (k & 3) < kept)
          for (int b = 0; b < esz; ++b) vph[(size_t)r * 16 + k * esz + b] = vtile[r * 16 + k * esz + b];
    }
  }
}

template <typename TIn, int CACHE>
hipError_t launch_pack(const PackArgs &a, hipStream_t stream) {
  hipError_t e = launch(pack_plan_kernel, dim3(1), dim3(kPackPlanThreads), 0, stream, a);
  if (e != hipSuccess || a.max_key_len == 0) return e;
  const int pages_per_seq = (a.max_key_len + a.cache.page_size - 1) / a.cache.page_size;
  const long long blocks = (long long)a.num_seqs * pages_per_seq;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  return launch(pack_kernel<TIn, CACHE>, dim3((unsigned)blocks, (unsigned)a.cache.num_kv_heads), dim3(256), 0,
                stream, a, pages_per_seq);
}

}  // namespace

hipError_t launch_attention_pack(const PackArgs &a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  ProfileScope prof("attention_pack", stream);
  if (a.in_dtype == NK_F32 && a.cache.dtype == NK_F32) return launch_pack<float, kCacheF32>(a, stream);
  if (a.in_dtype == NK_BF16 && a.cache.dtype == NK_BF16) return launch_pack<bf16_t, kCacheBF16>(a, stream);
  if (a.in_dtype == NK_BF16 && a.cache.dtype == NK_E4M3) return launch_pack<bf16_t, kCacheE4M3>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace nk
