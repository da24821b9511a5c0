// Split-KV decode attention: single-query rows over a paged bf16 or e4m3
// cache, the query heads of one KV head sharing every K/V load.
//
// What it computes: NumKong matrix-kernels page, attention_packed, for a
// segment with one query row (it sits at position kv_len - 1 and sees every
// key, or the last window_left + 1 keys); aria_kernel `attention` (single
// query step against the KV cache, GQA layout).  The keys are cut into
// chunks whose states are merged by log-sum-exp as on the Algenta page's
// flash-attention walkthrough (running max, rescale by exp(old - new)).
// e4m3 caches: a stored code times its per-(token, head) scale is the value;
// the K scale multiplies the score, the V scale the probability.
//
// Design (HBM-bound):
//   * one wave per work item (sequence, KV head, chunk of keys, block of 16
//     query heads): no LDS, no barriers; chunks are sized so that a batch
//     yields a few thousand waves and the whole grid is resident at once;
//   * the chunk is walked 16 keys at a time (one 16-token page, or half a
//     32-token page), so every load instruction reads one page: a wave-uniform
//     page base plus a per-lane offset;
//   * scores S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (16 keys x 16 query
//     heads, unused head columns zero) and O^T += V^T P^T on
//     v_mfma_f32_16x16x16_bf16: the score tile's lane layout (lane holds keys
//     4*(lane/16)..+3 of head lane%16) is exactly the P^T operand's, so the
//     probabilities never move between lanes;
//   * K pages are stored in 32-dim blocks ([dim/32][token][32]) and V pages
//     dimension-major ([dim][token]): each MFMA operand load of a wave is one
//     contiguous 1 KiB (bf16) / 512 B (e4m3) block of K or 512 B / 256 B of
//     V, read straight from HBM into registers; e4m3 codes widen to bf16
//     exactly in registers;
//   * a ring of NPF pages is in flight per wave: page i+NPF is requested
//     before page i is consumed;
//   * the row's final output (one chunk) or a float32 partial (several
//     chunks) is written straight from the accumulator lanes.

#include "common.h"
#include "internal.h"

// Pages in flight per wave and the waves-per-SIMD the register allocation
// aims for (compile-time; chosen by measurement on MI355X).
#ifndef NK_DECODE_NPF_BF16
#define NK_DECODE_NPF_BF16 3
#endif
#ifndef NK_DECODE_NPF_FP8
#define NK_DECODE_NPF_FP8 6
#endif
#ifndef NK_DECODE_WAVES_PER_EU
#define NK_DECODE_WAVES_PER_EU 2
#endif
// K/V pages are read once per call: non-temporal loads keep them from
// displacing other lines in the caches (measured: +8% for bf16 pages, a
// small loss for e4m3 pages)
#ifndef NK_DECODE_NT_BF16
#define NK_DECODE_NT_BF16 1
#endif
#ifndef NK_DECODE_NT_FP8
#define NK_DECODE_NT_FP8 0
#endif

namespace nk {
namespace {

template <int D, bool FP8>
struct Page {
  static constexpr int KK = D / 32;   // k-steps of the score MFMA
  static constexpr int DT = D / 16;   // d-tiles of the output MFMA
  using KVec = typename std::conditional<FP8, u32x2_t, bf16x8_t>::type;   // 8 dims of one key
  using VVec = typename std::conditional<FP8, uint32_t, bf16x4_t>::type;  // 4 keys of one dim
  KVec k[KK];
  VVec v[DT];
  f32x4_t ks, vs;                     // e4m3: scales of this lane's 4 keys
};

template <bool NT, typename T>
NK_DEVICE T stream_load(const T *p) {
  if constexpr (NT) {
    if constexpr (sizeof(T) == 16) return __builtin_bit_cast(T, __builtin_nontemporal_load((const u32x4_t *)p));
    else if constexpr (sizeof(T) == 8) return __builtin_bit_cast(T, __builtin_nontemporal_load((const u32x2_t *)p));
    else return __builtin_bit_cast(T, __builtin_nontemporal_load((const uint32_t *)p));
  } else {
    return *p;
  }
}

// Per-lane byte offsets inside one page, fixed for the whole kernel.
struct LaneOffsets {
  uint32_t k, v, sc;
};

template <int D, int P, bool FP8>
NK_DEVICE LaneOffsets lane_offsets(int lane) {
  constexpr int esz = FP8 ? 1 : 2;
  const int lr = lane & 15, lg = lane >> 4;
  return LaneOffsets{(uint32_t)((lr * 32 + 8 * lg) * esz),    // K: key lr, dims 8*lg.. of a block
                     (uint32_t)((lr * P + 4 * lg) * esz),     // V: dim lr, keys 4*lg..
                     (uint32_t)(4 * lg * sizeof(float))};     // scales of keys 4*lg..
}

// Load one 16-key step: the page's base pointer is wave-uniform (scalar
// registers), each lane adds its fixed offset.
template <int D, int P, bool FP8>
NK_DEVICE void load_page(Page<D, FP8> &pg, const nk_paged_kv_t &c, int page, int sb, int g,
                         const LaneOffsets &lo) {
  using PG = Page<D, FP8>;
  constexpr int esz = FP8 ? 1 : 2;
  const int hkv = c.num_kv_heads;
  const size_t ph = (size_t)page * hkv + g;
  // K page-head: [dim/32][slot][32]; block kk of the 16 keys is contiguous
  const uint8_t *kpage = (const uint8_t *)c.k_pages + (ph * P * D + sb * 32) * esz;
  const uint8_t *vpage = (const uint8_t *)c.v_pages + (ph * D * P + sb) * esz;
#pragma unroll
  for (int kk = 0; kk < PG::KK; ++kk)
    pg.k[kk] = stream_load<FP8 ? NK_DECODE_NT_FP8 : NK_DECODE_NT_BF16>((const typename PG::KVec *)(kpage + lo.k + kk * P * 32 * esz));
#pragma unroll
  for (int dt = 0; dt < PG::DT; ++dt)
    pg.v[dt] = stream_load<FP8 ? NK_DECODE_NT_FP8 : NK_DECODE_NT_BF16>((const typename PG::VVec *)(vpage + lo.v + 16 * dt * P * esz));
  if constexpr (FP8) {
    const uint8_t *sk = (const uint8_t *)(c.k_scales + ph * P + sb);
    const uint8_t *sv = (const uint8_t *)(c.v_scales + ph * P + sb);
    pg.ks = stream_load<NK_DECODE_NT_FP8>((const f32x4_t *)(sk + lo.sc));
    pg.vs = stream_load<NK_DECODE_NT_FP8>((const f32x4_t *)(sv + lo.sc));
  }
}

NK_DEVICE bf16x4_t fp8x4_to_bf16x4(uint32_t w) {
  bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return bf16x4_t{a[0], a[1], b[0], b[1]};
}

template <int D, int P, bool FP8, int NPF, int CH>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(NK_DECODE_WAVES_PER_EU)))
attn_decode_kernel(AttnArgs a) {
  using PG = Page<D, FP8>;
  constexpr int KK = PG::KK, DT = PG::DT;
  constexpr int SUB = P / 16;                 // 16-key steps per page

  // linear work index, KV head fastest: the KV heads of one chunk are
  // dispatched together, so a page's heads (contiguous in memory) are
  // fetched at the same time
  const int B = a.num_seqs;
  const int hkv_ = a.cache.num_kv_heads;
  const int g = blockIdx.x % hkv_;
  const int sc = blockIdx.x / hkv_;
  const int s = sc % B;
  const int c = sc / B;
  const int hb = blockIdx.y;                  // block of 16 query heads
  const int lane = threadIdx.x;
  const int hkv = a.cache.num_kv_heads;
  const int G = a.hq / hkv;

  const int q0 = a.q_offsets[s];
  if (a.q_offsets[s + 1] - q0 != 1) return;
  const int L = a.kv_lens[s];
  const int hi = L - 1;
  const int lo = a.window_left < 0 ? 0 : max(0, hi - a.window_left);
  const int c0 = (lo / 32) * 32;              // chunks are aligned to 32 keys
  // (clamped to the grid: a kv_len above max_kv_len violates the
  // precondition, and its row then covers only the first max_chunks chunks)
  const int n_chunks = L > 0 ? min((hi + 1 - c0 + a.split_tokens - 1) / a.split_tokens, a.max_chunks) : 1;
  if (c >= n_chunks) return;
  const int cs = c0 + c * a.split_tokens;
  const int ce = min(cs + a.split_tokens, hi + 1);
  const int vlo = max(cs, lo);                // valid keys [vlo, ce)
  const int nsteps = L > 0 ? (ce - cs + 15) / 16 : 0;
  const int32_t *pt = a.cache.page_table + (size_t)s * a.cache.page_table_stride;
  const LaneOffsets loff = lane_offsets<D, P, FP8>(lane);

  const int n = lane & 15;
  const int lg = lane >> 4;
  const int hq_local = hb * 16 + n;
  const bool col_valid = hq_local < G;
  // Q operand (B of the score product); a column past the group's heads
  // computes a copy of the group's first head and is never written
  bf16x8_t qop[KK];
  {
    const bf16_t *qrow = (const bf16_t *)a.q + ((size_t)q0 * a.hq + g * G + (col_valid ? hq_local : hb * 16)) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qop[kk] = *(const bf16x8_t *)(qrow + 32 * kk + 8 * lg);
  }

  const float qk_scale = a.softmax_scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // step i covers keys cs + 16 i .. +15: page (cs + 16 i) / P, sub-block
  auto issue = [&](PG &pg, int i) {
    const int key0 = cs + 16 * min(i, nsteps - 1);   // past the end: reload the last page (cache hit)
    const int page = pt[key0 / P];
    load_page<D, P, FP8>(pg, a.cache, page, SUB == 1 ? 0 : (key0 % P), g, loff);
  };

  auto consume = [&](const PG &pg, int i) {
    const int kb = cs + 16 * i;
    f32x4_t sacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      bf16x8_t kop;
      if constexpr (FP8) kop = fp8x8_to_bf16x8(pg.k[kk]); else kop = pg.k[kk];
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[kk], sacc, 0, 0, 0);
    }
    // lane holds keys kb + 4*lg + r of head column n
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = FP8 ? sacc[r] * qk_scale * pg.ks[r] : sacc[r] * qk_scale;
    const bool edge = kb < vlo || kb + 16 > ce;
    if (edge) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb + 4 * lg + r;
        if (key < vlo || key >= ce) x[r] = -INFINITY;
      }
    }
    float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    tmax = fmaxf(tmax, shfl_xor_f32(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor_f32(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    if (__any(m_new > m_run)) {
      const float corr = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
      l_run *= corr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= corr;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = fast_exp2(x[r] - m_use);
      l_run += p[r];
    }
    if constexpr (FP8) {
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] *= pg.vs[r];
    }
    bf16x4_t pop;
#pragma unroll
    for (int r = 0; r < 4; ++r) pop[r] = (bf16_t)p[r];
    if (edge) {
      // masked keys may hold anything (unwritten slots, NaN scales): zero them
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb + 4 * lg + r;
        if (key < vlo || key >= ce) pop[r] = (bf16_t)0.f;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        bf16x4_t vv;
        if constexpr (FP8) vv = fp8x4_to_bf16x4(pg.v[dt]); else vv = pg.v[dt];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kb + 4 * lg + r < vlo || kb + 4 * lg + r >= ce) vv[r] = (bf16_t)0.f;
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vv, pop, o[dt], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        bf16x4_t vv;
        if constexpr (FP8) vv = fp8x4_to_bf16x4(pg.v[dt]); else vv = pg.v[dt];
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vv, pop, o[dt], 0, 0, 0);
      }
    }
  };

  // Software pipeline, NPF pages in flight, fully unrolled over a sub-chunk
  // of CH steps (no loop back-edge inside the pipeline: the compiler's wait
  // counts stay exact, each consume waits only for its own page).  A chunk
  // is one or more sub-chunks; steps past the chunk's end are skipped (their
  // loads re-read the last page, a cache hit).
  for (int sub = 0; sub * CH < nsteps; ++sub) {
    const int base = sub * CH;
    PG ring[NPF];
#pragma unroll
    for (int j = 0; j < NPF; ++j) issue(ring[j], base + j);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (base + j < nsteps) consume(ring[j % NPF], base + j);
      if (j + NPF < CH) issue(ring[j % NPF], base + j + NPF);
    }
  }

  // per-column sum over the four lane groups
  l_run += shfl_xor_f32(l_run, 16);
  l_run += shfl_xor_f32(l_run, 32);

  if (!col_valid) return;
  const int head = g * G + hq_local;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  const float lse = l_run > 0.f ? (m_run + fast_log2(l_run)) * kLn2 : -INFINITY;
  if (n_chunks == 1) {
    bf16_t *orow = (bf16_t *)a.out + ((size_t)q0 * a.hq + head) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      bf16x4_t v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (bf16_t)(o[dt][r] * inv);
      *(bf16x4_t *)(orow + 16 * dt + 4 * lg) = v;
    }
    if (a.lse && lg == 0) a.lse[(size_t)q0 * a.hq + head] = lse;
  } else {
    const size_t slot = (size_t)s * a.max_chunks + c;
    float *prow = a.part_out + (slot * a.hq + head) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *(f32x4_t *)(prow + 16 * dt + 4 * lg) = o[dt] * inv;
    if (lg == 0) a.part_lse[slot * a.hq + head] = lse;
  }
}

template <int D, int P, bool FP8>
hipError_t launch_cfg(const AttnArgs &a, hipStream_t stream) {
  constexpr int NPF = FP8 ? NK_DECODE_NPF_FP8 : (D == 256 ? 2 : NK_DECODE_NPF_BF16);
  const int hkv = a.cache.num_kv_heads;
  const int G = a.hq / hkv;
  dim3 grid((unsigned)(a.num_seqs * a.max_chunks * hkv), (unsigned)((G + 15) / 16), 1);
  // sub-chunks of 32 steps (512 keys) when the chunk size allows, else 16
  if (a.split_tokens % 512 == 0)
    attn_decode_kernel<D, P, FP8, NPF, 32><<<grid, 64, 0, stream>>>(a);
  else
    attn_decode_kernel<D, P, FP8, NPF, 16><<<grid, 64, 0, stream>>>(a);
  return hipGetLastError();
}

template <int D, int P>
hipError_t launch_dp(const AttnArgs &a, hipStream_t stream) {
  if (a.cache.dtype == NK_E4M3) return launch_cfg<D, P, true>(a, stream);
  return launch_cfg<D, P, false>(a, stream);
}

}  // namespace

hipError_t launch_attn_decode(const AttnArgs &a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  ProfileScope prof("attn_decode", stream);
  const int D = a.cache.head_dim, P = a.cache.page_size;
  if (D == 64 && P == 16) return launch_dp<64, 16>(a, stream);
  if (D == 64 && P == 32) return launch_dp<64, 32>(a, stream);
  if (D == 128 && P == 16) return launch_dp<128, 16>(a, stream);
  if (D == 128 && P == 32) return launch_dp<128, 32>(a, stream);
  if (D == 256 && P == 16) return launch_dp<256, 16>(a, stream);
  if (D == 256 && P == 32) return launch_dp<256, 32>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace nk
