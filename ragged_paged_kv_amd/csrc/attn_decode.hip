// Split-KV decode attention: single-query rows over a paged bf16 or e4m3
// cache, the query heads of one KV head sharing every K/V load.
//
// What it computes: NumKong matrix-kernels page, attention_packed, for a
// segment with one query row (it sits at position kv_len - 1 and sees every
// key, or the last window_left + 1 keys, plus the first sink_keys keys beside a
// window: Algenta, "Ten named techniques, one scalar formula each",
// StreamingLLM sinks); aria_kernel `attention` (single
// query step against the KV cache, GQA layout).  The sink keys left of the
// window form one chunk of their own.  The keys are cut into
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
//   * K pages are stored in blocks of 32 dims (64 for e4m3, the two 32-dim
//     halves interleaved in 8-element runs) and V pages as 16-byte runs in
//     the lane order of the V^T operand (include/nk.h): every load
//     instruction of a wave reads one contiguous 1 KiB with 16 bytes per
//     lane, which hold 1 (bf16) or 2 (e4m3) K operands or 2 (bf16) or 4
//     (e4m3) V operands, straight from HBM into registers with non-temporal
//     loads; e4m3 codes widen to bf16 exactly in registers;
//   * a ring of NPF pages is in flight per wave: page i+NPF is requested
//     before page i is consumed;
//   * the row's final output (one chunk) or a float32 partial (several
//     chunks) is written straight from the accumulator lanes.

#include "common.h"
#include "internal.h"

// Pages in flight per wave and the waves-per-SIMD the register allocation
// aims for (compile-time; chosen by measurement on MI355X).  More bf16 pages
// in flight only lengthen the memory queues: 2 waves x 2 pages per SIMD read
// the batched-decode pages 3-4 % faster than 2 x 4 or 1 x 8.
#ifndef NK_DECODE_NPF_BF16
#define NK_DECODE_NPF_BF16 2
#endif
#ifndef NK_DECODE_NPF_FP8
#define NK_DECODE_NPF_FP8 6
#endif
#ifndef NK_DECODE_NPF_D256        // head_dim 256: a second page in flight spills
#define NK_DECODE_NPF_D256 1
#endif
#ifndef NK_DECODE_WAVES_PER_EU
#define NK_DECODE_WAVES_PER_EU 2
#endif
// 16-key steps that share one softmax update (1 or 2)
#ifndef NK_DECODE_STEPS_PER_UPDATE
#define NK_DECODE_STEPS_PER_UPDATE 2
#endif
// K/V pages are read once per call: non-temporal loads keep them from
// displacing other lines in the caches (measured: +8% for bf16 pages, +5%
// for e4m3 pages with their 16-byte runs, and the split-KV partials then
// stay cached for the merge)
#ifndef NK_DECODE_NT_BF16
#define NK_DECODE_NT_BF16 1
#endif
#ifndef NK_DECODE_NT_FP8
#define NK_DECODE_NT_FP8 1
#endif

// e4m3 scales: 1 = the 16 lanes of a row each load the scales of a
// different 16-key step (one load instruction covers 16 steps) and a step's
// scales reach the lanes that use them by a DPP row broadcast; 0 = every
// step loads its own (two load instructions of 64 bytes each per step)
#ifndef NK_DECODE_SCALE_BCAST
#define NK_DECODE_SCALE_BCAST 1
#endif

// Grid order of the chunks (slowest index), bf16 caches: 1 = last chunk
// first, so that the work-groups of chunks most rows do not have come first
// and exit at once, and the long rows' last chunks do not wait behind them
// for a slot (batched decode 52.6 -> 51.9 us; the e4m3 long-context batch,
// many grids' worth of work-groups, ran 0.3 % slower that way, and calls
// with sink keys, whose sink chunk is the last index, 3.7 %)
#ifndef NK_DECODE_CHUNKS_REVERSED
#define NK_DECODE_CHUNKS_REVERSED 1
#endif

namespace nk {
namespace {

template <int D, bool FP8>
struct Page {
  static constexpr int KK = D / 32;   // k-steps of the score MFMA
  static constexpr int DT = D / 16;   // d-tiles of the output MFMA
  static constexpr int NV = FP8 ? 4 : 2;   // d-tiles per 16-byte V run
  static constexpr int NK = FP8 ? 2 : 1;   // k-steps per 16-byte K run
  u32x4_t k[KK / NK];                 // K runs: 8 dims of this lane's key for NK k-steps each
  u32x4_t v[DT / NV];                 // V runs: this lane's 4 keys of NV d-tiles each
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
  constexpr int NK = FP8 ? 2 : 1;
  return LaneOffsets{(uint32_t)((lr * 32 * NK + 8 * NK * lg) * esz),   // K: key lr, run lg of a block
                     (uint32_t)(16 * lane),                   // V: run `lane` of a dim group
                     (uint32_t)(4 * lg * sizeof(float))};     // scales of keys 4*lg..
}

NK_DEVICE bf16x4_t fp8x4_to_bf16x4(uint32_t w);

// Operand of k-step kk (K, lane lr + 16 lg: key lr, dims 32 kk + 8 lg..)
template <int D, bool FP8>
NK_DEVICE bf16x8_t k_operand(const Page<D, FP8> &pg, int kk) {
  if constexpr (FP8) {
    const u32x4_t r = pg.k[kk >> 1];
    return fp8x8_to_bf16x8(u32x2_t{r[2 * (kk & 1)], r[2 * (kk & 1) + 1]});
  } else {
    return __builtin_bit_cast(bf16x8_t, pg.k[kk]);
  }
}

// Operand of d-tile dt (V^T, lane lr + 16 lg: dim 16 dt + lr, keys 4 lg..)
template <int D, bool FP8>
NK_DEVICE bf16x4_t v_operand(const Page<D, FP8> &pg, int dt) {
  if constexpr (FP8) {
    return fp8x4_to_bf16x4(pg.v[dt >> 2][dt & 3]);
  } else {
    const u32x4_t r = pg.v[dt >> 1];
    return __builtin_bit_cast(bf16x4_t, u32x2_t{r[2 * (dt & 1)], r[2 * (dt & 1) + 1]});
  }
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
  // K page-head: [dim/(32 NK)][slot][32 NK]; block r of the 16 keys is contiguous
  const uint8_t *kpage = (const uint8_t *)c.k_pages + (ph * P * D + sb * 32 * PG::NK) * esz;
  // V page-head: 16-key blocks of 16-byte runs in MFMA operand order, one
  // run per lane and dim group
  const uint8_t *vpage = (const uint8_t *)c.v_pages + (ph * D * P + sb * D) * esz;
#pragma unroll
  for (int r = 0; r < PG::KK / PG::NK; ++r)
    pg.k[r] = stream_load<FP8 ? NK_DECODE_NT_FP8 : NK_DECODE_NT_BF16>((const u32x4_t *)(kpage + lo.k + r * P * 32 * PG::NK * esz));
#pragma unroll
  for (int r = 0; r < PG::DT / PG::NV; ++r)
    pg.v[r] = stream_load<FP8 ? NK_DECODE_NT_FP8 : NK_DECODE_NT_BF16>((const u32x4_t *)(vpage + lo.v + 1024 * r));
  if constexpr (FP8 && !NK_DECODE_SCALE_BCAST) {
    const uint8_t *sk = (const uint8_t *)(c.k_scales + ph * P + sb);
    const uint8_t *sv = (const uint8_t *)(c.v_scales + ph * P + sb);
    // the scales of a page's heads share cache lines read by the waves of
    // the other heads: ordinary loads let those reads hit (measured +2 %)
    pg.ks = stream_load<false>((const f32x4_t *)(sk + lo.sc));
    pg.vs = stream_load<false>((const f32x4_t *)(sv + lo.sc));
  }
}

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32,
// l^48), on the VALU: v_permlane16_swap / v_permlane32_swap exchange rows of
// a register pair, so one of the two outputs holds the partner row's value
// whichever row the lane is in.
NK_DEVICE float rows_max(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
  u = __builtin_bit_cast(uint32_t, v);
  r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

NK_DEVICE float rows_sum(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
  u = __builtin_bit_cast(uint32_t, v);
  r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Lane n of each 16-lane row, broadcast to its row (DPP row_newbcast).
// With every row and bank enabled each lane takes the broadcast value and
// `dep` is never selected; it only ties the move to the step whose value it
// is (otherwise the compiler hoists every step's broadcasts to the start of
// the unrolled sub-chunk and keeps them all live).
template <int N>
NK_DEVICE float row_bcast(float v, float dep) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, dep), __builtin_bit_cast(int, v),
                                                               0x150 + N, 0xf, 0xf, false));
}
// the same for an index that is a constant once the caller is unrolled
NK_DEVICE float row_bcast_n(float v, int n, float dep) {
  switch (n & 15) {
    case 0: return row_bcast<0>(v, dep);   case 1: return row_bcast<1>(v, dep);
    case 2: return row_bcast<2>(v, dep);   case 3: return row_bcast<3>(v, dep);
    case 4: return row_bcast<4>(v, dep);   case 5: return row_bcast<5>(v, dep);
    case 6: return row_bcast<6>(v, dep);   case 7: return row_bcast<7>(v, dep);
    case 8: return row_bcast<8>(v, dep);   case 9: return row_bcast<9>(v, dep);
    case 10: return row_bcast<10>(v, dep); case 11: return row_bcast<11>(v, dep);
    case 12: return row_bcast<12>(v, dep); case 13: return row_bcast<13>(v, dep);
    case 14: return row_bcast<14>(v, dep); default: return row_bcast<15>(v, dep);
  }
}

NK_DEVICE float dot2_ones(bf16x2_t p, float acc) {
  const bf16x2_t ones = {(bf16_t)1.0f, (bf16_t)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(p, ones, acc, false);
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
  constexpr int NS = (NPF % 2 == 0 && D <= 128) ? NK_DECODE_STEPS_PER_UPDATE : 1;   // steps per softmax update
  static_assert(CH % NS == 0 && NPF % NS == 0, "steps per update must divide the ring and the sub-chunk");
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
  const int c = NK_DECODE_CHUNKS_REVERSED && !FP8 && a.sink_keys == 0 ? a.max_chunks - 1 - sc / B : sc / B;
  const int hb = blockIdx.y;                  // block of 16 query heads
  const int lane = threadIdx.x;
  const int hkv = a.cache.num_kv_heads;
  const int G = a.hq / hkv;

  const int q0 = a.q_offsets[s];
  if (a.q_offsets[s + 1] - q0 != 1) return;
  const int L = a.kv_lens[s];
  const int hi = L - 1;
  // band chunks from c0 (32-key aligned), then the chunk of the sink keys
  // before the band, if any (clamped to the grid: a kv_len above max_kv_len
  // violates the precondition, and its row covers only max_chunks chunks)
  const DecodeChunks dc = decode_chunks(L, a.window_left, a.sink_keys, a.split_tokens, a.max_chunks);
  const int n_chunks = dc.n;
  if (c >= n_chunks) return;
  const bool sink_chunk = c >= dc.n_band;
  const int cs = sink_chunk ? 0 : dc.c0 + c * a.split_tokens;
  const int ce = sink_chunk ? dc.sink_end : min(cs + a.split_tokens, hi + 1);
  const int vlo = sink_chunk ? 0 : max(cs, dc.lo);          // valid keys [vlo, ce)
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

  // step i covers keys cs + 16 i .. +15: page (cs + 16 i) / P, sub-block.
  // The page ids of a sub-chunk's steps are fetched with one vector load
  // (lane j: step base + j) and read back per step into scalar registers.
  int step_page = 0;
  auto fetch_pages = [&](int base) {
    const int i = min(base + (lane % CH), nsteps - 1);   // past the end: the last page (cache hit)
    step_page = pt[(cs + 16 * i) / P];
  };
  auto issue = [&](PG &pg, int i, int j) {
    const int key0 = cs + 16 * min(i, nsteps - 1);
    const int page = __builtin_amdgcn_readlane(step_page, j);
    load_page<D, P, FP8>(pg, a.cache, page, SUB == 1 ? 0 : (key0 % P), g, loff);
  };
  // e4m3 scales of a sub-chunk (NK_DECODE_SCALE_BCAST): for its 16-step
  // group gi, lane lr + 16 lg holds the K and V scales of keys 4 lg .. 4 lg + 3
  // of step 16 gi + lr
  constexpr bool SB = FP8 && NK_DECODE_SCALE_BCAST;
  constexpr int NG = SB ? CH / 16 : 1;
  f32x4_t ksg[NG], vsg[NG];
  auto fetch_scales = [&](int base) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int key0 = cs + 16 * min(base + 16 * gi + n, nsteps - 1);
      const size_t off = ((size_t)pt[key0 / P] * hkv + g) * P + key0 % P + 4 * lg;
      ksg[gi] = *(const f32x4_t *)(a.cache.k_scales + off);
      vsg[gi] = *(const f32x4_t *)(a.cache.v_scales + off);
    }
  };
  // scales of this lane's 4 keys at step jl of the sub-chunk (jl a constant
  // once the step loop is unrolled)
  auto k_scale = [&](const PG &pg, int jl, int r, float dep) {
    if constexpr (SB) return row_bcast_n(ksg[jl / 16][r], jl, dep);
    else return pg.ks[r];
  };
  auto v_scale = [&](const PG &pg, int jl, int r, float dep) {
    if constexpr (SB) return row_bcast_n(vsg[jl / 16][r], jl, dep);
    else return pg.vs[r];
  };

  // NS consecutive 16-key steps (pages pg[0..NS-1], steps i..i+NS-1) share
  // one update of the running maximum; the maximum is replaced only when a
  // score exceeds it by more than 2^8 (exact either way: each term is
  // exp2(x - m_used)), and the normaliser sums the probabilities as rounded
  // to bf16 for the P.V product
  auto consume = [&](const PG *const *pg, int i, int jl) {
    float x[NS][4];
    bool edge = false;
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int kb = cs + 16 * (i + u);
      f32x4_t sacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<D, FP8>(*pg[u], kk), qop[kk], sacc, 0, 0, 0);
      }
      // lane holds keys kb + 4*lg + r of head column n
#pragma unroll
      for (int r = 0; r < 4; ++r)
        x[u][r] = FP8 ? sacc[r] * qk_scale * k_scale(*pg[u], jl + u, r, sacc[r]) : sacc[r] * qk_scale;
      edge |= kb < vlo || kb + 16 > ce || i + u >= nsteps;
    }
    if (edge) {
#pragma unroll
      for (int u = 0; u < NS; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = cs + 16 * (i + u) + 4 * lg + r;
          if (key < vlo || key >= ce) x[u][r] = -INFINITY;
        }
    }
    float tmax = x[0][0];
#pragma unroll
    for (int u = 0; u < NS; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, x[u][r]);
    tmax = rows_max(tmax);
    const bool grow = tmax > m_run + 8.f;
    if (__any(grow)) {
      const float m_new = grow ? tmax : m_run;
      const float corr = grow ? fast_exp2(m_run - m_new) : 1.f;   // 0 when m_run = -inf
      l_run *= corr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= corr;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int kb = cs + 16 * (i + u);
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = fast_exp2(x[u][r] - m_use);
      bf16x4_t pop;
      if constexpr (FP8) {
#pragma unroll
        for (int r = 0; r < 4; ++r) l_run += p[r];
#pragma unroll
        for (int r = 0; r < 4; ++r) pop[r] = (bf16_t)(p[r] * v_scale(*pg[u], jl + u, r, p[r]));
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) pop[r] = (bf16_t)p[r];
        l_run = dot2_ones(bf16x2_t{pop[0], pop[1]}, l_run);
        l_run = dot2_ones(bf16x2_t{pop[2], pop[3]}, l_run);
      }
      if (edge) {
        // masked keys may hold anything (unwritten slots, NaN scales): zero them
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kb + 4 * lg + r;
          if (key < vlo || key >= ce) pop[r] = (bf16_t)0.f;
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          bf16x4_t vv = v_operand<D, FP8>(*pg[u], dt);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kb + 4 * lg + r < vlo || kb + 4 * lg + r >= ce) vv[r] = (bf16_t)0.f;
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vv, pop, o[dt], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v_operand<D, FP8>(*pg[u], dt), pop, o[dt], 0, 0, 0);
        }
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
    fetch_pages(base);
    if constexpr (SB) fetch_scales(base);       // requested before the pages that need them
    PG ring[NPF];
#pragma unroll
    for (int j = 0; j < NPF; ++j) issue(ring[j], base + j, j);
#pragma unroll
    for (int j = 0; j < CH; j += NS) {
      if (base + j < nsteps) {
        const PG *pgs[NS];
#pragma unroll
        for (int u = 0; u < NS; ++u) pgs[u] = &ring[(j + u) % NPF];
        consume(pgs, base + j, j);
      }
#pragma unroll
      for (int u = 0; u < NS; ++u)
        if (j + u + NPF < CH) issue(ring[(j + u) % NPF], base + j + u + NPF, j + u + NPF);
    }
  }

  // per-column sum over the four lane groups
  l_run = rows_sum(l_run);

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
  constexpr int NPF = D == 256 ? NK_DECODE_NPF_D256 : (FP8 ? NK_DECODE_NPF_FP8 : NK_DECODE_NPF_BF16);
  const int hkv = a.cache.num_kv_heads;
  const int G = a.hq / hkv;
  dim3 grid((unsigned)(a.num_seqs * a.max_chunks * hkv), (unsigned)((G + 15) / 16), 1);
  // sub-chunks of 32 steps (512 keys) when the chunk size allows, else 16
  if (a.split_tokens % 512 == 0) return launch(attn_decode_kernel<D, P, FP8, NPF, 32>, grid, dim3(64), 0, stream, a);
  return launch(attn_decode_kernel<D, P, FP8, NPF, 16>, grid, dim3(64), 0, stream, a);
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
