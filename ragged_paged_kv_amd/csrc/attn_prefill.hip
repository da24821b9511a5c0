// Ragged causal (optionally windowed) prefill attention over a paged bf16 or
// e4m3 cache, on bf16 MFMA.
//
// What it computes: NumKong matrix-kernels page, attention_packed: query
// row i of a segment with q_len rows over kv_len keys sits at
// i + kv_len - q_len and sees the keys of its causal band (the last
// window_left + 1 of them when a window is set); aria_kernel
// `attention_causal_with_scale` (explicit scale, optional sliding window).
// A general band (keys up to window_right past the row) and, beside a
// window, the segment's first sink_keys keys (Algenta, "Ten named
// techniques, one scalar formula each", StreamingLLM sinks) widen the set;
// the sink keys' tiles are visited before the band's.
// The softmax is accumulated online, tile by tile, as on the Algenta page's
// flash-attention walkthrough: a running maximum, a running sum and a
// running output, rescaled by exp(old - new) when the maximum rises.
//
// Design (MFMA-bound):
//   * a work-group owns BM query rows of one segment and GW query heads of one
//     KV head (each wave owns 32 rows of one head; at head_dim 256 each wave
//     owns 16 rows, whose scores and full 256-dim output fit its registers),
//     so every K/V tile staged in LDS serves all GW heads;
//   * KV tiles of 64 keys (four 16-token or two 32-token pages).  Each page's
//     K or V block of one head is contiguous in the cache, so a wave's load
//     instruction reads one contiguous 1 KiB (bf16) piece of one page, at a
//     scalar page base plus a per-lane offset fixed for the whole kernel;
//     e4m3 codes are widened to bf16 on the way to LDS, their scales kept
//     beside the tile;
//   * LDS rows are padded by 16 bytes (no swizzle): the MFMA operand reads of
//     8 consecutive lanes hit 8 consecutive rows and so 32 distinct banks,
//     and every operand address is a per-lane base plus an immediate;
//   * per wave: S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (32 keys x 32 rows).
//     K rows sit in LDS in a permuted key order (bits 2 and 3 of the key
//     swapped) that makes the score tile's lane layout the P^T operand layout
//     of the second product O^T += V^T P^T (32 dims x 32 rows), so the
//     probabilities never leave their lanes.  16-row waves use
//     v_mfma_f32_16x16x32_bf16 (16 keys x 16 rows; 16 dims x 16 rows) with K
//     in key order and the V^T columns permuted instead;
//   * software pipeline: K runs one tile ahead of V; K and V tiles are
//     double-buffered and the global loads of tiles t+3 (K) and t+2 (V) are
//     in flight during iteration t.  Where two waves share a SIMD (8 waves
//     per work-group) they run one barrier apart: while one issues the score
//     and P.V MFMAs of its tile, the other runs its softmax and tile loads;
//   * online softmax in the exp2 domain, one fused multiply-add and one exp
//     per score; the running maximum is replaced only when the tile's
//     maximum exceeds it by more than 2^8 (exact either way: each term is
//     exp2(x - m_used)); the normaliser sums the probabilities as rounded to
//     bf16 for the P.V product (v_dot2_f32_bf16 on the packed pairs);
//   * persistent work-groups: a one-work-group plan kernel lists every
//     (segment, q-block) item, heaviest first, with the segment's offsets;
//     work-groups pull (item, head block) units from one atomic queue per
//     XCD, so the head blocks of a queue share that XCD's L2.

#include "common.h"
#include "internal.h"

// Waves per work-group for head dims up to 128 (compile-time, measured):
// 8 = one work-group per CU, 4 = two work-groups per CU whose barriers are
// independent.
#ifndef NK_PREFILL_NW
#define NK_PREFILL_NW 8
#endif
// head_dim 256: the output dimensions of a row block are split over this
// many waves, each computing the full scores (1 = no split, 4 waves per
// work-group; 2 = 8 waves, two per SIMD, each holding half of O)
#ifndef NK_PREFILL_D256_SPLIT
#define NK_PREFILL_D256_SPLIT 2
#endif
// Query rows per wave: 32 (v_mfma_f32_32x32x16_bf16 tiles) or 16
// (v_mfma_f32_16x16x32_bf16 tiles), for head dims up to 128 and for 256
#ifndef NK_PREFILL_RW
#define NK_PREFILL_RW 32
#endif
#ifndef NK_PREFILL_D256_RW
#define NK_PREFILL_D256_RW 16
#endif
// LDS operand reads in flight ahead of the MFMA that consumes them (head
// dims up to 128; 256: measured, fewer reads in flight are faster there)
#ifndef NK_PREFILL_VPAIR
#define NK_PREFILL_VPAIR 1
#endif
#ifndef NK_PREFILL_LDS_AHEAD
#define NK_PREFILL_LDS_AHEAD 4
#endif
#ifndef NK_PREFILL_LDS_AHEAD_D256
#define NK_PREFILL_LDS_AHEAD_D256 2
#endif
// Page ids of the K tile a load step requests are read one load step
// earlier (1), so that its global loads do not wait for scalar loads
// (head_dim 256: 2 % faster on the sliding-window batch; at 128 within
// noise, so left off there)
#ifndef NK_PREFILL_EARLY_IDS
#define NK_PREFILL_EARLY_IDS 1
#endif

namespace nk {
namespace {

constexpr int BN = 64;     // keys per KV tile

// Key (within a 32-key subtile) held by LDS row r of a K tile: bits 2 and 3
// of r swapped.  An involution.
NK_DEVICE constexpr int perm_key(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// The page table is read-only while a kernel runs: reading it through the
// constant address space lets wave-uniform lookups use scalar loads.
typedef __attribute__((address_space(4))) const int32_t *const_i32_ptr;

template <int D, int P, bool FP8, int NW>
struct Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int KROW = 2 * D + 16;             // bytes per K row (key) in LDS
  static constexpr int VROW = 2 * BN + 16;            // bytes per V^T row (dim) in LDS
  static constexpr int KBUF = BN * KROW;
  static constexpr int VBUF = D * VROW;
  static constexpr int SBUF = FP8 ? BN * 4 : 0;       // K scales, one per LDS row
  static constexpr int V_OFF = 2 * KBUF;
  static constexpr int KS_OFF = 2 * KBUF + 2 * VBUF;
  static constexpr int LDS = 2 * (KBUF + VBUF + SBUF);
  static constexpr int ESZ = FP8 ? 1 : 2;
  static constexpr int PAGE_CH = D * P / 8;            // 8-element chunks per page block
  static constexpr int PER = BN * D / 8 / NT;          // chunks per thread per tile (K or V)
  static constexpr int NPG = BN / P;                   // pages per tile
  // a 16-token block of one head's V is 16 D elements = 2 D chunks of 8:
  // when that is one chunk per thread, a thread's chunks i and i + 1 (even i)
  // cover the same dims for tokens 16 apart
  static constexpr bool V_PAIRS = NK_PREFILL_VPAIR && 2 * D == NT && PER % 2 == 0;
  static_assert(PAGE_CH % 64 == 0, "a wave's chunk must lie in one page");
  static_assert((BN * D / 8) % NT == 0, "tile chunks must divide over the threads");
};

NK_DEVICE uint32_t pack_bf16(float lo, float hi) {
  bf16x2_t v = {(bf16_t)lo, (bf16_t)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// max over the lane pair (l, l ^ 32): v_permlane32_swap exchanges the two
// 32-lane halves of a register pair, so one of the two outputs holds the
// partner's value whichever half the lane is in
NK_DEVICE float halves_max(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

NK_DEVICE float halves_sum(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// the same over the four 16-lane rows (l, l ^ 16, l ^ 32, l ^ 48):
// v_permlane16_swap first exchanges rows 0/1 and 2/3
NK_DEVICE float quarters_max(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return halves_max(fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])));
}

NK_DEVICE float quarters_sum(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return halves_sum(__builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]));
}

// One MFMA tile: 32 x 32 (k 16) or 16 x 16 (k 32), chosen by the accumulator
NK_DEVICE f32x16_t mma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
NK_DEVICE f32x4_t mma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS column of V^T that holds key k of a tile, 16-row waves: within each
// 32 keys, key 16h + 4q + i goes to column 8q + 4h + i, so that the 8
// columns a lane reads for the P.V product's k-step hold the keys of its
// score entries (keys 4q.. of both 16-key subtiles).  32-row waves keep
// V^T in key order and permute the K rows instead.
template <int RW>
NK_DEVICE constexpr int v_column(int k) {
  return RW == 32 ? k : (k & ~31) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}

NK_DEVICE float dot2_ones(uint32_t pk, float acc) {
  const bf16x2_t ones = {(bf16_t)1.0f, (bf16_t)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk), ones, acc, false);
}

// Key tiles of the sink keys left of a work item's band: the tiles that hold
// keys 0 .. sink_keys-1 below the band's first tile tb0 (sink keys in tile
// tb0 or later are visited with the band).
NK_DEVICE int sink_tiles(int sink_keys, int tb0, int bn) {
  return sink_keys > 0 ? min((sink_keys + bn - 1) / bn, tb0) : 0;
}

// Output dims split over the waves of a row block (32-row waves at head_dim
// 256 only)
template <int D, int RW>
constexpr int out_split() { return D == 256 && RW == 32 ? NK_PREFILL_D256_SPLIT : 1; }

// One work item: BM query rows (q-block qb) of segment s for the GW query
// heads of head block hy (KV head hy / HB).  Every thread of the work-group
// calls it with the same arguments.  A wave owns RW rows of one head.
template <int D, int P, bool FP8, int NW, int RW, bool SINKS>
NK_DEVICE void prefill_item(const AttnArgs &a, int GW, int s, int qb, int q0, int q_len, int L, int hy,
                            uint8_t *lds) {
  using C = Cfg<D, P, FP8, NW>;
  using Acc = typename std::conditional<RW == 32, f32x16_t, f32x4_t>::type;
  constexpr int NT = C::NT;
  constexpr int KW = 512 / RW;    // dims (score product) or keys (P.V) per MFMA k-step: 16 or 32
  constexpr int KD = D / KW;      // k-steps of the score MFMA
  constexpr int NSB = BN / RW;    // score subtiles (RW keys each) per tile
  constexpr int NA = RW * RW / 64; // accumulator entries per lane per subtile (16 or 4)
  constexpr int DH = out_split<D, RW>();   // waves sharing a row block's output dims
  constexpr int DT = D / RW / DH; // RW-dim tiles of the output MFMA held by a wave
  constexpr int PER = C::PER;
  constexpr int NPG = C::NPG;
  static_assert(sizeof(Acc) == NA * sizeof(float), "accumulator entries per lane");
  static_assert(RW * DT * DH == D, "output tiles cover the head dims");
  using Raw = typename std::conditional<FP8, u32x2_t, bf16x8_t>::type;

  const int hkv = a.cache.num_kv_heads;
  const int G = a.hq / hkv;
  const int HB = G / GW;                      // head blocks per KV head
  const int TB = NW / (GW * DH);              // RW-row blocks per work-group
  const int BM = RW * TB;
  const int g = hy / HB;
  const int hblk = hy % HB;

  const int r0 = qb * BM;
  const int shift = L - q_len;                // row r sits at position r + shift
  const int r_last = min(r0 + BM, q_len) - 1;
  const int kmax_wg = band_hi(r_last + shift, L, a.window_right);
  const int kmin_wg = band_lo(r0 + shift, a.window_left);
  if (kmax_wg < kmin_wg || L <= 0) {
    // no row of the group sees a key (q_len > kv_len): zeros, -inf
    for (int e = threadIdx.x; e < (r_last - r0 + 1) * GW * D; e += NT) {
      const int rr = e / (GW * D), rem = e % (GW * D);
      const int head = g * G + hblk * GW + rem / D;
      ((bf16_t *)a.out)[((size_t)(q0 + r0 + rr) * a.hq + head) * D + rem % D] = (bf16_t)0.f;
      if (a.lse && rem % D == 0) a.lse[(size_t)(q0 + r0 + rr) * a.hq + head] = -INFINITY;
    }
    return;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = wv % GW;
  const int dh = (wv / GW) % DH;              // which part of the output dims
  const int tb = wv / (GW * DH);
  const int head = g * G + hblk * GW + hl;
  const int rw = r0 + RW * tb;                // wave's first row
  const int qcol = lane % RW;                 // this lane's query row (column of S^T)
  const int half = lane / RW;                 // which 8 elements of a k-step the lane holds
  const int my_row = rw + qcol;
  const bool row_valid = my_row < q_len;
  const int my_pos = my_row + shift;
  const int my_lo = band_lo(my_pos, a.window_left);
  const int my_hi = band_hi(my_pos, L, a.window_right);
  // the wave's key range (over its valid rows)
  const bool wave_active = rw < q_len;
  const int w_rows_last = min(rw + RW - 1, q_len - 1);
  const int wk_hi = band_hi(w_rows_last + shift, L, a.window_right);
  const int wk_lo = band_lo(rw + shift, a.window_left);

  // ---- Q operand (B of the score product): lane holds Q[row][KW kk + 8 half .. +8].
  // A negative scale is folded into Q's sign (exact), a zero scale into a
  // zero Q, so that the exp2-domain factor c2 is positive.
  float c2 = a.softmax_scale * kLog2e;
  uint32_t qxor = 0;
  bool qzero = !row_valid;
  if (c2 < 0.f) { c2 = -c2; qxor = 0x80008000u; }
  else if (c2 == 0.f) { c2 = 1.f; qzero = true; }
  bf16x8_t qop[KD];
  {
    const bf16_t *qrow = (const bf16_t *)a.q + ((size_t)(q0 + (row_valid ? my_row : 0)) * a.hq + head) * D;
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
      u32x4_t v = *(const u32x4_t *)(qrow + KW * kk + 8 * half);
      v ^= qxor;
      if (qzero) v = u32x4_t{};
      qop[kk] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // ---- loader geometry, fixed per thread
  const int last_page = (L - 1) / P;
  const int32_t *pt = a.cache.page_table + (size_t)s * a.cache.page_table_stride;
  const const_i32_ptr ptc = (const_i32_ptr)pt;
  const size_t head_bytes = (size_t)P * D * C::ESZ;     // one page's K (or V) block of one head
  const size_t page_bytes = (size_t)hkv * head_bytes;
  const uint8_t *kb = (const uint8_t *)a.cache.k_pages + (size_t)g * head_bytes;
  const uint8_t *vb = (const uint8_t *)a.cache.v_pages + (size_t)g * head_bytes;
  // tiles are visited in the order t0 .. t1 of a virtual index: first the
  // ns sink tiles (physical tiles 0 .. ns-1), then the band's tiles, whose
  // virtual index is their physical one (calls without sink keys run an
  // instantiation where the index is the physical one throughout)
  const int tb0 = kmin_wg / BN, t1 = kmax_wg / BN;
  const int ns = SINKS ? sink_tiles(a.sink_keys, tb0, BN) : 0;
  const int t0 = tb0 - ns;
  auto phys = [&](int t) { return SINKS && t < tb0 ? t - t0 : t; };

  int pit[PER];                                         // page of the tile (wave-uniform)
  uint32_t kg[PER], vg[PER], kl[PER], vl[PER], vkey[PER];
  constexpr int NV = FP8 ? 4 : 2;                        // 16-dim groups per 16-byte V run
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + i * NT;
    pit[i] = (wv * 64 + i * NT) / C::PAGE_CH;
    const int w = c % C::PAGE_CH;
    // K: lanes take consecutive LDS rows; the page block is
    // [dim/(32 NK)][token][run (4)][half (NK)][8], NK 2 for e4m3, else 1
    constexpr int NK = FP8 ? 2 : 1;
    const int kslot = w % P, e8 = (w / P) & 3, blk = w / (4 * P);
    const int ksrc = RW == 32 ? perm_key(kslot) : kslot;
    kg[i] = (uint32_t)((((blk / NK) * P + ksrc) * 32 * NK + e8 * NK * 8 + (blk % NK) * 8) * C::ESZ);
    kl[i] = (uint32_t)((pit[i] * P + kslot) * C::KROW + (blk * 32 + e8 * 8) * 2);
    // V: the page block is 16-token blocks of 16-byte runs in MFMA operand
    // order; a chunk (8 elements) is 4 tokens of 2 dims 16 apart: run
    // R = w * 8 / (4 NV) holds dims 16 (c NV + j) + l of tokens 16 sb + 4 gq..
    const int e0 = 8 * w, R = e0 / (4 * NV), jq = (e0 % (4 * NV)) / 4;
    const int runs_per_block = (D / (16 * NV)) * 64;
    const int sb = R / runs_per_block, rr = R % runs_per_block;
    const int cg = rr / 64, L = rr % 64, gq = L / 16, l = L % 16;
    const int dim0 = 16 * (cg * NV + jq) + l;              // and dim0 + 16
    vg[i] = (uint32_t)(e0 * C::ESZ);
    vkey[i] = (uint32_t)(pit[i] * P + 16 * sb + 4 * gq);
    vl[i] = (uint32_t)(dim0 * C::VROW + v_column<RW>(vkey[i]) * 2);
  }

  Raw kst[PER], vst[PER];
  f32x4_t vsc[PER];                                     // e4m3: the scales of a V chunk's 4 keys
  float kss = 0.f;                                      // e4m3: K scale of LDS row tid
  auto page_of = [&](int tile, int j) -> size_t {
    return (size_t)(uint32_t)ptc[min(tile * NPG + j, last_page)];
  };
  // pages of the K tile last requested: the V tile requested one step later
  // is the same tile
  size_t pgk[PER];
  constexpr bool EARLY_IDS = NK_PREFILL_EARLY_IDS && D == 256;
  // page ids read ahead for the next load_k (EARLY_IDS)
  int pid_next[PER];
  auto fetch_ids = [&](int vtile) {
    const int tile = phys(vtile);
#pragma unroll
    for (int i = 0; i < PER; ++i) pid_next[i] = ptc[min(tile * NPG + pit[i], last_page)];
  };
  // K of `tile` into the given staging registers; `early`: its page ids are
  // the ones fetch_ids read
  auto load_k_to = [&](int vtile, Raw (&dst)[PER], float &dss, bool early) {
    const int tile = phys(vtile);
    if (early) {
#pragma unroll
      for (int i = 0; i < PER; ++i) pgk[i] = (size_t)(uint32_t)pid_next[i];
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) pgk[i] = page_of(tile, pit[i]);
      __builtin_amdgcn_sched_barrier(0);     // all page lookups in flight together
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) dst[i] = *(const Raw *)(kb + pgk[i] * page_bytes + kg[i]);
    if (FP8 && tid < BN) {
      const int key = tile * BN + (RW == 32 ? 32 * (tid >> 5) + perm_key(tid & 31) : tid);
      const int page = pt[min(key / P, last_page)];
      dss = a.cache.k_scales[((size_t)page * hkv + g) * P + key % P];
    }
  };
  auto load_k = [&](int tile) { load_k_to(tile, kst, kss, false); };
  // V of `tile` through the given pages
  auto load_v = [&](const size_t (&pg)[PER]) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      vst[i] = *(const Raw *)(vb + pg[i] * page_bytes + vg[i]);
      if constexpr (FP8) {
        vsc[i] = *(const f32x4_t *)(a.cache.v_scales + (pg[i] * hkv + g) * P + (vkey[i] % P));
      }
    }
  };
  auto store_k_from = [&](int buf, const Raw (&src)[PER], float sss) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      bf16x8_t x;
      if constexpr (FP8) x = fp8x8_to_bf16x8(src[i]); else x = src[i];
      *(bf16x8_t *)(lds + buf * C::KBUF + kl[i]) = x;
    }
    if (FP8 && tid < BN) ((float *)(lds + C::KS_OFF + buf * C::SBUF))[tid] = sss;
  };
  auto store_k = [&](int buf) { store_k_from(buf, kst, kss); };
  // e4m3 V enters LDS as bf16(code * scale); keys >= L become zeros (their
  // slots may hold anything, and 0 * NaN is NaN)
  auto store_v = [&](int buf, int vtile) {
    const int base = phys(vtile) * BN;
    // chunk i as bf16: elements 0..3 dim dim0, tokens vkey..+3; 4..7 dim dim0 + 16
    auto chunk = [&](int i) {
      bf16x8_t x;
      if constexpr (FP8) {
        const bf16x8_t c = fp8x8_to_bf16x8(vst[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (bf16_t)((float)c[e] * vsc[i][e & 3]);
      } else {
        x = vst[i];
      }
      if (base + BN > L) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (base + (int)vkey[i] + (e & 3) >= L) x[e] = (bf16_t)0.f;
      }
      return x;
    };
    if constexpr (C::V_PAIRS && RW == 16) {
      // chunks i and i + 1 hold the same dims for tokens 16 apart, which the
      // 16-row column order places side by side: one 16-byte store per dim
#pragma unroll
      for (int i = 0; i < PER; i += 2) {
        const bf16x8_t x0 = chunk(i), x1 = chunk(i + 1);
        uint8_t *dst = lds + C::V_OFF + buf * C::VBUF + vl[i];
        *(bf16x8_t *)dst = bf16x8_t{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        *(bf16x8_t *)(dst + 16 * C::VROW) = bf16x8_t{x0[4], x0[5], x0[6], x0[7], x1[4], x1[5], x1[6], x1[7]};
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const bf16x8_t x = chunk(i);
        uint8_t *dst = lds + C::V_OFF + buf * C::VBUF + vl[i];
        *(bf16x4_t *)dst = bf16x4_t{x[0], x[1], x[2], x[3]};
        *(bf16x4_t *)(dst + 16 * C::VROW) = bf16x4_t{x[4], x[5], x[6], x[7]};
      }
    }
  };

  // ---- MFMA operand bases: per-lane base plus immediates
  const uint8_t *klane = lds + qcol * C::KROW + 16 * half;
  const uint8_t *vlane = lds + C::V_OFF + (dh * DT * RW + qcol) * C::VROW + 16 * half;

  float m_run = -INFINITY, l_run = 0.f;
  Acc o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = Acc{};
  Acc sc[NSB];             // scores S^T of the next tile (NSB subtiles of RW keys)
  constexpr int NPK = NSB * NA / 2;
  uint32_t pk[NPK];        // probabilities of the current tile, bf16 pairs
#pragma unroll
  for (int j = 0; j < NPK; ++j) pk[j] = 0u;

  auto active = [&](int t) {
    const int b = phys(t) * BN;
    return wave_active && b <= wk_hi && (b + BN - 1 >= wk_lo || (SINKS && b < a.sink_keys));
  };

  // M(t), t >= t0: S(t+1) = K(t+1) Q^T and O^T += V(t)^T P(t)^T -- MFMA
  // work only, one straight block (past the last tile S reads a stale
  // buffer and is never used; P is zero where the wave sees no key of the
  // tile, and V(t) is a loaded tile, finite).  The LDS operand reads run
  // NK_PREFILL_LDS_AHEAD MFMAs ahead.
  auto mfma_step = [&](int t) {
    const uint8_t *kt = klane + ((t + 1) & 1) * C::KBUF;
    const uint8_t *vt = vlane + (t & 1) * C::VBUF;
    auto kop = [&](int i) { return *(const bf16x8_t *)(kt + (i / KD) * RW * C::KROW + 2 * KW * (i % KD)); };
    auto vop = [&](int i) { return *(const bf16x8_t *)(vt + (i % DT) * RW * C::VROW + 2 * KW * (i / DT)); };
    constexpr int NS = NSB * KD, NP = (BN / KW) * DT;
    constexpr int AH = D == 256 ? NK_PREFILL_LDS_AHEAD_D256 : NK_PREFILL_LDS_AHEAD;
    bf16x8_t ring[AH];
#pragma unroll
    for (int i = 0; i < AH; ++i) ring[i] = i < NS ? kop(i) : vop(i - NS);
#pragma unroll
    for (int i = 0; i < NS + NP; ++i) {
      const bf16x8_t opnd = ring[i % AH];
      if (i + AH < NS + NP) ring[i % AH] = i + AH < NS ? kop(i + AH) : vop(i + AH - NS);
      if (i < NS) {
        const int st = i / KD, kk = i % KD;
        sc[st] = mma(opnd, qop[kk], kk == 0 ? Acc{} : sc[st]);
      } else {
        // k-step c of P^T: 32-row waves take the pairs 8(c/2) + 4(c%2) ..
        // (the permuted K rows), 16-row waves the pairs 4c .. (entries 0..3
        // of subtiles 2c and 2c + 1, matching the permuted V^T columns)
        const int c = (i - NS) / DT, dt = (i - NS) % DT, b = RW == 32 ? 8 * (c >> 1) + 4 * (c & 1) : 4 * c;
        const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[b], pk[b + 1], pk[b + 2], pk[b + 3]});
        o[dt] = mma(opnd, pop, o[dt]);
      }
    }
#pragma unroll
    for (int i = 0; i < AH; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // one LDS read
    }
#pragma unroll
    for (int i = 0; i < NS + NP; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
      if (i + AH < NS + NP) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  // V(t): softmax of S(t+1) into P(t+1), with the running maximum and sum
  // -- VALU work only.  Entry v of subtile st holds key
  // 32st + 16(v>>3) + 8half + (v&7) of the tile (32-row waves: C row
  // 8(v>>2) + 4half + (v&3), through the K row permutation) or
  // 16st + 4half + v (16-row waves: C row 4half + v, K rows in key order).
  // S is dead afterwards and is overwritten in place.
  auto softmax_step = [&](int t) {
    const int tn = t + 1;
    if (tn > t1 || !active(tn)) {
#pragma unroll
      for (int j = 0; j < NPK; ++j) pk[j] = 0u;
      return;
    }
    const int tile_base = phys(tn) * BN;
    if constexpr (FP8) {
      // K scales are stored per LDS row: C rows 4 apart, 4 at a time
      const float *ks = (const float *)(lds + C::KS_OFF + (tn & 1) * C::SBUF);
#pragma unroll
      for (int st = 0; st < NSB; ++st)
#pragma unroll
        for (int j = 0; j < NA / 4; ++j) {
          const f32x4_t k4 = *(const f32x4_t *)(ks + RW * st + 8 * j + 4 * half);
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[st][4 * j + r] *= k4[r];
        }
    }
    const bool mask = tile_base + BN - 1 > band_hi(rw + shift, L, a.window_right) ||
                      (a.window_left >= 0 && tile_base < band_lo(w_rows_last + shift, a.window_left));
    if (mask) {
      constexpr int KOFF = RW == 32 ? 8 : 4;                      // key offset per lane group
      const int rel_hi = row_valid ? my_hi - tile_base - KOFF * half : -1000000;
      const int rel_lo = my_lo - tile_base - KOFF * half;
      const int rel_sink = a.sink_keys - tile_base - KOFF * half;    // keys below it are sinks
      if (!SINKS && a.window_left < 0) {
        // no left bound (plain causal): one compare per entry
#pragma unroll
        for (int st = 0; st < NSB; ++st)
#pragma unroll
          for (int v = 0; v < NA; ++v) {
            const int kv = RW == 32 ? 32 * st + 16 * (v >> 3) + (v & 7) : 16 * st + v;
            if (kv > rel_hi) sc[st][v] = -INFINITY;
          }
      } else {
#pragma unroll
        for (int st = 0; st < NSB; ++st)
#pragma unroll
          for (int v = 0; v < NA; ++v) {
            const int kv = RW == 32 ? 32 * st + 16 * (v >> 3) + (v & 7) : 16 * st + v;
            if (kv > rel_hi || (kv < rel_lo && (!SINKS || kv >= rel_sink))) sc[st][v] = -INFINITY;
          }
      }
    }
    float tmax = sc[0][0];
#pragma unroll
    for (int i = 1; i < NSB * NA; ++i) tmax = fmaxf(tmax, sc[i / NA][i % NA]);
    tmax = RW == 32 ? halves_max(tmax) : quarters_max(tmax);
    const float tm = tmax * c2;
    const bool grow = tm > m_run + 8.f;
    if (__any(grow)) {
      const float m_new = grow ? tm : m_run;
      const float corr = grow ? fast_exp2(m_run - m_new) : 1.f;   // 0 when m_run = -inf
      l_run *= corr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= corr;
      m_run = m_new;
    }
    const float nm = m_run == -INFINITY ? 0.f : -m_run;
    float l0 = 0.f, l1 = 0.f;
#pragma unroll
    for (int j = 0; j < NPK; ++j) {
      const int st = 2 * j / NA, v = 2 * j % NA;
      pk[j] = pack_bf16(fast_exp2(fmaf(sc[st][v], c2, nm)), fast_exp2(fmaf(sc[st][v + 1], c2, nm)));
      if (j & 1) l1 = dot2_ones(pk[j], l1); else l0 = dot2_ones(pk[j], l0);
    }
    l_run += l0 + l1;
  };

  // L(t): K(t+2) and V(t+1) from the staging registers into LDS (replacing
  // K(t) and V(t-1)), then request K(t+3) and V(t+2)
  auto load_step = [&](int t) {
    if (t + 2 <= t1) store_k(t & 1);
    if (t + 1 <= t1) store_v((t + 1) & 1, t + 1);
    size_t pgv[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) pgv[i] = pgk[i];
    if (EARLY_IDS) {
      if (t + 3 <= t1) load_k_to(t + 3, kst, kss, true);
      if (t + 4 <= t1) fetch_ids(t + 4);
    } else {
      if (t + 3 <= t1) load_k(t + 3);
    }
    if (t + 2 <= t1) load_v(pgv);
  };

  // ---- prologue: K(t0) in LDS; K(t0+1), V(t0) staged.  All three are
  // requested before the first is waited for.
  {
    Raw k0[PER];
    float ks0 = 0.f;
    load_k_to(t0, k0, ks0, false);
    size_t pgv[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) pgv[i] = pgk[i];
    if (t0 + 1 <= t1) load_k(t0 + 1);
    load_v(pgv);
    // the first load step requests K(t0 + 2)
    if (EARLY_IDS && t0 + 2 <= t1) fetch_ids(t0 + 2);
    store_k_from(t0 & 1, k0, ks0);
  }
  __syncthreads();

  // ---- ping-pong: waves w and w + NW/2 share a SIMD.  Both groups run the
  // same sequence M(it), barrier, V(it) + L, barrier; group 1 starts one
  // barrier later, so that between two barriers one wave of each SIMD issues
  // MFMAs while the other works on the VALU.  M(it) of either group reads
  // K(it+1) and V(it); the loads of group 0 (L(it), after its V(it)) and of
  // group 1 (L(it+1), after its V(it), i.e. during group 0's M(it+1)) write
  // the other buffers.
  // (only where two waves share a SIMD: with 4 waves per work-group each
  // SIMD holds one, and an offset group would only wait)
  const int grp = NW >= 8 && wv >= NW / 2 ? 1 : 0;
  if (grp) {
    load_step(t0 - 1);
    __syncthreads();
  }
  // M(t0 - 1): S(t0) only (no V tile before t0)
  {
    const uint8_t *kt = klane + (t0 & 1) * C::KBUF;
#pragma unroll
    for (int st = 0; st < NSB; ++st) {
      sc[st] = Acc{};
#pragma unroll
      for (int kk = 0; kk < KD; ++kk)
        sc[st] = mma(*(const bf16x8_t *)(kt + st * RW * C::KROW + 2 * KW * kk), qop[kk], sc[st]);
    }
  }
  __syncthreads();
  softmax_step(t0 - 1);
  load_step(t0 - 1 + grp);
  __syncthreads();
  for (int it = t0; it <= t1; ++it) {
    mfma_step(it);
    __syncthreads();
    softmax_step(it);
    load_step(it + grp);
    if (grp == 0 || it < t1) __syncthreads();
  }

  if (!wave_active) return;
  l_run = RW == 32 ? halves_sum(l_run) : quarters_sum(l_run);
  if (!row_valid) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  bf16_t *orow = (bf16_t *)a.out + ((size_t)(q0 + my_row) * a.hq + head) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < NA / 4; ++j) {
      // values v = 4j..4j+3 are dims RW dt + 8j + 4 half + 0..3
      bf16x4_t ov;
#pragma unroll
      for (int r = 0; r < 4; ++r) ov[r] = (bf16_t)(o[dt][4 * j + r] * inv);
      *(bf16x4_t *)(orow + RW * (dh * DT + dt) + 8 * j + 4 * half) = ov;
    }
  if (a.lse && half == 0 && dh == 0)
    a.lse[(size_t)(q0 + my_row) * a.hq + head] = l_run > 0.f ? (m_run + fast_log2(l_run)) * kLn2 : -INFINITY;
}

// Key tiles a work item visits (0 when none of its rows sees a key); the
// same bounds as prefill_item.
NK_DEVICE int item_tiles(const AttnArgs &a, int BM, int q_len, int L, int qb) {
  const int shift = L - q_len;
  const int r0 = qb * BM;
  const int r_last = min(r0 + BM, q_len) - 1;
  const int kmax = band_hi(r_last + shift, L, a.window_right);
  const int kmin = band_lo(r0 + shift, a.window_left);
  return (kmax < kmin || L <= 0) ? 0 : kmax / BN - kmin / BN + 1 + sink_tiles(a.sink_keys, kmin / BN, BN);
}

constexpr int kPlanThreads = 1024;
constexpr int kPlanBins = 4096;        // work classes (tiles, capped)

// Exclusive prefix sum over the work-group (kPlanThreads threads); *total
// receives the sum.  `part` holds one int per wave.
NK_DEVICE int block_exclusive_scan(int v, int *part, int *total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  if (lane == 63) part[w] = x;
  __syncthreads();
  if (w == 0) {
    int p = lane < kPlanThreads / 64 ? part[lane] : 0;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int y = __shfl_up(p, d, kWave);
      if (lane >= d) p += y;
    }
    if (lane < kPlanThreads / 64) part[lane] = p;          // inclusive wave totals
  }
  __syncthreads();
  const int before = (w > 0 ? part[w - 1] : 0) + x - v;
  *total = part[kPlanThreads / 64 - 1];
  __syncthreads();                                          // part is reused by the next call
  return before;
}

NK_DEVICE int segment_of_item(const int32_t *segoff, int num_seqs, int i) {
  int lo = 0, hi = num_seqs - 1;                            // last s with segoff[s] <= i
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (segoff[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Builds the prefill work list: every (segment, q-block) of the segments
// with more than one row, ordered by the key tiles it visits, most first
// (a counting sort; equal classes in any order), and zeroes the queue
// counters.  q-blocks whose rows see no key at all (rows placed before a
// segment's first key, or a segment without keys) sort last; this kernel
// writes their zeros and -inf itself and leaves them out of the item count
// the attention kernels read.  One work-group.  Batches of up to
// kPlanLdsSegs segments keep the segments' item offsets, row offsets and
// key counts in LDS, so the per-item segment search and band bounds make no
// dependent global reads; larger batches search the offsets in the
// workspace.
constexpr int kPlanLdsSegs = 2048;

__global__ void __launch_bounds__(kPlanThreads) prefill_plan_kernel(AttnArgs a, int BM) {
  __shared__ int hist[kPlanBins];
  __shared__ int part[kPlanThreads / 64];
  __shared__ int l_segoff[kPlanLdsSegs + 1];
  __shared__ int l_qoff[kPlanLdsSegs + 1];
  __shared__ int l_kvl[kPlanLdsSegs];
  int32_t *sc = a.sched;
  int32_t *segoff = sc + kSchedSegOff;
  int4 *items = (int4 *)(sc + sched_items_offset(a.num_seqs));   // two int4 per item
  const int tid = threadIdx.x;
  const bool small = a.num_seqs <= kPlanLdsSegs;
  for (int i = tid; i < kPlanBins; i += kPlanThreads) hist[i] = 0;
  if (tid < kSchedQueues) sc[tid * kSchedCounterStride] = 0;

  int base = 0;
  for (int c0 = 0; c0 < a.num_seqs; c0 += kPlanThreads) {
    const int s = c0 + tid;
    int n = 0;
    if (s < a.num_seqs) {
      const int q0 = a.q_offsets[s], q1 = a.q_offsets[s + 1];
      const int q_len = q1 - q0;
      n = q_len > 1 ? (q_len + BM - 1) / BM : 0;
      if (small) {
        l_qoff[s] = q0;
        l_kvl[s] = a.kv_lens[s];
        if (s == a.num_seqs - 1) l_qoff[s + 1] = q1;
      }
    }
    int tot;
    const int ex = block_exclusive_scan(n, part, &tot);
    if (s < a.num_seqs) {
      segoff[s] = base + ex;
      if (small) l_segoff[s] = base + ex;
    }
    base += tot;
  }
  const int n_items = min(base, a.sched_items_max);
  if (tid == 0) {
    segoff[a.num_seqs] = base;
    if (small) l_segoff[a.num_seqs] = base;
  }
  __syncthreads();
  // generic pointers: LDS copies for small batches, else global memory
  const int32_t *so = small ? (const int32_t *)l_segoff : (const int32_t *)segoff;
  const int32_t *qo = small ? (const int32_t *)l_qoff : a.q_offsets;
  const int32_t *kl = small ? (const int32_t *)l_kvl : a.kv_lens;

  for (int i = tid; i < n_items; i += kPlanThreads) {
    const int s = segment_of_item(so, a.num_seqs, i);
    const int w = item_tiles(a, BM, qo[s + 1] - qo[s], kl[s], i - so[s]);
    atomicAdd(&hist[kPlanBins - 1 - min(w, kPlanBins - 1)], 1);
  }
  __syncthreads();
  {
    // bins ascend as work descends; 4 bins per thread
    int v[kPlanBins / kPlanThreads], sum = 0;
#pragma unroll
    for (int j = 0; j < kPlanBins / kPlanThreads; ++j) { v[j] = hist[tid * (kPlanBins / kPlanThreads) + j]; sum += v[j]; }
    int tot;
    int run = block_exclusive_scan(sum, part, &tot);
#pragma unroll
    for (int j = 0; j < kPlanBins / kPlanThreads; ++j) {
      hist[tid * (kPlanBins / kPlanThreads) + j] = run;
      run += v[j];
    }
  }
  __syncthreads();
  for (int i = tid; i < n_items; i += kPlanThreads) {
    const int s = segment_of_item(so, a.num_seqs, i);
    const int qb = i - so[s];
    const int q0 = qo[s], q_len = qo[s + 1] - q0, L = kl[s];
    const int w = item_tiles(a, BM, q_len, L, qb);
    const int pos = atomicAdd(&hist[kPlanBins - 1 - min(w, kPlanBins - 1)], 1);
    items[2 * pos] = int4{s, qb, q0, q_len};
    items[2 * pos + 1] = int4{L, 0, 0, 0};
  }
  // the items without keys are the last ones (bin kPlanBins - 1 ends the
  // order); after the loop above hist[kPlanBins - 1] is the end of that bin
  __syncthreads();
  const int n_keyed = n_items - (hist[kPlanBins - 1] - (kPlanBins > 1 ? hist[kPlanBins - 2] : 0));
  if (tid == 0) sc[kSchedCount] = n_keyed;
  const int D = a.cache.head_dim;
  for (int i = n_keyed; i < n_items; ++i) {
    const int4 rec = items[2 * i];                // {s, qb, q0, q_len}: every row of the block, every head
    const int r0 = rec.y * BM, rows = min(BM, rec.w - r0);
    const long long n = (long long)rows * a.hq * D;
    bf16_t *o = (bf16_t *)a.out + ((size_t)(rec.z + r0) * a.hq) * D;
    for (long long e = tid; e < n; e += kPlanThreads) o[e] = (bf16_t)0.f;
    if (a.lse)
      for (int e = tid; e < rows * a.hq; e += kPlanThreads) a.lse[(size_t)(rec.z + r0) * a.hq + e] = -INFINITY;
  }
}

// Persistent prefill: each work-group takes work units from its queue until
// the queue is empty.  Queue q serves the work-groups with blockIdx % NQ == q
// (one queue per XCD under round-robin dispatch, so that the head blocks of
// one queue share that XCD's L2); a unit is (item, head block).  An item
// record carries its segment's row offset, row count and key count, so a
// unit starts after one read.
template <int D, int P, bool FP8, int NW, int RW, bool SINKS>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW == 4 ? 1 : 2)))
attn_prefill_kernel(AttnArgs a, int GW, int NQ) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int unit_slot;
  const int hkv = a.cache.num_kv_heads;
  const int NH = hkv * (a.hq / hkv / GW);       // head blocks per item
  const int NHq = NH / NQ;                      // of them in this queue
  const int q = blockIdx.x % NQ;
  int32_t *ctr = a.sched + q * kSchedCounterStride;
  const int4 *items = (const int4 *)(a.sched + sched_items_offset(a.num_seqs));
  const long long units = (long long)a.sched[kSchedCount] * NHq;
  if (threadIdx.x == 0) unit_slot = atomicAdd(ctr, 1);
  __syncthreads();
  int u = unit_slot;
  while (u < units) {
    __syncthreads();                            // every thread has read unit_slot
    int next = 0;
    if (threadIdx.x == 0) next = atomicAdd(ctr, 1);   // in flight while the item runs
    const int4 rec = items[2 * (u / NHq)];      // {segment, q-block, q0, q_len}
    const int kv = items[2 * (u / NHq) + 1].x;
    prefill_item<D, P, FP8, NW, RW, SINKS>(a, GW, rec.x, rec.y, rec.z, rec.w, kv, q + NQ * (u % NHq), lds);
    if (threadIdx.x == 0) unit_slot = next;
    __syncthreads();
    u = unit_slot;
  }
}

struct DeviceShape { int cus = 0; };
DeviceShape &device_shape(int dev) {
  static DeviceShape shapes[64];
  return shapes[dev & 63];
}

template <int D, int P, bool FP8, bool SINKS>
hipError_t launch_cfg(const AttnArgs &a, hipStream_t stream) {
  constexpr int RW = D == 256 ? NK_PREFILL_D256_RW : NK_PREFILL_RW;
  constexpr int DH = out_split<D, RW>();
  constexpr int NW = D == 256 && RW == 32 ? 4 * DH : NK_PREFILL_NW;
  using C = Cfg<D, P, FP8, NW>;
  const int hkv = a.cache.num_kv_heads;
  const int G = a.hq / hkv;
  int GW = 1;                                  // heads per work-group: power of 2 dividing G
  while (GW * 2 * DH <= NW && G % (GW * 2) == 0) GW *= 2;
  const int BM = RW * (NW / (GW * DH));
  static_assert(RW >= kMinPrefillBlock, "the work list is sized for q-blocks of kMinPrefillBlock rows or more");
  const int NH = hkv * (G / GW);
  const int NQ = NH % kSchedQueues == 0 ? kSchedQueues : 1;
  if (!a.sched) return hipErrorInvalidValue;
  auto kern = attn_prefill_kernel<D, P, FP8, NW, RW, SINKS>;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static int per_cu[64];                       // resident work-groups per CU, per device
  int &res = per_cu[dev & 63];
  if (res == 0) {                              // idempotent; a race only repeats the queries
    if (C::LDS > 65536) {
      e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
      if (e != hipSuccess) return e;
    }
    int n = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, NW * 64, C::LDS);
    if (e != hipSuccess) return e;
    if (n <= 0) return hipErrorInvalidConfiguration;
    res = n;
  }
  DeviceShape &ds = device_shape(dev);
  if (ds.cus == 0) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    ds.cus = cus;
  }
  // enough work-groups to fill every CU, at least one per queue
  int grid = ds.cus * res;
  grid = (grid + NQ - 1) / NQ * NQ;
  e = launch(prefill_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a, BM);
  if (e != hipSuccess) return e;
  return launch(kern, dim3(grid), dim3(NW * 64), C::LDS, stream, a, GW, NQ);
}

template <int D, int P>
hipError_t launch_dp(const AttnArgs &a, hipStream_t stream) {
  const bool sinks = a.sink_keys > 0;
  if (a.cache.dtype == NK_E4M3)
    return sinks ? launch_cfg<D, P, true, true>(a, stream) : launch_cfg<D, P, true, false>(a, stream);
  return sinks ? launch_cfg<D, P, false, true>(a, stream) : launch_cfg<D, P, false, false>(a, stream);
}

}  // namespace

hipError_t launch_attn_prefill(const AttnArgs &a, hipStream_t stream) {
  if (a.num_seqs == 0 || a.max_q_len <= 1) return hipSuccess;
  ProfileScope prof("attn_prefill", stream);
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
