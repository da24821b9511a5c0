// Ragged causal (optionally windowed) prefill attention over a paged bf16 or
// e4m3 cache, on bf16 MFMA.
//
// What it computes: NumKong matrix-kernels page, attention_packed: query
// row i of a segment with q_len rows over kv_len keys sits at
// i + kv_len - q_len and sees the keys of its causal band (the last
// window_left + 1 of them when a window is set); aria_kernel
// `attention_causal_with_scale` (explicit scale, optional sliding window).
// The softmax is accumulated online, tile by tile, as on the Algenta page's
// flash-attention walkthrough: a running maximum, a running sum and a
// running output, rescaled by exp(old - new) when the maximum rises.
//
// Design (MFMA-bound):
//   * a work-group owns BM query rows of one segment and GW query heads of one
//     KV head (GW * BM/32 = waves; each wave owns 32 rows of one head), so
//     every K/V tile staged in LDS serves all GW heads;
//   * KV tiles of 64 keys (four 16-token or two 32-token pages) are gathered
//     through the page table into LDS with contiguous 16-byte reads: K as
//     [key][dim] (from the cache's 32-dim blocks), V as [dim][key] (the cache
//     already stores V dimension-major per page), 16-byte chunks XOR-swizzled
//     against bank conflicts; e4m3 codes are widened to bf16 on the way in,
//     their scales kept beside the tile;
//   * per wave: S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (32 keys x 32 rows),
//     with K rows read in a permuted key order that makes the score tile's
//     lane layout the P^T operand layout of the second product
//     O^T += V^T P^T (32 dims x 32 rows), so probabilities never leave their
//     lanes;
//   * online softmax in the exp2 domain with the maximum kept per row in
//     registers, rescaling the output only when the maximum has grown by more
//     than 2^8 (results are exact either way: each term is exp2(x - m_used));
//   * the next tile's global loads are in flight while the current tile is
//     computed; segments' q-blocks are dispatched heaviest-first, and
//     consecutive work-groups take the KV heads of one q-block so that the
//     groups of one KV head land on one XCD (round-robin dispatch) and share
//     its L2.

#include "common.h"
#include "internal.h"

namespace nk {
namespace {

constexpr int BN = 64;     // keys per KV tile

// 16-byte slot swizzle of an LDS row: rows of 128 bytes (V^T tiles, D = 64
// K tiles) pair up in a 256-byte bank window, wider rows span it.
template <int ROW_BYTES>
NK_DEVICE int swz(int row, int slot) {
  if (ROW_BYTES == 128) return slot ^ ((row >> 1) & 7);
  return slot ^ (row & 15);
}

// Physical key (within a 32-key subtile) that score-tile row rho holds:
// bits 2 and 3 of rho swapped.
NK_DEVICE int perm_key(int rho) {
  return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

template <int D, int P, bool FP8, int NT>
struct Loader {
  static constexpr int CH = BN * D / 8;             // chunks per tile (K or V)
  static constexpr int PER = CH / NT;               // chunks per thread
  static_assert(CH % NT == 0, "tile chunks must divide over the threads");
  using Raw = typename std::conditional<FP8, u32x2_t, bf16x8_t>::type;
  Raw k[PER], v[PER];
  float ks, vs;                                     // fp8: one key's scales (threads < BN)

  NK_DEVICE void load(const AttnArgs &a, const int32_t *pt, int tile_base, int L, int g, int tid) {
    const int hkv = a.cache.num_kv_heads;
    const int last_page = (L - 1) / P;
    constexpr int esz = FP8 ? 1 : 2;
    const uint8_t *kb = (const uint8_t *)a.cache.k_pages;
    const uint8_t *vb = (const uint8_t *)a.cache.v_pages;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * NT;
      // K: chunk c -> (page of the tile, 32-dim block, key in page, 8 dims);
      // consecutive chunks are consecutive in the page's [dim/32][key][32]
      {
        const int e8 = c & 3, rest = c >> 2;
        const int kip = rest % P, rest2 = rest / P;
        const int blk = rest2 % (D / 32), pit = rest2 / (D / 32);
        const int kk = tile_base + pit * P + kip;
        const int page = pt[min(kk / P, last_page)];
        const size_t ph = (size_t)page * hkv + g;
        k[i] = *(const Raw *)(kb + (ph * P * D + ((size_t)blk * P + kip) * 32 + 8 * e8) * esz);
      }
      // V: chunk c -> dim c / 8, keys 8*(c % 8) ..
      {
        const int d = c / 8, ks8 = c % 8;
        const int kk = tile_base + 8 * ks8;
        const int page = pt[min(kk / P, last_page)];
        v[i] = *(const Raw *)(vb + ((((size_t)page * hkv + g) * D + d) * P + (kk % P)) * esz);
      }
    }
    if (FP8 && tid < BN) {
      const int kk = tile_base + tid;
      const int page = pt[min(kk / P, last_page)];
      const size_t idx = ((size_t)page * hkv + g) * P + (kk % P);
      ks = a.cache.k_scales[idx];
      vs = a.cache.v_scales[idx];
    }
  }

  // Write to LDS; keys >= L become zeros (their slots may hold anything).
  NK_DEVICE void store(bf16_t *sk, bf16_t *sv, float *sks, float *svs, int tile_base, int L, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * NT;
      {
        const int e8 = c & 3, rest = c >> 2;
        const int kip = rest % P, rest2 = rest / P;
        const int blk = rest2 % (D / 32), pit = rest2 / (D / 32);
        const int key = pit * P + kip, slot = blk * 4 + e8;
        bf16x8_t x;
        if constexpr (FP8) x = fp8x8_to_bf16x8(k[i]); else x = k[i];
        if (tile_base + key >= L) x = bf16x8_t{};
        *(bf16x8_t *)(sk + key * D + 8 * swz<D * 2>(key, slot)) = x;
      }
      {
        const int d = c / 8, ks8 = c % 8;
        bf16x8_t x;
        if constexpr (FP8) x = fp8x8_to_bf16x8(v[i]); else x = v[i];
        const int k0 = tile_base + 8 * ks8;
        if (k0 + 8 > L) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (k0 + e >= L) x[e] = (bf16_t)0.f;
        }
        *(bf16x8_t *)(sv + d * BN + 8 * swz<BN * 2>(d, ks8)) = x;
      }
    }
    if (FP8 && tid < BN) {
      const bool in = tile_base + tid < L;
      sks[tid] = in ? ks : 0.f;
      svs[tid] = in ? vs : 0.f;
    }
  }
};

template <int D, int P, bool FP8, int NWAVES>
__global__ void __launch_bounds__(NWAVES * 64) attn_prefill_kernel(AttnArgs a, int GW, int max_qb) {
  constexpr int NT = NWAVES * 64;
  constexpr int KD = D / 16;      // k-steps of the score MFMA (16 dims each)
  constexpr int DT = D / 32;      // 32-dim tiles of the output MFMA
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
  bf16_t *sk = (bf16_t *)smem_raw;                       // [BN][D]
  bf16_t *sv = sk + BN * D;                              // [D][BN]
  float *sks = (float *)(sv + D * BN);                   // [BN] (e4m3 only)
  float *svs = sks + BN;

  const int hkv = a.cache.num_kv_heads;
  const int G = a.hq / hkv;
  const int HB = G / GW;                      // head blocks per KV head
  const int NH = hkv * HB;
  const int B = a.num_seqs;
  const int TB = NWAVES / GW;                 // 32-row blocks per work-group
  const int BM = 32 * TB;

  // heaviest-first: q-block index descends along the grid; the KV heads of
  // one q-block are consecutive
  const long long lin = blockIdx.x;
  const int hy = (int)(lin % NH);
  const long long rest = lin / NH;
  const int s = (int)(rest % B);
  const int qb = max_qb - 1 - (int)(rest / B);
  const int g = hy / HB;
  const int hblk = hy % HB;

  const int q0 = a.q_offsets[s];
  const int q_len = a.q_offsets[s + 1] - q0;
  if (q_len <= 1) return;
  const int r0 = qb * BM;
  if (r0 >= q_len) return;
  const int L = a.kv_lens[s];
  const int shift = L - q_len;                // row r sits at position r + shift
  const int r_last = min(r0 + BM, q_len) - 1;
  const int kmax_wg = min(r_last + shift, L - 1);
  const int kmin_wg = a.window_left < 0 ? 0 : max(0, r0 + shift - a.window_left);
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
  const int32_t *pt = a.cache.page_table + (size_t)s * a.cache.page_table_stride;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hl = w % GW;
  const int tb = w / GW;
  const int head = g * G + hblk * GW + hl;
  const int rw = r0 + 32 * tb;                // wave's first row
  const int qcol = lane & 31;                 // this lane's query row (column of S^T)
  const int half = lane >> 5;
  const int my_row = rw + qcol;
  const bool row_valid = my_row < q_len;
  const int my_pos = my_row + shift;
  const int my_lo = a.window_left < 0 ? 0 : max(0, my_pos - a.window_left);
  const int my_hi = min(my_pos, L - 1);
  // wave key range
  const int w_rows_last = min(rw + 31, q_len - 1);
  const bool wave_active = rw < q_len;
  const int wk_hi = min(w_rows_last + shift, L - 1);
  const int wk_lo = a.window_left < 0 ? 0 : max(0, rw + shift - a.window_left);

  // Q operand (B of the score product): lane holds Q[row][16kk + 8*half .. +8]
  bf16x8_t qop[KD];
  {
    const bf16_t *qrow = (const bf16_t *)a.q + ((size_t)(q0 + (row_valid ? my_row : 0)) * a.hq + head) * D;
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
      bf16x8_t v = *(const bf16x8_t *)(qrow + 16 * kk + 8 * half);
      qop[kk] = row_valid ? v : bf16x8_t{};
    }
  }

  const float qk_scale = a.softmax_scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16_t{};

  Loader<D, P, FP8, NT> ld;
  const int t_first = kmin_wg / BN, t_last = kmax_wg / BN;
  ld.load(a, pt, t_first * BN, L, g, tid);

  for (int t = t_first; t <= t_last; ++t) {
    const int tile_base = t * BN;
    __syncthreads();
    ld.store(sk, sv, sks, svs, tile_base, L, tid);
    __syncthreads();
    if (t < t_last) ld.load(a, pt, (t + 1) * BN, L, g, tid);

    if (!wave_active || tile_base > wk_hi || tile_base + BN - 1 < wk_lo) continue;

    // ---- scores S^T for two 32-key subtiles
    f32x16_t sacc[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      sacc[st] = f32x16_t{};
      const int key = 32 * st + perm_key(qcol);        // A row = lane % 32
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) {
        const int slot = 2 * kk + half;
        const bf16x8_t kop = *(const bf16x8_t *)(sk + key * D + 8 * swz<D * 2>(key, slot));
        sacc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[kk], sacc[st], 0, 0, 0);
      }
    }
    // element v of subtile st holds key tile_base + 32st + perm_key(rho),
    // rho = 8*(v/4) + 4*half + v%4
    float x[32];
    const bool need_mask = tile_base + BN - 1 > rw + shift || tile_base + BN > L ||
                           (a.window_left >= 0 && tile_base < w_rows_last + shift - a.window_left) ||
                           !row_valid || rw + 31 >= q_len;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float xv = sacc[st][v] * qk_scale;
        if (FP8) {
          const int key = 32 * st + perm_key(8 * (v >> 2) + 4 * half + (v & 3));
          xv *= sks[key];
        }
        x[16 * st + v] = xv;
      }
    if (need_mask) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = tile_base + 32 * st + perm_key(8 * (v >> 2) + 4 * half + (v & 3));
          if (!row_valid || key < my_lo || key > my_hi) x[16 * st + v] = -INFINITY;
        }
    }
    float tmax = x[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) tmax = fmaxf(tmax, x[i]);
    tmax = fmaxf(tmax, shfl_xor_f32(tmax, 32));
    // lazy rescale: keep the used maximum unless the new one exceeds it by 8
    const bool grow = tmax > m_run + 8.f || (m_run == -INFINITY && tmax != -INFINITY);
    if (__any(grow)) {
      const float m_new = grow ? tmax : m_run;
      const float corr = (m_run == -INFINITY || !grow) ? (grow ? 0.f : 1.f) : fast_exp2(m_run - m_new);
      l_run *= corr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= corr;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float p[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) p[i] = fast_exp2(x[i] - m_use);
    if (FP8) {
#pragma unroll
      for (int i = 0; i < 32; ++i) l_run += p[i];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = 32 * st + perm_key(8 * (v >> 2) + 4 * half + (v & 3));
          p[16 * st + v] *= svs[key];
        }
    } else {
      // the normaliser sums the probabilities as the P.V product sees them
      // (rounded to bf16), so the weights stay self-consistent: a dominant
      // key reproduces its value row exactly even when p is up to 2^8
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        p[i] = (float)(bf16_t)p[i];
        l_run += p[i];
      }
    }
    // ---- O^T += V^T P^T over four 16-key chunks
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8_t pop;
#pragma unroll
      for (int e = 0; e < 8; ++e) pop[e] = (bf16_t)p[16 * (c >> 1) + 8 * (c & 1) + e];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 32 * dt + qcol;                  // A row = lane % 32
        const int slot = 2 * c + half;                 // keys 16c + 8*half ..
        const bf16x8_t vop = *(const bf16x8_t *)(sv + d * BN + 8 * swz<BN * 2>(d, slot));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop, o[dt], 0, 0, 0);
      }
    }
  }

  if (!wave_active) return;
  l_run += shfl_xor_f32(l_run, 32);
  if (!row_valid) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  bf16_t *orow = (bf16_t *)a.out + ((size_t)(q0 + my_row) * a.hq + head) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // values v = 4j..4j+3 are dims 32dt + 8j + 4*half + 0..3
      bf16x4_t pk;
#pragma unroll
      for (int r = 0; r < 4; ++r) pk[r] = (bf16_t)(o[dt][4 * j + r] * inv);
      *(bf16x4_t *)(orow + 32 * dt + 8 * j + 4 * half) = pk;
    }
  if (a.lse && half == 0)
    a.lse[(size_t)(q0 + my_row) * a.hq + head] = l_run > 0.f ? (m_run + fast_log2(l_run)) * kLn2 : -INFINITY;
}

template <int D, int P, bool FP8>
hipError_t launch_cfg(const AttnArgs &a, hipStream_t stream) {
  constexpr int NWAVES = D == 256 ? 4 : 8;
  const int hkv = a.cache.num_kv_heads;
  const int G = a.hq / hkv;
  int GW = 1;                                  // heads per work-group: power of 2 dividing G
  while (GW * 2 <= NWAVES && G % (GW * 2) == 0) GW *= 2;
  const int BM = 32 * (NWAVES / GW);
  const int max_qb = (a.max_q_len + BM - 1) / BM;
  const long long grid = (long long)max_qb * a.num_seqs * hkv * (G / GW);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const size_t lds = (size_t)2 * BN * D * sizeof(bf16_t) + (FP8 ? 2 * BN * sizeof(float) : 0);
  auto kern = attn_prefill_kernel<D, P, FP8, NWAVES>;
  if (lds > 65536) {
    static bool attr_set = false;     // idempotent; a race only repeats the call
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
  }
  kern<<<(unsigned)grid, NWAVES * 64, lds, stream>>>(a, GW, max_qb);
  return hipGetLastError();
}

template <int D, int P>
hipError_t launch_dp(const AttnArgs &a, hipStream_t stream) {
  if (a.cache.dtype == NK_E4M3) return launch_cfg<D, P, true>(a, stream);
  return launch_cfg<D, P, false>(a, stream);
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
