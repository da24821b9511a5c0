// Split-KV decode attention: single-query rows over a paged bf16 or e4m3
// cache, grouped-query heads sharing every K/V load.
//
// What it computes: NumKong matrix-kernels page, attention_packed, for a
// segment with one query row (it sits at position kv_len - 1 and sees every
// key, or the last window_left + 1 keys); aria_kernel `attention` (single
// query step against the KV cache, GQA layout).  The keys are cut into
// chunks; each chunk's state is merged by log-sum-exp as on the Algenta
// page's flash-attention walkthrough (running max, rescale by
// exp(old - new)).  float8 caches: the stored code times its per-(token,
// head) scale is the value -- the K scale multiplies the score, the V scale
// the probability.
//
// Design (HBM-bound; one work-group per (sequence, kv head, chunk)):
//   * a chunk is walked in steps of 32 keys (two 16-token pages or one
//     32-token page); the NW waves of the group take steps round-robin and
//     prefetch their next step while computing the current one;
//   * scores S^T = K Q^T and the update O^T += V^T P^T run on
//     v_mfma_f32_16x16x32_bf16: 16 keys x 16 query heads per tile, the query
//     heads of one KV head on the N axis (unused columns are zero);
//   * K pages are [token][dim] and V pages [dim][token], so both MFMA
//     operands are plain 16-byte (bf16) or 8-byte (e4m3) loads straight from
//     HBM into registers, in the lane order the instruction wants: the K rows
//     are loaded in a permuted key order that makes the score tile's lane
//     layout coincide with the P^T operand layout, so no data moves between
//     lanes except the max reduction;
//   * e4m3 codes are widened to bf16 exactly in registers;
//   * at the end the waves combine their (max, sum, O) through LDS and write
//     either the final row (one chunk) or a float32 partial for the merge.

#include "common.h"
#include "internal.h"

namespace nk {
namespace {

template <int D, bool FP8>
struct Step {
  static constexpr int KK = D / 32;   // k-steps of the score MFMA
  static constexpr int DT = D / 16;   // d-tiles of the output MFMA
  using KVec = typename std::conditional<FP8, u32x2_t, bf16x8_t>::type;
  KVec k[2][KK];
  KVec v[DT];
  f32x4_t ks[2];   // fp8: K scales of this lane's keys (tile m)
  f32x4_t vs[2];   // fp8: V scales of keys 8h..8h+3, 8h+4..8h+7
};

template <int D, int P, bool FP8>
NK_DEVICE void load_step(Step<D, FP8> &st, const AttnArgs &a, const int32_t *pt, int kb, int last_page,
                         int g, int lane) {
  const int hkv = a.cache.num_kv_heads;
  const int lg = lane >> 4;         // lane group 0..3
  const int lr = lane & 15;
  int pg[2];
  if (P == 16) {
    pg[0] = pt[kb / 16];
    pg[1] = pt[min(kb / 16 + 1, last_page)];
  } else {
    pg[0] = pg[1] = pt[kb / 32];
  }
  constexpr int esz = FP8 ? 1 : 2;
  const uint8_t *kbase = (const uint8_t *)a.cache.k_pages;
  const uint8_t *vbase = (const uint8_t *)a.cache.v_pages;
  // K rows: score-tile row rho = lr holds key 8*(rho/4) + 4m + rho%4
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int kappa = 8 * (lr >> 2) + 4 * m + (lr & 3);
    const int page = pg[kappa / P];
    const size_t row = ((size_t)page * hkv + g) * P + (kappa % P);
#pragma unroll
    for (int kk = 0; kk < Step<D, FP8>::KK; ++kk) {
      const int d0 = 32 * kk + 8 * lg;
      st.k[m][kk] = *(const typename Step<D, FP8>::KVec *)(kbase + (row * D + d0) * esz);
    }
  }
  // V columns: lane holds keys 8*lg .. 8*lg+7 of dim 16*dt + lr
  {
    const int kappa0 = 8 * lg;
    const int page = pg[kappa0 / P];
    const size_t base = ((size_t)page * hkv + g) * D;
#pragma unroll
    for (int dt = 0; dt < Step<D, FP8>::DT; ++dt) {
      const int d = 16 * dt + lr;
      st.v[dt] = *(const typename Step<D, FP8>::KVec *)(vbase + ((base + d) * P + (kappa0 % P)) * esz);
    }
  }
  if (FP8) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int kappa = 8 * lg + 4 * m;
      const size_t idx = ((size_t)pg[kappa / P] * hkv + g) * P + (kappa % P);
      st.ks[m] = *(const f32x4_t *)(a.cache.k_scales + idx);
      st.vs[m] = *(const f32x4_t *)(a.cache.v_scales + idx);
    }
  }
}

template <int D, bool FP8>
NK_DEVICE bf16x8_t as_bf16x8(const typename Step<D, FP8>::KVec &x) {
  if constexpr (FP8) return fp8x8_to_bf16x8(x);
  else return x;
}

template <int D, int P, bool FP8, int NW>
__global__ void __launch_bounds__(NW * 64) attn_decode_kernel(AttnArgs a) {
  static_assert(NW >= 2, "the waves combine through LDS");
  using St = Step<D, FP8>;
  constexpr int KK = St::KK, DT = St::DT;
  extern __shared__ float smem[];           // [NW][DT][4][64] O, then m[NW][16], l[NW][16]

  const int B = a.num_seqs;
  const int s = blockIdx.x % B;
  const int c = blockIdx.x / B;
  const int g = blockIdx.y;
  const int hb = blockIdx.z;                // block of 16 query heads
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int hkv = a.cache.num_kv_heads;
  const int G = a.hq / hkv;

  const int q0 = a.q_offsets[s];
  if (a.q_offsets[s + 1] - q0 != 1) return;
  const int L = a.kv_lens[s];
  const int hi = L - 1;
  const int lo = a.window_left < 0 ? 0 : max(0, hi - a.window_left);
  const int c0 = (lo / 32) * 32;                         // chunks are aligned to 32 keys
  // (clamped to the grid: a kv_len above max_kv_len violates the precondition,
  // and its row then covers only the first max_chunks chunks)
  const int n_chunks = L > 0 ? min((hi + 1 - c0 + a.split_tokens - 1) / a.split_tokens, a.max_chunks) : 1;
  if (c >= n_chunks) return;
  const int cs = c0 + c * a.split_tokens;
  const int ce = min(cs + a.split_tokens, hi + 1);
  const int vs_lo = max(cs, lo);                         // valid keys [vs_lo, ce)
  const int nsteps = L > 0 ? (ce - cs + 31) / 32 : 0;
  const int last_page = L > 0 ? hi / P : 0;
  const int32_t *pt = a.cache.page_table + (size_t)s * a.cache.page_table_stride;

  // Q operand: column n = lane%16 is query head g*G + hb*16 + n
  const int n = lane & 15;
  const int lg = lane >> 4;
  const int hq_local = hb * 16 + n;
  const bool col_valid = hq_local < G;
  bf16x8_t qop[KK];
  {
    const bf16_t *qrow = (const bf16_t *)a.q + ((size_t)q0 * a.hq + g * G + (col_valid ? hq_local : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      bf16x8_t v = *(const bf16x8_t *)(qrow + 32 * kk + 8 * lg);
      qop[kk] = col_valid ? v : bf16x8_t{};
    }
  }

  const float qk_scale = a.softmax_scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const St &st, int kb) {
    f32x4_t sacc[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      sacc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        sacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8<D, FP8>(st.k[m][kk]), qop[kk], sacc[m], 0, 0, 0);
    }
    // lane holds keys kb + 8*lg + 4m + r  (m = 0,1; r = 0..3)
    float x[8];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = sacc[m][r] * qk_scale;
        if (FP8) v *= st.ks[m][r];
        x[4 * m + r] = v;
      }
    const bool edge = kb < vs_lo || kb + 32 > ce;
    if (edge) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int key = kb + 8 * lg + i;
        if (key < vs_lo || key >= ce) x[i] = -INFINITY;
      }
    }
    float tmax = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, x[i]);
    tmax = fmaxf(tmax, shfl_xor_f32(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor_f32(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    if (__any(m_new > m_run)) {
      const float corr = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
      l_run *= corr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= corr;
    }
    m_run = m_new;
    float p[8];
    const bool live = m_new != -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = live ? fast_exp2(x[i] - m_new) : 0.f;
      l_run += p[i];
    }
    if (FP8) {
#pragma unroll
      for (int r = 0; r < 4; ++r) { p[r] *= st.vs[0][r]; p[4 + r] *= st.vs[1][r]; }
      if (edge) {   // a masked key's scale may be anything (unwritten slot)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int key = kb + 8 * lg + i;
          if (key < vs_lo || key >= ce) p[i] = 0.f;
        }
      }
    }
    bf16x8_t pop;
#pragma unroll
    for (int i = 0; i < 8; ++i) pop[i] = (bf16_t)p[i];
    if (edge) {
      // masked keys may hold anything (unwritten slots): zero their V
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        bf16x8_t vv = as_bf16x8<D, FP8>(st.v[dt]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int key = kb + 8 * lg + i;
          if (key < vs_lo || key >= ce) vv[i] = (bf16_t)0.f;
        }
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pop, o[dt], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8<D, FP8>(st.v[dt]), pop, o[dt], 0, 0, 0);
    }
  };

  {
    St bufA, bufB;
    int k = w;
    if (k < nsteps) load_step<D, P, FP8>(bufA, a, pt, cs + 32 * k, last_page, g, lane);
    while (k < nsteps) {
      const int k1 = k + NW;
      if (k1 < nsteps) load_step<D, P, FP8>(bufB, a, pt, cs + 32 * k1, last_page, g, lane);
      compute(bufA, cs + 32 * k);
      if (k1 >= nsteps) break;
      const int k2 = k1 + NW;
      if (k2 < nsteps) load_step<D, P, FP8>(bufA, a, pt, cs + 32 * k2, last_page, g, lane);
      compute(bufB, cs + 32 * k1);
      k = k2;
    }
  }

  // per-column sum over the four lane groups
  l_run += shfl_xor_f32(l_run, 16);
  l_run += shfl_xor_f32(l_run, 32);

  float *sm_o = smem;
  float *sm_m = smem + NW * DT * 4 * 64;
  float *sm_l = sm_m + NW * 16;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm_o[((w * DT + dt) * 4 + r) * 64 + lane] = o[dt][r];
  if (lane < 16) { sm_m[w * 16 + lane] = m_run; sm_l[w * 16 + lane] = l_run; }
  __syncthreads();

  const int G_blk = min(16, G - hb * 16);
  const bool single = n_chunks == 1;
  const size_t slot = (size_t)s * a.max_chunks + c;
  for (int e = threadIdx.x; e < G_blk * D; e += NW * 64) {
    const int col = e / D, d = e % D;
    const int src_lane = col + 16 * ((d & 15) >> 2);
    const int dt = d >> 4, r = d & 3;
    float M = -INFINITY;
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm_m[ww * 16 + col]);
    float num = 0.f, den = 0.f;
    for (int ww = 0; ww < NW; ++ww) {
      const float mw = sm_m[ww * 16 + col];
      const float f = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
      num += f * sm_o[((ww * DT + dt) * 4 + r) * 64 + src_lane];
      den += f * sm_l[ww * 16 + col];
    }
    const float val = den > 0.f ? num / den : 0.f;
    const float lse = den > 0.f ? (M + fast_log2(den)) * kLn2 : -INFINITY;
    const int head = g * G + hb * 16 + col;
    if (single) {
      ((bf16_t *)a.out)[((size_t)q0 * a.hq + head) * D + d] = (bf16_t)val;
      if (a.lse && d == 0) a.lse[(size_t)q0 * a.hq + head] = lse;
    } else {
      a.part_out[(slot * a.hq + head) * D + d] = val;
      if (d == 0) a.part_lse[slot * a.hq + head] = lse;
    }
  }
}

template <int D, int P, bool FP8, int NW>
hipError_t launch_cfg(const AttnArgs &a, hipStream_t stream) {
  const int hkv = a.cache.num_kv_heads;
  const int G = a.hq / hkv;
  dim3 grid((unsigned)(a.num_seqs * a.max_chunks), (unsigned)hkv, (unsigned)((G + 15) / 16));
  const size_t lds = (size_t)(NW * (D / 16) * 4 * 64 + 2 * NW * 16) * sizeof(float);
  attn_decode_kernel<D, P, FP8, NW><<<grid, NW * 64, lds, stream>>>(a);
  return hipGetLastError();
}

// Waves per work-group: 4, or 2 for D = 256 (the LDS combine buffer holds
// NW * D * 64 bytes and must stay within 64 KiB).
template <int D, int P>
hipError_t launch_dp(const AttnArgs &a, hipStream_t stream) {
  constexpr int NW = D == 256 ? 2 : 4;
  if (a.cache.dtype == NK_E4M3) return launch_cfg<D, P, true, NW>(a, stream);
  return launch_cfg<D, P, false, NW>(a, stream);
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
