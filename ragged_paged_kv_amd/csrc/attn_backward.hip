// Gradients of ragged paged attention with respect to Q, K and V.
//
// What it computes: NumKong matrix-kernels page, attention_packed_gradients
// -- from the forward's output O, its gradient dO and its log-sum-exp, the
// query, key and value gradients under the same band (and sink keys) as the
// forward.  With scores s_ij = scale * q_i.k_j over the keys row i sees and
// P_ij = exp(s_ij - lse_i):
//   dV_j  = sum_i P_ij dO_i
//   dS_ij = P_ij (dO_i.v_j - dO_i.O_i)
//   dQ_i  = scale * sum_j dS_ij k_j
//   dK_j  = scale * sum_i dS_ij q_i
// summed over the query heads that share a KV head (GQA).  This is the
// softmax's Jacobian applied row by row (the running-state identities of the
// Algenta page's flash-attention walkthrough give the same P from lse).
//
// Design of the float32 path (and of bf16 at head dims other than 64 and
// 128; the MFMA path below takes bf16 at 64 and 128): two VALU kernels.
//   * dQ: one wave per (query row, up to 4 query heads of one KV head); lanes
//     take 64 visible keys at a time, each lane loading its key's K and V once
//     and computing q.k and dO.v for every head, then lanes over head
//     dimensions accumulate dS_j k_j;
//   * dK/dV: one wave per (8 consecutive keys of a segment, KV head); lanes
//     take 64 (row, head) pairs of the rows that see one of the keys, each
//     loading the pair's rows once and computing dO.O and, per key, q.k and
//     dO.v, then lanes over dimensions accumulate P dO and dS q per key.
// Every key of a segment gets its rows written (zeros when no row sees it).
// Scores are recomputed from the cache, as the forward computes them.

#include "common.h"
#include "internal.h"

namespace nk {
namespace {

template <typename T> NK_DEVICE float ld(const T *p) { return (float)*p; }

// 8 consecutive elements (16-byte aligned) as float32: one 16-byte load for
// bf16, two for float32
NK_DEVICE void ld8(const bf16_t *p, float *x) {
  const bf16x8_t v = *(const bf16x8_t *)p;
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
}
NK_DEVICE void ld8(const float *p, float *x) {
  const f32x4_t a = *(const f32x4_t *)p, b = *(const f32x4_t *)(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
}

// Element (dim d, key t of its page) of a K or V page-head block (include/nk.h
// layouts; NV = 4 / element bytes for V's 16-byte runs).
template <typename T> NK_DEVICE size_t k_elem(int d, int t, int P) {
  return ((size_t)(d >> 5) * P + t) * 32 + (d & 31);
}
template <typename T> NK_DEVICE size_t v_elem(int d, int t, int D) {
  constexpr int NV = 4 / (int)sizeof(T);
  return ((size_t)(t >> 4) * (D / (16 * NV)) + ((d >> 4) / NV)) * (64 * 4 * NV) +
         (size_t)(16 * ((t & 15) >> 2) + (d & 15)) * (4 * NV) + ((d >> 4) % NV) * 4 + (t & 3);
}

// Keys a row at position p sees: [lo, hi] plus the sink keys 0..n_sink-1
// left of lo, walked as one list (entry v: key v if v < n_sink, else
// lo + v - n_sink).
struct RowKeys {
  int lo, hi, n_sink, n;
  NK_DEVICE int key(int v) const { return v < n_sink ? v : lo + v - n_sink; }
};
NK_DEVICE RowKeys row_keys(const BackwardArgs &a, int p, int L) {
  RowKeys r;
  r.hi = band_hi(p, L, a.window_right);
  r.lo = band_lo(p, a.window_left);
  const int sinks = a.window_left < 0 ? 0 : a.sink_keys;
  r.n_sink = max(0, min(sinks, min(r.lo, r.hi + 1)));
  r.n = r.n_sink + max(0, r.hi - r.lo + 1);
  return r;
}

// dQ of one query row for HB query heads of one KV head per wave: each
// visible key's K and V are loaded once for the HB heads.
template <typename T, int HB>
__global__ void __launch_bounds__(64) attn_dq_kernel(BackwardArgs a) {
  const int t = blockIdx.x, h0 = blockIdx.y * HB, lane = threadIdx.x;
  const int D = a.cache.head_dim, P = a.cache.page_size, hkv = a.cache.num_kv_heads;
  const int g = h0 / (a.hq / hkv);
  __shared__ float qs[HB][256], dos[HB][256];
  const int s = find_segment(a.q_offsets, a.num_seqs, t);
  const int q0 = a.q_offsets[s];
  const int q_len = a.q_offsets[s + 1] - q0;
  const int L = a.kv_lens[s];
  const RowKeys rk = row_keys(a, (t - q0) + L - q_len, L);
  float di[HB], lse[HB];                            // dO.O and the forward's lse of each head
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const size_t row = (size_t)t * a.hq + h0 + hb;
    float x = 0.f;
    for (int d = lane; d < D; d += kWave) {
      qs[hb][d] = ld((const T *)a.q + row * D + d);
      dos[hb][d] = ld((const T *)a.dout + row * D + d);
      x += dos[hb][d] * ld((const T *)a.out + row * D + d);
    }
    di[hb] = wave_sum(x);
    lse[hb] = a.lse[row];
  }
  __syncthreads();
  const T *kp = (const T *)a.cache.k_pages;
  const T *vp = (const T *)a.cache.v_pages;
  const int32_t *pt = a.cache.page_table + (size_t)s * a.cache.page_table_stride;
  float dq[HB][4];                                  // dims lane, lane+64, ...
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int r = 0; r < 4; ++r) dq[hb][r] = 0.f;
  for (int base = 0; base < rk.n; base += kWave) {
    const bool valid = base + lane < rk.n;
    float ds[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) ds[hb] = 0.f;
    if (valid) {
      const int key = rk.key(base + lane);
      const size_t blk = ((size_t)pt[key / P] * hkv + g) * P * D;
      float qk[HB], dv[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) qk[hb] = dv[hb] = 0.f;
      for (int d0 = 0; d0 < D; d0 += 8) {            // a key's 8 dims of one block are contiguous
        float kx[8];
        ld8(kp + blk + k_elem<T>(d0, key % P, P), kx);
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) qk[hb] = fmaf(qs[hb][d0 + e], kx[e], qk[hb]);
      }
      for (int d = 0; d < D; ++d) {
        const float vd = ld(vp + blk + v_elem<T>(d, key % P, D));
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) dv[hb] = fmaf(dos[hb][d], vd, dv[hb]);
      }
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const float p = expf(a.softmax_scale * qk[hb] - lse[hb]);
        ds[hb] = p * (dv[hb] - di[hb]);
      }
    }
    const int nk = min(kWave, rk.n - base);
    for (int i = 0; i < nk; ++i) {
      float dsi[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) dsi[hb] = __shfl(ds[hb], i, kWave);
      const int key = rk.key(base + i);
      const size_t blk = ((size_t)pt[key / P] * hkv + g) * P * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = lane + r * kWave;
        if (d < D) {
          const float kd = ld(kp + blk + k_elem<T>(d, key % P, P));
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) dq[hb][r] = fmaf(dsi[hb], kd, dq[hb][r]);
        }
      }
    }
  }
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const size_t row = (size_t)t * a.hq + h0 + hb;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = lane + r * kWave;
      if (d < D) a.dq[row * D + d] = a.softmax_scale * dq[hb][r];
    }
  }
}

// dK/dV of KB consecutive keys of one segment and KV head per wave: each
// (row, head) pair's q, dO and O rows are loaded once for all KB keys.
constexpr int kDkvKeys = 8;

template <typename T>
__global__ void __launch_bounds__(64) attn_dkv_kernel(BackwardArgs a, int blocks_per_seq) {
  constexpr int KB = kDkvKeys;
  const int s = blockIdx.x / blocks_per_seq, j0 = (blockIdx.x % blocks_per_seq) * KB, g = blockIdx.y;
  const int lane = threadIdx.x;
  const int D = a.cache.head_dim, P = a.cache.page_size, hkv = a.cache.num_kv_heads;
  const int G = a.hq / hkv;
  const int L = a.kv_lens[s];
  if (j0 >= L) return;
  const int nkeys = min(KB, L - j0);
  __shared__ float ks[KB][256], vs[KB][256];
  const int32_t *pt = a.cache.page_table + (size_t)s * a.cache.page_table_stride;
  for (int kk = 0; kk < KB; ++kk) {
    const int j = j0 + min(kk, nkeys - 1);       // past the segment: a copy of its last key, never written
    const size_t blk = ((size_t)pt[j / P] * hkv + g) * P * D;
    for (int d = lane; d < D; d += kWave) {
      ks[kk][d] = ld((const T *)a.cache.k_pages + blk + k_elem<T>(d, j % P, P));
      vs[kk][d] = ld((const T *)a.cache.v_pages + blk + v_elem<T>(d, j % P, D));
    }
  }
  __syncthreads();
  const int q0 = a.q_offsets[s];
  const int q_len = a.q_offsets[s + 1] - q0;
  const int shift = L - q_len;
  const int jl = j0 + nkeys - 1;
  // rows that may see a key of the block: hi >= j0 from i_min on, lo <= jl
  // up to i_max (no upper limit when a key of the block is a sink key); each
  // (pair, key) is checked exactly below
  const int i_min = a.window_right < 0 ? 0 : (int)max(0LL, (long long)j0 - a.window_right - shift);
  const bool sink = a.window_left >= 0 && j0 < a.sink_keys;
  const int i_max = (a.window_left < 0 || sink) ? q_len - 1
                                                 : (int)min((long long)q_len - 1, (long long)jl + a.window_left - shift);
  const int n_pairs = max(0, i_max - i_min + 1) * G;
  float dk[KB][4], dv[KB][4];
#pragma unroll
  for (int kk = 0; kk < KB; ++kk)
#pragma unroll
    for (int r = 0; r < 4; ++r) dk[kk][r] = dv[kk][r] = 0.f;
  for (int base = 0; base < n_pairs; base += kWave) {
    const int e = base + lane;
    float p[KB], ds[KB];
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) p[kk] = ds[kk] = 0.f;
    if (e < n_pairs) {
      const int i = i_min + e / G, h = g * G + e % G;
      const RowKeys rk = row_keys(a, i + shift, L);
      const size_t row = (size_t)(q0 + i) * a.hq + h;
      const T *q = (const T *)a.q + row * D, *dout = (const T *)a.dout + row * D, *o = (const T *)a.out + row * D;
      float qk[KB], dov[KB], doo = 0.f;
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) qk[kk] = dov[kk] = 0.f;
      for (int d0 = 0; d0 < D; d0 += 8) {
        float qx[8], dx[8], ox[8];
        ld8(q + d0, qx);
        ld8(dout + d0, dx);
        ld8(o + d0, ox);
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          doo = fmaf(dx[x], ox[x], doo);
#pragma unroll
          for (int kk = 0; kk < KB; ++kk) {
            qk[kk] = fmaf(qx[x], ks[kk][d0 + x], qk[kk]);
            dov[kk] = fmaf(dx[x], vs[kk][d0 + x], dov[kk]);
          }
        }
      }
      const float lse = a.lse[row];
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        const int j = j0 + kk;
        const bool sees = kk < nkeys && j <= rk.hi && (j >= rk.lo || j < rk.n_sink);
        if (sees) {
          p[kk] = expf(a.softmax_scale * qk[kk] - lse);
          ds[kk] = p[kk] * (dov[kk] - doo);
        }
      }
    }
    const int np = min(kWave, n_pairs - base);
    for (int u = 0; u < np; ++u) {
      float pu[KB], dsu[KB];
      bool any = false;
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        pu[kk] = __shfl(p[kk], u, kWave);
        dsu[kk] = __shfl(ds[kk], u, kWave);
        any |= pu[kk] != 0.f || dsu[kk] != 0.f;
      }
      if (!any) continue;                              // wave-uniform (shuffled values)
      const int i = i_min + (base + u) / G, h = g * G + (base + u) % G;
      const size_t row = (size_t)(q0 + i) * a.hq + h;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = lane + r * kWave;
        if (d < D) {
          const float dd = ld((const T *)a.dout + row * D + d), qd = ld((const T *)a.q + row * D + d);
#pragma unroll
          for (int kk = 0; kk < KB; ++kk) {
            dv[kk][r] = fmaf(pu[kk], dd, dv[kk][r]);
            dk[kk][r] = fmaf(dsu[kk], qd, dk[kk][r]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int kk = 0; kk < KB; ++kk) {
    if (kk >= nkeys) break;
    const size_t orow = ((size_t)a.key_offsets[s] + j0 + kk) * hkv + g;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = lane + r * kWave;
      if (d < D) {
        a.dk[orow * D + d] = a.softmax_scale * dk[kk][r];
        a.dv[orow * D + d] = dv[kk][r];
      }
    }
  }
}

// ---------------------------------------------------------------- MFMA path
// bf16 queries and cache, head_dim 64 or 128: the same gradients on
// v_mfma_f32_32x32x16_bf16 (32 x 32 tiles, k = 16), P and dS rounded to bf16
// for their products, float32 accumulation.
//
// Two kernels, each recomputing the scores and dP = dO V^T of its tiles:
//   * dK/dV: a work-group of 4 waves owns 128 keys of one KV head (32 per
//     wave, K and V held as MFMA operands) and walks the 32-row query tiles
//     of every query head of the group that can see them.  Per tile the
//     waves stage Q and dO row-major in LDS with the rows' log-sum-exp and
//     dO.O; the score products read rows of these tiles, dV = P^T dO and
//     dK = dS^T Q (contraction over rows) read down their columns with
//     transposing LDS reads;
//   * dQ: a work-group of 4 waves owns 32-row query tiles of up to 4 query
//     heads of one KV head (Q and dO held as operands) and walks the 32-key
//     tiles the rows see, staging K and V row-major (dQ = dS K reads down
//     K's columns).
// Both pipelines load the next tile's global data into registers while the
// current one is computed (LDS double buffered, one barrier per tile).
// Row (dK/dV) or key (dQ) order inside a tile is permuted (bits 2 and 3 of
// the index swapped) for the score products, which makes their output lane
// layout the A operand layout of the next product: P and dS never move
// between lanes.  In a 32 x 32 output lane l holds column l % 32 and rows
// 8 (v / 4) + 4 (l / 32) + v % 4 (v < 16); under the permutation entry v is
// row 16 (v / 8) + 8 (l / 32) + v % 8, i.e. entries 8 s .. 8 s + 7 are the
// eight consecutive rows of k-step s.

NK_DEVICE constexpr int bperm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

NK_DEVICE uint32_t pack2_bf16(float lo, float hi) {
  bf16x2_t v = {(bf16_t)lo, (bf16_t)hi};
  return __builtin_bit_cast(uint32_t, v);
}

NK_DEVICE bf16x8_t pack8(const float *x) {
  return __builtin_bit_cast(bf16x8_t, u32x4_t{pack2_bf16(x[0], x[1]), pack2_bf16(x[2], x[3]),
                                              pack2_bf16(x[4], x[5]), pack2_bf16(x[6], x[7])});
}

// Four 16-bit values down a column of a row-major LDS tile: within each
// 16-lane group, ds_read_b64_tr_b16 hands lane 4a + b element b of the 8
// bytes addressed by lane 4e + a, as its element e (measured on gfx950).  So
// if lane j of the group addresses row k0 + j / 4, columns c0 + 4 (j % 4)
// .. + 3, lane i receives rows k0 .. k0 + 3 of column c0 + i; lds_col8 reads
// rows k0 .. k0 + 7 (the second half `row_bytes` x 4 further on).
typedef short i16x4_t __attribute__((ext_vector_type(4)));
NK_DEVICE bf16x8_t lds_col8(const uint8_t *p, int row_bytes) {
  typedef __attribute__((address_space(3))) i16x4_t *lds_ptr;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)p);
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(p + 4 * row_bytes));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int D>
struct BwdTile {
  // bytes per row-major row in LDS: 2D + 48 puts 16 consecutive rows on
  // distinct banks for 16-byte row reads and 4 rows x 32 bytes apart for the
  // column reads above
  static constexpr int RM = 2 * D + 48;
  static constexpr int KD = D / 16;         // k-steps over head dims
  static constexpr int DC = D / 32;         // 32-dim output tiles
  static constexpr int CH = 32 * D / 8;     // 16-byte chunks of a 32 x D tile
  static constexpr int PER = CH / 256;      // of them per thread (4 waves)
  static_assert(CH % 256 == 0, "tile chunks must divide over the work-group");
};

// ---- dK / dV
template <int D>
struct DkvLds {
  using B = BwdTile<D>;
  static constexpr int Q = 0, DO = 32 * B::RM, LSE = 64 * B::RM, DI = LSE + 128, SIZE = DI + 128;
  static constexpr int TOTAL = 2 * SIZE;
};

template <int D>
__global__ void __launch_bounds__(256) attn_dkv_mfma_kernel(BackwardArgs a, int tiles_per_seq, int HC) {
  using B = BwdTile<D>;
  using LY = DkvLds<D>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];      // two buffers of LY::SIZE
  // KV head fastest (consecutive work-groups go to different XCDs, so each
  // XCD's L2 holds the rows of its own heads), then head chunk, segment and
  // key tile: a causal segment's first key tiles carry the most rows, so
  // every segment's heaviest work-groups are dispatched first.  With HC > 1
  // the G query heads of a KV head are split into HC chunks on separate
  // work-groups, which add their dK/dV into the (zeroed) outputs.
  const int nh = a.cache.num_kv_heads;
  const int g = blockIdx.x % nh, rest0 = blockIdx.x / nh;
  const int hc = rest0 % HC, rest = rest0 / HC;
  const int s = rest % a.num_seqs, kt0 = (rest / a.num_seqs) * 128;
  const int L = a.kv_lens[s];
  if (kt0 >= L) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int hkv = a.cache.num_kv_heads, G = a.hq / hkv, P = a.cache.page_size;
  const int q0 = a.q_offsets[s];
  const int q_len = a.q_offsets[s + 1] - q0;
  const int shift = L - q_len;
  const int32_t *pt = a.cache.page_table + (size_t)s * a.cache.page_table_stride;

  // this wave's 32 keys as operands: K (B of S = Q K^T: lane = key l32,
  // dims 16 kk + 8 h ..) and V (B of dP = dO V^T); keys past the segment are
  // zeros
  const int k0 = kt0 + 32 * w;
  const int key = k0 + l32;
  bf16x8_t kop[B::KD], vop[B::KD];
  {
    const bool kv = key < L;
    const size_t blk = ((size_t)pt[min(key, L - 1) / P] * hkv + g) * P * D;
    const bf16_t *kp = (const bf16_t *)a.cache.k_pages + blk;
    const bf16_t *vp = (const bf16_t *)a.cache.v_pages + blk;
    const int t = min(key, L - 1) % P;
#pragma unroll
    for (int kk = 0; kk < B::KD; ++kk) {
      const int d0 = 16 * kk + 8 * h;
      bf16x8_t x = *(const bf16x8_t *)(kp + k_elem<bf16_t>(d0, t, P));
      bf16x8_t y;
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = vp[v_elem<bf16_t>(d0 + e, t, D)];
      if (!kv) { x = bf16x8_t{}; y = bf16x8_t{}; }
      kop[kk] = x;
      vop[kk] = y;
    }
  }

  // query rows that may see one of the work-group's keys (each (row, key)
  // checked exactly when a tile straddles the band)
  const int kmax = min(kt0 + 128, L) - 1;
  const int i_min = a.window_right < 0 ? 0 : (int)max(0LL, (long long)kt0 - a.window_right - shift);
  const bool sink = a.window_left >= 0 && kt0 < a.sink_keys;
  const int i_max = (a.window_left < 0 || sink) ? q_len - 1
                                                 : (int)min((long long)q_len - 1, (long long)kmax + a.window_left - shift);
  const int rt0 = i_min / 32, rt1 = i_max < i_min ? rt0 - 1 : i_max / 32;
  const int Gc = G / HC;                        // query heads of this work-group: g G + hc Gc ..
  const int n_pairs = (rt1 - rt0 + 1) * Gc;

  f32x16_t dk[B::DC], dv[B::DC];
#pragma unroll
  for (int c = 0; c < B::DC; ++c) { dk[c] = f32x16_t{}; dv[c] = f32x16_t{}; }
  const float c2 = a.softmax_scale * kLog2e;
  // positions p of the rows that see this lane's key: p >= key - window_right
  // (a row sees keys up to p + window_right), p <= key + window_left (its
  // band starts at p - window_left) unless the key is a sink key, which
  // every row whose band reaches past it sees; none for keys past the segment
  const int sinks = a.window_left < 0 ? 0 : a.sink_keys;
  const int p_min = key >= L ? 1 << 30 : (a.window_right < 0 ? -(1 << 30) : key - a.window_right);
  const int p_max = (a.window_left < 0 || key < sinks) ? (1 << 30) : key + a.window_left;

  // software pipeline over the (row tile, head) pairs: the global loads of
  // pair pr + 1 are in flight while pair pr is computed; LDS is double
  // buffered, so one barrier per pair separates a buffer's writes from its
  // reads (a buffer is rewritten two pairs later, after the next barrier)
  // the loads of pair pr + 1 are in flight while pair pr is computed
  // dO.O of each (row, head) comes precomputed in the dq buffer (rows x
  // heads floats), which the dQ kernel overwrites only after this kernel
  const float *rowdot = a.dq;
  struct Regs { bf16x8_t q[B::PER], d[B::PER]; float lse[B::PER], di[B::PER]; };
  Regs R0;
  auto fetch = [&](int pr, Regs &R) {
    bf16x8_t *gq = R.q, *gd = R.d;
    float *glse = R.lse, *gdi = R.di;
    const int r0 = (rt0 + pr / Gc) * 32, head = g * G + hc * Gc + pr % Gc;
#pragma unroll
    for (int i = 0; i < B::PER; ++i) {
      const int c = tid + 256 * i;
      // rows past the segment read its last row (in bounds; their P is zero)
      const int row = min(r0 + c / (D / 8), q_len - 1), d0 = 8 * (c % (D / 8));
      const size_t rh = (size_t)(q0 + row) * a.hq + head;
      gq[i] = *(const bf16x8_t *)((const bf16_t *)a.q + rh * D + d0);
      gd[i] = *(const bf16x8_t *)((const bf16_t *)a.dout + rh * D + d0);
      glse[i] = a.lse[rh];
      gdi[i] = rowdot[rh];
    }
  };
  auto stage = [&](int pr, uint8_t *buf, const Regs &R) {
    const bf16x8_t *gq = R.q, *gd = R.d;
    const float *glse = R.lse, *gdi = R.di;
    const int r0 = (rt0 + pr / Gc) * 32;
#pragma unroll
    for (int i = 0; i < B::PER; ++i) {
      const int c = tid + 256 * i;
      const int r = c / (D / 8), d0 = 8 * (c % (D / 8));
      const int row = r0 + r;
      *(bf16x8_t *)(buf + LY::Q + r * B::RM + 2 * d0) = gq[i];
      *(bf16x8_t *)(buf + LY::DO + r * B::RM + 2 * d0) = gd[i];
      if (c % (D / 8) == 0) {
        ((float *)(buf + LY::DI))[r] = gdi[i];
        // log2-domain lse; rows past the segment get +inf (P = 0)
        ((float *)(buf + LY::LSE))[r] = row < q_len ? glse[i] * kLog2e : INFINITY;
      }
    }
  };

  auto step = [&](int pr, Regs &R) {
    const int r0 = (rt0 + pr / Gc) * 32;
    uint8_t *buf = lds + (pr & 1) * LY::SIZE;
    stage(pr, buf, R);
    __syncthreads();
    if (pr + 1 < n_pairs) fetch(pr + 1, R);

    // ---- S = Q K^T and dP = dO V^T (rows permuted)
    f32x16_t sc = f32x16_t{}, dp = f32x16_t{};
    {
      const uint8_t *qa = buf + LY::Q + bperm(l32) * B::RM + 16 * h;
      const uint8_t *da = buf + LY::DO + bperm(l32) * B::RM + 16 * h;
#pragma unroll
      for (int kk = 0; kk < B::KD; ++kk) {
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8_t *)(qa + 32 * kk), kop[kk], sc, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8_t *)(da + 32 * kk), vop[kk], dp, 0, 0, 0);
      }
    }
    // ---- P and dS: entry v is row 16 (v/8) + 8 h + v % 8 of the tile, key `key`
    float pv[16], dsv[16];
    {
      // the log-sum-exp and dO.O of rows 8 h + rl (rl = 0..7, 16..23) as
      // 16-byte reads
      float lse2[24], dis[24];
      {
        const f32x4_t *l4 = (const f32x4_t *)(buf + LY::LSE), *d4 = (const f32x4_t *)(buf + LY::DI);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int rl0 = 16 * (q4 >> 1) + 4 * (q4 & 1);
          const f32x4_t lv = l4[(rl0 >> 2) + 2 * h], dv4 = d4[(rl0 >> 2) + 2 * h];
#pragma unroll
          for (int e = 0; e < 4; ++e) { lse2[rl0 + e] = lv[e]; dis[rl0 + e] = dv4[e]; }
        }
      }
      // tile rows (relative to 8 h) that see the key: [lo_r, hi_r]
      const int base = r0 + shift + 8 * h;
      const int lo_r = p_min - base, hi_r = min(p_max - base, q_len - 1 - r0 - 8 * h);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rl = 16 * (v >> 3) + (v & 7);
        const bool ok = rl >= lo_r && rl <= hi_r;
        // exp of every entry, then a select: no branch per entry (the scores of
        // entries not seen are finite, and rows past the segment have lse +inf)
        const float ex = fast_exp2(fmaf(sc[v], c2, -lse2[rl]));
        const float pe = ok ? ex : 0.f;
        pv[v] = pe;
        dsv[v] = pe * (dp[v] - dis[rl]);
      }
    }
    // ---- dV += P^T dO and dK += dS^T Q (contraction over the tile's rows)
    {
      const bf16x8_t pa0 = pack8(pv), pa1 = pack8(pv + 8);
      const bf16x8_t sa0 = pack8(dsv), sa1 = pack8(dsv + 8);
      // B operands (rows 16 s + 8 h .. + 7 of dim 32 c + l32) read down the
      // columns of the row-major dO and Q tiles
      const int i16 = lane & 15;
      const int cb = (8 * h + (i16 >> 2)) * B::RM + 32 * ((lane >> 4) & 1) + 8 * (i16 & 3);
      const uint8_t *dob = buf + LY::DO + cb;
      const uint8_t *qbb = buf + LY::Q + cb;
#pragma unroll
      for (int c = 0; c < B::DC; ++c) {
        dv[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa0, lds_col8(dob + 64 * c, B::RM), dv[c], 0, 0, 0);
        dv[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa1, lds_col8(dob + 64 * c + 16 * B::RM, B::RM), dv[c], 0, 0, 0);
        dk[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa0, lds_col8(qbb + 64 * c, B::RM), dk[c], 0, 0, 0);
        dk[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa1, lds_col8(qbb + 64 * c + 16 * B::RM, B::RM), dk[c], 0, 0, 0);
      }
    }
  };
  if (n_pairs > 0) fetch(0, R0);
  for (int pr = 0; pr < n_pairs; ++pr) step(pr, R0);

  // ---- write: output entry v of tile c is key k0 + 8 (v/4) + 4 h + v % 4, dim 32 c + l32
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int kk = k0 + 8 * (v >> 2) + 4 * h + (v & 3);
    if (kk >= L) continue;
    const size_t orow = ((size_t)a.key_offsets[s] + kk) * hkv + g;
#pragma unroll
    for (int c = 0; c < B::DC; ++c) {
      if (HC == 1) {
        a.dk[orow * D + 32 * c + l32] = a.softmax_scale * dk[c][v];
        a.dv[orow * D + 32 * c + l32] = dv[c][v];
      } else {
        unsafeAtomicAdd(a.dk + orow * D + 32 * c + l32, a.softmax_scale * dk[c][v]);
        unsafeAtomicAdd(a.dv + orow * D + 32 * c + l32, dv[c][v]);
      }
    }
  }
}

// ---- dQ
template <int D>
struct DqLds {
  using B = BwdTile<D>;
  // V is staged as the cache stores it, 16-byte runs (4 keys x dims l and
  // l + 16), with 64 bytes of padding after every 16 runs so that the
  // transposing reads of one 16-lane group hit distinct banks
  static constexpr int RUNS = D / 32 * 64;             // runs per 16-key block
  static NK_DEVICE constexpr int run_at(int run) { return 16 * run + 64 * (run / 16); }
  static constexpr int K = 0, V = 32 * B::RM, SIZE = V + run_at(2 * RUNS);
};

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) attn_dq_mfma_kernel(BackwardArgs a, int blocks_per_seq, int GW) {
  using B = BwdTile<D>;
  using LY = DqLds<D>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * LY::SIZE];   // two buffers
  const int TB = 4 / GW;
  const int hkv = a.cache.num_kv_heads, G = a.hq / hkv, P = a.cache.page_size;
  // head block fastest (XCD-local rows and keys), then segment, then row
  // block, last row blocks first: under a causal band they see the most keys
  const int nhb = hkv * (G / GW);
  const int hy = blockIdx.x % nhb, rest = blockIdx.x / nhb;
  const int s = rest % a.num_seqs, rb = blocks_per_seq - 1 - rest / a.num_seqs;
  const int g = hy / (G / GW), hblk = hy % (G / GW);
  const int q0 = a.q_offsets[s];
  const int q_len = a.q_offsets[s + 1] - q0;
  const int L = a.kv_lens[s];
  const int R0 = rb * 32 * TB;
  if (R0 >= q_len) return;
  const int shift = L - q_len;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int head = g * G + hblk * GW + w % GW;
  const int r0 = R0 + 32 * (w / GW);
  const int row = r0 + l32;                       // this lane's row (column of S^T)
  const bool rvalid = row < q_len;
  const int32_t *pt = a.cache.page_table + (size_t)s * a.cache.page_table_stride;

  // Q and dO of the lane's row as B operands (dims 16 kk + 8 h ..), dO.O and lse
  bf16x8_t qb[B::KD], db[B::KD];
  float di = 0.f, lse2 = INFINITY;
  {
    const size_t off = ((size_t)(q0 + min(row, q_len - 1)) * a.hq + head) * D;
#pragma unroll
    for (int kk = 0; kk < B::KD; ++kk) {
      const int d0 = 16 * kk + 8 * h;
      bf16x8_t qx = *(const bf16x8_t *)((const bf16_t *)a.q + off + d0);
      bf16x8_t dx = *(const bf16x8_t *)((const bf16_t *)a.dout + off + d0);
      const bf16x8_t ox = *(const bf16x8_t *)((const bf16_t *)a.out + off + d0);
      if (!rvalid) { qx = bf16x8_t{}; dx = bf16x8_t{}; }
#pragma unroll
      for (int e = 0; e < 8; ++e) di = fmaf((float)dx[e], (float)ox[e], di);
      qb[kk] = qx;
      db[kk] = dx;
    }
    di += shfl_xor_f32(di, 32);
    if (rvalid) lse2 = a.lse[(size_t)(q0 + row) * a.hq + head] * kLog2e;
  }

  // keys the work-group's rows may see: the band of its first and last rows,
  // plus the sink keys
  const int p_lo = R0 + shift, p_hi = min(R0 + 32 * TB, q_len) - 1 + shift;
  const int kh = band_hi(p_hi, L, a.window_right), kl = band_lo(p_lo, a.window_left);
  const int sinks = a.window_left < 0 ? 0 : min(a.sink_keys, L);
  // wave's own range (for skipping tiles it cannot see)
  const int w_hi = band_hi(min(r0 + 31, q_len - 1) + shift, L, a.window_right);
  const int w_lo = band_lo(r0 + shift, a.window_left);
  const bool w_active = r0 < q_len;
  // tiles: the sink tiles below the band's first tile, then the band's
  const int tb0 = kl / 32, tb1 = kh < kl ? tb0 - 1 : kh / 32;
  const int ns = sinks > 0 ? min((sinks + 31) / 32, max(tb0, 0)) : 0;
  const int n_tiles = ns + max(0, tb1 - tb0 + 1);

  f32x16_t dq[B::DC];
#pragma unroll
  for (int c = 0; c < B::DC; ++c) dq[c] = f32x16_t{};
  const float c2 = a.softmax_scale * kLog2e;
  // transposing-read source of this lane for the V operand (see the score
  // loop): key group 4 (lane/16 % 2) + swap(lane % 4), dim 8 h + lane/4 % 4
  // of a k-step; the second read of an operand (dims + 4) is 4 runs on, 64
  // bytes (lds_col8's step of 4 rows of 16 bytes)
  const int va_off = [&] {
    const int j = lane & 15, a2 = j & 3;
    const int kg = 4 * ((lane >> 4) & 1) + (((a2 & 1) << 1) | (a2 >> 1));
    const int sb = kg / 4, gq = kg % 4, l = 8 * h + (j >> 2);
    return LY::run_at(sb * LY::RUNS + 16 * gq + l);
  }();
  // keys the lane's row sees (none for rows past the segment)
  const int pos = row + shift;
  const int k_lo = band_lo(pos, a.window_left);
  const int k_hi = rvalid ? band_hi(pos, L, a.window_right) : -1;
  const int n_sink = rvalid ? max(0, min(sinks, min(k_lo, k_hi + 1))) : 0;

  // software pipeline over the key tiles: the global loads of tile it + 1
  // are in flight while tile it is computed; LDS double buffered (one
  // barrier per tile, as in the dK/dV kernel)
  auto tile_base = [&](int it) { return 32 * (it < ns ? it : tb0 + (it - ns)); };
  constexpr int RUNS = LY::RUNS;
  // this thread's K chunk is key c % 32 (the same key for every i, since
  // 256 is a multiple of 32); its V chunks are runs of the 16-key block i
  const int k_key = tid % 32;
  auto v_key = [&](int i) { const int rr = (tid + 256 * i) % RUNS; return 16 * ((tid + 256 * i) / RUNS) + 4 * ((rr % 64) / 16); };
  // the registers hold the data of tile t (loaded one tile ahead of its
  // use) and the page ids of tile t + 1 (read one tile ahead of the data
  // that needs them)
  struct Regs { bf16x8_t k[B::PER], v[B::PER]; int pk, pv[B::PER]; };
  Regs RA;
  auto fetch_pages = [&](int it, Regs &R) {
    const int kb = tile_base(it);
    R.pk = pt[min(kb + k_key, L - 1) / P];
#pragma unroll
    for (int i = 0; i < B::PER; ++i) R.pv[i] = pt[min(kb + v_key(i), L - 1) / P];
  };
  auto fetch = [&](int it, Regs &R) {
    const int kb = tile_base(it);
#pragma unroll
    for (int i = 0; i < B::PER; ++i) {
      const int c = tid + 256 * i;
      {
        // keys past the segment read its last key (in bounds) and are zeroed when staged
        const int k = min(kb + k_key, L - 1), d0 = 8 * (c / 32);
        const size_t blk = ((size_t)R.pk * hkv + g) * P * D;
        R.k[i] = *(const bf16x8_t *)((const bf16_t *)a.cache.k_pages + blk + k_elem<bf16_t>(d0, k % P, P));
      }
      {
        const int rr = c % RUNS, cg = rr / 64, l = rr % 16;
        const int k = min(kb + v_key(i), L - 1);   // the run's 4 keys share a page
        const size_t blk = ((size_t)R.pv[i] * hkv + g) * P * D;
        R.v[i] = *(const bf16x8_t *)((const bf16_t *)a.cache.v_pages + blk + v_elem<bf16_t>(32 * cg + l, (k % P) & ~3, D));
      }
    }
  };
  auto stage = [&](int it, uint8_t *buf, const Regs &R) {
    const bf16x8_t *gk = R.k, *gv = R.v;
    const int kb = tile_base(it);
#pragma unroll
    for (int i = 0; i < B::PER; ++i) {
      const int c = tid + 256 * i;
      {
        const int kr = c % 32, d0 = 8 * (c / 32);
        *(bf16x8_t *)(buf + LY::K + kr * B::RM + 2 * d0) = kb + kr < L ? gk[i] : bf16x8_t{};
      }
      {
        // run c of the tile (its two 16-key blocks in page order); keys past
        // the segment become zeros
        const int lim = L - (kb + v_key(i));
        u32x4_t x = __builtin_bit_cast(u32x4_t, gv[i]);
        if (lim < 4) {
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2) {
            const int k = 2 * (w2 & 1);                     // words 0, 1: dim l keys 0-3; 2, 3: dim l + 16
            x[w2] &= (k < lim ? 0xffffu : 0u) | (k + 1 < lim ? 0xffff0000u : 0u);
          }
        }
        *(u32x4_t *)(buf + LY::V + LY::run_at(c)) = x;
      }
    }
  };

  auto step = [&](int it, Regs &R) {
    const int kb = tile_base(it);
    uint8_t *buf = lds + (it & 1) * LY::SIZE;
    stage(it, buf, R);
    __syncthreads();
    if (it + 1 < n_tiles) {
      fetch(it + 1, R);
      if (it + 2 < n_tiles) fetch_pages(it + 2, R);
    }

    const bool act = w_active && kb <= w_hi && (kb + 31 >= w_lo || kb < sinks);
    if (act) {
      const uint8_t *va = buf + LY::V + va_off;
      // ---- S^T = K Q^T and dP^T = V dO^T (keys permuted)
      f32x16_t sc = f32x16_t{}, dp = f32x16_t{};
      const uint8_t *ka = buf + LY::K + bperm(l32) * B::RM + 16 * h;
#pragma unroll
      for (int kk = 0; kk < B::KD; ++kk) {
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8_t *)(ka + 32 * kk), qb[kk], sc, 0, 0, 0);
        // A = V rows of keys bperm(l32), dims 16 kk + 8 h ..: transposing
        // reads of the runs (lane 4 e + a of a group addresses the run of
        // dim 16 kk + 8 h + e for the key group that output lanes 4 a ..
        // 4 a + 3 need)
        const int off = 1280 * (kk / 2) + 8 * (kk % 2);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_col8(va + off, 16), db[kk], dp, 0, 0, 0);
      }
      // entry v: key kb + 16 (v/8) + 8 h + v % 8 of row `row`
      // the lane's row sees keys [k_lo, k_hi] and the sink keys below n_sink;
      // relative to kb + 8 h
      const int base = kb + 8 * h;
      const int lo_k = k_lo - base, hi_k = k_hi - base, sk_k = n_sink - base;
      float dsv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kv = 16 * (v >> 3) + (v & 7);
        const bool ok = (kv >= lo_k && kv <= hi_k) || kv < sk_k;
        const float ex = fast_exp2(fmaf(sc[v], c2, -lse2));
        const float pe = ok ? ex : 0.f;
        dsv[v] = pe * (dp[v] - di);
      }
      // ---- dQ += dS K: A = dS (row l32, keys of k-step s), B = keys
      // 16 s + 8 h .. + 7 of dim 32 c + l32, read down the K tile's columns
      const bf16x8_t sa0 = pack8(dsv), sa1 = pack8(dsv + 8);
      const int i16 = lane & 15;
      const uint8_t *kb_ = buf + LY::K + (8 * h + (i16 >> 2)) * B::RM + 32 * ((lane >> 4) & 1) + 8 * (i16 & 3);
#pragma unroll
      for (int c = 0; c < B::DC; ++c) {
        dq[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa0, lds_col8(kb_ + 64 * c, B::RM), dq[c], 0, 0, 0);
        dq[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa1, lds_col8(kb_ + 64 * c + 16 * B::RM, B::RM), dq[c], 0, 0, 0);
      }
    }
  };
  if (n_tiles > 0) {
    fetch_pages(0, RA);
    fetch(0, RA);
    if (n_tiles > 1) fetch_pages(1, RA);
  }
  for (int it = 0; it < n_tiles; ++it) step(it, RA);

  // ---- write: entry v of tile c is row r0 + 8 (v/4) + 4 h + v % 4, dim 32 c + l32
  if (!w_active) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = r0 + 8 * (v >> 2) + 4 * h + (v & 3);
    if (r >= q_len) continue;
    float *drow = a.dq + ((size_t)(q0 + r) * a.hq + head) * D;
#pragma unroll
    for (int c = 0; c < B::DC; ++c) drow[32 * c + l32] = a.softmax_scale * dq[c][v];
  }
}

// dO.O of every (row, query head), as float32, into the first total_q x hq
// floats of the dq buffer, for the dK/dV kernel (the dQ kernel, launched
// after it, computes its own and overwrites the buffer): D/8 consecutive
// lanes per (row, head), 16-byte loads, a lane-group sum.
template <int D>
__global__ void __launch_bounds__(256) bwd_rowdot_kernel(BackwardArgs a) {
  constexpr int LG = D / 8;                       // lanes per (row, head)
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long rh = t / LG;
  const bool live = rh < (long long)a.total_q * a.hq;
  const int j = (int)(t % LG);
  float x = 0.f;
  if (live) {
    const bf16x8_t d = *(const bf16x8_t *)((const bf16_t *)a.dout + rh * D + 8 * j);
    const bf16x8_t o = *(const bf16x8_t *)((const bf16_t *)a.out + rh * D + 8 * j);
#pragma unroll
    for (int e = 0; e < 8; ++e) x = fmaf((float)d[e], (float)o[e], x);
  }
#pragma unroll
  for (int m = 1; m < LG; m <<= 1) x += shfl_xor_f32(x, m);
  if (live && j == 0) a.dq[rh] = x;
}

// Zeros of the dK/dV rows of every segment's keys (rows key_offsets[s] ..
// key_offsets[s] + kv_lens[s] - 1), before work-groups add into them: one
// work-group per (segment, 16 keys).
__global__ void __launch_bounds__(256) bwd_zero_kernel(BackwardArgs a, int per_seq) {
  const int s = blockIdx.x / per_seq, k0 = (blockIdx.x % per_seq) * 16;
  const int L = a.kv_lens[s];
  if (k0 >= L) return;
  const int width = a.cache.num_kv_heads * a.cache.head_dim;      // floats per key row, a multiple of 4
  const size_t first = ((size_t)a.key_offsets[s] + k0) * width;
  const int n4 = min(16, L - k0) * width / 4;
  for (int i = threadIdx.x; i < n4; i += 256) {
    ((f32x4_t *)(a.dk + first))[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    ((f32x4_t *)(a.dv + first))[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
}

template <int D>
hipError_t launch_mfma(const BackwardArgs &a, int max_q_len, hipStream_t stream) {
  const int hkv = a.cache.num_kv_heads, G = a.hq / hkv;
  int GW = 1;                                      // heads per dQ work-group: power of 2 dividing G, at most 4
  while (GW * 2 <= 4 && G % (GW * 2) == 0) GW *= 2;
  const int rows_per_block = 32 * (4 / GW);
  hipError_t e = hipSuccess;
  // dQ last: the dK/dV kernel reads dO.O from the dq buffer
  auto launch_dq = [&]() -> hipError_t {
    if (a.total_q <= 0 || max_q_len <= 0) return hipSuccess;
    const int per_seq = (max_q_len + rows_per_block - 1) / rows_per_block;
    const long long blocks = (long long)a.num_seqs * per_seq * hkv * (G / GW);
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    return launch(attn_dq_mfma_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, stream, a, per_seq, GW);
  };
  if (a.max_kv_len == 0 || a.total_q <= 0) return launch_dq();
  {
    const long long threads = (long long)a.total_q * a.hq * (D / 8);
    const long long rblocks = (threads + 255) / 256;
    if (rblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    e = launch(bwd_rowdot_kernel<D>, dim3((unsigned)rblocks), dim3(256), 0, stream, a);
    if (e != hipSuccess) return e;
  }
  // query heads of a KV head split over HC work-groups (a power of two
  // dividing G, at most 4): shorter work-groups, added into zeroed outputs
  int HC = 1;
  while (HC * 2 <= 4 && G % (HC * 2) == 0) HC *= 2;
  if (HC > 1) {
    const int zper = (a.max_kv_len + 15) / 16;
    const long long zblocks = (long long)a.num_seqs * zper;
    if (zblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    e = launch(bwd_zero_kernel, dim3((unsigned)zblocks), dim3(256), 0, stream, a, zper);
    if (e != hipSuccess) return e;
  }
  const int per_seq = (a.max_kv_len + 127) / 128;
  const long long blocks = (long long)a.num_seqs * per_seq * hkv * HC;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  static bool attr_set[64];                     // per device; idempotent, a race only repeats the call
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (!attr_set[dev & 63]) {
    e = hipFuncSetAttribute((const void *)attn_dkv_mfma_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            DkvLds<D>::TOTAL);
    if (e != hipSuccess) return e;
    attr_set[dev & 63] = true;
  }
  e = launch(attn_dkv_mfma_kernel<D>, dim3((unsigned)blocks), dim3(256), DkvLds<D>::TOTAL, stream, a, per_seq, HC);
  if (e != hipSuccess) return e;
  return launch_dq();
}

template <typename T>
hipError_t launch_t(const BackwardArgs &a, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (a.total_q > 0) {
    const int G = a.hq / a.cache.num_kv_heads;       // heads per wave: 4, 2 or 1, dividing the group
    const int HB = G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
    const dim3 grid((unsigned)a.total_q, (unsigned)(a.hq / HB));
    e = HB == 4 ? launch(attn_dq_kernel<T, 4>, grid, dim3(kWave), 0, stream, a)
        : HB == 2 ? launch(attn_dq_kernel<T, 2>, grid, dim3(kWave), 0, stream, a)
                  : launch(attn_dq_kernel<T, 1>, grid, dim3(kWave), 0, stream, a);
  }
  if (e != hipSuccess || a.max_kv_len == 0) return e;
  const int per_seq = (a.max_kv_len + kDkvKeys - 1) / kDkvKeys;
  const long long blocks = (long long)a.num_seqs * per_seq;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  return launch(attn_dkv_kernel<T>, dim3((unsigned)blocks, (unsigned)a.cache.num_kv_heads), dim3(kWave), 0,
                stream, a, per_seq);
}

}  // namespace

hipError_t launch_attn_backward(const BackwardArgs &a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  ProfileScope prof("attn_backward", stream);
  if (a.q_dtype == NK_F32) return launch_t<float>(a, stream);
  // bf16 on MFMA for head dims 64 and 128 (the row-tile grid is bounded by
  // total_q, the longest a segment can be)
  const int D = a.cache.head_dim;
  if (D == 128) return launch_mfma<128>(a, a.total_q, stream);
  if (D == 64) return launch_mfma<64>(a, a.total_q, stream);
  return launch_t<bf16_t>(a, stream);
}

}  // namespace nk
