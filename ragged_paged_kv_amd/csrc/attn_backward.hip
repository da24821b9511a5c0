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
// Design (float32 VALU, correctness first): two kernels.
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
  return launch_t<bf16_t>(a, stream);
}

}  // namespace nk
