// Log-sum-exp merge of partial attention states.
//
// What it computes: Algenta "Attention variant kernels", "Flash attention's
// running state reproduces the same softmax": states over disjoint key
// chunks combine by rescaling with exp(old_max - new_max); for normalised
// chunk outputs o_i with log-sum-exp lse_i the merge is
//   M = max lse_i, w_i = exp(lse_i - M), out = sum w_i o_i / sum w_i,
//   lse = M + ln(sum w_i);
// rows whose chunks are all empty (-inf) give zeros and -inf.
//
// Design: one wave per (row, head); lanes hold head dimensions (two floats
// each, up to D = 512 in a loop); the chunk loop reads one lse per chunk
// (wave-uniform) and streams the chunk outputs -- HBM-bound, tiny.  Two
// row->partials maps: explicit merge offsets (the public entry point) and
// the split-KV decode layout (chunks of a decode row at row*max_chunks).

#include "common.h"
#include "internal.h"

namespace nk {
namespace {

template <typename TOut> NK_DEVICE void store2(TOut *p, float a, float b);
template <> NK_DEVICE void store2<float>(float *p, float a, float b) {
  *(f32x2_t *)p = f32x2_t{a, b};
}
template <> NK_DEVICE void store2<bf16_t>(bf16_t *p, float a, float b) {
  *(bf16x2_t *)p = bf16x2_t{(bf16_t)a, (bf16_t)b};
}

// Merge `n` partials starting at `first` (stride `heads` between chunks) for
// head `h`; write row `out_row`.  The chunks' lse values are read by the lanes
// in parallel (64 at a time), the maximum and the weight sum are wave
// reductions, and each chunk's weight is broadcast from its lane while the
// partial outputs stream in four chunks at a time.
template <typename TOut>
NK_DEVICE void merge_row(const float *__restrict__ po, const float *__restrict__ pl, long long first,
                         int n, int heads, int h, int D, TOut *__restrict__ out_row,
                         float *__restrict__ lse_out) {
  const int lane = threadIdx.x;
  float M = -INFINITY;
  for (int b = 0; b < n; b += kWave) {
    const int i = b + lane;
    if (i < n) M = fmaxf(M, pl[(first + i) * heads + h]);
  }
  M = wave_max(M);
  constexpr int kMaxPairs = 4;                       // D <= 512: two floats per lane per pass
  float acc[2 * kMaxPairs] = {};
  float tot = 0.f;
  if (M != -INFINITY) {
    for (int b = 0; b < n; b += kWave) {
      const int i = b + lane;
      const float li = i < n ? pl[(first + i) * heads + h] : -INFINITY;
      const float wl = li == -INFINITY ? 0.f : expf(li - M);     // weight of chunk b + lane
      tot += wl;
      const int cnt = min(kWave, n - b);
      int k = 0;
      for (; k + 4 <= cnt; k += 4) {
        float w4[4];
        f32x2_t v4[4][kMaxPairs];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          w4[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), k + u));
          const float *o = po + ((first + b + k + u) * heads + h) * (long long)D;
#pragma unroll
          for (int r = 0; r < kMaxPairs; ++r) {
            const int d = 2 * (lane + r * kWave);
            v4[u][r] = d < D ? *(const f32x2_t *)(o + d) : f32x2_t{0.f, 0.f};
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int r = 0; r < kMaxPairs; ++r) {
            acc[2 * r] = fmaf(w4[u], v4[u][r][0], acc[2 * r]);
            acc[2 * r + 1] = fmaf(w4[u], v4[u][r][1], acc[2 * r + 1]);
          }
      }
      for (; k < cnt; ++k) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), k));
        const float *o = po + ((first + b + k) * heads + h) * (long long)D;
#pragma unroll
        for (int r = 0; r < kMaxPairs; ++r) {
          const int d = 2 * (lane + r * kWave);
          if (d < D) {
            const f32x2_t v = *(const f32x2_t *)(o + d);
            acc[2 * r] = fmaf(w, v[0], acc[2 * r]);
            acc[2 * r + 1] = fmaf(w, v[1], acc[2 * r + 1]);
          }
        }
      }
    }
    tot = wave_sum(tot);
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
  for (int r = 0; r < kMaxPairs; ++r) {
    const int d = 2 * (lane + r * kWave);
    if (d < D) store2<TOut>(out_row + d, acc[2 * r] * inv, acc[2 * r + 1] * inv);
  }
  if (lse_out && lane == 0) *lse_out = tot > 0.f ? M + logf(tot) : -INFINITY;
}

template <typename TOut>
__global__ void __launch_bounds__(64) lse_merge_kernel(const float *po, const float *pl,
                                                       const int32_t *offsets, int heads, int D,
                                                       TOut *out, float *lse_out) {
  const int r = blockIdx.x, h = blockIdx.y;
  const int a = offsets[r], b = offsets[r + 1];
  merge_row<TOut>(po, pl, a, b - a, heads, h, D, out + ((size_t)r * heads + h) * D,
                  lse_out ? lse_out + (size_t)r * heads + h : nullptr);
}

// Split-KV decode rows: sequence s (a single query row) has its chunks at
// s*max_chunks ... ; rows with one chunk were finished by the decode kernel.
template <typename TOut>
__global__ void __launch_bounds__(64) decode_merge_kernel(AttnArgs a) {
  const int s = blockIdx.x, h = blockIdx.y;
  const int q0 = a.q_offsets[s];
  if (a.q_offsets[s + 1] - q0 != 1) return;
  const int L = a.kv_lens[s];
  if (L <= 0) return;
  const int hi = L - 1;
  const int lo = a.window_left < 0 ? 0 : max(0, hi - a.window_left);
  const int c0 = (lo / 32) * 32;              // the decode kernel's chunk origin
  const int n = min((hi + 1 - c0 + a.split_tokens - 1) / a.split_tokens, a.max_chunks);
  if (n <= 1) return;
  merge_row<TOut>(a.part_out, a.part_lse, (long long)s * a.max_chunks, n, a.hq, h,
                  a.cache.head_dim, (TOut *)a.out + ((size_t)q0 * a.hq + h) * a.cache.head_dim,
                  a.lse ? a.lse + (size_t)q0 * a.hq + h : nullptr);
}

}  // namespace

hipError_t launch_lse_merge(const float *po, const float *pl, const int32_t *offsets, int32_t rows,
                            int32_t heads, int32_t head_dim, void *out, int32_t out_dtype,
                            float *lse_out, hipStream_t stream) {
  if (rows == 0 || heads == 0) return hipSuccess;
  ProfileScope prof("lse_merge", stream);
  dim3 grid((unsigned)rows, (unsigned)heads);
  if (out_dtype == NK_F32)
    lse_merge_kernel<float><<<grid, kWave, 0, stream>>>(po, pl, offsets, heads, head_dim, (float *)out, lse_out);
  else
    lse_merge_kernel<bf16_t><<<grid, kWave, 0, stream>>>(po, pl, offsets, heads, head_dim, (bf16_t *)out, lse_out);
  return hipGetLastError();
}

hipError_t launch_decode_merge(const AttnArgs &a, hipStream_t stream) {
  if (a.max_chunks <= 1 || a.num_seqs == 0) return hipSuccess;
  ProfileScope prof("lse_merge", stream);
  dim3 grid((unsigned)a.num_seqs, (unsigned)a.hq);
  if (a.q_dtype == NK_F32)
    decode_merge_kernel<float><<<grid, kWave, 0, stream>>>(a);
  else
    decode_merge_kernel<bf16_t><<<grid, kWave, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace nk
