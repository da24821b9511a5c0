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
// Design: one wave per (row, head), the heads of a row on consecutive
// work-groups (their partials are adjacent); four 16-lane groups stream
// every fourth chunk, lanes over head dimensions -- HBM-bound.  Two
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
// head `h`; write row `out_row`.  The wave splits into four 16-lane groups
// that take every fourth chunk (two of them in flight per group), each lane
// holding MAXP pairs of dimensions 2(l + 16 r), r < MAXP; the groups' sums
// are added across lanes at the end.  The maximum lse and the weight sum are
// wave reductions over the chunks' lse values read by the lanes in parallel.
template <typename TOut, int MAXP>
NK_DEVICE void merge_row(const float *__restrict__ po, const float *__restrict__ pl, long long first,
                         int n, int heads, int h, int D, TOut *__restrict__ out_row,
                         float *__restrict__ lse_out) {
  const int lane = threadIdx.x;
  const int grp = lane >> 4, l16 = lane & 15;
  float M = -INFINITY;
  for (int b = 0; b < n; b += kWave) {
    const int i = b + lane;
    if (i < n) M = fmaxf(M, pl[(first + i) * heads + h]);
  }
  M = wave_max(M);
  f32x2_t acc[MAXP];
#pragma unroll
  for (int r = 0; r < MAXP; ++r) acc[r] = f32x2_t{0.f, 0.f};
  float tot = 0.f;
  if (M != -INFINITY) {
    for (int b = 0; b < n; b += kWave) {
      const int i = b + lane;
      const float li = i < n ? pl[(first + i) * heads + h] : -INFINITY;
      tot += li == -INFINITY ? 0.f : expf(li - M);
    }
    tot = wave_sum(tot);
    auto weight = [&](int c) {
      const float lc = pl[(first + c) * heads + h];          // same address across the group
      return lc == -INFINITY ? 0.f : expf(lc - M);
    };
    int c = grp;
    for (; c + 4 < n; c += 8) {
      const float w0 = weight(c), w1 = weight(c + 4);
      const float *o0 = po + ((first + c) * heads + h) * (long long)D;
      const float *o1 = po + ((first + c + 4) * heads + h) * (long long)D;
      f32x2_t v0[MAXP], v1[MAXP];
#pragma unroll
      for (int r = 0; r < MAXP; ++r) {
        const int d = 2 * (l16 + 16 * r);
        v0[r] = d < D ? *(const f32x2_t *)(o0 + d) : f32x2_t{0.f, 0.f};
        v1[r] = d < D ? *(const f32x2_t *)(o1 + d) : f32x2_t{0.f, 0.f};
      }
#pragma unroll
      for (int r = 0; r < MAXP; ++r) {
        acc[r][0] = fmaf(w0, v0[r][0], acc[r][0]);
        acc[r][1] = fmaf(w0, v0[r][1], acc[r][1]);
        acc[r][0] = fmaf(w1, v1[r][0], acc[r][0]);
        acc[r][1] = fmaf(w1, v1[r][1], acc[r][1]);
      }
    }
    if (c < n) {
      const float w0 = weight(c);
      const float *o0 = po + ((first + c) * heads + h) * (long long)D;
#pragma unroll
      for (int r = 0; r < MAXP; ++r) {
        const int d = 2 * (l16 + 16 * r);
        if (d < D) {
          const f32x2_t v = *(const f32x2_t *)(o0 + d);
          acc[r][0] = fmaf(w0, v[0], acc[r][0]);
          acc[r][1] = fmaf(w0, v[1], acc[r][1]);
        }
      }
    }
    // the four groups hold the same dimensions: lanes l, l^16, l^32, l^48
#pragma unroll
    for (int r = 0; r < MAXP; ++r)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        acc[r][e] += shfl_xor_f32(acc[r][e], 16);
        acc[r][e] += shfl_xor_f32(acc[r][e], 32);
      }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  if (grp == 0) {
#pragma unroll
    for (int r = 0; r < MAXP; ++r) {
      const int d = 2 * (l16 + 16 * r);
      if (d < D) store2<TOut>(out_row + d, acc[r][0] * inv, acc[r][1] * inv);
    }
  }
  if (lse_out && lane == 0) *lse_out = tot > 0.f ? M + logf(tot) : -INFINITY;
}

template <typename TOut, int MAXP>
__global__ void __launch_bounds__(64) lse_merge_kernel(const float *po, const float *pl,
                                                       const int32_t *offsets, int heads, int D,
                                                       TOut *out, float *lse_out) {
  const int h = (int)(blockIdx.x % (unsigned)heads), r = (int)(blockIdx.x / (unsigned)heads);   // heads fastest
  const int a = offsets[r], b = offsets[r + 1];
  merge_row<TOut, MAXP>(po, pl, a, b - a, heads, h, D, out + ((size_t)r * heads + h) * D,
                        lse_out ? lse_out + (size_t)r * heads + h : nullptr);
}

// Split-KV decode rows: sequence s (a single query row) has its chunks at
// s*max_chunks ... ; rows with one chunk were finished by the decode kernel.
template <typename TOut, int MAXP>
__global__ void __launch_bounds__(64) decode_merge_kernel(AttnArgs a) {
  const int h = (int)(blockIdx.x % (unsigned)a.hq), s = (int)(blockIdx.x / (unsigned)a.hq);     // heads fastest
  const int q0 = a.q_offsets[s];
  if (a.q_offsets[s + 1] - q0 != 1) return;
  const int L = a.kv_lens[s];
  if (L <= 0) return;
  const int hi = L - 1;
  const int lo = a.window_left < 0 ? 0 : max(0, hi - a.window_left);
  const int c0 = (lo / 32) * 32;              // the decode kernel's chunk origin
  const int n = min((hi + 1 - c0 + a.split_tokens - 1) / a.split_tokens, a.max_chunks);
  if (n <= 1) return;
  merge_row<TOut, MAXP>(a.part_out, a.part_lse, (long long)s * a.max_chunks, n, a.hq, h,
                  a.cache.head_dim, (TOut *)a.out + ((size_t)q0 * a.hq + h) * a.cache.head_dim,
                  a.lse ? a.lse + (size_t)q0 * a.hq + h : nullptr);
}

}  // namespace

hipError_t launch_lse_merge(const float *po, const float *pl, const int32_t *offsets, int32_t rows,
                            int32_t heads, int32_t head_dim, void *out, int32_t out_dtype,
                            float *lse_out, hipStream_t stream) {
  if (rows == 0 || heads == 0) return hipSuccess;
  ProfileScope prof("lse_merge", stream);
  const long long n = (long long)rows * heads;
  if (n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const unsigned grid = (unsigned)n;
  auto go = [&](auto tag) {
    using TOut = decltype(tag);
    TOut *o = (TOut *)out;
    if (head_dim <= 128) lse_merge_kernel<TOut, 4><<<grid, kWave, 0, stream>>>(po, pl, offsets, heads, head_dim, o, lse_out);
    else if (head_dim <= 256) lse_merge_kernel<TOut, 8><<<grid, kWave, 0, stream>>>(po, pl, offsets, heads, head_dim, o, lse_out);
    else lse_merge_kernel<TOut, 16><<<grid, kWave, 0, stream>>>(po, pl, offsets, heads, head_dim, o, lse_out);
  };
  if (out_dtype == NK_F32) go(float{}); else go(bf16_t{});
  return hipGetLastError();
}

hipError_t launch_decode_merge(const AttnArgs &a, hipStream_t stream) {
  if (a.max_chunks <= 1 || a.num_seqs == 0) return hipSuccess;
  ProfileScope prof("lse_merge", stream);
  const long long n = (long long)a.hq * a.num_seqs;
  if (n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const unsigned grid = (unsigned)n;
  auto go = [&](auto tag) {
    using TOut = decltype(tag);
    const int D = a.cache.head_dim;
    if (D <= 128) decode_merge_kernel<TOut, 4><<<grid, kWave, 0, stream>>>(a);
    else decode_merge_kernel<TOut, 8><<<grid, kWave, 0, stream>>>(a);
  };
  if (a.q_dtype == NK_F32) go(float{}); else go(bf16_t{});
  return hipGetLastError();
}

}  // namespace nk
