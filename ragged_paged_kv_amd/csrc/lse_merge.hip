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
// work-groups (their partials are adjacent); four 16-lane groups take every
// fourth chunk, lanes over head dimensions.  A call moves little data, so
// its time is the chain of dependent memory accesses, kept short: a row's
// partials and lse values are requested together (for a decode row, before
// its chunk count is read), then the output is written.  Two
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

// Where a merged row goes: its chunk count (negative: nothing to write) and
// output locations.
template <typename TOut> struct RowTarget {
  int n;
  TOut *out_row;
  float *lse_out;
};

// Merge the partials of one row for head `h`: chunk c's state sits at
// `first + c` (stride `heads` between chunks).  `target()` reads the row's
// chunk count and output locations; at most `n_issue` chunks are requested
// before it returns (an upper bound on the count, within the row's slots),
// so that those requests and its own are in flight together.  The wave
// splits into four 16-lane groups that take every fourth chunk, each lane
// holding MAXP pairs of dimensions 2(l + 16 r), r < MAXP; the groups' sums
// are added across lanes at the end.  Latency-bound: the first batch of
// partial outputs (4 chunks per group) is requested together with the
// chunks' lse values.  Lane i holds chunk i's lse and weight; a group reads
// its chunks' weights from those lanes.
template <typename TOut, int MAXP, typename Target>
NK_DEVICE void merge_row(const float *__restrict__ po, const float *__restrict__ pl, long long first,
                         int n_issue, int heads, int h, int D, Target &&target) {
  constexpr int CB = 4;                       // chunks per group and batch
  const int lane = threadIdx.x;
  const int grp = lane >> 4, l16 = lane & 15;
  f32x2_t v[CB][MAXP];
  auto load_batch = [&](int c0, int n) {
#pragma unroll
    for (int k = 0; k < CB; ++k) {
      const int c = c0 + grp + 4 * k;
      const float *o = po + ((first + c) * heads + h) * (long long)D;
#pragma unroll
      for (int r = 0; r < MAXP; ++r) {
        const int d = 2 * (l16 + 16 * r);
        v[k][r] = c < n && d < D ? *(const f32x2_t *)(o + d) : f32x2_t{0.f, 0.f};
      }
    }
  };
  auto lse_of = [&](int c) { return pl[(first + c) * heads + h]; };
  load_batch(0, n_issue);
  const float l_issued = lane < n_issue ? lse_of(lane) : -INFINITY;
  const RowTarget<TOut> t = target();
  if (t.n < 0) return;
  const int n = t.n;
  const float l0 = lane < n ? l_issued : -INFINITY;
  float M = l0;
  for (int b = kWave; b < n; b += kWave)
    if (b + lane < n) M = fmaxf(M, lse_of(b + lane));
  M = wave_max(M);
  f32x2_t acc[MAXP];
#pragma unroll
  for (int r = 0; r < MAXP; ++r) acc[r] = f32x2_t{0.f, 0.f};
  float tot = 0.f;
  if (M != -INFINITY) {
    auto weight_of = [&](float lc) { return lc == -INFINITY ? 0.f : expf(lc - M); };
    const float w0 = weight_of(l0);           // chunk `lane` (0 past n)
    float ws = w0;
    for (int b = kWave; b < n; b += kWave)
      if (b + lane < n) ws += weight_of(lse_of(b + lane));
    tot = wave_sum(ws);
    for (int c0 = 0;;) {
#pragma unroll
      for (int k = 0; k < CB; ++k) {
        const int c = c0 + grp + 4 * k;
        const float wl = __shfl(w0, c & (kWave - 1), kWave);          // every lane takes part
        if (c < n) {                          // (requested chunks past n hold anything)
          const float w = c < kWave ? wl : weight_of(lse_of(c));
#pragma unroll
          for (int r = 0; r < MAXP; ++r) {
            acc[r][0] = fmaf(w, v[k][r][0], acc[r][0]);
            acc[r][1] = fmaf(w, v[k][r][1], acc[r][1]);
          }
        }
      }
      c0 += 4 * CB;
      if (c0 >= n) break;
      load_batch(c0, n);
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
      if (d < D) store2<TOut>(t.out_row + d, acc[r][0] * inv, acc[r][1] * inv);
    }
  }
  if (t.lse_out && lane == 0) *t.lse_out = tot > 0.f ? M + logf(tot) : -INFINITY;
}

template <typename TOut, int MAXP>
__global__ void __launch_bounds__(64) lse_merge_kernel(const float *po, const float *pl,
                                                       const int32_t *offsets, int heads, int D,
                                                       TOut *out, float *lse_out) {
  const int h = (int)(blockIdx.x % (unsigned)heads), r = (int)(blockIdx.x / (unsigned)heads);   // heads fastest
  const int a = offsets[r], b = offsets[r + 1];
  merge_row<TOut, MAXP>(po, pl, a, b - a, heads, h, D, [&]() {
    return RowTarget<TOut>{b - a, out + ((size_t)r * heads + h) * D, lse_out ? lse_out + (size_t)r * heads + h : nullptr};
  });
}

// Split-KV decode rows: sequence s (a single query row) has its chunks at
// s*max_chunks ... ; rows with one chunk were finished by the decode kernel.
// The row's slots are known before its chunk count, so they are requested
// first.
template <typename TOut, int MAXP>
__global__ void __launch_bounds__(64) decode_merge_kernel(AttnArgs a) {
  const int h = (int)(blockIdx.x % (unsigned)a.hq), s = (int)(blockIdx.x / (unsigned)a.hq);     // heads fastest
  merge_row<TOut, MAXP>(a.part_out, a.part_lse, (long long)s * a.max_chunks, a.max_chunks, a.hq, h,
                        a.cache.head_dim, [&]() {
    const int q0 = a.q_offsets[s];
    const int q1 = a.q_offsets[s + 1];
    const int L = a.kv_lens[s];
    RowTarget<TOut> t{-1, nullptr, nullptr};
    if (q1 - q0 != 1 || L <= 0) return t;
    const int n = decode_chunks(L, a.window_left, a.sink_keys, a.split_tokens, a.max_chunks).n;   // the decode kernel's
    if (n <= 1) return t;
    t.n = n;
    t.out_row = (TOut *)a.out + ((size_t)q0 * a.hq + h) * a.cache.head_dim;
    t.lse_out = a.lse ? a.lse + (size_t)q0 * a.hq + h : nullptr;
    return t;
  });
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
    auto k = head_dim <= 128 ? lse_merge_kernel<TOut, 4> : head_dim <= 256 ? lse_merge_kernel<TOut, 8>
                                                                          : lse_merge_kernel<TOut, 16>;
    return launch(k, dim3(grid), dim3(kWave), 0, stream, po, pl, offsets, heads, head_dim, o, lse_out);
  };
  return out_dtype == NK_F32 ? go(float{}) : go(bf16_t{});
}

hipError_t launch_decode_merge(const AttnArgs &a, hipStream_t stream) {
  if (a.max_chunks <= 1 || a.num_seqs == 0) return hipSuccess;
  ProfileScope prof("lse_merge", stream);
  const long long n = (long long)a.hq * a.num_seqs;
  if (n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const unsigned grid = (unsigned)n;
  auto go = [&](auto tag) {
    using TOut = decltype(tag);
    auto k = a.cache.head_dim <= 128 ? decode_merge_kernel<TOut, 4> : decode_merge_kernel<TOut, 8>;
    return launch(k, dim3(grid), dim3(kWave), 0, stream, a);
  };
  return a.q_dtype == NK_F32 ? go(float{}) : go(bf16_t{});
}

}  // namespace nk
