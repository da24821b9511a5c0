// Ragged paged attention for float32 queries and a float32 cache (VALU).
//
// What it computes: NumKong matrix-kernels page, attention_packed -- query
// row i of a segment sits at i + kv_len - q_len and sees the causal band
// (optionally windowed: window_left keys before it, window_right after it,
// and beside a window the segment's first sink_keys keys -- Algenta, "Ten
// named techniques, one scalar formula each", StreamingLLM sinks); rows with no key give
// zeros; the log-sum-exp is filled alongside.  Scores are
// softmax_scale * q.k (Algenta "A scalar reference, not a buffer kernel";
// explicit scale as in aria_kernel `attention_with_scale`).
//
// Design: float32 parity path.  One wave per (query row, query head); lanes
// take 64 keys at a time, each lane computing a full dot product, followed by
// an online-softmax update (running max / sum, rescale on a new max, as on
// the Algenta page's flash-attention walkthrough) and the P.V accumulation
// with lanes over head dimensions.  Throughput is not the goal here: the
// float32 workloads are small; the bf16 / fp8 paths use MFMA kernels.

#include "common.h"
#include "internal.h"

namespace nk {
namespace {

__global__ void __launch_bounds__(64) attn_f32_kernel(AttnArgs a) {
  const int t = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const int D = a.cache.head_dim;
  const int P = a.cache.page_size;
  const int hkv = a.cache.num_kv_heads;
  const int g = h / (a.hq / hkv);
  __shared__ float qs[256];

  const int s = find_segment(a.q_offsets, a.num_seqs, t);
  const int q0 = a.q_offsets[s];
  const int q_len = a.q_offsets[s + 1] - q0;
  const int L = a.kv_lens[s];
  const int p = (t - q0) + L - q_len;
  const int hi = band_hi(p, L, a.window_right);
  const int lo = band_lo(p, a.window_left);

  const float *q = (const float *)a.q + ((size_t)t * a.hq + h) * D;
  for (int d = lane; d < D; d += kWave) qs[d] = q[d];
  __syncthreads();

  const float *kp = (const float *)a.cache.k_pages;
  const float *vp = (const float *)a.cache.v_pages;
  const int32_t *pt = a.cache.page_table + (size_t)s * a.cache.page_table_stride;

  // visible keys: the sink keys before the band, then the band; walked as
  // one list, entry v being key v (v < n_sink) or lo + v - n_sink
  const int n_sink = max(0, min(a.sink_keys, min(lo, hi + 1)));
  const int n_keys = n_sink + max(0, hi - lo + 1);
  auto key_of = [&](int v) { return v < n_sink ? v : lo + v - n_sink; };
  float m = -INFINITY, l = 0.f;
  float o[4] = {0.f, 0.f, 0.f, 0.f};     // dims lane, lane+64, lane+128, lane+192
  for (int base = 0; base < n_keys; base += kWave) {
    const bool valid = base + lane < n_keys;
    const int key = key_of(base + lane);
    float sc = -INFINITY;
    if (valid) {
      const int page = pt[key / P];
      // K page-head: [dim/32][slot][32]
      const float *kph = kp + ((size_t)page * hkv + g) * P * D + (key % P) * 32;
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = fmaf(qs[d], kph[(d >> 5) * P * 32 + (d & 31)], acc);
      sc = a.softmax_scale * acc;
    }
    const float cm = wave_max(sc);
    const float nm = fmaxf(m, cm);
    const float corr = expf(m - nm);                 // 0 when m = -inf
    const float pj = valid ? expf(sc - nm) : 0.f;
    l = l * corr + wave_sum(pj);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] *= corr;
    const int nk = min(kWave, n_keys - base);
    for (int i = 0; i < nk; ++i) {
      const float pi = __shfl(pj, i, kWave);
      const int kk = key_of(base + i);
      const int page = pt[kk / P];
      // V page-head block in MFMA operand order (one 16-dim tile per
      // 16-byte run for float32): element (d, t) at
      // ((t/16)*(D/16) + d/16)*256 + (16*((t%16)/4) + d%16)*4 + t%4
      const int t = kk % P;
      const float *vblk = vp + ((size_t)page * hkv + g) * D * P + (t >> 4) * 16 * D + 64 * ((t & 15) >> 2) + (t & 3);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = lane + r * kWave;
        if (d < D) o[r] = fmaf(pi, vblk[(d >> 4) * 256 + (d & 15) * 4], o[r]);
      }
    }
    m = nm;
  }

  float *out = (float *)a.out + ((size_t)t * a.hq + h) * D;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int d = lane + r * kWave;
    if (d < D) out[d] = o[r] * inv;
  }
  if (a.lse && lane == 0) a.lse[(size_t)t * a.hq + h] = l > 0.f ? m + logf(l) : -INFINITY;
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t stream) {
  if (a.total_q == 0) return hipSuccess;
  ProfileScope prof("attn_f32", stream);
  dim3 grid((unsigned)a.total_q, (unsigned)a.hq);
  return launch(attn_f32_kernel, grid, dim3(kWave), 0, stream, a);
}

}  // namespace nk
