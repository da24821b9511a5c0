// Launch descriptors shared between the C-ABI layer (api.hip) and the
// kernel files: argument structs, the workspace layout of the prefill work
// list, and the launcher prototypes.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/nk.h"

namespace nk {

constexpr int kMaxMropeSections = 4;

struct RopeArgs {
  const void *q, *k, *v;
  void *q_out;
  const int32_t *q_offsets, *kv_lens, *position_ids;
  const float *freqs;
  int32_t rotary_dim, layout, in_dtype, max_pos;
  int32_t num_seqs, total_tokens, hq;
  nk_paged_kv_t cache;
  // M-RoPE: position_ids is [mrope_sections][total_tokens]; section s holds
  // rotated pairs [mrope_end[s-1], mrope_end[s]) (0: one position per token)
  int32_t mrope_sections;
  int32_t mrope_end[kMaxMropeSections];
};

struct AttnArgs {
  const void *q;
  int32_t q_dtype;
  const int32_t *q_offsets, *kv_lens;
  nk_paged_kv_t cache;
  float softmax_scale;
  int32_t window_left;      // keys before a row's position it sees (-1: all)
  int32_t window_right;     // keys after it (0: causal; -1: all)
  int32_t sink_keys;        // first keys of a segment every row also sees, up to its band's right edge
  void *out;
  float *lse;
  int32_t num_seqs, total_q, max_q_len, max_kv_len, hq;
  // split-KV decode
  int32_t split_tokens;     // keys per chunk
  int32_t max_chunks;       // chunks per decode row (upper bound)
  float *part_out;          // [num_seqs * max_chunks][hq][D]
  float *part_lse;          // [num_seqs * max_chunks][hq]
  // prefill work list (workspace): queue counters, item count, per-segment
  // item offsets and the items, heaviest first (segment, q-block and the
  // segment's row offset, row count and key count)
  int32_t *sched;
  int32_t sched_items_max;
};

// Prefill schedule layout inside the workspace (int32 offsets).
constexpr int kSchedQueues = 8;               // one work queue per XCD
constexpr int kSchedCounterStride = 32;       // one 128-byte line per counter
constexpr int kSchedCount = kSchedQueues * kSchedCounterStride;   // item count
constexpr int kSchedSegOff = kSchedCount + 64;                    // [num_seqs + 1]
constexpr int kSchedItemInts = 8;             // {s, q-block, q0, q_len, kv_len, 0, 0, 0}
__host__ __device__ inline size_t sched_items_offset(int num_seqs) {                  // 32-byte items
  return ((size_t)kSchedSegOff + num_seqs + 1 + 63) / 64 * 64;
}
// Smallest q-block of the prefill kernels (rows): 16-row waves, one row
// block per work-group
constexpr int kMinPrefillBlock = 16;
// q-blocks of a prefill batch: at most one per kMinPrefillBlock rows plus one
// per segment
__host__ __device__ inline int sched_items_max(int num_seqs, int total_q) {
  return total_q / kMinPrefillBlock + num_seqs + 1;
}
__host__ __device__ inline size_t sched_bytes(int num_seqs, int total_q) {
  return (sched_items_offset(num_seqs) + (size_t)kSchedItemInts * sched_items_max(num_seqs, total_q)) * 4;
}

// Each launcher enqueues its kernel(s) on `stream` and returns a
// hipError_t (hipSuccess when the launch was accepted).
// Packing ragged K/V token rows into cache pages (no rotation): segment s
// keeps its first kept-length rows from row key_offsets[s]
struct PackArgs {
  const void *k, *v;
  int32_t in_dtype;
  const int32_t *key_offsets, *key_lengths;   // [num_seqs + 1], [num_seqs] or null
  nk_paged_kv_t cache;                         // pages, scales and page table written
  int32_t *kv_lens_out;                        // [num_seqs]
  int32_t num_seqs, max_key_len;
};

// Gradients of the attention: dq [total_q][hq][D], dk/dv [rows][Hkv][D]
// (segment s's key j at row key_offsets[s] + j), all float32
struct BackwardArgs {
  const void *q, *out, *dout;          // q_dtype [total_q][hq][D]
  int32_t q_dtype;
  const float *lse;                    // [total_q][hq]
  const int32_t *q_offsets, *kv_lens, *key_offsets;
  nk_paged_kv_t cache;
  float softmax_scale;
  int32_t window_left, window_right, sink_keys;
  float *dq, *dk, *dv;
  int32_t num_seqs, total_q, max_kv_len, hq;
};

hipError_t launch_rope_write(const RopeArgs &a, hipStream_t stream);
hipError_t launch_attn_backward(const BackwardArgs &a, hipStream_t stream);
hipError_t launch_attention_pack(const PackArgs &a, hipStream_t stream);
hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t stream);
hipError_t launch_attn_decode(const AttnArgs &a, hipStream_t stream);
hipError_t launch_attn_prefill(const AttnArgs &a, hipStream_t stream);
hipError_t launch_decode_merge(const AttnArgs &a, hipStream_t stream);
hipError_t launch_lse_merge(const float *po, const float *pl, const int32_t *offsets,
                            int32_t rows, int32_t heads, int32_t head_dim, void *out,
                            int32_t out_dtype, float *lse_out, hipStream_t stream);

// Kernel timing (diagnostics, nk_profile_enable).  While enabled for its
// family, a scope owns a pair of events, and the kernels launched inside it
// through launch() carry them: the scope's first launch the start event,
// every launch the stop event (the last one recorded counts).  The events
// then take the kernels' own dispatch start and end times, with no marker
// packets of their own on the stream.
struct ProfileScope {
  ProfileScope(const char *family, hipStream_t stream);
  ~ProfileScope();
  ProfileScope(const ProfileScope &) = delete;
  ProfileScope &operator=(const ProfileScope &) = delete;
  // events for the next launch in the innermost scope of this thread (null
  // when none is enabled)
  static void launch_events(hipEvent_t *start, hipEvent_t *stop);
  int slot;
  bool started = false, stopped = false;
  ProfileScope *outer;
};

// Every kernel launch of the library: hipExtLaunchKernel with the current
// scope's events (plain launch when timing is off).
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                  Args... args) {
  hipEvent_t start = nullptr, stop = nullptr;
  ProfileScope::launch_events(&start, &stop);
  hipExtLaunchKernelGGL(kernel, grid, block, (std::uint32_t)shmem, stream, start, stop, 0u, args...);
  return hipGetLastError();
}

}  // namespace nk
