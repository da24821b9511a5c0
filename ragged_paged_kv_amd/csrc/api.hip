// C ABI of libnk.so: argument validation, launch planning, dispatch.
//
// Every check here is a host-side check of scalars and pointer nullness, made
// before anything is launched; device-array contents are preconditions
// (include/nk.h).  Planning uses host scalars only: the split-KV chunk size,
// the grid bounds and the workspace carve-up.  Which rows are single-token
// decode rows and which are prefill rows is decided inside the kernels from
// the device offsets, so a call never reads device memory on the host and
// never synchronises.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "internal.h"

using namespace nk;

namespace {

constexpr int kVersion = 10000;   // 1.0.0

bool head_dim_ok(int d) { return d == 64 || d == 128 || d == 256; }
bool page_size_ok(int p) { return p == 16 || p == 32; }

int check_cache(const nk_paged_kv_t *c) {
  if (!c || !c->k_pages || !c->v_pages || !c->page_table) return NK_ERR_INVALID_ARG;
  if (c->num_pages < 0 || c->num_kv_heads <= 0 || c->page_table_stride < 0) return NK_ERR_INVALID_ARG;
  if (c->dtype != NK_F32 && c->dtype != NK_BF16 && c->dtype != NK_E4M3) return NK_ERR_UNSUPPORTED;
  if (c->dtype == NK_E4M3 && (!c->k_scales || !c->v_scales)) return NK_ERR_INVALID_ARG;
  if (!head_dim_ok(c->head_dim) || !page_size_ok(c->page_size)) return NK_ERR_UNSUPPORTED;
  return NK_OK;
}

// Keys per split-KV chunk of a decode row: about 4096 single-wave work items
// over the batch at head_dim 128 (four per SIMD of a 256-CU part, all
// resident at once), proportionally fewer for wider heads (each step moves
// more bytes), chunks of 128..4096 keys, a multiple of 32.
int split_tokens(int num_seqs, int max_kv_len, int hq, int hkv, int head_dim, int window_left,
                 int requested) {
  if (requested > 0) return requested;
  const long long span = window_left < 0 ? max_kv_len : std::min<long long>(max_kv_len, (long long)window_left + 32);
  if (span <= 0) return 128;
  const long long rows = (long long)std::max(num_seqs, 1) * hkv * ((hq / hkv + 15) / 16);
  const long long target = 4096LL * 128 / std::max(head_dim, 1);
  const long long per_row = std::max(1LL, target / std::max(1LL, rows));
  long long s = (span + per_row - 1) / per_row;
  s = std::max(128LL, std::min(4096LL, s));
  return (int)((s + 31) / 32 * 32);
}

int max_chunks(int max_kv_len, int window_left, int split) {
  long long span = window_left < 0 ? max_kv_len : std::min<long long>(max_kv_len, (long long)window_left + 32);
  if (span <= 0) return 1;
  return (int)((span + split - 1) / split);
}

bool uses_split(int q_dtype, int cache_dtype) { return q_dtype == NK_BF16 && cache_dtype != NK_F32; }

// A windowed call may also attend to sink keys left of its band: those take
// one more split-KV chunk per decode row, which the workspace always reserves
// for windowed calls (the size query does not see the sink count).
bool sink_chunk_possible(int max_kv_len, int window_left) {
  return window_left >= 0 && (long long)max_kv_len > (long long)window_left + 1;
}

// Workspace: the split-KV partials of decode rows (when a row spans several
// chunks), then the prefill work list (when any row block may be a prefill
// one), each 256-byte aligned.
struct WorkspacePlan {
  int split = 0;
  int band_chunks = 1;      // chunks of a row's band
  int chunks = 1;           // capacity per row: band chunks + a sink chunk when possible
  size_t part_lse = 0, sched = 0, total = 0;
  bool partials = false, prefill = false;
};

WorkspacePlan plan_workspace(int q_dtype, int cache_dtype, int num_seqs, int total_q, int max_q_len,
                             int max_kv_len, int hq, int hkv, int head_dim, int window_left,
                             int requested_split) {
  WorkspacePlan w;
  w.split = split_tokens(num_seqs, max_kv_len, hq, hkv, head_dim, window_left, requested_split);
  w.band_chunks = max_chunks(max_kv_len, window_left, w.split);
  w.chunks = w.band_chunks + (sink_chunk_possible(max_kv_len, window_left) ? 1 : 0);
  if (!uses_split(q_dtype, cache_dtype)) return w;
  size_t off = 0;
  if (w.chunks > 1) {
    const size_t slots = (size_t)num_seqs * w.chunks;
    off = (slots * hq * head_dim * sizeof(float) + 255) / 256 * 256;     // partial outputs
    w.part_lse = off;
    off = (off + slots * hq * sizeof(float) + 255) / 256 * 256;          // partial lse
    w.partials = true;
  }
  if (max_q_len > 1) {
    w.sched = off;
    off = (off + sched_bytes(num_seqs, total_q) + 255) / 256 * 256;
    w.prefill = true;
  }
  w.total = off;
  return w;
}

// ------------------------------------------------------------------ profiling
// Timing-only events: no system-scope fence when recorded (no cache
// writeback and invalidation around the bracketed launch, which would cost
// the stream time and the kernel its warm caches).
constexpr unsigned kProfileEventFlags = hipEventDisableSystemFence;

struct ProfileState {
  std::mutex mu;
  int mask = 0;
  struct Rec { const char *family; hipEvent_t a, b; bool pending; };
  std::vector<Rec> recs;
  std::vector<std::pair<std::string, std::pair<double, int64_t>>> totals;
};
ProfileState &prof() {
  static ProfileState p;
  return p;
}

void flush_pending(ProfileState &p) {
  for (auto &r : p.recs) {
    if (!r.pending) continue;
    hipEventSynchronize(r.b);
    float ms = 0.f;
    hipEventElapsedTime(&ms, r.a, r.b);
    bool found = false;
    for (auto &t : p.totals)
      if (t.first == r.family) { t.second.first += ms; t.second.second += 1; found = true; }
    if (!found) p.totals.push_back({r.family, {ms, 1}});
    r.pending = false;
  }
}

}  // namespace

namespace nk {

static int family_bit(const char *family) {
  static const char *const names[] = {"rope_write", "attn_decode", "attn_prefill", "attn_f32", "lse_merge",
                                      "attention_pack", "attn_backward"};
  for (int i = 0; i < 7; ++i)
    if (std::strcmp(family, names[i]) == 0) return 1 << i;
  return 0;
}

namespace {
ProfileScope *&current_scope() {
  static thread_local ProfileScope *cur = nullptr;
  return cur;
}
}  // namespace

ProfileScope::ProfileScope(const char *family, hipStream_t) : slot(-1), outer(current_scope()) {
  current_scope() = this;
  ProfileState &p = prof();
  if (!(p.mask & family_bit(family))) return;
  std::lock_guard<std::mutex> lock(p.mu);
  int idx = -1;
  for (size_t i = 0; i < p.recs.size(); ++i)
    if (!p.recs[i].pending) { idx = (int)i; break; }
  if (idx < 0) {
    if (p.recs.size() >= 4096) flush_pending(p), idx = 0;
    else {
      ProfileState::Rec r{family, nullptr, nullptr, false};
      if (hipEventCreateWithFlags(&r.a, kProfileEventFlags) != hipSuccess ||
          hipEventCreateWithFlags(&r.b, kProfileEventFlags) != hipSuccess)
        return;
      p.recs.push_back(r);
      idx = (int)p.recs.size() - 1;
    }
  }
  p.recs[idx].family = family;
  p.recs[idx].pending = true;
  slot = idx;
}

void ProfileScope::launch_events(hipEvent_t *start, hipEvent_t *stop) {
  ProfileScope *ps = current_scope();
  if (!ps || ps->slot < 0) return;
  ProfileState &p = prof();
  std::lock_guard<std::mutex> lock(p.mu);
  if (!ps->started) *start = p.recs[ps->slot].a;
  *stop = p.recs[ps->slot].b;
  ps->started = ps->stopped = true;
}

ProfileScope::~ProfileScope() {
  current_scope() = outer;
  if (slot < 0 || (started && stopped)) return;
  ProfileState &p = prof();                  // nothing was launched: no record
  std::lock_guard<std::mutex> lock(p.mu);
  p.recs[slot].pending = false;
}

}  // namespace nk

// ------------------------------------------------------------------ static scratch
// The allocation-free attention entry point keeps its split-KV partials and
// prefill work list in this file-scope device array instead of a caller
// workspace: every device the library runs on holds one copy, at its own
// address, until the process ends.  In host code `scratch` only names the
// symbol; its device address comes from hipGetSymbolAddress, taken once per
// device (with that device current) and kept per device below; kernels are
// handed that address, never the symbol itself.
static __device__ __align__(256) uint8_t scratch[NK_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kStaticScratchBytes = NK_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__global__ void __launch_bounds__(256) zero_scratch_kernel(uint4 *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = uint4{0u, 0u, 0u, 0u};
}

struct StaticScratch {
  std::mutex mu;
  void *ptr[kMaxDevices] = {};
};
StaticScratch &static_scratch_state() {
  static StaticScratch st;
  return st;
}

// This device's scratch address; on the first call for a device it is looked
// up and the array cleared on `stream` (a fill kernel, so that the clearing
// may also be captured into a graph).
hipError_t static_scratch(hipStream_t stream, void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  StaticScratch &st = static_scratch_state();
  std::lock_guard<std::mutex> lock(st.mu);
  if (!st.ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    hipLaunchKernelGGL(zero_scratch_kernel, dim3(1024), dim3(256), 0, stream, (uint4 *)ptr,
                       kStaticScratchBytes / sizeof(uint4));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    st.ptr[dev] = ptr;
  }
  *out = st.ptr[dev];
  return hipSuccess;
}

// The attention call behind both entry points: the caller's workspace, or
// (use_static) this device's static scratch buffer.
int attention_call(const void *q, int32_t q_dtype, const int32_t *q_offsets, const int32_t *kv_lens,
                   const nk_paged_kv_t *cache, float softmax_scale, int32_t window_left, int32_t window_right,
                   int32_t sink_keys, void *out, float *lse, int32_t num_seqs, int32_t total_q, int32_t min_q_len,
                   int32_t max_q_len, int32_t max_kv_len, int32_t num_q_heads, int32_t kv_split_tokens,
                   void *workspace, size_t workspace_bytes_given, bool use_static, void *stream) {
  if (num_seqs < 0 || total_q < 0 || min_q_len < 0 || max_q_len < 0 || max_kv_len < 0 || num_q_heads <= 0)
    return NK_ERR_INVALID_ARG;
  if (min_q_len > max_q_len) return NK_ERR_INVALID_ARG;
  if (window_left < -1 || window_right < -1 || sink_keys < 0) return NK_ERR_INVALID_ARG;
  if (kv_split_tokens < 0 || kv_split_tokens % 32) return NK_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return NK_ERR_INVALID_ARG;
  int st = check_cache(cache);
  if (st != NK_OK) return st;
  if (num_q_heads % cache->num_kv_heads) return NK_ERR_INVALID_ARG;
  const bool ok_types = (q_dtype == NK_F32 && cache->dtype == NK_F32) ||
                        (q_dtype == NK_BF16 && (cache->dtype == NK_BF16 || cache->dtype == NK_E4M3));
  if (!ok_types) return NK_ERR_UNSUPPORTED;
  if (q_dtype == NK_BF16 && num_q_heads / cache->num_kv_heads > 64) return NK_ERR_UNSUPPORTED;
  if (total_q == 0) return NK_OK;
  if (num_seqs == 0) return NK_ERR_INVALID_ARG;
  if (!q || !q_offsets || !kv_lens || !out) return NK_ERR_INVALID_ARG;

  AttnArgs a{};
  a.q = q; a.q_dtype = q_dtype; a.q_offsets = q_offsets; a.kv_lens = kv_lens;
  a.cache = *cache; a.softmax_scale = softmax_scale;
  a.window_left = window_left; a.window_right = window_right;
  a.sink_keys = window_left < 0 ? 0 : sink_keys;     // a full left side already holds them
  a.out = out; a.lse = lse;
  a.num_seqs = num_seqs; a.total_q = total_q; a.max_q_len = max_q_len; a.max_kv_len = max_kv_len;
  a.hq = num_q_heads;

  if (q_dtype == NK_F32) return launch_attn_f32(a, (hipStream_t)stream) == hipSuccess ? NK_OK : NK_ERR_DEVICE;

  const WorkspacePlan wp = plan_workspace(q_dtype, cache->dtype, num_seqs, total_q, max_q_len,
                                         max_kv_len, num_q_heads, cache->num_kv_heads,
                                         cache->head_dim, window_left, kv_split_tokens);
  hipStream_t s = (hipStream_t)stream;
  if (use_static) {
    if (wp.total > kStaticScratchBytes) return NK_ERR_WORKSPACE;
    if (wp.total > 0) {
      if (static_scratch(s, &workspace) != hipSuccess) return NK_ERR_DEVICE;
      workspace_bytes_given = kStaticScratchBytes;
    }
  }
  if (wp.total > 0 && (!workspace || workspace_bytes_given < wp.total)) return NK_ERR_WORKSPACE;
  a.split_tokens = wp.split;
  // grid and partials stride: the sink chunk only when there are sink keys
  a.max_chunks = a.sink_keys > 0 ? wp.chunks : wp.band_chunks;
  if (wp.partials) {
    a.part_out = (float *)workspace;
    a.part_lse = (float *)((char *)workspace + wp.part_lse);
  }
  if (wp.prefill) {
    a.sched = (int32_t *)((char *)workspace + wp.sched);
    a.sched_items_max = sched_items_max(num_seqs, total_q);
  }
  // prefill rows (q_len > 1) and decode rows (q_len == 1) run as separate
  // launches on the same stream; each kernel skips the rows of the other
  // kind.  The host bounds say which kinds a batch can hold: no prefill
  // launch when max_q_len <= 1, no decode launch (nor merge) when
  // min_q_len >= 2.
  const bool decode_rows = min_q_len <= 1;
  if (wp.prefill && launch_attn_prefill(a, s) != hipSuccess) return NK_ERR_DEVICE;
  if (decode_rows && launch_attn_decode(a, s) != hipSuccess) return NK_ERR_DEVICE;
  if (decode_rows && wp.partials && launch_decode_merge(a, s) != hipSuccess) return NK_ERR_DEVICE;
  return NK_OK;
}

}  // namespace

extern "C" {

const char *nk_status_string(int status) {
  switch (status) {
    case NK_OK: return "ok";
    case NK_ERR_INVALID_ARG: return "invalid argument";
    case NK_ERR_UNSUPPORTED: return "unsupported configuration";
    case NK_ERR_WORKSPACE: return "workspace missing or too small";
    case NK_ERR_DEVICE: return "device launch failed";
    default: return "unknown status";
  }
}

int nk_version(void) { return kVersion; }

int nk_rope_qk_write_paged(const void *q, const void *k, const void *v, int32_t in_dtype,
                           void *q_out, const int32_t *q_offsets, const int32_t *kv_lens,
                           const int32_t *position_ids, const float *freqs, int32_t max_pos,
                           int32_t rotary_dim, int32_t layout, int32_t num_seqs,
                           int32_t total_tokens, int32_t num_q_heads,
                           const nk_paged_kv_t *cache, void *stream) {
  return nk_rope_qk_write_paged_mrope(q, k, v, in_dtype, q_out, q_offsets, kv_lens, position_ids, 0, nullptr,
                                      freqs, max_pos, rotary_dim, layout, num_seqs, total_tokens,
                                      num_q_heads, cache, stream);
}

int nk_rope_qk_write_paged_mrope(const void *q, const void *k, const void *v, int32_t in_dtype,
                                 void *q_out, const int32_t *q_offsets, const int32_t *kv_lens,
                                 const int32_t *position_ids, int32_t num_sections,
                                 const int32_t *section_pairs_host, const float *freqs, int32_t max_pos,
                                 int32_t rotary_dim, int32_t layout, int32_t num_seqs,
                                 int32_t total_tokens, int32_t num_q_heads,
                                 const nk_paged_kv_t *cache, void *stream) {
  if (num_seqs < 0 || total_tokens < 0 || num_q_heads <= 0 || max_pos <= 0) return NK_ERR_INVALID_ARG;
  if (num_sections < 0 || num_sections > kMaxMropeSections) return NK_ERR_INVALID_ARG;
  int32_t mrope_end[kMaxMropeSections] = {};
  if (num_sections > 0) {
    if (!section_pairs_host || !position_ids) return NK_ERR_INVALID_ARG;
    int32_t sum = 0;
    for (int s = 0; s < num_sections; ++s) {
      if (section_pairs_host[s] <= 0 || section_pairs_host[s] % 8) return NK_ERR_UNSUPPORTED;
      sum += section_pairs_host[s];
      mrope_end[s] = sum;
    }
    if (sum != rotary_dim / 2) return NK_ERR_INVALID_ARG;
  }
  int st = check_cache(cache);
  if (st != NK_OK) return st;
  if (num_q_heads % cache->num_kv_heads) return NK_ERR_INVALID_ARG;
  if (layout != NK_ROPE_HALF && layout != NK_ROPE_INTERLEAVED && layout != NK_ROPE_HALF_PROPORTIONAL)
    return NK_ERR_INVALID_ARG;
  if (rotary_dim <= 0 || rotary_dim > cache->head_dim || rotary_dim % 16) return NK_ERR_UNSUPPORTED;
  const bool ok_types = (in_dtype == NK_F32 && cache->dtype == NK_F32) ||
                        (in_dtype == NK_BF16 && (cache->dtype == NK_BF16 || cache->dtype == NK_E4M3));
  if (!ok_types) return NK_ERR_UNSUPPORTED;
  if (total_tokens == 0) return NK_OK;
  if (num_seqs == 0) return NK_ERR_INVALID_ARG;
  if (!q || !k || !v || !q_out || !q_offsets || !kv_lens || !freqs) return NK_ERR_INVALID_ARG;
  RopeArgs a{};
  a.q = q; a.k = k; a.v = v; a.q_out = q_out;
  a.q_offsets = q_offsets; a.kv_lens = kv_lens; a.position_ids = position_ids;
  a.freqs = freqs; a.rotary_dim = rotary_dim; a.layout = layout; a.in_dtype = in_dtype;
  a.max_pos = max_pos;
  a.num_seqs = num_seqs; a.total_tokens = total_tokens; a.hq = num_q_heads;
  a.cache = *cache;
  a.mrope_sections = num_sections;
  for (int s = 0; s < kMaxMropeSections; ++s) a.mrope_end[s] = mrope_end[s];
  return launch_rope_write(a, (hipStream_t)stream) == hipSuccess ? NK_OK : NK_ERR_DEVICE;
}

size_t nk_ragged_paged_attention_workspace_size(int32_t q_dtype, int32_t cache_dtype,
                                                int32_t num_seqs, int32_t total_q,
                                                int32_t max_q_len, int32_t max_kv_len,
                                                int32_t num_q_heads, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t window_left,
                                                int32_t kv_split_tokens) {
  if (num_seqs <= 0 || total_q < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_kv_len <= 0)
    return 0;
  return plan_workspace(q_dtype, cache_dtype, num_seqs, total_q, max_q_len, max_kv_len, num_q_heads,
                        num_kv_heads, head_dim, window_left, kv_split_tokens).total;
}

int32_t nk_ragged_paged_attention_split_tokens(int32_t num_seqs, int32_t max_kv_len,
                                               int32_t num_q_heads, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t window_left,
                                               int32_t kv_split_tokens) {
  return split_tokens(num_seqs, max_kv_len, num_q_heads, num_kv_heads, head_dim, window_left,
                      kv_split_tokens);
}

int nk_ragged_paged_attention(const void *q, int32_t q_dtype, const int32_t *q_offsets,
                              const int32_t *kv_lens, const nk_paged_kv_t *cache,
                              float softmax_scale, int32_t window_left, void *out, float *lse,
                              int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                              int32_t max_kv_len, int32_t num_q_heads, int32_t kv_split_tokens,
                              void *workspace, size_t workspace_bytes_given, void *stream) {
  return nk_ragged_paged_attention_band(q, q_dtype, q_offsets, kv_lens, cache, softmax_scale, window_left, 0,
                                        0, out, lse, num_seqs, total_q, 0, max_q_len, max_kv_len, num_q_heads,
                                        kv_split_tokens, workspace, workspace_bytes_given, stream);
}

int nk_ragged_paged_attention_band(const void *q, int32_t q_dtype, const int32_t *q_offsets,
                                   const int32_t *kv_lens, const nk_paged_kv_t *cache,
                                   float softmax_scale, int32_t window_left, int32_t window_right,
                                   int32_t sink_keys, void *out, float *lse, int32_t num_seqs, int32_t total_q,
                                   int32_t min_q_len, int32_t max_q_len, int32_t max_kv_len, int32_t num_q_heads,
                                   int32_t kv_split_tokens, void *workspace,
                                   size_t workspace_bytes_given, void *stream) {
  return attention_call(q, q_dtype, q_offsets, kv_lens, cache, softmax_scale, window_left, window_right, sink_keys,
                        out, lse, num_seqs, total_q, min_q_len, max_q_len, max_kv_len, num_q_heads, kv_split_tokens,
                        workspace, workspace_bytes_given, false, stream);
}

int nk_ragged_paged_attention_noalloc(const void *q, int32_t q_dtype, const int32_t *q_offsets,
                                      const int32_t *kv_lens, const nk_paged_kv_t *cache,
                                      float softmax_scale, int32_t window_left, int32_t window_right,
                                      int32_t sink_keys, void *out, float *lse, int32_t num_seqs,
                                      int32_t total_q, int32_t min_q_len, int32_t max_q_len, int32_t max_kv_len,
                                      int32_t num_q_heads, int32_t kv_split_tokens, void *stream) {
  return attention_call(q, q_dtype, q_offsets, kv_lens, cache, softmax_scale, window_left, window_right, sink_keys,
                        out, lse, num_seqs, total_q, min_q_len, max_q_len, max_kv_len, num_q_heads, kv_split_tokens,
                        nullptr, 0, true, stream);
}

int nk_attention_pack(const void *k, const void *v, int32_t in_dtype, const int32_t *key_offsets,
                      const int32_t *key_lengths, const nk_paged_kv_t *cache, int32_t *kv_lens_out,
                      int32_t num_seqs, int32_t max_key_len, void *stream) {
  if (num_seqs < 0 || max_key_len < 0) return NK_ERR_INVALID_ARG;
  int st = check_cache(cache);
  if (st != NK_OK) return st;
  const bool ok_types = (in_dtype == NK_F32 && cache->dtype == NK_F32) ||
                        (in_dtype == NK_BF16 && (cache->dtype == NK_BF16 || cache->dtype == NK_E4M3));
  if (!ok_types) return NK_ERR_UNSUPPORTED;
  if (num_seqs == 0) return NK_OK;
  if (!key_offsets || !kv_lens_out) return NK_ERR_INVALID_ARG;
  if (max_key_len > 0 && (!k || !v || cache->num_pages <= 0)) return NK_ERR_INVALID_ARG;
  if ((long long)cache->page_table_stride * cache->page_size < (long long)max_key_len) return NK_ERR_INVALID_ARG;
  PackArgs a{};
  a.k = k; a.v = v; a.in_dtype = in_dtype;
  a.key_offsets = key_offsets; a.key_lengths = key_lengths;
  a.cache = *cache; a.kv_lens_out = kv_lens_out;
  a.num_seqs = num_seqs; a.max_key_len = max_key_len;
  return launch_attention_pack(a, (hipStream_t)stream) == hipSuccess ? NK_OK : NK_ERR_DEVICE;
}

int nk_ragged_paged_attention_backward(const void *q, int32_t q_dtype, const int32_t *q_offsets,
                                       const int32_t *kv_lens, const nk_paged_kv_t *cache, float softmax_scale,
                                       int32_t window_left, int32_t window_right, int32_t sink_keys,
                                       const void *out, const void *dout, const float *lse,
                                       const int32_t *key_offsets, float *dq, float *dk, float *dv,
                                       int32_t num_seqs, int32_t total_q, int32_t max_kv_len,
                                       int32_t num_q_heads, void *stream) {
  if (num_seqs < 0 || total_q < 0 || max_kv_len < 0 || num_q_heads <= 0) return NK_ERR_INVALID_ARG;
  if (window_left < -1 || window_right < -1 || sink_keys < 0) return NK_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return NK_ERR_INVALID_ARG;
  int st = check_cache(cache);
  if (st != NK_OK) return st;
  if (num_q_heads % cache->num_kv_heads) return NK_ERR_INVALID_ARG;
  const bool ok_types = (q_dtype == NK_F32 && cache->dtype == NK_F32) ||
                        (q_dtype == NK_BF16 && cache->dtype == NK_BF16);
  if (!ok_types) return NK_ERR_UNSUPPORTED;
  if (num_seqs == 0) return total_q == 0 ? NK_OK : NK_ERR_INVALID_ARG;
  if (!q_offsets || !kv_lens || !key_offsets) return NK_ERR_INVALID_ARG;
  if (total_q > 0 && (!q || !out || !dout || !lse || !dq)) return NK_ERR_INVALID_ARG;
  if (max_kv_len > 0 && (!dk || !dv)) return NK_ERR_INVALID_ARG;
  BackwardArgs a{};
  a.q = q; a.out = out; a.dout = dout; a.q_dtype = q_dtype; a.lse = lse;
  a.q_offsets = q_offsets; a.kv_lens = kv_lens; a.key_offsets = key_offsets;
  a.cache = *cache; a.softmax_scale = softmax_scale;
  a.window_left = window_left; a.window_right = window_right; a.sink_keys = sink_keys;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.num_seqs = num_seqs; a.total_q = total_q; a.max_kv_len = max_kv_len; a.hq = num_q_heads;
  return launch_attn_backward(a, (hipStream_t)stream) == hipSuccess ? NK_OK : NK_ERR_DEVICE;
}

int nk_attention_lse_merge(const float *partial_out, const float *partial_lse,
                           const int32_t *merge_offsets, int32_t num_rows, int32_t num_heads,
                           int32_t head_dim, void *out, int32_t out_dtype, float *lse_out,
                           void *stream) {
  if (num_rows < 0 || num_heads <= 0 || head_dim <= 0 || head_dim % 2 || head_dim > 512)
    return NK_ERR_INVALID_ARG;
  if (out_dtype != NK_F32 && out_dtype != NK_BF16) return NK_ERR_UNSUPPORTED;
  if (num_rows == 0) return NK_OK;
  if (!partial_out || !partial_lse || !merge_offsets || !out) return NK_ERR_INVALID_ARG;
  return launch_lse_merge(partial_out, partial_lse, merge_offsets, num_rows, num_heads, head_dim,
                          out, out_dtype, lse_out, (hipStream_t)stream) == hipSuccess
             ? NK_OK : NK_ERR_DEVICE;
}

int nk_profile_enable(int family_mask) {
  if (family_mask & ~NK_PROF_ALL) return NK_ERR_INVALID_ARG;
  prof().mask = family_mask;
  return NK_OK;
}

int nk_profile_reset(void) {
  ProfileState &p = prof();
  std::lock_guard<std::mutex> lock(p.mu);
  flush_pending(p);
  p.totals.clear();
  return NK_OK;
}

int nk_profile_read(const char *kernel, double *total_ms_host, int64_t *launches_host) {
  if (!kernel || !total_ms_host || !launches_host) return NK_ERR_INVALID_ARG;
  ProfileState &p = prof();
  std::lock_guard<std::mutex> lock(p.mu);
  flush_pending(p);
  *total_ms_host = 0.0;
  *launches_host = 0;
  for (auto &t : p.totals)
    if (t.first == kernel) { *total_ms_host = t.second.first; *launches_host = t.second.second; }
  return NK_OK;
}

}  // extern "C"
