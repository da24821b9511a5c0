// Host-side checks of the C ABI's validation paths, built with
// AddressSanitizer and UndefinedBehaviorSanitizer (host code only) by
// tests/test_host_sanitizer.py.  Every call here must return before any
// device work: pointers are non-null stand-ins that the host never
// dereferences, and the kernel launchers are stand-ins that abort if called.
// Exit status: the number of failed checks (0 = all passed).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "../../include/nk.h"

static int failures = 0;
static void expect(int got, int want, const char *what, int line) {
  if (got != want) {
    std::fprintf(stderr, "line %d: %s: status %d, expected %d\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

static void *P = (void *)0x1000;              // never dereferenced on the host
static const int32_t *PI = (const int32_t *)0x1000;

static nk_paged_kv_t cache(int dtype = NK_BF16, int head_dim = 128, int page_size = 16, int heads = 2) {
  nk_paged_kv_t c;
  std::memset(&c, 0, sizeof c);
  c.k_pages = P;
  c.v_pages = P;
  c.k_scales = dtype == NK_E4M3 ? (float *)P : nullptr;
  c.v_scales = dtype == NK_E4M3 ? (float *)P : nullptr;
  c.dtype = dtype;
  c.num_pages = 4;
  c.page_size = page_size;
  c.num_kv_heads = heads;
  c.head_dim = head_dim;
  c.page_table = PI;
  c.page_table_stride = 4;
  return c;
}

static int rope(const nk_paged_kv_t *c, int in_dtype = NK_BF16, int rotary = 128, int seqs = 1, int hq = 4,
                const void *q = P) {
  return nk_rope_qk_write_paged(q, P, P, in_dtype, P, PI, PI, nullptr, (const float *)P, 16, rotary, NK_ROPE_HALF,
                                seqs, 4, hq, c, nullptr);
}

static int band(const nk_paged_kv_t *c, int q_dtype = NK_BF16, float scale = 0.1f, int wl = -1, int wr = 0,
                int sinks = 0, int seqs = 1, int min_q = 0, int max_q = 4, int max_kv = 64, int hq = 4,
                int split = 0, void *ws = nullptr, size_t ws_bytes = 0, void *out = P) {
  return nk_ragged_paged_attention_band(P, q_dtype, PI, PI, c, scale, wl, wr, sinks, out, nullptr, seqs, 4, min_q,
                                        max_q, max_kv, hq, split, ws, ws_bytes, nullptr);
}

int main() {
  // ---- status strings, version
  for (int s = -3; s < 8; ++s) {
    const char *t = nk_status_string(s);
    if (!t || !*t) { std::fprintf(stderr, "empty status string %d\n", s); ++failures; }
  }
  if (nk_version() < 10000) { std::fprintf(stderr, "version\n"); ++failures; }

  const nk_paged_kv_t c = cache();
  // ---- RoPE + append
  EXPECT(rope(nullptr), NK_ERR_INVALID_ARG);
  EXPECT(rope(&c, NK_BF16, 130), NK_ERR_UNSUPPORTED);          // rotary_dim not a multiple of 16
  EXPECT(rope(&c, NK_BF16, 256), NK_ERR_UNSUPPORTED);          // beyond head_dim
  EXPECT(rope(&c, NK_BF16, 128, -1), NK_ERR_INVALID_ARG);
  EXPECT(rope(&c, NK_BF16, 128, 1, 3), NK_ERR_INVALID_ARG);    // heads not a multiple of KV heads
  EXPECT(rope(&c, NK_F32), NK_ERR_UNSUPPORTED);                // f32 input into a bf16 cache
  EXPECT(rope(&c, NK_BF16, 128, 1, 4, nullptr), NK_ERR_INVALID_ARG);
  EXPECT(rope(&c, 7), NK_ERR_UNSUPPORTED);
  {
    nk_paged_kv_t bad = cache(NK_BF16, 96);
    EXPECT(rope(&bad), NK_ERR_UNSUPPORTED);
    bad = cache(NK_BF16, 128, 24);
    EXPECT(rope(&bad), NK_ERR_UNSUPPORTED);
    bad = cache(NK_E4M3);
    bad.v_scales = nullptr;
    EXPECT(rope(&bad), NK_ERR_INVALID_ARG);
    bad = cache(9);
    EXPECT(rope(&bad), NK_ERR_UNSUPPORTED);
    bad = cache();
    bad.num_kv_heads = 0;
    EXPECT(rope(&bad), NK_ERR_INVALID_ARG);
  }
  {
    const int32_t five[5] = {16, 16, 16, 8, 8}, odd[3] = {16, 20, 28}, short_sum[2] = {16, 16};
    EXPECT(nk_rope_qk_write_paged_mrope(P, P, P, NK_BF16, P, PI, PI, PI, 5, five, (const float *)P, 16, 128,
                                        NK_ROPE_HALF, 1, 4, 4, &c, nullptr), NK_ERR_INVALID_ARG);
    EXPECT(nk_rope_qk_write_paged_mrope(P, P, P, NK_BF16, P, PI, PI, PI, 3, odd, (const float *)P, 16, 128,
                                        NK_ROPE_HALF, 1, 4, 4, &c, nullptr), NK_ERR_UNSUPPORTED);
    EXPECT(nk_rope_qk_write_paged_mrope(P, P, P, NK_BF16, P, PI, PI, PI, 2, short_sum, (const float *)P, 16, 128,
                                        NK_ROPE_HALF, 1, 4, 4, &c, nullptr), NK_ERR_INVALID_ARG);
    EXPECT(nk_rope_qk_write_paged_mrope(P, P, P, NK_BF16, P, PI, PI, nullptr, 2, short_sum, (const float *)P, 16,
                                        64, NK_ROPE_HALF, 1, 4, 4, &c, nullptr), NK_ERR_INVALID_ARG);
  }

  // ---- attention
  EXPECT(band(nullptr), NK_ERR_INVALID_ARG);
  EXPECT(band(&c, NK_BF16, std::numeric_limits<float>::quiet_NaN()), NK_ERR_INVALID_ARG);
  EXPECT(band(&c, NK_BF16, std::numeric_limits<float>::infinity()), NK_ERR_INVALID_ARG);
  EXPECT(band(&c, NK_BF16, 0.1f, -2), NK_ERR_INVALID_ARG);
  EXPECT(band(&c, NK_BF16, 0.1f, -1, -2), NK_ERR_INVALID_ARG);
  EXPECT(band(&c, NK_BF16, 0.1f, 8, 0, -1), NK_ERR_INVALID_ARG);
  EXPECT(band(&c, NK_BF16, 0.1f, -1, 0, 0, 0), NK_ERR_INVALID_ARG);            // no sequences
  EXPECT(band(&c, NK_BF16, 0.1f, -1, 0, 0, 1, 5, 4), NK_ERR_INVALID_ARG);     // min_q_len > max_q_len
  EXPECT(band(&c, NK_BF16, 0.1f, -1, 0, 0, 1, 0, 4, 64, 3), NK_ERR_INVALID_ARG);
  EXPECT(band(&c, NK_BF16, 0.1f, -1, 0, 0, 1, 0, 4, 64, 4, 48), NK_ERR_INVALID_ARG);   // split not /32
  EXPECT(band(&c, NK_BF16, 0.1f, -1, 0, 0, 1, 0, 4, 64, 4, 0, nullptr, 0, nullptr), NK_ERR_INVALID_ARG);
  EXPECT(band(&c, NK_BF16, 0.1f, -1, 0, 0, 1, 0, 4, 64, 2 * 65), NK_ERR_UNSUPPORTED);  // group > 64
  EXPECT(band(&c, NK_F32), NK_ERR_UNSUPPORTED);                                 // f32 q over bf16 pages
  {
    // a decode + prefill call needs a workspace: none, then one byte short
    const size_t need = nk_ragged_paged_attention_workspace_size(NK_BF16, NK_BF16, 1, 4, 4, 4096, 4, 2, 128, -1, 0);
    if (need == 0) { std::fprintf(stderr, "workspace size 0\n"); ++failures; }
    EXPECT(band(&c, NK_BF16, 0.1f, -1, 0, 0, 1, 0, 4, 4096), NK_ERR_WORKSPACE);
    EXPECT(band(&c, NK_BF16, 0.1f, -1, 0, 0, 1, 0, 4, 4096, 4, 0, P, need - 1), NK_ERR_WORKSPACE);
    // the no-allocation call rejects a batch whose workspace exceeds its array
    EXPECT(nk_ragged_paged_attention_noalloc(P, NK_BF16, PI, PI, &c, 0.1f, -1, 0, 0, P, nullptr, 4096, 4096, 0, 1,
                                             1 << 20, 4, 128, nullptr), NK_ERR_WORKSPACE);
    EXPECT(nk_ragged_paged_attention(P, NK_BF16, PI, PI, &c, 0.1f, -1, P, nullptr, 1, 4, 4, 4096, 4, 0, nullptr, 0,
                                     nullptr), NK_ERR_WORKSPACE);
  }
  // host planning queries over extreme sizes (UBSan watches the arithmetic)
  {
    const int32_t big = std::numeric_limits<int32_t>::max();
    volatile size_t sink = 0;
    for (int seqs : {1, 7, 4096, big})
      for (int kv : {0, 1, 4096, big})
        for (int wl : {-1, 0, 1023, big - 1})
          for (int split : {0, 32, 4096}) {
            sink += nk_ragged_paged_attention_workspace_size(NK_BF16, NK_E4M3, seqs, seqs, 1, kv, 64, 8, 128, wl,
                                                             split);
            sink += (size_t)nk_ragged_paged_attention_split_tokens(seqs, kv, 64, 8, 256, wl, split);
          }
    (void)sink;
  }

  // ---- merge
  EXPECT(nk_attention_lse_merge(nullptr, (float *)P, PI, 1, 1, 128, P, NK_BF16, nullptr, nullptr),
         NK_ERR_INVALID_ARG);
  EXPECT(nk_attention_lse_merge((float *)P, (float *)P, PI, 1, 1, 128, P, NK_E4M3, nullptr, nullptr),
         NK_ERR_UNSUPPORTED);
  EXPECT(nk_attention_lse_merge((float *)P, (float *)P, PI, -1, 1, 128, P, NK_BF16, nullptr, nullptr),
         NK_ERR_INVALID_ARG);
  EXPECT(nk_attention_lse_merge((float *)P, (float *)P, PI, 1, 1, 129, P, NK_BF16, nullptr, nullptr),
         NK_ERR_INVALID_ARG);
  EXPECT(nk_attention_lse_merge((float *)P, (float *)P, PI, 0, 1, 128, P, NK_BF16, nullptr, nullptr), NK_OK);

  // ---- pack
  {
    int32_t *lens_out = (int32_t *)P;
    EXPECT(nk_attention_pack(P, P, NK_BF16, nullptr, nullptr, &c, lens_out, 1, 16, nullptr), NK_ERR_INVALID_ARG);
    EXPECT(nk_attention_pack(P, P, NK_BF16, PI, nullptr, &c, lens_out, -1, 16, nullptr), NK_ERR_INVALID_ARG);
    EXPECT(nk_attention_pack(P, P, NK_F32, PI, nullptr, &c, lens_out, 1, 16, nullptr), NK_ERR_UNSUPPORTED);
    EXPECT(nk_attention_pack(P, P, NK_BF16, PI, nullptr, &c, lens_out, 1, 4 * 16 + 1, nullptr),
           NK_ERR_INVALID_ARG);                                              // beyond the table's row
    EXPECT(nk_attention_pack(P, P, NK_BF16, PI, nullptr, nullptr, lens_out, 1, 16, nullptr), NK_ERR_INVALID_ARG);
  }

  // ---- backward
  {
    const nk_paged_kv_t e = cache(NK_E4M3);
    float *F = (float *)P;
    EXPECT(nk_ragged_paged_attention_backward(P, NK_BF16, PI, PI, &e, 0.1f, -1, 0, 0, P, P, F, PI, F, F, F, 1, 4,
                                              64, 4, nullptr), NK_ERR_UNSUPPORTED);
    EXPECT(nk_ragged_paged_attention_backward(P, NK_BF16, PI, PI, &c, NAN, -1, 0, 0, P, P, F, PI, F, F, F, 1, 4, 64,
                                              4, nullptr), NK_ERR_INVALID_ARG);
    EXPECT(nk_ragged_paged_attention_backward(P, NK_BF16, PI, PI, &c, 0.1f, -1, 0, 0, P, P, F, PI, nullptr, F, F, 1,
                                              4, 64, 4, nullptr), NK_ERR_INVALID_ARG);
    EXPECT(nk_ragged_paged_attention_backward(P, NK_BF16, PI, PI, &c, 0.1f, -1, 0, 0, P, P, F, PI, F, nullptr, F,
                                              1, 4, 64, 4, nullptr), NK_ERR_INVALID_ARG);
    EXPECT(nk_ragged_paged_attention_backward(P, NK_BF16, PI, PI, &c, 0.1f, -1, 0, 0, P, P, F, PI, F, F, F, 0, 0,
                                              0, 4, nullptr), NK_OK);        // nothing to do
    EXPECT(nk_ragged_paged_attention_backward(P, NK_BF16, PI, PI, &c, 0.1f, -1, 0, 0, P, P, F, PI, F, F, F, 0, 3,
                                              0, 4, nullptr), NK_ERR_INVALID_ARG);
  }

  // ---- timing diagnostics (host state only)
  EXPECT(nk_profile_enable(1 << 12), NK_ERR_INVALID_ARG);
  EXPECT(nk_profile_enable(0), NK_OK);
  EXPECT(nk_profile_reset(), NK_OK);
  {
    double ms = -1.0;
    int64_t n = -1;
    EXPECT(nk_profile_read(nullptr, &ms, &n), NK_ERR_INVALID_ARG);
    EXPECT(nk_profile_read("attn_decode", nullptr, &n), NK_ERR_INVALID_ARG);
    EXPECT(nk_profile_read("attn_decode", &ms, &n), NK_OK);
    if (ms != 0.0 || n != 0) { std::fprintf(stderr, "profile totals not zero\n"); ++failures; }
    ms = -1.0;
    n = -1;
    EXPECT(nk_profile_read("no_such_family", &ms, &n), NK_OK);       // a name never timed reads as zero
    if (ms != 0.0 || n != 0) { std::fprintf(stderr, "unknown family not zero\n"); ++failures; }
  }

  std::printf("abi checks: %d failed\n", failures);
  return failures;
}
