// Stand-ins for the kernel launchers, so that the C-ABI layer (api.hip) links
// into a host-only program built with AddressSanitizer and UBSan.  The
// checks in abi_checks.cpp only reach paths that return before any launch;
// every stand-in reports failure if it is ever called.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#include "../../ragged_paged_kv_amd/csrc/internal.h"

namespace nk {
static hipError_t called(const char *what) {
  std::fprintf(stderr, "unexpected launch: %s\n", what);
  std::abort();
}
hipError_t launch_rope_write(const RopeArgs &, hipStream_t) { return called("rope_write"); }
hipError_t launch_attn_backward(const BackwardArgs &, hipStream_t) { return called("attn_backward"); }
hipError_t launch_attention_pack(const PackArgs &, hipStream_t) { return called("attention_pack"); }
hipError_t launch_attn_f32(const AttnArgs &, hipStream_t) { return called("attn_f32"); }
hipError_t launch_attn_decode(const AttnArgs &, hipStream_t) { return called("attn_decode"); }
hipError_t launch_attn_prefill(const AttnArgs &, hipStream_t) { return called("attn_prefill"); }
hipError_t launch_decode_merge(const AttnArgs &, hipStream_t) { return called("decode_merge"); }
hipError_t launch_lse_merge(const float *, const float *, const int32_t *, int32_t, int32_t, int32_t, void *,
                            int32_t, float *, hipStream_t) {
  return called("lse_merge");
}
}  // namespace nk
