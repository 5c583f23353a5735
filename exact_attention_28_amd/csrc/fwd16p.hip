// fwd16p.hip — the pipelined 16-bit forward's launches (kernel and launch
// shapes in fwd16p_kernel.h).

#include "fwd16p_kernel.h"

namespace xattn {

bool fwd16_pipelined_enabled() {
  const char* env = std::getenv("ATTN_FWD_PIPELINE");
  return env == nullptr || std::atoi(env) != 0;
}

hipError_t launch_fwd16_pipelined(const void* q, const void* k, const void* v, void* o,
                                  float* lse, int B, int Hq, int Hkv, int Sq, int Skv, int D,
                                  int causal, float scale, const double2* rope_tab, int dtype,
                                  hipStream_t stream, const int* kv_lens, int kv_rows) {
  return launch_fwdp<false>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale, rope_tab,
                            dtype, stream, kv_lens, kv_rows);
}

}  // namespace xattn
