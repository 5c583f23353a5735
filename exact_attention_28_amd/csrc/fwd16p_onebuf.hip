// fwd16p_onebuf.hip — the single-buffer instances of the pipelined 16-bit
// forward (fwd16p_kernel.h), a check of its LDS double buffering: same
// arguments and, bit for bit, the same results as launch_fwd16_pipelined.
// Compiled on their own so that the two sets of instances build in parallel.

#include "fwd16p_kernel.h"

namespace xattn {

hipError_t launch_fwd16_pipelined_onebuf(const void* q, const void* k, const void* v, void* o,
                                         float* lse, int B, int Hq, int Hkv, int Sq, int Skv,
                                         int D, int causal, float scale, const double2* rope_tab,
                                         int dtype, hipStream_t stream, const int* kv_lens,
                                         int kv_rows) {
  return launch_fwdp<true>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale, rope_tab,
                           dtype, stream, kv_lens, kv_rows);
}

}  // namespace xattn
