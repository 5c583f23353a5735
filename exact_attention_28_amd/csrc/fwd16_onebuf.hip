// fwd16_onebuf.hip — the single-buffer instances of the masked / key-split
// 16-bit forward (fwd16_kernel.h), a check of its LDS double buffering: same
// arguments and, bit for bit, the same results as launch_fwd16's own
// launches.  Compiled on their own so that the two sets of instances build in
// parallel.

#include "fwd16_kernel.h"

namespace xattn {

hipError_t launch_fwd16_onebuf(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                               float scale, const double2* rope_tab, int dtype, hipStream_t stream,
                               const int* kv_lens, int kv_rows, MaskView mask, KeySplit ks) {
  return launch_fwd16_kernel<true>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale,
                                   rope_tab, dtype, stream, kv_lens, kv_rows, mask, ks);
}

}  // namespace xattn
