// fwd16.hip — launches of the 16-bit forward (kernel and launch shapes in
// fwd16_kernel.h, the pipelined kernel in fwd16p_kernel.h) and the merge of
// its key splits.

#include "fwd16_kernel.h"

namespace xattn {

// Merge of the key splits: row r (O's row order) gets L = log sum_i exp(lse_i)
// over its partial LSEs (empty runs carry -inf and weigh 0) and
// O = sum_i exp(lse_i - L) O_i, stored in the input format; the LSE (nullable)
// goes to [B, Hq, Sq].  A row with every run empty gets O = 0, LSE = -inf.
// D / 4 threads per row, 16 bytes of each partial per thread.
template <typename T, int D>
__global__ __launch_bounds__(256) void fwd16_combine_kernel(const float* __restrict__ Op,
                                                            const float* __restrict__ Lp,
                                                            u16* __restrict__ O,
                                                            float* __restrict__ LSE,
                                                            long long rows, int Sq, int Hq,
                                                            int ns) {
  constexpr int TPR = D / 4;
  const long long r = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int d = (threadIdx.x % TPR) * 4;
  if (r >= rows) return;
  const float* lp = Lp + r * ns;
  float m2 = -INFINITY;  // in log2 units
  for (int i = 0; i < ns; ++i) m2 = fmaxf(m2, lp[i] * kLog2e);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float L2 = -INFINITY;
  if (m2 != -INFINITY) {
    float sum = 0.f;
    for (int i = 0; i < ns; ++i) sum += __builtin_amdgcn_exp2f(lp[i] * kLog2e - m2);
    L2 = m2 + __log2f(sum);
    for (int i = 0; i < ns; ++i) {
      const float wgt = __builtin_amdgcn_exp2f(lp[i] * kLog2e - L2);
      const f32x4 x = *reinterpret_cast<const f32x4*>(Op + (r * ns + i) * D + d);
      acc += wgt * x;
    }
  }
  u32x2 pk;
  pk[0] = Fmt16<T>::pack(acc[0], acc[1]);
  pk[1] = Fmt16<T>::pack(acc[2], acc[3]);
  *reinterpret_cast<u32x2*>(O + r * D + d) = pk;
  if (LSE != nullptr && d == 0) {
    const long long bs = r / Hq;  // b * Sq + pos
    LSE[((bs / Sq) * Hq + r % Hq) * Sq + bs % Sq] = L2 * kLn2;
  }
}

hipError_t launch_fwd16_merge(const float* op, const float* lp, void* o, float* lse,
                              long long rows, int Sq, int Hq, int ns, int D, int dtype,
                              hipStream_t stream) {
#define XATTN_MERGE_CASE(TT, DD)                                                              \
  {                                                                                          \
    constexpr int RPB = 256 / (DD / 4); /* rows per block */                                 \
    launch_kernel(fwd16_combine_kernel<TT, DD>, dim3((unsigned)((rows + RPB - 1) / RPB)),    \
                  dim3(256), stream, op, lp, static_cast<u16*>(o), lse, rows, Sq, Hq, ns);   \
    return hipGetLastError();                                                                \
  }
  if (dtype == 1 && D == 64) XATTN_MERGE_CASE(__bf16, 64)
  if (dtype == 1 && D == 128) XATTN_MERGE_CASE(__bf16, 128)
  if (dtype == 2 && D == 64) XATTN_MERGE_CASE(_Float16, 64)
  if (dtype == 2 && D == 128) XATTN_MERGE_CASE(_Float16, 128)
#undef XATTN_MERGE_CASE
  return hipErrorInvalidValue;
}

bool lds_single_buffer_enabled() {
  const char* env = std::getenv("ATTN_LDS_SINGLE_BUFFER");
  return env != nullptr && std::atoi(env) != 0;
}

hipError_t launch_fwd16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int Hq, int Hkv, int Sq, int Skv, int D, int causal, float scale,
                        const double2* rope_tab, int dtype, hipStream_t stream,
                        const int* kv_lens, int kv_rows, MaskView mask, KeySplit ks) {
  const bool onebuf = lds_single_buffer_enabled();
  if (mask.p == nullptr && ks.n <= 1 && fwd16_pipelined_enabled())
    return (onebuf ? launch_fwd16_pipelined_onebuf : launch_fwd16_pipelined)(
        q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale, rope_tab, dtype, stream, kv_lens,
        kv_rows);
  if (kv_lens == nullptr) kv_rows = Skv;
  if (onebuf)
    return launch_fwd16_onebuf(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale, rope_tab,
                               dtype, stream, kv_lens, kv_rows, mask, ks);
  return launch_fwd16_kernel<false>(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale,
                                    rope_tab, dtype, stream, kv_lens, kv_rows, mask, ks);
}

int fwd16_key_splits(int B, int Hq, int Hkv, int Sq, int kv_rows, int D) {
  const int G = Hq / Hkv;
  const int HPW = G % 8 == 0 ? 8 : G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1;
  const long long n_bh = (long long)B * (Hq / HPW);
  const int tiles = (kv_rows + 63) / 64;
  long long ns = 1;
  const char* env = std::getenv("ATTN_FWD_SPLITS");
  if (env != nullptr && *env != '\0') {
    ns = std::atoll(env);
  } else {
    // the launch go16 makes without splits: two query blocks per wave
    // (D = 64) when that still gives two workgroups per CU, else one.
    // Measured (whole calls, 11 under-filled shapes from 16 to 256
    // workgroups): a split costs a combine pass and the partials' traffic,
    // which pays once a query tile has >= 32 key tiles and the launch has
    // < 256 workgroups; then about 512 workgroups in total, >= 8 key tiles
    // per split and <= 8 splits come within 4 % of the best count.
    if (D == 64 && (long long)((Sq + 256 / HPW - 1) / (256 / HPW)) * n_bh >= 512) return 1;
    const long long wg = (long long)((Sq + 128 / HPW - 1) / (128 / HPW)) * n_bh;
    if (wg >= 256 || tiles < 32) return 1;
    ns = std::min((512 + wg - 1) / wg, std::min((long long)(tiles / 8), 8LL));
  }
  return (int)std::max(1LL, std::min(ns, std::min(16LL, (long long)std::max(tiles, 1))));
}

size_t fwd16_split_ws_bytes(int B, int Hq, int Sq, int D, int ns) {
  const size_t rows = (size_t)B * Sq * Hq;
  return ((rows * ns * D * 4 + 255) & ~(size_t)255) + rows * ns * 4;
}

}  // namespace xattn
