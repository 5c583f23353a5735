// kernels.h — host-side launchers of the gfx950 kernels (internal to libattn.so).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace xattn {

// Event pair that the forward-kernel launches of the calling thread record
// while the library's kernel-timing session brackets them: the first launch
// records `start` as the kernel begins, every launch records `stop` as it
// ends.  The events ride on the dispatch itself (hipExtLaunchKernel), so no
// marker packet sits between the kernel and the work before it.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
inline LaunchEvents& launch_events() {
  static thread_local LaunchEvents ev;
  return ev;
}

// kernel<<<grid, block, 0, stream>>>(args...), recording the thread's launch
// events when a timing session has set them.
template <typename... P, typename... A>
inline void launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream,
                          A... args) {
  LaunchEvents& ev = launch_events();
  if (ev.stop == nullptr) {
    kernel<<<grid, block, 0, stream>>>(static_cast<P>(args)...);
    return;
  }
  hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev.start, ev.stop, 0,
                        static_cast<P>(args)...);
  ev.start = nullptr;
}

// Additive fp32 mask for the forward: element (b, h, i, j) at
// p[b*bs + h*hs + i*rs + j] (strides in elements; 0 broadcasts), added to the
// scaled score of query row i and key j of batch b, query head h.  vec: p and
// the strides allow 16-byte loads (p 16-byte aligned, strides multiples of 4).
struct MaskView {
  const float* p = nullptr;
  long long bs = 0, hs = 0, rs = 0;
  bool vec = false;
};

// Key splits of an under-filled 16-bit forward launch (unmasked only): n runs
// of key tiles per query tile, each writing its partial O (normalised by its
// own sum) to o [rows][n][D] and its natural-log LSE to l [rows][n], fp32,
// rows = B*Sq*Hq in O's row order; a combine pass merges them by log-sum-exp.
// n = 1: no splits (o, l unused).
struct KeySplit {
  int n = 1;
  float* o = nullptr;
  float* l = nullptr;
};

// Split count for a forward launch of this shape (kv_rows: keys, or the cache
// capacity): 1 when the unsplit launch has >= 256 workgroups or a query tile
// has < 32 key tiles, else min(512 / workgroups, tiles / 8, 8).
// ATTN_FWD_SPLITS in the environment overrides it (clamped to
// [1, min(16, tiles)]).
int fwd16_key_splits(int B, int Hq, int Hkv, int Sq, int kv_rows, int D);
// Merge of key-split partials op [rows, ns, D] fp32 (normalised) and lp
// [rows, ns] (natural-log LSE) into o [rows, D] (dtype 1 bf16, 2 fp16) and
// lse [B, Hq, Sq] (nullable); rows = B * Sq * Hq in O's row order.
hipError_t launch_fwd16_merge(const float* op, const float* lp, void* o, float* lse,
                              long long rows, int Sq, int Hq, int ns, int D, int dtype,
                              hipStream_t stream);
size_t fwd16_split_ws_bytes(int B, int Hq, int Sq, int D, int ns);

// Prefill: q [B,Sq,Hq,D], k/v [B,Skv,Hkv,D], o like q, lse [B,Hq,Sq] (nullable).
// rope_tab: table rows for positions [0, Skv); query row i uses row Skv-Sq+i.
// The 16-bit kernels (dtype 1 bf16, 2 fp16) rotate only the queries (keys
// arrive rotated); fp32 rotates queries and keys.  Null disables rotation.
// 16-bit with kv_lens non-null: k/v are caches of kv_rows rows per batch and
// batch b attends to its first min(kv_lens[b], kv_rows - Sq) + Sq rows (Skv
// is then unused; the table must cover kv_rows positions).  mask.p non-null
// adds the mask to the scores (all formats).
hipError_t launch_fwd16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int Hq, int Hkv, int Sq, int Skv, int D, int causal, float scale,
                        const double2* rope_tab, int dtype, hipStream_t stream,
                        const int* kv_lens = nullptr, int kv_rows = 0,
                        MaskView mask = MaskView(), KeySplit ks = KeySplit());

// The unmasked, unsplit 16-bit forward with the software-pipelined key loop
// (fwd16p_kernel.h): same arguments and results as launch_fwd16 without a
// mask or key splits.  ATTN_FWD_PIPELINE=0 in the environment turns it off
// (launch_fwd16 then runs fwd16_kernel for those launches too).
bool fwd16_pipelined_enabled();
hipError_t launch_fwd16_pipelined(const void* q, const void* k, const void* v, void* o,
                                  float* lse, int B, int Hq, int Hkv, int Sq, int Skv, int D,
                                  int causal, float scale, const double2* rope_tab, int dtype,
                                  hipStream_t stream, const int* kv_lens, int kv_rows);

// Single-buffer instances of both 16-bit forwards, a check of their LDS
// double buffering: one K and one V buffer, refilled only after a barrier
// that follows every wave's last read of it, with the loads waited for before
// the next read.  Same arguments as launch_fwd16 / launch_fwd16_pipelined and
// bit-identical results.  launch_fwd16 routes every 16-bit forward through
// them, and launch_bwd16 its two streaming kernels through their own
// single-buffer instances, when ATTN_LDS_SINGLE_BUFFER=1 is set in the
// environment (read per call).
bool lds_single_buffer_enabled();
hipError_t launch_fwd16_onebuf(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                               float scale, const double2* rope_tab, int dtype, hipStream_t stream,
                               const int* kv_lens, int kv_rows, MaskView mask, KeySplit ks);
hipError_t launch_fwd16_pipelined_onebuf(const void* q, const void* k, const void* v, void* o,
                                         float* lse, int B, int Hq, int Hkv, int Sq, int Skv,
                                         int D, int causal, float scale, const double2* rope_tab,
                                         int dtype, hipStream_t stream, const int* kv_lens,
                                         int kv_rows);

// Cache append: rows t < Sq of k_new/v_new [B,Sq,Hkv,D] (bf16) go to rows
// L_b + t of kcache/vcache [B,rows,Hkv,D] with L_b = min(max(lens[b], 0),
// rows - Sq); keys are rotated at position L_b + t (table row L_b + t, fp64,
// rounded to bf16) when tab is non-null.
hipError_t launch_cache_append(const void* k_new, const void* v_new, void* kcache, void* vcache,
                               const int* lens, int B, int Sq, int Hkv, int D, int rows,
                               const double2* tab, hipStream_t stream);
hipError_t launch_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                          float scale, const double2* rope_tab, hipStream_t stream,
                          MaskView mask = MaskView());

// RoPE: row t of the table holds (cos, sin)((pos0 + t) / base^(2i/D)) for
// t < npos, i < D/2, in fp64.
hipError_t launch_rope_table(double2* tab, int pos0, int npos, int D, double base,
                             hipStream_t stream);
// Rotate x [B,S,H,D] (dtype 0 fp32 / 1 bf16 / 2 fp16) into y (y may equal x);
// token t uses table row t.
hipError_t launch_rope_rotate(const void* x, void* y, int B, int S, int H, int D,
                              const double2* tab, int dtype, hipStream_t stream);
// Rotate an attention call's q [B,Sq,Hq,D] into qo (q non-null) and k
// [B,Skv,Hkv,D] into ko (k non-null) in one launch, dtype 1 bf16 / 2 fp16,
// D % 8 == 0, B <= 65535, Sq <= Skv when q is given: key row t uses table row
// t, query row t table row Skv - Sq + t.
hipError_t launch_rope_rotate_qk(const void* q, void* qo, int B, int Sq, int Hq, const void* k,
                                 void* ko, int Skv, int Hkv, int D, const double2* tab, int dtype,
                                 hipStream_t stream);

// Backward (16-bit: dtype 1 bf16, 2 fp16; D = 64): q, k, v, o, dout like the
// forward's tensors, lse its [B,Hq,Sq] output; dq like q, dk and dv like k.
// rope_tab: table rows for positions [0, Skv) (null: no RoPE).  workspace:
// bwd_workspace_bytes bytes (per-row -D and log2 lse, then, with RoPE, the
// rotated Q and K).
size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv, int D, bool rope);
hipError_t launch_bwd16(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                        int Hq, int Hkv, int Sq, int Skv, int D, int causal, float scale,
                        const double2* rope_tab, int dtype, void* workspace, hipStream_t stream);

// Head dims other than 64/128: copy x [B,S,H,D] into y [B,S,H,Dp] with zero
// columns past D (dtype 0 fp32 / 1 bf16 / 2 fp16), rotating pair i < D/2 of token t by
// table row pos0 + t when tab is non-null; and back: o [rows, D] from the first
// D columns of op [rows, Dp].
hipError_t launch_pack_heads(const void* x, void* y, int B, int S, int H, int D, int Dp,
                             const double2* tab, int pos0, int dtype, hipStream_t stream);
hipError_t launch_unpack_heads(const void* op, void* o, long long rows, int D, int Dp, int dtype,
                               hipStream_t stream);

// Decode: split pass into the workspace, then the merge pass.
size_t decode_workspace_bytes(int B, int Hq, int D, int num_splits);
hipError_t launch_decode(const void* q, const void* kc, const void* vc, const int* seqlens,
                         void* o, float* lse, int B, int Hq, int Hkv, int D, int num_splits,
                         float scale, int max_seqlen, void* workspace, hipStream_t stream);

}  // namespace xattn
