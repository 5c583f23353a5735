/*
 * attn.h — C ABI of the exact-attention library for AMD Instinct MI355X (gfx950).
 *
 * Exact scaled-dot-product attention O = softmax(scale * Q K^T) V computed by
 * tiles with an online softmax (a running row maximum m and row sum l, rescaled
 * per key/value tile), with causal masking, grouped-query heads, rotary position
 * embedding on Q and K, and flash-decoding (split-KV partial results merged by
 * log-sum-exp).
 *
 * Definitions follow these docs.rs source pages:
 *   [FA]  scirs2-neural 0.4.3, src/layers/flash_attention.rs
 *   [GQA] scirs2-neural 0.4.4, src/layers/grouped_query_attention.rs
 *   [WH]  whisper-apr 0.3.1, src/model/attention_generated.rs
 *   [FD]  oxibonsai-model 0.1.4, src/layers/flash_decode.rs
 *   [LF]  whisper-apr 0.3.1, src/model/lfm2/gqa.rs
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never frees caller memory.  Tensors are dense and contiguous, and start
 *    16-byte aligned (as hipMalloc and torch allocations, and row views of
 *    them at D = 64 or 128, do): the kernels move rows in 16-byte loads and
 *    stores.  This is a precondition, not checked.
 *  - Calls are asynchronous on `stream` (0 = the null stream): arguments are
 *    validated synchronously on the host before anything is enqueued, then
 *    the kernels are launched and the call returns without synchronising.
 *  - Return value: ATTN_OK (0) or a negative attn_status_t; on error nothing is
 *    enqueued and attn_last_error() describes the problem.  Nothing throws
 *    across the ABI.
 *  - Library-owned device buffers (RoPE tables, rotated-K staging, key-split
 *    partials, the default decode and backward workspaces) are allocated on
 *    first need, grow only, and are kept per device until the process ends;
 *    calls that use them concurrently on different streams of one device
 *    must be ordered by the caller.
 *  - The fp64 RoPE (cos, sin) table is built on the call's stream when a call
 *    needs positions, a head dim or a base that the table does not hold, or
 *    runs on another stream than the one that built it; otherwise it is
 *    reused (the same values, ordered before the call by its stream).
 *  - HIP graph capture: a call can be captured once the library-owned buffers
 *    it uses are large enough (an earlier call of the same or a larger shape;
 *    or pass the workspaces explicitly), since capture cannot allocate.  A
 *    captured call records its RoPE table build.  Every library buffer that a
 *    capture references is kept alive until the process ends: when a later
 *    call needs it larger, the library allocates a new one and retires the
 *    old one instead of freeing it, so a graph never replays into freed
 *    memory.  A replay rewrites its table buffer at times the host does not
 *    see, so an eager call after a capture builds its table in a new buffer
 *    rather than trusting the cache.  The library's buffers are shared, so
 *    replays must still be ordered with other calls that use them.
 *  - Environment variables (read on every call): ATTN_DEBUG=1 (host checks of
 *    device-resident lengths, see attn_decode_splitkv), ATTN_FWD_SPLITS=n
 *    (see attn_fwd), ATTN_FWD_PIPELINE=0 (unmasked 16-bit forwards run the
 *    tile kernel instead of the pipelined one; same results up to fp32
 *    rounding order) and ATTN_LDS_SINGLE_BUFFER=1 (the 16-bit forward and
 *    backward kernels run with one LDS tile buffer instead of two, each
 *    refilled only when no wave reads it: slower, bit-identical results; a
 *    check of the double buffering's waits and barriers).
 */
#ifndef EXACT_ATTN_H
#define EXACT_ATTN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_F32 = 0,  /* IEEE binary32 */
  ATTN_BF16 = 1, /* bfloat16 (8 significant bits) */
  ATTN_F16 = 2,  /* IEEE binary16 (11 significant bits, subnormals kept) */
} attn_dtype_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID = -1,     /* null pointer, size < 1, Hq not a multiple of Hkv,
                                odd D with RoPE, scale not finite or <= 0, ... */
  ATTN_ERR_UNSUPPORTED = -2, /* valid but not built: D not 64/128, dtype, ... */
  ATTN_ERR_HIP = -3,         /* a HIP runtime call or kernel launch failed */
  ATTN_ERR_EMPTY_KV = -4,    /* zero keys ([FD] FlashDecodeError::EmptyKv) */
} attn_status_t;

/*
 * attn_fwd — exact attention forward pass with per-row log-sum-exp.
 *
 * Computes, for batch b, query head h, query row i and d < D:
 *   g        = h / (Hq / Hkv)                         (contiguous GQA groups:
 *                                                      [GQA] forward loop, [LF]
 *                                                      fn attention_scalar)
 *   s_ij     = scale * <q~[b,i,h,:], k~[b,j,g,:]>     ([FA] compute_block_scores)
 *   s_ij     = -inf  if causal and j > i + (Skv - Sq)  ([FA] apply_causal_mask for
 *                                                      Sq == Skv; bottom-right
 *                                                      alignment otherwise, the
 *                                                      cached-generation rule of
 *                                                      [GQA] forward_with_cache)
 *   O[b,i,h,d] = sum_j exp(s_ij - m_i) v[b,j,g,d] / l_i,  m_i = max_j s_ij,
 *   l_i = sum_j exp(s_ij - m_i),  lse[b,h,i] = m_i + ln l_i
 * by the tiled forward with online softmax of [FA] flash_attention_forward /
 * online_softmax_update.  A row with no visible key (causal with Sq > Skv)
 * gets O = 0 and lse = -inf.
 * q~, k~ are Q and K after rotary embedding when rope_base > 0 ([GQA]
 * RotaryPositionEmbedding::apply: pair (2i, 2i+1) rotated by the angle
 * pos / rope_base^(2i/D)), with query row i at position Skv - Sq + i and key j
 * at position j; the rotation is evaluated in fp64 and rounded to `dtype`
 * (nearest, ties to even) before the dot products.  V is not rotated.
 *
 * Arguments:
 *   q    [B, Sq, Hq, D]  dtype          k, v [B, Skv, Hkv, D] dtype
 *   o    [B, Sq, Hq, D]  dtype (output) lse  [B, Hq, Sq] fp32 (output; may be NULL)
 *   B, Hq, Hkv, Sq, Skv, D >= 1; Hq % Hkv == 0; D <= 128.  D = 64 and 128 run
 *   the kernels directly; any other D runs them on zero-padded copies (64 or
 *   128 columns; Q and K rotated with the angles of the true D), which is
 *   exact: the head-dim padding of [LF] GqaConfig::pad_head_dim_to (36 -> 40
 *   for Moonshine), with the scale passed explicitly (1/sqrt(D), not the
 *   padded width's).  The padded copies live in a library-owned buffer.
 *   causal: 0 or 1;  scale: finite and > 0, used as given (the pages' default
 *   is 1/sqrt(D));  rope_base: > 0 enables RoPE (D even), <= 0 disables it
 *   dtype: ATTN_BF16 or ATTN_F16 (16-bit MFMA of that format, fp32
 *          accumulation; P enters the second product in the input format), or
 *          ATTN_F32 (fp32 throughout)
 * Errors: ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED (also for 16-bit inputs whose
 *   one batch of K or V, at 64 or 128 columns, reaches 2 GiB: the kernels use
 *   32-bit buffer offsets), ATTN_ERR_EMPTY_KV (Skv == 0),
 *   ATTN_ERR_HIP.  With rope_base > 0 and a 16-bit dtype, the call may allocate the
 *   library's rotated-K staging buffer (B*Skv*Hkv*D*2 bytes) and RoPE table.
 * Key splits (16-bit, no mask): a launch with fewer than 256 workgroups whose
 *   query tiles each have >= 32 key tiles of 64 splits each query tile's keys
 *   into n <= 8 runs, one workgroup per run, and merges the runs' partial O
 *   and LSE by log-sum-exp in a second kernel, as decode merges its splits
 *   ([FD] fn combine_tile_outputs; the same result up to fp32 rounding
 *   order); the partials live in a library-owned buffer of
 *   B*Sq*Hq*n*(D+1)*4 bytes.  ATTN_FWD_SPLITS=n in the environment forces n
 *   (1 disables splitting; clamped to 16 and to the key-tile count).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
             int Hkv, int Sq, int Skv, int D, int causal, float scale, float rope_base,
             int dtype, hipStream_t stream);

/*
 * attn_fwd_masked — attn_fwd with an additive float mask on the scores.
 *
 * As attn_fwd, with the score of query row i and key j of batch b, head h
 *   s_ij = scale * <q~[b,i,h,:], k~[b,j,g,:]> + mask[b*mask_bstride +
 *          h*mask_hstride + i*mask_rstride + j]
 * (the mask term of [WH] compute_block_scores, added to the scaled dot
 * product; the attn_mask of scaled_dot_product_attention), then the causal
 * rule and the softmax as in attn_fwd.  The mask is an fp32 device array owned
 * by the caller; strides are in elements and may be 0 to broadcast (e.g.
 * mask_bstride = mask_hstride = 0 for one [Sq, Skv] mask shared by every batch
 * and head, mask_rstride = 0 for a per-key padding mask); the columns j are
 * contiguous.  Entries must be finite or -inf: -inf hides a key, and a row
 * whose keys are all hidden gets O = 0 and lse = -inf.  Every address
 * b*mask_bstride + h*mask_hstride + i*mask_rstride + j (b < B, h < Hq, i < Sq,
 * j < Skv) must lie in the array.
 * Errors: as attn_fwd, and ATTN_ERR_INVALID for a null mask or a negative
 *   stride.
 */
int attn_fwd_masked(const void* q, const void* k, const void* v, const float* mask,
                    long long mask_bstride, long long mask_hstride, long long mask_rstride,
                    void* o, float* lse, int B, int Hq, int Hkv, int Sq, int Skv, int D,
                    int causal, float scale, float rope_base, int dtype, hipStream_t stream);

/*
 * attn_bwd_workspace_bytes — size of the workspace attn_bwd needs: the per-row
 * -D_i and log2 lse ([B, Hq, Sq] fp32 each) and, with rope_base > 0, the rotated
 * Q and K (B*Sq*Hq*D and B*Skv*Hkv*D 16-bit values), each part rounded up to 256 bytes.
 * Returns 0 for invalid sizes.
 */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv, int D, float rope_base);

/*
 * attn_bwd — gradients of attn_fwd with respect to q, k and v.
 *
 * The FA-2 backward per head of [FA] fn flash_backward_head, with dK and dV
 * summed over the query heads of each group and the gradients of the
 * pre-rotation Q and K obtained by the inverse rotation ([GQA] backward through
 * grouped attention).  With s_ij, g, q~, k~ as in attn_fwd and dO = dout:
 *   P_ij  = exp(s_ij - lse[b,h,i])         (0 where masked, and for a row whose
 *                                          lse is -inf)
 *   D_i   = sum_d dO[b,i,h,d] O[b,i,h,d]
 *   dS_ij = P_ij (<dO[b,i,h,:], v[b,j,g,:]> - D_i)
 *   dv[b,j,g,:] = sum over h in group g and rows i of P_ij dO[b,i,h,:]
 *   dq~[b,i,h,:] = scale sum_j dS_ij k~[b,j,g,:]
 *   dk~[b,j,g,:] = scale sum over h in group g and rows i of dS_ij q~[b,i,h,:]
 *   dq = R^T dq~, dk = R^T dk~  (R: the forward's rotation at the same
 *   positions; identity without RoPE)
 * P and dS enter the MFMA contractions in the input format (bf16 or fp16);
 * accumulation is fp32 and the inverse rotation fp64.  Deterministic: no
 * atomics, the same inputs give the same bits.
 *
 * Arguments:
 *   q, k, v, causal, scale, rope_base, dtype: as given to attn_fwd
 *   o    [B, Sq, Hq, D] dtype: attn_fwd's output for these inputs
 *   dout [B, Sq, Hq, D] dtype: gradient of the loss with respect to o
 *   lse  [B, Hq, Sq] fp32: attn_fwd's lse for these inputs (required)
 *   dq   [B, Sq, Hq, D] dtype, dk and dv [B, Skv, Hkv, D] dtype (outputs)
 *   workspace: attn_bwd_workspace_bytes(...) bytes of device memory, or NULL
 *          to use a library-owned buffer
 *   Built: dtype ATTN_BF16 or ATTN_F16 with D == 64; RoPE needs Sq <= Skv.
 * Errors: ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED (other dtype or D),
 *   ATTN_ERR_EMPTY_KV (Skv == 0), ATTN_ERR_HIP.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq,
             int Skv, int D, int causal, float scale, float rope_base, int dtype,
             void* workspace, hipStream_t stream);

/*
 * attn_decode_workspace_bytes — size of the workspace attn_decode_splitkv needs
 * for the per-split partial outputs and log-sum-exps: B*Hq*num_splits*(D+1)*4
 * bytes rounded up to 256.  Returns 0 for invalid sizes.
 */
size_t attn_decode_workspace_bytes(int B, int Hq, int D, int num_splits);

/*
 * attn_decode_splitkv — flash-decoding of one query token per sequence.
 *
 * For batch b and query head h (kv head g = h / (Hq/Hkv)), attends q[b,h,:]
 * to the first L_b = seqlens[b] positions of the caches, with no mask
 * ([LF] fn attention_cached).  The positions [0, L_b) are split into
 * num_splits chunks; each chunk yields a normalised partial output and its
 * log-sum-exp ([FD] fn flash_decode_tile); a second pass merges the chunks by
 * log-sum-exp, dropping empty chunks ([FD] fn combine_tile_outputs).  The
 * result equals exact attention over all L_b positions for any split.
 * L_b == 0 gives O = 0 and lse = -inf.
 *
 * Arguments:
 *   q       [B, Hq, D] bf16
 *   kcache, vcache [B, max_seqlen, Hkv, D] bf16, token-major ([FD]
 *           flash_decode_multi_head layout; [LF] KvCache); rows >= L_b are
 *           never read
 *   seqlens [B] int32 in device memory, 0 <= seqlens[b] <= max_seqlen
 *           (a precondition: it is not checked on the host because the values
 *           live on the device; larger values are clamped to max_seqlen).
 *           With ATTN_DEBUG=1 in the environment the call copies seqlens to
 *           the host first (synchronously on `stream`, so it waits for the
 *           work queued there; skipped during graph capture) and returns
 *           ATTN_ERR_INVALID, launching nothing, if a value is out of range.
 *   o       [B, Hq, D] bf16 (output);  lse [B, Hq] fp32 (output, may be NULL)
 *   B, Hq, Hkv >= 1; Hq % Hkv == 0; D in {64, 128}; 1 <= num_splits <= 64;
 *   max_seqlen >= 1; scale finite and > 0
 *   workspace: device buffer of attn_decode_workspace_bytes(B, Hq, D,
 *           num_splits) bytes, or NULL to use a library-owned buffer
 * Errors: ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP.
 */
int attn_decode_splitkv(const void* q, const void* kcache, const void* vcache,
                        const int* seqlens, void* o, int B, int Hq, int Hkv, int D,
                        int num_splits, float scale, int max_seqlen, float* lse,
                        void* workspace, hipStream_t stream);

/*
 * attn_decode_splitkv_noalloc — attn_decode_splitkv for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): it allocates nothing (no hipMalloc,
 * hipFree or allocating library call) and keeps the per-split partials in a
 * scratch array built into the library, 16 MiB per GPU, which each GPU the
 * library runs on holds until the process ends.
 *
 * Arguments, result and errors are those of attn_decode_splitkv without the
 * workspace (and without the ATTN_DEBUG length check, which copies to the
 * host); the same kernels run, so o and lse are bit-identical to
 * attn_decode_splitkv's.  Shapes whose partials need more than the scratch,
 * attn_decode_workspace_bytes(B, Hq, D, num_splits) > 16 MiB (for example
 * B*Hq*num_splits > 32513 at D = 128), return ATTN_ERR_UNSUPPORTED and launch
 * nothing.  Every call on one GPU uses that GPU's one scratch array and leaves
 * its partials there (every split of a call writes its own, so nothing needs
 * clearing): calls that can overlap on one GPU (different streams, or
 * different host threads) race and must be serialised by the caller.  The
 * first call on a device looks the array's address up there
 * (hipGetSymbolAddress); ATTN_ERR_HIP if that fails.
 */
int attn_decode_splitkv_noalloc(const void* q, const void* kcache, const void* vcache,
                                const int* seqlens, void* o, int B, int Hq, int Hkv, int D,
                                int num_splits, float scale, int max_seqlen, float* lse,
                                hipStream_t stream);

/*
 * attn_prefill_kvcache — one chunk of a streaming (chunked) prefill against a
 * token-major KV cache: append, then attend.
 *
 * For batch b, with L_b = cache_lens[b] positions already in the cache (keys
 * stored rotated, as this call stores them):
 *  1. kcache[b, L_b + t, g, :] = R(L_b + t) k_new[b, t, g, :] (fp64 rotation
 *     rounded to bf16) and vcache[b, L_b + t, g, :] = v_new[b, t, g, :] for
 *     t < Sq — the position_offset of [GQA] RotaryPositionEmbedding::apply and
 *     the cache append of [GQA] forward_with_cache;
 *  2. O and lse of q[b, i] (rotated at position L_b + i) against cache rows
 *     [0, L_b + Sq): exactly attn_fwd with Skv = L_b + Sq (bottom-right causal:
 *     key j is hidden from row i iff j > L_b + i, the cached-generation rule
 *     of [GQA] forward_with_cache).
 * Sq == 1 is one decode step that also appends its token.  The call does not
 * update cache_lens: the caller adds Sq once the call is ordered before the
 * next use.  Without RoPE (rope_base <= 0) nothing is rotated.
 *
 * Arguments:
 *   q [B, Sq, Hq, D] bf16;  k_new, v_new [B, Sq, Hkv, D] bf16
 *   kcache, vcache [B, max_seqlen, Hkv, D] bf16 (rows < L_b are read, rows
 *          [L_b, L_b + Sq) written, later rows neither read nor written)
 *   cache_lens [B] int32 in device memory, 0 <= cache_lens[b] <= max_seqlen - Sq
 *          (a precondition, as for attn_decode_splitkv: values outside are
 *          clamped into that range; checked on the host, as there, with
 *          ATTN_DEBUG=1)
 *   o [B, Sq, Hq, D] bf16 (output);  lse [B, Hq, Sq] fp32 (output, may be NULL)
 *   B, Hq, Hkv, Sq >= 1; Hq % Hkv == 0; D in {64, 128}; 1 <= Sq <= max_seqlen;
 *   causal 0 or 1; scale finite and > 0; rope_base > 0 enables RoPE (D even)
 * Errors: ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP.  With RoPE the
 *   call uses the library's RoPE table for max_seqlen positions (built on the
 *   first such call on a stream and reused by the next ones).  The attention
 *   step splits keys as attn_fwd does, counting key tiles from max_seqlen.
 */
int attn_prefill_kvcache(const void* q, const void* k_new, const void* v_new, void* kcache,
                         void* vcache, const int* cache_lens, void* o, float* lse, int B, int Hq,
                         int Hkv, int Sq, int D, int max_seqlen, int causal, float scale,
                         float rope_base, hipStream_t stream);

/*
 * rope_apply — rotary position embedding, in place ([GQA]
 * RotaryPositionEmbedding::apply with its position_offset argument).
 *
 * x [B, S, H, D] of dtype; token t is at position pos_offset + t; pair
 * (2i, 2i+1) is rotated by pos / rope_base^(2i/D), evaluated in fp64 and
 * rounded to dtype (nearest, ties to even).
 *   B, S, H >= 1; D even, 2 <= D <= 256; pos_offset >= 0; rope_base > 0
 * Errors: ATTN_ERR_INVALID (odd D: "RoPE head_dim must be even" in [GQA]),
 *   ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP.
 */
int rope_apply(void* x, int B, int S, int H, int D, int pos_offset, float rope_base, int dtype,
               hipStream_t stream);

/* Text of the last error raised on the calling thread ("" if none). */
const char* attn_last_error(void);

/*
 * Kernel timing (tracing; not part of the method).  A forward call launches
 * up to three kernels (the RoPE table build, the key rotation, the attention
 * kernel); a caller's events around the call time all of them.  Between
 * attn_profile_begin() and attn_profile_end(), every attn_fwd,
 * attn_fwd_masked and attn_prefill_kvcache call has its attention kernel
 * (with the key-split merge when the keys are split) record a pair of HIP
 * events on the call's stream, attached to the kernel dispatches themselves
 * (hipExtLaunchKernel): start as the kernel begins, stop as the last one
 * ends, so their difference is that kernel's GPU time, and no marker packet
 * delays the kernel.  The events carry no system-scope fence.  Calls on a
 * stream being captured into a graph record nothing.
 *   attn_profile_begin: starts a session (drops one still open).  Returns
 *     ATTN_OK, or ATTN_ERR_HIP if events cannot be created later.
 *   attn_profile_end: waits for the recorded events, writes up to `cap`
 *     per-launch times in milliseconds, in launch order, to ms (may be NULL
 *     when cap is 0) and the number of launches recorded to *n, and ends the
 *     session.  ATTN_ERR_INVALID for a null n or cap < 0; ATTN_ERR_HIP if an
 *     event query fails.
 * The session is process-wide (one at a time); the events are the library's.
 */
int attn_profile_begin(void);
int attn_profile_end(float* ms, int cap, int* n);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTN_H */
