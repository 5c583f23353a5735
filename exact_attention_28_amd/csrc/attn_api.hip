// attn_api.hip — the C ABI declared in include/attn.h: argument validation,
// library-owned device buffers, and kernel dispatch.  Host code only.
//
// Validation rules follow the pages' constructors and error types:
// scirs2-neural 0.4.4 src/layers/grouped_query_attention.rs
// (GroupedQueryAttention::new rejects zero sizes and a head count that is not a
// multiple of the kv-head count; RotaryPositionEmbedding::new rejects an odd
// head dim), whisper-apr 0.3.1 src/model/lfm2/gqa.rs (GqaConfig::validate),
// oxibonsai-model 0.1.4 src/layers/flash_decode.rs (FlashDecodeError::EmptyKv
// for zero keys).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "attn.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return ATTN_OK;
}

// Library-owned device buffers of one device: grow-only, kept until exit.
// A buffer that a stream capture has referenced is "frozen": the captured
// graph holds its address (and, for the RoPE table, replays a build into it),
// so it is never freed and never trusted as a cache afterwards.  When such a
// buffer must grow, or an eager call needs a table in it, the library moves
// to a new allocation and keeps the old one alive in `retired` until exit.
struct DevBuffers {
  void* rope_tab = nullptr;
  size_t rope_tab_bytes = 0;
  bool rope_tab_frozen = false;
  // what the RoPE table holds: positions [tab_pos0, tab_pos0 + tab_npos) for
  // head dim tab_D and base tab_base, written on tab_stream
  bool tab_ok = false;
  int tab_pos0 = 0, tab_npos = 0, tab_D = 0;
  double tab_base = 0.0;
  hipStream_t tab_stream = nullptr;
  void* kstage = nullptr;
  size_t kstage_bytes = 0;
  bool kstage_frozen = false;
  void* dec_ws = nullptr;
  size_t dec_ws_bytes = 0;
  bool dec_ws_frozen = false;
  void* bwd_ws = nullptr;
  size_t bwd_ws_bytes = 0;
  bool bwd_ws_frozen = false;
  void* pad_ws = nullptr;
  size_t pad_ws_bytes = 0;
  bool pad_ws_frozen = false;
  void* split_ws = nullptr;  // key-split partials of under-filled forward launches
  size_t split_ws_bytes = 0;
  bool split_ws_frozen = false;
  std::vector<void*> retired;  // frozen buffers that were replaced; never freed
};

std::mutex g_mu;
std::map<int, DevBuffers> g_dev;

// Kernel-timing session (attn_profile_begin / attn_profile_end): event pairs
// recorded around the attention-kernel launches of forward calls.  Events
// are created on demand and reused by later sessions, without the
// system-scope fence of a default event: that fence writes back and
// invalidates the caches when the event is reached, which leaves the GPU idle
// for microseconds before the next kernel (a kernel trace shows ~5 us per
// default event between two kernels on MI355X).
struct ProfEvents {
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfEvents> g_prof_pool;  // every event pair created so far
size_t g_prof_used = 0;               // pairs recorded in this session

// Whether `stream` is being captured into a graph (a query error counts as no).
bool capturing(hipStream_t stream) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess) {
    (void)hipGetLastError();  // not left for the launch checks that follow
    return false;
  }
  return cap != hipStreamCaptureStatusNone;
}

// With a profiling session open and `stream` not capturing, the event pair
// that brackets the next attention-kernel launch (nullptr otherwise).
ProfEvents* prof_pair(hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  if (!g_prof_on || capturing(stream)) return nullptr;
  if (g_prof_used == g_prof_pool.size()) {
    ProfEvents pe;
    if (hipEventCreateWithFlags(&pe.start, hipEventDisableSystemFence) != hipSuccess)
      return nullptr;
    if (hipEventCreateWithFlags(&pe.stop, hipEventDisableSystemFence) != hipSuccess) {
      (void)hipEventDestroy(pe.start);
      return nullptr;
    }
    g_prof_pool.push_back(pe);
  }
  return &g_prof_pool[g_prof_used++];
}

// Launch `launch` (returning hipError_t) with a profiling event pair recorded
// by its kernels (start as the first begins, stop as the last ends) when a
// session is open.
template <typename F>
hipError_t timed_launch(hipStream_t stream, F&& launch) {
  ProfEvents* pe = prof_pair(stream);
  if (pe == nullptr) return launch();
  xattn::launch_events() = xattn::LaunchEvents{pe->start, pe->stop};
  hipError_t e = launch();
  xattn::launch_events() = xattn::LaunchEvents{};
  return e;
}

// Make *p hold at least `need` bytes on the current device, for a call on
// `stream`.  A buffer used while `stream` is captured becomes frozen; a frozen
// buffer (or any buffer while capturing, where hipFree would have to
// synchronise) is retired instead of freed when it has to grow.
int grow(DevBuffers* db, void** p, size_t* cap, bool* frozen, size_t need, const char* what,
         hipStream_t stream) {
  const bool cap_now = capturing(stream);
  if (*cap >= need && *p != nullptr) {
    if (cap_now) *frozen = true;
    return ATTN_OK;
  }
  if (*p != nullptr) {
    if (*frozen || cap_now) {
      db->retired.push_back(*p);
    } else {
      hipError_t e = hipFree(*p);  // synchronises the device before the buffer goes
      if (e != hipSuccess) {
        *p = nullptr;
        *cap = 0;
        return fail(ATTN_ERR_HIP, "hipFree(%s): %s", what, hipGetErrorString(e));
      }
    }
    *p = nullptr;
    *cap = 0;
  }
  hipError_t e = hipMalloc(p, need);
  if (e != hipSuccess) {
    *p = nullptr;
    return fail(ATTN_ERR_HIP, "hipMalloc(%s, %zu bytes)%s: %s", what, need,
                cap_now ? " during stream capture (run the call once before capturing)" : "",
                hipGetErrorString(e));
  }
  *cap = need;
  *frozen = cap_now;
  return ATTN_OK;
}

DevBuffers* buffers(int* status) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *status = fail(ATTN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    return nullptr;
  }
  *status = ATTN_OK;
  return &g_dev[dev];
}

bool finite_pos(float x) { return std::isfinite(x) && x > 0.f; }

// With ATTN_DEBUG=1 in the environment, lengths that live in device memory
// (decode seqlens, cache_lens) are copied to the host and checked against
// [lo, hi] before the launch.  The copy is synchronous on the call's stream,
// so the call first waits for the work already queued there; during graph
// capture, where such a copy cannot run, the check is skipped.
int debug_check_lens(const char* fn, const char* what, const int* lens, int B, int lo, int hi,
                     hipStream_t stream) {
  const char* env = std::getenv("ATTN_DEBUG");
  if (env == nullptr || std::strcmp(env, "1") != 0) return ATTN_OK;
  if (capturing(stream)) return ATTN_OK;
  std::vector<int> h((size_t)B);
  hipError_t e = hipMemcpyAsync(h.data(), lens, (size_t)B * sizeof(int), hipMemcpyDeviceToHost,
                                stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess)
    return fail(ATTN_ERR_HIP, "%s: ATTN_DEBUG copy of %s: %s", fn, what, hipGetErrorString(e));
  for (int b = 0; b < B; ++b)
    if (h[(size_t)b] < lo || h[(size_t)b] > hi)
      return fail(ATTN_ERR_INVALID, "%s: %s[%d] = %d outside [%d, %d] (ATTN_DEBUG)", fn, what, b,
                  h[(size_t)b], lo, hi);
  return ATTN_OK;
}

// Key splits for a 16-bit forward launch (unmasked; kv_rows = keys, or the
// cache capacity) and, when there are any, the library-owned partial buffer.
// The caller holds g_mu.
int plan_splits_locked(DevBuffers* db, int B, int Hq, int Hkv, int Sq, int kv_rows, int D,
                       bool masked, xattn::KeySplit* ks, hipStream_t stream) {
  *ks = xattn::KeySplit();
  if (masked) return ATTN_OK;
  const int n = xattn::fwd16_key_splits(B, Hq, Hkv, Sq, kv_rows, D);
  if (n <= 1) return ATTN_OK;
  const size_t rows = (size_t)B * Sq * Hq;
  const size_t obytes = (rows * n * D * 4 + 255) & ~(size_t)255;
  int st = grow(db, &db->split_ws, &db->split_ws_bytes, &db->split_ws_frozen,
                xattn::fwd16_split_ws_bytes(B, Hq, Sq, D, n), "key-split partials", stream);
  if (st != ATTN_OK) return st;
  ks->n = n;
  ks->o = static_cast<float*>(db->split_ws);
  ks->l = reinterpret_cast<float*>(static_cast<char*>(db->split_ws) + obytes);
  return ATTN_OK;
}

int plan_splits(int B, int Hq, int Hkv, int Sq, int kv_rows, int D, bool masked,
                xattn::KeySplit* ks, hipStream_t stream) {
  *ks = xattn::KeySplit();
  if (masked || xattn::fwd16_key_splits(B, Hq, Hkv, Sq, kv_rows, D) <= 1) return ATTN_OK;
  std::lock_guard<std::mutex> lock(g_mu);
  int st;
  DevBuffers* db = buffers(&st);
  if (!db) return st;
  return plan_splits_locked(db, B, Hq, Hkv, Sq, kv_rows, D, masked, ks, stream);
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The fp64 (cos, sin) table for positions [pos0, pos0 + npos) at head dim D
// (caller holds g_mu).  A table built earlier on the same stream for the same
// first position, D and base that covers npos positions is reused (its values
// are the same; stream order puts its build before this call's kernels);
// otherwise the table is rebuilt on `stream`.  While `stream` is being
// captured into a graph the build is always recorded (a replay must not
// depend on what the buffer holds then), the buffer is frozen and the cache is
// dropped: replays rewrite that buffer at times the host does not see, so an
// eager call afterwards builds its table in a new buffer.
int rope_table(DevBuffers* db, int pos0, int npos, int D, float base, hipStream_t stream,
               const double2** tab, const char* fn) {
  const bool cap_now = capturing(stream);
  if (!cap_now && db->tab_ok && db->tab_stream == stream && db->tab_pos0 == pos0 &&
      db->tab_D == D && db->tab_base == (double)base && db->tab_npos >= npos) {
    *tab = static_cast<const double2*>(db->rope_tab);
    return ATTN_OK;
  }
  db->tab_ok = false;
  if (!cap_now && db->rope_tab_frozen && db->rope_tab != nullptr) {
    db->retired.push_back(db->rope_tab);
    db->rope_tab = nullptr;
    db->rope_tab_bytes = 0;
    db->rope_tab_frozen = false;
  }
  const size_t bytes = (size_t)npos * (D / 2) * sizeof(double2);
  int st = grow(db, &db->rope_tab, &db->rope_tab_bytes, &db->rope_tab_frozen, bytes, "rope table",
                stream);
  if (st != ATTN_OK) return st;
  hipError_t e = xattn::launch_rope_table(static_cast<double2*>(db->rope_tab), pos0, npos, D,
                                          (double)base, stream);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: rope table launch: %s", fn, hipGetErrorString(e));
  db->tab_ok = !cap_now;
  db->tab_pos0 = pos0;
  db->tab_npos = npos;
  db->tab_D = D;
  db->tab_base = (double)base;
  db->tab_stream = stream;
  *tab = static_cast<const double2*>(db->rope_tab);
  return ATTN_OK;
}

// attn_fwd for a head dim other than 64 and 128: zero-padded copies of Q, K,
// V (Q and K rotated with the angles of the true D), the kernel at the padded
// width without rotation, then O's first D columns.
int fwd_padded(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
               int Hkv, int Sq, int Skv, int D, int causal, float scale, float rope_base,
               int dtype, xattn::MaskView mask, hipStream_t stream) {
  const int Dp = D <= 64 ? 64 : 128;
  const size_t es = dtype == ATTN_F32 ? 4 : 2;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t qb = up((size_t)B * Sq * Hq * Dp * es), kb = up((size_t)B * Skv * Hkv * Dp * es);
  std::lock_guard<std::mutex> lock(g_mu);
  int st;
  DevBuffers* db = buffers(&st);
  if (!db) return st;
  if ((st = grow(db, &db->pad_ws, &db->pad_ws_bytes, &db->pad_ws_frozen, 2 * qb + 2 * kb,
                 "padded head dim staging", stream)) != ATTN_OK)
    return st;
  char* base = static_cast<char*>(db->pad_ws);
  void *qp = base, *kp = base + qb, *vp = base + qb + kb, *op = base + qb + 2 * kb;
  const double2* tab = nullptr;
  hipError_t e;
  if (rope_base > 0.f &&
      (st = rope_table(db, 0, Skv, D, rope_base, stream, &tab, "attn_fwd")) != ATTN_OK)
    return st;
  const int dt = dtype;  // kernel format codes: 0 fp32, 1 bf16, 2 fp16
  xattn::KeySplit ks;
  if (dtype != ATTN_F32 &&
      (st = plan_splits_locked(db, B, Hq, Hkv, Sq, Skv, Dp, mask.p != nullptr, &ks, stream)) !=
          ATTN_OK)
    return st;
  if ((e = xattn::launch_pack_heads(q, qp, B, Sq, Hq, D, Dp, tab, Skv - Sq, dt, stream)) !=
          hipSuccess ||
      (e = xattn::launch_pack_heads(k, kp, B, Skv, Hkv, D, Dp, tab, 0, dt, stream)) != hipSuccess ||
      (e = xattn::launch_pack_heads(v, vp, B, Skv, Hkv, D, Dp, nullptr, 0, dt, stream)) !=
          hipSuccess)
    return hip_status(e, "attn_fwd: head-dim padding launch");
  e = timed_launch(stream, [&] {
    if (dtype != ATTN_F32)
      return xattn::launch_fwd16(qp, kp, vp, op, lse, B, Hq, Hkv, Sq, Skv, Dp, causal, scale,
                                 nullptr, dt, stream, nullptr, 0, mask, ks);
    return xattn::launch_fwd_f32(qp, kp, vp, op, lse, B, Hq, Hkv, Sq, Skv, Dp, causal, scale,
                                 nullptr, stream, mask);
  });
  if (e != hipSuccess) return hip_status(e, "attn_fwd: kernel launch");
  e = xattn::launch_unpack_heads(op, o, (long long)B * Sq * Hq, D, Dp, dt, stream);
  return hip_status(e, "attn_fwd: head-dim unpadding launch");
}

// attn_fwd and attn_fwd_masked (mask.p null: no mask); `fn` names the entry
// point in error messages.
int fwd(const char* fn, const void* q, const void* k, const void* v, void* o, float* lse, int B,
        int Hq, int Hkv, int Sq, int Skv, int D, int causal, float scale, float rope_base,
        int dtype, xattn::MaskView mask, hipStream_t stream) {
  if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID, "%s: null q, k, v or o", fn);
  if (Skv == 0) return fail(ATTN_ERR_EMPTY_KV, "%s: no keys (Skv == 0)", fn);
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1 || D < 1)
    return fail(ATTN_ERR_INVALID, "%s: sizes must be >= 1 (B=%d Hq=%d Hkv=%d Sq=%d Skv=%d D=%d)",
                fn, B, Hq, Hkv, Sq, Skv, D);
  if (Hq % Hkv != 0)
    return fail(ATTN_ERR_INVALID, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID, "%s: causal must be 0 or 1", fn);
  if (!finite_pos(scale)) return fail(ATTN_ERR_INVALID, "%s: scale must be finite and > 0", fn);
  if (std::isnan(rope_base) || std::isinf(rope_base))
    return fail(ATTN_ERR_INVALID, "%s: rope_base must be finite", fn);
  const bool rope = rope_base > 0.f;
  if (rope && D % 2 != 0) return fail(ATTN_ERR_INVALID, "%s: RoPE needs an even head dim", fn);
  if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_F16)
    return fail(ATTN_ERR_INVALID, "%s: unknown dtype %d", fn, dtype);
  if (D > 128) return fail(ATTN_ERR_UNSUPPORTED, "%s: D=%d (built: up to 128)", fn, D);
  if (rope && Sq > Skv)
    return fail(ATTN_ERR_UNSUPPORTED,
                "%s: RoPE with Sq > Skv would place queries at negative positions", fn);
  if ((long long)B * Hq * ((Sq + 15) / 16) > 0x7fffffffLL || B > 65535 || Hq > 65535)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: grid too large", fn);
  // the 16-bit kernels address one batch's K and V (at their 64- or 128-wide
  // rows) through 32-bit buffer offsets
  if (dtype != ATTN_F32 && (long long)Skv * Hkv * (D <= 64 ? 64 : 128) * 2 >= 0x7fffffffLL)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: one batch's K or V exceeds 2 GiB", fn);
  if (D != 64 && D != 128)
    return fwd_padded(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale, rope_base, dtype,
                      mask, stream);

  // RoPE: the fp32 kernel rotates queries and keys as it loads them; the
  // 16-bit kernel rotates its query fragments in its prologue, and the keys,
  // which every query tile reads, are rotated once by a pass into a
  // library-owned copy
  const double2* tab = nullptr;
  const void* kin = k;
  if (rope) {
    std::lock_guard<std::mutex> lock(g_mu);
    int st;
    DevBuffers* db = buffers(&st);
    if (!db) return st;
    if ((st = rope_table(db, 0, Skv, D, rope_base, stream, &tab, fn)) != ATTN_OK) return st;
    if (dtype != ATTN_F32) {
      const size_t kb = (size_t)B * Skv * Hkv * D * 2;
      if ((st = grow(db, &db->kstage, &db->kstage_bytes, &db->kstage_frozen, kb, "rotated K",
                     stream)) != ATTN_OK)
        return st;
      hipError_t e = xattn::launch_rope_rotate_qk(nullptr, nullptr, B, Sq, Hq, k, db->kstage, Skv,
                                                  Hkv, D, tab, dtype, stream);
      if (e != hipSuccess) return hip_status(e, "attn_fwd: K rotation launch");
      kin = db->kstage;
    }
  }
  hipError_t e;
  if (dtype != ATTN_F32) {
    xattn::KeySplit ks;
    if (int st = plan_splits(B, Hq, Hkv, Sq, Skv, D, mask.p != nullptr, &ks, stream)) return st;
    e = timed_launch(stream, [&] {
      return xattn::launch_fwd16(q, kin, v, o, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale, tab,
                                 dtype, stream, nullptr, 0, mask, ks);
    });
  } else {
    e = timed_launch(stream, [&] {
      return xattn::launch_fwd_f32(q, kin, v, o, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale, tab,
                                   stream, mask);
    });
  }
  return hip_status(e, "attn_fwd: kernel launch");
}

// Argument checks shared by the split-KV decode entry points (`fn` names the
// entry point in messages).
int check_decode_args(const char* fn, const void* q, const void* kcache, const void* vcache,
                      const int* seqlens, const void* o, int B, int Hq, int Hkv, int D,
                      int num_splits, float scale, int max_seqlen) {
  if (!q || !kcache || !vcache || !seqlens || !o)
    return fail(ATTN_ERR_INVALID, "%s: null q, kcache, vcache, seqlens or o", fn);
  if (B < 1 || Hq < 1 || Hkv < 1 || D < 1)
    return fail(ATTN_ERR_INVALID, "%s: sizes must be >= 1", fn);
  if (Hq % Hkv != 0)
    return fail(ATTN_ERR_INVALID, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (num_splits < 1 || num_splits > 64)
    return fail(ATTN_ERR_INVALID, "%s: num_splits=%d outside [1, 64]", fn, num_splits);
  if (max_seqlen < 1) return fail(ATTN_ERR_INVALID, "%s: max_seqlen < 1", fn);
  if (!finite_pos(scale)) return fail(ATTN_ERR_INVALID, "%s: scale must be finite and > 0", fn);
  if (D != 64 && D != 128) return fail(ATTN_ERR_UNSUPPORTED, "%s: D=%d (built: 64, 128)", fn, D);
  if (B > 65535 || Hq > 65535 || (long long)B * Hq > 0x7fffffffLL)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: grid too large", fn);
  return ATTN_OK;
}

}  // namespace

// Scratch of attn_decode_splitkv_noalloc: the decode partials live in this
// array, which the code object brings into every GPU's memory when the
// library is loaded there (each GPU holds its own copy, at its own address,
// until the process ends).  In host code `scratch` names a host-side stand-in,
// not device memory: kernels and copies get the per-device address that
// hipGetSymbolAddress returns, fetched once per device on the entry point's
// first call there.
static constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
static std::mutex g_scratch_mu;
static std::map<int, void*> g_scratch_ptr;  // device -> device address of `scratch`

// Device address of `scratch` on the current device (looked up once per device).
static int scratch_on_device(const char* fn, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *ptr = it->second;
    return ATTN_OK;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || p == nullptr)
    return fail(ATTN_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                hipGetErrorString(e));
  g_scratch_ptr[dev] = p;
  *ptr = p;
  return ATTN_OK;
}

extern "C" {

const char* attn_last_error(void) { return g_err.c_str(); }

int attn_profile_begin(void) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  g_prof_on = true;
  g_prof_used = 0;
  return ok();
}

int attn_profile_end(float* ms, int cap, int* n) {
  if (n == nullptr || cap < 0) return fail(ATTN_ERR_INVALID, "attn_profile_end: null n or cap < 0");
  if (cap > 0 && ms == nullptr) return fail(ATTN_ERR_INVALID, "attn_profile_end: null ms");
  std::lock_guard<std::mutex> lock(g_prof_mu);
  g_prof_on = false;
  *n = (int)g_prof_used;
  for (size_t i = 0; i < g_prof_used; ++i) {
    hipError_t e = hipEventSynchronize(g_prof_pool[i].stop);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, g_prof_pool[i].start, g_prof_pool[i].stop);
    if (e != hipSuccess) {
      g_prof_used = 0;
      return fail(ATTN_ERR_HIP, "attn_profile_end: event %zu: %s", i, hipGetErrorString(e));
    }
    if ((int)i < cap) ms[i] = t;
  }
  g_prof_used = 0;
  return ok();
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
             int Hkv, int Sq, int Skv, int D, int causal, float scale, float rope_base,
             int dtype, hipStream_t stream) {
  return fwd("attn_fwd", q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale, rope_base, dtype,
             xattn::MaskView(), stream);
}

int attn_fwd_masked(const void* q, const void* k, const void* v, const float* mask,
                    long long mask_bstride, long long mask_hstride, long long mask_rstride,
                    void* o, float* lse, int B, int Hq, int Hkv, int Sq, int Skv, int D,
                    int causal, float scale, float rope_base, int dtype, hipStream_t stream) {
  if (!mask) return fail(ATTN_ERR_INVALID, "attn_fwd_masked: null mask");
  if (mask_bstride < 0 || mask_hstride < 0 || mask_rstride < 0)
    return fail(ATTN_ERR_INVALID, "attn_fwd_masked: mask strides must be >= 0");
  xattn::MaskView m;
  m.p = mask;
  m.bs = mask_bstride;
  m.hs = mask_hstride;
  m.rs = mask_rstride;
  m.vec = (reinterpret_cast<uintptr_t>(mask) % 16 == 0) && mask_bstride % 4 == 0 &&
          mask_hstride % 4 == 0 && mask_rstride % 4 == 0;
  return fwd("attn_fwd_masked", q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale,
             rope_base, dtype, m, stream);
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv, int D, float rope_base) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1 || D < 1) return 0;
  return xattn::bwd_workspace_bytes(B, Hq, Hkv, Sq, Skv, D, rope_base > 0.f);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq,
             int Skv, int D, int causal, float scale, float rope_base, int dtype,
             void* workspace, hipStream_t stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)
    return fail(ATTN_ERR_INVALID, "attn_bwd: null q, k, v, o, dout, lse, dq, dk or dv");
  if (Skv == 0) return fail(ATTN_ERR_EMPTY_KV, "attn_bwd: no keys (Skv == 0)");
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1 || D < 1)
    return fail(ATTN_ERR_INVALID, "attn_bwd: sizes must be >= 1 (B=%d Hq=%d Hkv=%d Sq=%d Skv=%d D=%d)",
                B, Hq, Hkv, Sq, Skv, D);
  if (Hq % Hkv != 0)
    return fail(ATTN_ERR_INVALID, "attn_bwd: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID, "attn_bwd: causal must be 0 or 1");
  if (!finite_pos(scale)) return fail(ATTN_ERR_INVALID, "attn_bwd: scale must be finite and > 0");
  if (std::isnan(rope_base) || std::isinf(rope_base))
    return fail(ATTN_ERR_INVALID, "attn_bwd: rope_base must be finite");
  const bool rope = rope_base > 0.f;
  if (rope && D % 2 != 0) return fail(ATTN_ERR_INVALID, "attn_bwd: RoPE needs an even head dim");
  if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_F16)
    return fail(ATTN_ERR_INVALID, "attn_bwd: unknown dtype %d", dtype);
  if (dtype == ATTN_F32 || D != 64)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd: built for bf16 and fp16 with D=64 (dtype=%d D=%d)",
                dtype, D);
  if (rope && Sq > Skv)
    return fail(ATTN_ERR_UNSUPPORTED,
                "attn_bwd: RoPE with Sq > Skv would place queries at negative positions");
  // 32-bit buffer offsets within one batch; grid sizes
  if ((long long)Sq * Hq * D * 2 >= 0x7fffffffLL || (long long)Skv * Hkv * D * 2 >= 0x7fffffffLL)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd: one batch's Q or K exceeds 2 GiB");
  if ((long long)B * Hq * ((Sq + 31) / 32) > 0x7fffffffLL || (rope && B > 65535))
    return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd: grid too large");

  std::lock_guard<std::mutex> lock(g_mu);
  int st;
  DevBuffers* db = buffers(&st);
  if (!db) return st;
  const double2* tab = nullptr;
  if (rope && (st = rope_table(db, 0, Skv, D, rope_base, stream, &tab, "attn_bwd")) != ATTN_OK)
    return st;
  void* ws = workspace;
  if (ws == nullptr) {
    if ((st = grow(db, &db->bwd_ws, &db->bwd_ws_bytes, &db->bwd_ws_frozen,
                   xattn::bwd_workspace_bytes(B, Hq, Hkv, Sq, Skv, D, rope), "backward workspace",
                   stream)) != ATTN_OK)
      return st;
    ws = db->bwd_ws;
  }
  hipError_t e = xattn::launch_bwd16(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D,
                                     causal, scale, tab, dtype, ws, stream);
  return hip_status(e, "attn_bwd: kernel launch");
}

size_t attn_decode_workspace_bytes(int B, int Hq, int D, int num_splits) {
  if (B < 1 || Hq < 1 || D < 1 || num_splits < 1) return 0;
  return xattn::decode_workspace_bytes(B, Hq, D, num_splits);
}

int attn_decode_splitkv(const void* q, const void* kcache, const void* vcache,
                        const int* seqlens, void* o, int B, int Hq, int Hkv, int D,
                        int num_splits, float scale, int max_seqlen, float* lse,
                        void* workspace, hipStream_t stream) {
  if (int st = check_decode_args("attn_decode_splitkv", q, kcache, vcache, seqlens, o, B, Hq, Hkv,
                                 D, num_splits, scale, max_seqlen))
    return st;
  if (int st = debug_check_lens("attn_decode_splitkv", "seqlens", seqlens, B, 0, max_seqlen,
                                stream))
    return st;

  void* ws = workspace;
  if (ws == nullptr) {
    std::lock_guard<std::mutex> lock(g_mu);
    int st;
    DevBuffers* db = buffers(&st);
    if (!db) return st;
    if ((st = grow(db, &db->dec_ws, &db->dec_ws_bytes, &db->dec_ws_frozen,
                   xattn::decode_workspace_bytes(B, Hq, D, num_splits), "decode workspace",
                   stream)) != ATTN_OK)
      return st;
    ws = db->dec_ws;
  }
  hipError_t e = xattn::launch_decode(q, kcache, vcache, seqlens, o, lse, B, Hq, Hkv, D,
                                      num_splits, scale, max_seqlen, ws, stream);
  return hip_status(e, "attn_decode_splitkv: kernel launch");
}

int attn_decode_splitkv_noalloc(const void* q, const void* kcache, const void* vcache,
                                const int* seqlens, void* o, int B, int Hq, int Hkv, int D,
                                int num_splits, float scale, int max_seqlen, float* lse,
                                hipStream_t stream) {
  const char* fn = "attn_decode_splitkv_noalloc";
  if (int st = check_decode_args(fn, q, kcache, vcache, seqlens, o, B, Hq, Hkv, D, num_splits,
                                 scale, max_seqlen))
    return st;
  const size_t need = xattn::decode_workspace_bytes(B, Hq, D, num_splits);
  if (need > kNoAllocScratchBytes)
    return fail(ATTN_ERR_UNSUPPORTED,
                "%s: the partials need %zu bytes (B*Hq*num_splits*(D+1)*4, rounded to 256); the "
                "built-in scratch holds %zu",
                fn, need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (int st = scratch_on_device(fn, &ws)) return st;
  // every split writes its partial (an empty one too), so the scratch needs
  // no clearing between calls
  hipError_t e = xattn::launch_decode(q, kcache, vcache, seqlens, o, lse, B, Hq, Hkv, D,
                                      num_splits, scale, max_seqlen, ws, stream);
  return hip_status(e, "attn_decode_splitkv_noalloc: kernel launch");
}

int attn_prefill_kvcache(const void* q, const void* k_new, const void* v_new, void* kcache,
                         void* vcache, const int* cache_lens, void* o, float* lse, int B, int Hq,
                         int Hkv, int Sq, int D, int max_seqlen, int causal, float scale,
                         float rope_base, hipStream_t stream) {
  if (!q || !k_new || !v_new || !kcache || !vcache || !cache_lens || !o)
    return fail(ATTN_ERR_INVALID,
                "attn_prefill_kvcache: null q, k_new, v_new, kcache, vcache, cache_lens or o");
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || D < 1 || max_seqlen < 1)
    return fail(ATTN_ERR_INVALID, "attn_prefill_kvcache: sizes must be >= 1");
  if (Sq > max_seqlen)
    return fail(ATTN_ERR_INVALID, "attn_prefill_kvcache: Sq=%d exceeds max_seqlen=%d", Sq,
                max_seqlen);
  if (Hq % Hkv != 0)
    return fail(ATTN_ERR_INVALID, "attn_prefill_kvcache: Hq=%d is not a multiple of Hkv=%d", Hq,
                Hkv);
  if (causal != 0 && causal != 1)
    return fail(ATTN_ERR_INVALID, "attn_prefill_kvcache: causal must be 0 or 1");
  if (!finite_pos(scale))
    return fail(ATTN_ERR_INVALID, "attn_prefill_kvcache: scale must be finite and > 0");
  if (std::isnan(rope_base) || std::isinf(rope_base))
    return fail(ATTN_ERR_INVALID, "attn_prefill_kvcache: rope_base must be finite");
  const bool rope = rope_base > 0.f;
  if (rope && D % 2 != 0)
    return fail(ATTN_ERR_INVALID, "attn_prefill_kvcache: RoPE needs an even head dim");
  if (D != 64 && D != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill_kvcache: D=%d (built: 64, 128)", D);
  if ((long long)max_seqlen * Hkv * D * 2 >= 0x7fffffffLL)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill_kvcache: one batch's cache exceeds 2 GiB");
  if ((long long)B * Hq * ((Sq + 15) / 16) > 0x7fffffffLL || B > 65535 || Hq > 65535)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill_kvcache: grid too large");

  if (int st = debug_check_lens("attn_prefill_kvcache", "cache_lens", cache_lens, B, 0,
                                max_seqlen - Sq, stream))
    return st;

  const double2* tab = nullptr;
  if (rope) {
    std::lock_guard<std::mutex> lock(g_mu);
    int st;
    DevBuffers* db = buffers(&st);
    if (!db) return st;
    if ((st = rope_table(db, 0, max_seqlen, D, rope_base, stream, &tab, "attn_prefill_kvcache")) !=
        ATTN_OK)
      return st;
  }
  // every buffer is in place before the first launch, so a failure leaves the
  // caller's cache untouched
  xattn::KeySplit ks;
  if (int st = plan_splits(B, Hq, Hkv, Sq, max_seqlen, D, false, &ks, stream)) return st;
  hipError_t e = xattn::launch_cache_append(k_new, v_new, kcache, vcache, cache_lens, B, Sq, Hkv,
                                            D, max_seqlen, tab, stream);
  if (e != hipSuccess) return hip_status(e, "attn_prefill_kvcache: append launch");
  e = timed_launch(stream, [&] {
    return xattn::launch_fwd16(q, kcache, vcache, o, lse, B, Hq, Hkv, Sq, max_seqlen, D, causal,
                               scale, tab, ATTN_BF16, stream, cache_lens, max_seqlen,
                               xattn::MaskView(), ks);
  });
  return hip_status(e, "attn_prefill_kvcache: kernel launch");
}

int rope_apply(void* x, int B, int S, int H, int D, int pos_offset, float rope_base, int dtype,
               hipStream_t stream) {
  if (!x) return fail(ATTN_ERR_INVALID, "rope_apply: null x");
  if (B < 1 || S < 1 || H < 1 || D < 1) return fail(ATTN_ERR_INVALID, "rope_apply: sizes must be >= 1");
  if (D % 2 != 0) return fail(ATTN_ERR_INVALID, "rope_apply: RoPE head_dim must be even (D=%d)", D);
  if (pos_offset < 0) return fail(ATTN_ERR_INVALID, "rope_apply: pos_offset < 0");
  if ((long long)pos_offset + S > 0x7fffffffLL)
    return fail(ATTN_ERR_INVALID, "rope_apply: positions overflow");
  if (!finite_pos(rope_base)) return fail(ATTN_ERR_INVALID, "rope_apply: rope_base must be finite and > 0");
  if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_F16)
    return fail(ATTN_ERR_INVALID, "rope_apply: unknown dtype %d", dtype);
  if (D > 256) return fail(ATTN_ERR_UNSUPPORTED, "rope_apply: D=%d (built: up to 256)", D);

  std::lock_guard<std::mutex> lock(g_mu);
  int st;
  DevBuffers* db = buffers(&st);
  if (!db) return st;
  const double2* tab = nullptr;
  if ((st = rope_table(db, pos_offset, S, D, rope_base, stream, &tab, "rope_apply")) != ATTN_OK)
    return st;
  hipError_t e = xattn::launch_rope_rotate(x, x, B, S, H, D, tab, dtype, stream);
  return hip_status(e, "rope_apply: kernel launch");
}

}  // extern "C"
