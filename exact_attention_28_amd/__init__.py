"""Exact attention on AMD Instinct MI355X (gfx950): thin Python binding.

The work is done by ``libattn.so`` (hand-written HIP kernels behind the C ABI
of ``include/attn.h``).  This module only marshals torch tensors (device
memory) and the current HIP stream into those calls; it computes nothing
itself and has no fallback: if the library is missing or the tensors are not
on a GPU, the call raises.

Entry points (same names as the C ABI):
  attn_fwd(q, k, v, causal=False, scale=None, rope_base=0.0, o=None, lse=None)
  attn_fwd_masked(q, k, v, mask, causal=False, scale=None, rope_base=0.0, ...)
  attn_bwd(q, k, v, o, dout, lse, causal=False, scale=None, rope_base=0.0, ...)
  attn_prefill_kvcache(q, k_new, v_new, kcache, vcache, cache_lens, ...)
  attn_decode_splitkv(q, kcache, vcache, seqlens, num_splits, scale=None, ...)
  attn_decode_splitkv_noalloc(q, kcache, vcache, seqlens, num_splits, o, ...)
  rope_apply(x, pos_offset=0, rope_base=10000.0)
  attn_decode_workspace_bytes(B, Hq, D, num_splits)
  attn_profile_begin(), attn_profile_end() -> per-launch attention-kernel ms
"""
import ctypes
import math
import os

import torch  # loads the HIP runtime that libattn.so then binds to

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_F32, ATTN_BF16, ATTN_F16 = 0, 1, 2
ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP, ATTN_ERR_EMPTY_KV = 0, -1, -2, -3, -4
EXPORTS = ("attn_fwd", "attn_fwd_masked", "attn_bwd_workspace_bytes", "attn_bwd",
           "attn_decode_workspace_bytes", "attn_decode_splitkv", "attn_decode_splitkv_noalloc",
           "attn_prefill_kvcache",
           "rope_apply", "attn_last_error", "attn_profile_begin", "attn_profile_end")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def load():
    """Load libattn.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with exact_attention_28_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    ll = ctypes.c_longlong
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, f, i, vp]
    lib.attn_fwd_masked.argtypes = [vp, vp, vp, vp, ll, ll, ll, vp, vp, i, i, i, i, i, i, i, f, f,
                                    i, vp]
    lib.attn_fwd_masked.restype = i
    lib.attn_fwd.restype = i
    lib.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, f]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, f, i, vp,
                             vp]
    lib.attn_bwd.restype = i
    lib.attn_decode_workspace_bytes.argtypes = [i, i, i, i]
    lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_decode_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp, vp]
    lib.attn_decode_splitkv.restype = i
    lib.attn_decode_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp]
    lib.attn_decode_splitkv_noalloc.restype = i
    lib.attn_prefill_kvcache.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f,
                                         f, vp]
    lib.attn_prefill_kvcache.restype = i
    lib.rope_apply.argtypes = [vp, i, i, i, i, i, f, i, vp]
    lib.rope_apply.restype = i
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_profile_begin.argtypes = []
    lib.attn_profile_begin.restype = i
    lib.attn_profile_end.argtypes = [ctypes.POINTER(ctypes.c_float), i, ctypes.POINTER(i)]
    lib.attn_profile_end.restype = i
    _lib = lib
    return lib


def last_error():
    return load().attn_last_error().decode()


def _check(code):
    if code != ATTN_OK:
        raise AttnError(code, last_error())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float16:
        return ATTN_F16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16, float16 or float32)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need_gpu(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on a GPU device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on different devices ({dev} and {t.device})")


def _check_out(t, name, shape, dtype):
    """A caller-supplied output must have exactly the shape and dtype the
    kernels write (they take only its pointer)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _mask_view(mask, B, Hq, Sq, Skv):
    """The fp32 mask as a [B, Hq, Sq, Skv] view whose broadcast dimensions
    have stride 0 and whose keys are contiguous (the C ABI takes strides for
    batch, head and row only).  A mask broadcast over the keys (last dimension
    1, or a 0-d mask) is first expanded to Skv columns in memory, keeping its
    leading dimensions; a last dimension with another stride is copied."""
    if mask.dtype != torch.float32:
        raise TypeError("mask must be fp32")
    if mask.dim() > 4:
        raise ValueError("mask has more than 4 dimensions")
    if mask.dim() == 0 or mask.shape[-1] != Skv:
        lead = tuple(mask.shape[:-1]) if mask.dim() > 0 else ()
        if mask.dim() > 0 and mask.shape[-1] != 1:
            raise ValueError(f"mask {tuple(mask.shape)} does not broadcast to "
                             f"[{B}, {Hq}, {Sq}, {Skv}]")
        mask = mask.reshape(*lead, 1).expand(*lead, Skv).contiguous()
    elif mask.stride(-1) != 1:
        mask = mask.contiguous()
    try:
        m = mask.expand(B, Hq, Sq, Skv)
    except RuntimeError as e:
        raise ValueError(f"mask {tuple(mask.shape)} does not broadcast to "
                         f"[{B}, {Hq}, {Sq}, {Skv}]") from e
    if Skv > 1 and m.stride(3) != 1:
        raise ValueError("mask keys must be contiguous")
    return m


def attn_fwd(q, k, v, causal=False, scale=None, rope_base=0.0, o=None, lse=None, stream=None,
             want_lse=True):
    """O, LSE = exact attention.  q [B,Sq,Hq,D], k/v [B,Skv,Hkv,D] (bf16, fp16 or fp32).

    Returns (o [B,Sq,Hq,D] in q's dtype, lse [B,Hq,Sq] fp32 or None)."""
    _need_gpu(q, k, v, o, lse)
    B, Sq, Hq, D = q.shape
    Bk, Skv, Hkv, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    _check_out(o, "o", q.shape, q.dtype)
    _check_out(lse, "lse", (B, Hq, Sq), torch.float32)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check(load().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Sq, Skv, D,
                           int(bool(causal)), float(scale), float(rope_base), _dtype_code(q),
                           _stream(stream)))
    return o, lse


def attn_fwd_masked(q, k, v, mask, causal=False, scale=None, rope_base=0.0, o=None, lse=None,
                    stream=None, want_lse=True):
    """attn_fwd with an additive fp32 mask added to the scaled scores.

    mask: fp32 tensor broadcastable to [B, Hq, Sq, Skv] (e.g. [Sq, Skv],
    [B, 1, 1, Skv]); broadcast batch, head and row dimensions are passed as
    zero strides, so they are never expanded in memory.  The kernels read a
    row's keys at consecutive addresses: a mask whose last stride is not 1 is
    first made contiguous, and one broadcast over the keys (last dimension 1,
    or 0-d) is first expanded to Skv columns."""
    _need_gpu(q, k, v, o, lse)
    if not mask.is_cuda or mask.device != q.device:
        raise ValueError("mask must be on q's GPU device")
    B, Sq, Hq, D = q.shape
    Bk, Skv, Hkv, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    m = _mask_view(mask, B, Hq, Sq, Skv)
    _check_out(o, "o", q.shape, q.dtype)
    _check_out(lse, "lse", (B, Hq, Sq), torch.float32)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check(load().attn_fwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(m), m.stride(0), m.stride(1),
                                  m.stride(2), _ptr(o), _ptr(lse), B, Hq, Hkv, Sq, Skv, D,
                                  int(bool(causal)), float(scale), float(rope_base),
                                  _dtype_code(q), _stream(stream)))
    return o, lse


def attn_bwd_workspace_bytes(B, Hq, Hkv, Sq, Skv, D, rope_base=0.0):
    return int(load().attn_bwd_workspace_bytes(B, Hq, Hkv, Sq, Skv, D, float(rope_base)))


def attn_bwd(q, k, v, o, dout, lse, causal=False, scale=None, rope_base=0.0, dq=None, dk=None,
             dv=None, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of attn_fwd for the upstream gradient dout.

    q, k, v, causal, scale, rope_base as given to attn_fwd; o and lse its
    outputs; dout like o.  Returns dq like q, dk and dv like k."""
    _need_gpu(q, k, v, o, dout, lse, dq, dk, dv, workspace)
    B, Sq, Hq, D = q.shape
    Bk, Skv, Hkv, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o and dout must have q's shape")
    if tuple(lse.shape) != (B, Hq, Sq) or lse.dtype != torch.float32:
        raise ValueError("lse must be fp32 [B, Hq, Sq]")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype):
        raise TypeError("q, k, v, o, dout must share a dtype")
    if workspace is not None and workspace.numel() * workspace.element_size() < \
            attn_bwd_workspace_bytes(B, Hq, Hkv, Sq, Skv, D, rope_base):
        raise ValueError("workspace smaller than attn_bwd_workspace_bytes")
    _check_out(dq, "dq", q.shape, q.dtype)
    _check_out(dk, "dk", k.shape, k.dtype)
    _check_out(dv, "dv", v.shape, v.dtype)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check(load().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                           _ptr(dk), _ptr(dv), B, Hq, Hkv, Sq, Skv, D, int(bool(causal)),
                           float(scale), float(rope_base), _dtype_code(q), _ptr(workspace),
                           _stream(stream)))
    return dq, dk, dv


def attn_decode_workspace_bytes(B, Hq, D, num_splits):
    return int(load().attn_decode_workspace_bytes(B, Hq, D, num_splits))


def attn_decode_splitkv(q, kcache, vcache, seqlens, num_splits, scale=None, o=None, lse=None,
                        workspace=None, stream=None, want_lse=True):
    """Split-KV decode.  q [B,Hq,D] bf16, caches [B,Smax,Hkv,D] bf16, seqlens [B] int32.

    Returns (o [B,Hq,D] bf16, lse [B,Hq] fp32 or None)."""
    _need_gpu(q, kcache, vcache, seqlens, o, lse, workspace)
    B, Hq, D = q.shape
    Bk, Smax, Hkv, Dk = kcache.shape
    if tuple(vcache.shape) != tuple(kcache.shape) or Bk != B or Dk != D:
        raise ValueError("shape mismatch between q and the caches")
    if seqlens.dtype != torch.int32 or seqlens.numel() != B:
        raise ValueError("seqlens must be int32 [B]")
    if q.dtype != torch.bfloat16 or kcache.dtype != torch.bfloat16 or vcache.dtype != torch.bfloat16:
        raise TypeError("decode takes bf16 q and caches")
    _check_out(o, "o", q.shape, q.dtype)
    _check_out(lse, "lse", (B, Hq), torch.float32)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if workspace is not None and workspace.numel() * workspace.element_size() < \
            attn_decode_workspace_bytes(B, Hq, D, num_splits):
        raise ValueError("workspace too small")
    _check(load().attn_decode_splitkv(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(seqlens), _ptr(o),
                                      B, Hq, Hkv, D, int(num_splits), float(scale), Smax,
                                      _ptr(lse), _ptr(workspace), _stream(stream)))
    return o, lse


def attn_decode_splitkv_noalloc(q, kcache, vcache, seqlens, num_splits, o, lse=None, scale=None,
                                stream=None):
    """attn_decode_splitkv with the partials in the library's built-in
    scratch (no device allocation by the library; o, and lse if wanted, are
    the caller's).  Returns (o, lse)."""
    _need_gpu(q, kcache, vcache, seqlens, o, lse)
    B, Hq, D = q.shape
    Bk, Smax, Hkv, Dk = kcache.shape
    if tuple(vcache.shape) != tuple(kcache.shape) or Bk != B or Dk != D:
        raise ValueError("shape mismatch between q and the caches")
    if seqlens.dtype != torch.int32 or seqlens.numel() != B:
        raise ValueError("seqlens must be int32 [B]")
    if q.dtype != torch.bfloat16 or kcache.dtype != torch.bfloat16 or vcache.dtype != torch.bfloat16:
        raise TypeError("decode takes bf16 q and caches")
    if o is None:
        raise ValueError("o is required (this entry point allocates nothing)")
    _check_out(o, "o", q.shape, q.dtype)
    _check_out(lse, "lse", (B, Hq), torch.float32)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check(load().attn_decode_splitkv_noalloc(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(seqlens),
                                              _ptr(o), B, Hq, Hkv, D, int(num_splits),
                                              float(scale), Smax, _ptr(lse), _stream(stream)))
    return o, lse


def attn_prefill_kvcache(q, k_new, v_new, kcache, vcache, cache_lens, causal=True, scale=None,
                         rope_base=0.0, o=None, lse=None, stream=None, want_lse=True):
    """Append (k_new, v_new) to the caches after cache_lens[b] rows (keys
    rotated at their positions), then attend q to the first cache_lens[b] + Sq
    rows.  q [B,Sq,Hq,D], k_new/v_new [B,Sq,Hkv,D], caches [B,Smax,Hkv,D]
    (bf16), cache_lens [B] int32 (not updated).  Returns (o, lse)."""
    _need_gpu(q, k_new, v_new, kcache, vcache, cache_lens, o, lse)
    B, Sq, Hq, D = q.shape
    Bc, Smax, Hkv, Dc = kcache.shape
    if tuple(vcache.shape) != tuple(kcache.shape) or Bc != B or Dc != D:
        raise ValueError("cache shape mismatch")
    if tuple(k_new.shape) != (B, Sq, Hkv, D) or tuple(v_new.shape) != (B, Sq, Hkv, D):
        raise ValueError("k_new / v_new must be [B, Sq, Hkv, D]")
    if cache_lens.dtype != torch.int32 or tuple(cache_lens.shape) != (B,):
        raise ValueError("cache_lens must be int32 [B]")
    if not (q.dtype == k_new.dtype == v_new.dtype == kcache.dtype == vcache.dtype == torch.bfloat16):
        raise TypeError("bf16 tensors expected")
    _check_out(o, "o", q.shape, q.dtype)
    _check_out(lse, "lse", (B, Hq, Sq), torch.float32)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check(load().attn_prefill_kvcache(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(kcache),
                                       _ptr(vcache), _ptr(cache_lens), _ptr(o), _ptr(lse), B, Hq,
                                       Hkv, Sq, D, Smax, int(bool(causal)), float(scale),
                                       float(rope_base), _stream(stream)))
    return o, lse


def rope_apply(x, pos_offset=0, rope_base=10000.0, stream=None):
    """Rotate x [B,S,H,D] (bf16 or fp32) in place at positions pos_offset + t."""
    _need_gpu(x)
    B, S, H, D = x.shape
    _check(load().rope_apply(_ptr(x), B, S, H, D, int(pos_offset), float(rope_base),
                             _dtype_code(x), _stream(stream)))
    return x


def attn_profile_begin():
    """Start recording HIP events around the attention-kernel launch of every
    later forward call (attn_fwd, attn_fwd_masked, attn_prefill_kvcache)."""
    _check(load().attn_profile_begin())


def attn_profile_end(cap=4096):
    """Stop recording; returns the recorded launches' GPU times in ms, in
    launch order (waits for them)."""
    buf = (ctypes.c_float * max(cap, 0))()
    n = ctypes.c_int(0)
    _check(load().attn_profile_end(buf, int(cap), ctypes.byref(n)))
    return [float(buf[i]) for i in range(min(n.value, cap))]
