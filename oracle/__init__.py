"""fp64 CPU oracle for exact attention — TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never imports, links or
calls it, and it imports nothing from the HIP library.

This module only marshals numpy arrays into ``liboracle.so`` (compiled from
``oracle.c`` by ``oracle/build.py``); every step of the arithmetic is in
``oracle.c``.  Inputs may be float64, float32, float16 (IEEE binary16), or
uint16 arrays holding bf16 bit patterns; they are widened exactly inside the
oracle.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

F64, F32, BF16, F16 = 0, 1, 2, 3
ROUND_NONE, ROUND_BF16, ROUND_F16, ROUND_F32 = 0, 8, 11, 24

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)


def load(path=None):
    """Load (building if absent) liboracle.so; a path loads a private build."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        lib_path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(lib_path):
            _build.build()
        _lib = _declare(ctypes.CDLL(lib_path))
    return _lib


def _declare(lib):
    vp, i, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    ll = ctypes.c_longlong
    lib.oracle_attn_fwd.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, i, d, d, i, _ip, i, _ip, i,
                                    _dp, _dp, _dp, ll, ll, i]
    lib.oracle_attn_fwd.restype = i
    lib.oracle_decode.argtypes = [vp, vp, vp, i, _ip, i, i, i, i, i, d, _ip, i, _dp, _dp, i]
    lib.oracle_decode.restype = i
    lib.oracle_rope.argtypes = [vp, i, _dp, i, i, i, i, i, d, i]
    lib.oracle_rope.restype = i
    lib.oracle_lse_merge.argtypes = [_dp, _dp, i, i, _dp, _dp]
    lib.oracle_lse_merge.restype = None
    lib.oracle_flash_decode_head.argtypes = [_dp, _dp, _dp, i, i, i, d, _dp, _dp]
    lib.oracle_flash_decode_head.restype = i
    lib.oracle_attn_tiled_head.argtypes = [_dp, _dp, _dp, i, i, i, i, d, i, i, _dp, _dp]
    lib.oracle_attn_tiled_head.restype = i
    lib.oracle_attn_bwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, d, d, i, _ip, i,
                                    _dp, _dp, _dp, i]
    lib.oracle_attn_bwd.restype = i
    lib.oracle_round_sig.argtypes = [d, i]
    lib.oracle_round_sig.restype = d
    return lib


def _as_input(x):
    """Contiguous array + dtype code; uint16/int16 arrays are bf16 bit patterns."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float64:
        return x, F64
    if x.dtype == np.float32:
        return x, F32
    if x.dtype in (np.uint16, np.int16):
        return x.view(np.uint16), BF16
    if x.dtype == np.float16:
        return x.view(np.uint16), F16
    raise TypeError(f"unsupported oracle input dtype {x.dtype}")


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a, t=_dp):
    return a.ctypes.data_as(t)


def _ints(seq):
    if seq is None:
        return None, 0
    a = np.ascontiguousarray(np.asarray(seq, dtype=np.int32))
    return a, int(a.size)


def default_round_bits(dtype_code):
    return {F64: ROUND_NONE, F32: ROUND_F32, BF16: ROUND_BF16, F16: ROUND_F16}[dtype_code]


def attn_fwd(q, k, v, causal=False, scale=None, rope_base=0.0, round_bits=None, rows=None,
             units=None, nthreads=1, lib=None, mask=None):
    """Exact attention.  q [B,Sq,Hq,D], k and v [B,Skv,Hkv,D] (same dtype).

    Returns (o, lse).  With rows and units both None: o [B,Sq,Hq,D] and
    lse [B,Hq,Sq].  Otherwise o [len(units), len(rows), D] and
    lse [len(units), len(rows)] where a unit is b*Hq + h (None = all units /
    all rows).  round_bits: significant bits the rotated q/k are rounded to
    (default: the input format's).  mask: additive mask [Bm, Hm, Sq, Skv]
    with Bm in (1, B) and Hm in (1, Hq) (size 1 broadcasts), added to the
    scaled scores.
    """
    lib = lib or load()
    q, dt = _as_input(q)
    k, dtk = _as_input(k)
    v, dtv = _as_input(v)
    assert dt == dtk == dtv, "q, k, v must share a dtype"
    B, Sq, Hq, D = q.shape
    _, Skv, Hkv, _ = k.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if round_bits is None:
        round_bits = default_round_bits(dt)
    rows_a, nrows = _ints(rows)
    units_a, nunits = _ints(units)
    nr = nrows if rows_a is not None else Sq
    nu = nunits if units_a is not None else B * Hq
    o = np.empty((nu, nr, D), dtype=np.float64)
    lse = np.empty((nu, nr), dtype=np.float64)
    mbs = mhs = 0
    if mask is not None:
        mask = _f64(mask)
        Bm, Hm, Sm, Km = mask.shape
        if Bm not in (1, B) or Hm not in (1, Hq) or Sm != Sq or Km != Skv:
            raise ValueError(f"mask shape {mask.shape} for B={B} Hq={Hq} Sq={Sq} Skv={Skv}")
        mhs = Sq * Skv if Hm > 1 else 0
        mbs = Hm * Sq * Skv if Bm > 1 else 0
    st = lib.oracle_attn_fwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, dt, B, Hq, Hkv, Sq,
                             Skv, D, int(bool(causal)), float(scale), float(rope_base),
                             int(round_bits),
                             _ptr(rows_a, _ip) if rows_a is not None else None, nrows,
                             _ptr(units_a, _ip) if units_a is not None else None, nunits,
                             _ptr(o), _ptr(lse), _ptr(mask) if mask is not None else None,
                             mbs, mhs, int(nthreads))
    if st != 0:
        raise ValueError(f"oracle_attn_fwd rejected its arguments (status {st})")
    if rows is None and units is None:
        return o.reshape(B, Hq, Sq, D).transpose(0, 2, 1, 3).copy(), lse.reshape(B, Hq, Sq)
    return o, lse


def attn_bwd(q, k, v, dout, causal=False, scale=None, rope_base=0.0, round_bits=None,
             units=None, nthreads=1, lib=None):
    """Gradients (dq [B,Sq,Hq,D], dk and dv [B,Skv,Hkv,D], fp64) of the
    attention of attn_fwd for the upstream gradient dout [B,Sq,Hq,D].

    units: list of b*Hkv + g (a kv head with its query heads) to evaluate;
    None = all.  Slices of other units are returned as NaN."""
    lib = lib or load()
    q, dt = _as_input(q)
    k, dtk = _as_input(k)
    v, dtv = _as_input(v)
    do, dtd = _as_input(dout)
    assert dt == dtk == dtv == dtd, "q, k, v, dout must share a dtype"
    B, Sq, Hq, D = q.shape
    _, Skv, Hkv, _ = k.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D or do.shape != q.shape:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape} dout{do.shape}")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if round_bits is None:
        round_bits = default_round_bits(dt)
    units_a, nunits = _ints(units)
    dq = np.full((B, Sq, Hq, D), np.nan)
    dk = np.full((B, Skv, Hkv, D), np.nan)
    dv = np.full((B, Skv, Hkv, D), np.nan)
    st = lib.oracle_attn_bwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, do.ctypes.data, dt, B,
                             Hq, Hkv, Sq, Skv, D, int(bool(causal)), float(scale),
                             float(rope_base), int(round_bits),
                             _ptr(units_a, _ip) if units_a is not None else None, nunits,
                             _ptr(dq), _ptr(dk), _ptr(dv), int(nthreads))
    if st != 0:
        raise ValueError(f"oracle_attn_bwd rejected its arguments (status {st})")
    return dq, dk, dv


def decode(q, kcache, vcache, seqlens, scale=None, units=None, nthreads=1, lib=None):
    """Single-token attention against a token-major cache.

    q [B,Hq,D], caches [B,Smax,Hkv,D], seqlens [B].  Returns o [B,Hq,D] and
    lse [B,Hq] (or [len(units), D] / [len(units)] for a list of b*Hq + h)."""
    lib = lib or load()
    q, dt = _as_input(q)
    kc, dtk = _as_input(kcache)
    vc, dtv = _as_input(vcache)
    assert dt == dtk == dtv
    B, Hq, D = q.shape
    _, Smax, Hkv, _ = kc.shape
    if kc.shape != vc.shape or kc.shape[0] != B or kc.shape[3] != D or len(seqlens) != B:
        raise ValueError(f"shape mismatch q{q.shape} k{kc.shape} v{vc.shape}")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    sl, _ = _ints(seqlens)
    units_a, nunits = _ints(units)
    nu = nunits if units_a is not None else B * Hq
    o = np.empty((nu, D), dtype=np.float64)
    lse = np.empty((nu,), dtype=np.float64)
    st = lib.oracle_decode(q.ctypes.data, kc.ctypes.data, vc.ctypes.data, dt, _ptr(sl, _ip), B,
                           Hq, Hkv, D, Smax, float(scale),
                           _ptr(units_a, _ip) if units_a is not None else None, nunits,
                           _ptr(o), _ptr(lse), int(nthreads))
    if st != 0:
        raise ValueError(f"oracle_decode rejected its arguments (status {st})")
    if units is None:
        return o.reshape(B, Hq, D), lse.reshape(B, Hq)
    return o, lse


def rope(x, pos_offset=0, base=10000.0, round_bits=None, lib=None):
    """Pair rotation of x [B,S,H,D] at positions pos_offset + t; fp64 result
    rounded to `round_bits` significant bits (default: the input format's)."""
    lib = lib or load()
    x, dt = _as_input(x)
    B, S, H, D = x.shape
    if round_bits is None:
        round_bits = default_round_bits(dt)
    out = np.empty(x.shape, dtype=np.float64)
    st = lib.oracle_rope(x.ctypes.data, dt, _ptr(out), B, S, H, D, int(pos_offset), float(base),
                         int(round_bits))
    if st != 0:
        raise ValueError(f"oracle_rope rejected its arguments (status {st})")
    return out


def lse_merge(o_parts, lse_parts, lib=None):
    """Merge per-part (O_i [n,D], lse_i [n]) into (O [D], lse)."""
    lib = lib or load()
    op = _f64(o_parts)
    lp = _f64(lse_parts)
    n, D = op.shape
    o = np.empty(D, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    lib.oracle_lse_merge(_ptr(op), _ptr(lp), n, D, _ptr(o), _ptr(lse))
    return o, float(lse[0])


def flash_decode_head(q, k, v, num_tiles, scale=None, lib=None):
    """Split-KV decode of one head in the pages' order: q [D], k/v [S,D]."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    S, D = k.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.empty(D, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    st = lib.oracle_flash_decode_head(_ptr(q), _ptr(k), _ptr(v), S, D, int(num_tiles),
                                      float(scale), _ptr(o), _ptr(lse))
    if st != 0:
        raise ValueError(f"oracle_flash_decode_head status {st}")
    return o, float(lse[0])


def attn_tiled_head(q, k, v, causal=False, scale=None, block_q=64, block_kv=64, lib=None):
    """Tiled online-softmax forward of one head in the pages' loop order:
    q [Sq,D], k/v [Skv,D] (fp64).  Returns (o [Sq,D], lse [Sq])."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    Sq, D = q.shape
    Skv = k.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.empty((Sq, D), dtype=np.float64)
    lse = np.empty(Sq, dtype=np.float64)
    st = lib.oracle_attn_tiled_head(_ptr(q), _ptr(k), _ptr(v), Sq, Skv, D, int(bool(causal)),
                                    float(scale), int(block_q), int(block_kv), _ptr(o),
                                    _ptr(lse))
    if st != 0:
        raise ValueError(f"oracle_attn_tiled_head status {st}")
    return o, lse


def round_sig(x, bits, lib=None):
    lib = lib or load()
    return lib.oracle_round_sig(float(x), int(bits))
