"""GPU checks that the forward, decode and chunked-prefill entry points touch
only their own memory and give the same bits every time.

Every input sits between NaN guard regions (a read past an input would
bring a NaN into the result) and every output between canary regions that
must survive the call; the guarded call's outputs must equal, bit for bit,
those of the same call on plain tensors, and three repetitions of the plain
call must agree bit for bit (a missing barrier on a double-buffered LDS
tile, or any other race, shows up as run-to-run differences).  The shapes
cover the pipelined forward with one and two query blocks per wave and with
two key groups per workgroup, RoPE, ragged tiles, the masked forward, the
fp32 forward, the split-KV decode (workspace and built-in scratch) and the
chunked prefill against a KV cache.
"""
import math
import sys

import numpy as np
import pytest
import torch

import exact_attention_28_amd as xa

pytestmark = pytest.mark.gpu

GUARD = 4096  # elements on each side


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _guarded(like_shape, dtype, fill, src=None):
    n = math.prod(like_shape)
    buf = torch.full((n + 2 * GUARD,), fill, dtype=dtype, device="cuda")
    view = buf[GUARD:GUARD + n].view(like_shape)
    if src is not None:
        view.copy_(src)
    return buf, view


def _intact(buf, n, fill, what):
    ends = torch.cat([buf[:GUARD], buf[GUARD + n:]]).float()
    if math.isnan(fill):
        assert torch.isnan(ends).all(), f"{what}: guard region written"
    else:
        assert (ends == fill).all(), f"{what}: guard region written"


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


def _rand(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype).cuda()


FWD_CASES = [  # B, Hq, Hkv, Sq, Skv, D, causal, rope, dtype
    (2, 8, 2, 300, 300, 64, True, 10000.0, torch.bfloat16),    # one query block per wave, RoPE
    (8, 32, 8, 1024, 1024, 64, True, 10000.0, torch.bfloat16),  # two query blocks per wave
    (1, 4, 4, 200, 1100, 128, False, 0.0, torch.bfloat16),     # two key groups per workgroup
    (1, 6, 2, 77, 190, 64, False, 0.0, torch.float16),
    (1, 2, 1, 100, 150, 64, True, 0.0, torch.float32),         # fp32 kernel
]


@pytest.mark.parametrize("case", FWD_CASES, ids=[str(c[:8]) for c in FWD_CASES])
def test_forward_guards_and_repeatability(case):
    B, Hq, Hkv, Sq, Skv, D, causal, rope, dt = case
    say("case guards fwd", case)
    q, k, v = (_rand(s, dt, 11 + i) for i, s in
               enumerate(((B, Sq, Hq, D), (B, Skv, Hkv, D), (B, Skv, Hkv, D))))
    runs = []
    for _ in range(3):
        o, lse = xa.attn_fwd(q, k, v, causal=causal, rope_base=rope)
        runs.append((_bits(o), lse.cpu().numpy().view(np.int32)))
    torch.cuda.synchronize()
    for o_b, l_b in runs[1:]:
        np.testing.assert_array_equal(o_b, runs[0][0])
        np.testing.assert_array_equal(l_b, runs[0][1])
    bq, gq = _guarded(q.shape, dt, float("nan"), q)
    bk, gk = _guarded(k.shape, dt, float("nan"), k)
    bv, gv = _guarded(v.shape, dt, float("nan"), v)
    bo, go = _guarded(q.shape, dt, 7.0)
    bl, gl = _guarded((B, Hq, Sq), torch.float32, 7.0)
    xa.attn_fwd(gq, gk, gv, causal=causal, rope_base=rope, o=go, lse=gl)
    torch.cuda.synchronize()
    _intact(bo, go.numel(), 7.0, "o")
    _intact(bl, gl.numel(), 7.0, "lse")
    for b, t, name in ((bq, gq, "q"), (bk, gk, "k"), (bv, gv, "v")):
        _intact(b, t.numel(), float("nan"), name)
    np.testing.assert_array_equal(_bits(go), runs[0][0])
    np.testing.assert_array_equal(gl.cpu().numpy().view(np.int32), runs[0][1])


def test_masked_forward_guards():
    B, Hq, Hkv, Sq, Skv, D = 1, 4, 2, 130, 257, 64
    say("case guards masked", B, Hq, Hkv, Sq, Skv, D)
    q, k, v = (_rand(s, torch.bfloat16, 21 + i) for i, s in
               enumerate(((B, Sq, Hq, D), (B, Skv, Hkv, D), (B, Skv, Hkv, D))))
    mask = _rand((Sq, Skv), torch.float32, 24)
    o_ref, l_ref = xa.attn_fwd_masked(q, k, v, mask, causal=True)
    bm, gm = _guarded(mask.shape, torch.float32, float("nan"), mask)
    bo, go = _guarded(q.shape, torch.bfloat16, 7.0)
    bl, gl = _guarded((B, Hq, Sq), torch.float32, 7.0)
    xa.attn_fwd_masked(q, k, v, gm, causal=True, o=go, lse=gl)
    torch.cuda.synchronize()
    _intact(bm, gm.numel(), float("nan"), "mask")
    _intact(bo, go.numel(), 7.0, "o")
    _intact(bl, gl.numel(), 7.0, "lse")
    np.testing.assert_array_equal(_bits(go), _bits(o_ref))
    np.testing.assert_array_equal(gl.cpu().numpy(), l_ref.cpu().numpy())


@pytest.mark.parametrize("noalloc", [False, True])
def test_decode_guards_and_repeatability(noalloc):
    B, Hq, Hkv, D, Smax, ns = 3, 8, 2, 128, 700, 8
    lens = torch.tensor([0, 700, 33], dtype=torch.int32).cuda()
    say("case guards decode", B, Hq, Hkv, D, Smax, ns, "noalloc" if noalloc else "workspace")
    q = _rand((B, Hq, D), torch.bfloat16, 31)
    kc = _rand((B, Smax, Hkv, D), torch.bfloat16, 32)
    vc = _rand((B, Smax, Hkv, D), torch.bfloat16, 33)

    def call(q_, kc_, vc_, o_, l_):
        if noalloc:
            xa.attn_decode_splitkv_noalloc(q_, kc_, vc_, lens, ns, o_, l_)
        else:
            xa.attn_decode_splitkv(q_, kc_, vc_, lens, ns, o=o_, lse=l_)
    runs = []
    for _ in range(3):
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        call(q, kc, vc, o, lse)
        runs.append((_bits(o), lse.cpu().numpy()))
    for o_b, l_b in runs[1:]:
        np.testing.assert_array_equal(o_b, runs[0][0])
        np.testing.assert_array_equal(l_b, runs[0][1])
    bq, gq = _guarded(q.shape, torch.bfloat16, float("nan"), q)
    bk, gk = _guarded(kc.shape, torch.bfloat16, float("nan"), kc)
    bv, gv = _guarded(vc.shape, torch.bfloat16, float("nan"), vc)
    bo, go = _guarded(q.shape, torch.bfloat16, 7.0)
    bl, gl = _guarded((B, Hq), torch.float32, 7.0)
    call(gq, gk, gv, go, gl)
    torch.cuda.synchronize()
    _intact(bo, go.numel(), 7.0, "o")
    _intact(bl, gl.numel(), 7.0, "lse")
    for b, t, name in ((bq, gq, "q"), (bk, gk, "kcache"), (bv, gv, "vcache")):
        _intact(b, t.numel(), float("nan"), name)
    np.testing.assert_array_equal(_bits(go), runs[0][0])
    np.testing.assert_array_equal(gl.cpu().numpy(), runs[0][1])


def test_chunked_prefill_guards():
    B, Hq, Hkv, Sq, D, Smax = 2, 8, 2, 50, 64, 300
    lens = torch.tensor([0, 100], dtype=torch.int32).cuda()
    say("case guards kvcache", B, Hq, Hkv, Sq, D, Smax)
    q = _rand((B, Sq, Hq, D), torch.bfloat16, 41)
    kn = _rand((B, Sq, Hkv, D), torch.bfloat16, 42)
    vn = _rand((B, Sq, Hkv, D), torch.bfloat16, 43)
    kc0 = _rand((B, Smax, Hkv, D), torch.bfloat16, 44)
    vc0 = _rand((B, Smax, Hkv, D), torch.bfloat16, 45)
    kc, vc = kc0.clone(), vc0.clone()
    o_ref, l_ref = xa.attn_prefill_kvcache(q, kn, vn, kc, vc, lens, causal=True, rope_base=10000.0)
    bk, gk = _guarded(kc0.shape, torch.bfloat16, 7.0, kc0)
    bv, gv = _guarded(vc0.shape, torch.bfloat16, 7.0, vc0)
    bo, go = _guarded(q.shape, torch.bfloat16, 7.0)
    bl, gl = _guarded((B, Hq, Sq), torch.float32, 7.0)
    xa.attn_prefill_kvcache(q, kn, vn, gk, gv, lens, causal=True, rope_base=10000.0, o=go, lse=gl)
    torch.cuda.synchronize()
    for b, t, name in ((bk, gk, "kcache"), (bv, gv, "vcache"), (bo, go, "o"), (bl, gl, "lse")):
        _intact(b, t.numel(), 7.0, name)
    np.testing.assert_array_equal(_bits(gk), _bits(kc))
    np.testing.assert_array_equal(_bits(gv), _bits(vc))
    np.testing.assert_array_equal(_bits(go), _bits(o_ref))
    np.testing.assert_array_equal(gl.cpu().numpy(), l_ref.cpu().numpy())
