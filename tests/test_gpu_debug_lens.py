"""ATTN_DEBUG=1: host-side check of the device-resident length preconditions.

attn_decode_splitkv requires 0 <= seqlens[b] <= max_seqlen and
attn_prefill_kvcache 0 <= cache_lens[b] <= max_seqlen - Sq.  The values live
in device memory, so by default they are not checked (out-of-range values are
clamped).  With ATTN_DEBUG=1 the library copies them to the host first and
rejects a call with an out-of-range value with ATTN_ERR_INVALID before any
launch (the output keeps its sentinel); in-range calls give the same bits as
without the check.
"""
import sys

import numpy as np
import pytest
import torch

import exact_attention_28_amd as xa
import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _decode_case():
    cfg = W.Decode("debug", 3, 8, 2, 64, 256, 1, 256, 91)
    qn, kcn, vcn, sln = W.decode_inputs(cfg)
    return cfg, W.to_device(qn), W.to_device(kcn), W.to_device(vcn), sln


@pytest.mark.parametrize("bad", [257, -1, 100000])
def test_decode_lengths_checked_under_debug(monkeypatch, bad):
    say("case debug decode", bad)
    cfg, q, kc, vc, sln = _decode_case()
    good = torch.from_numpy(sln).cuda()
    o_ref, lse_ref = xa.attn_decode_splitkv(q, kc, vc, good, 4, scale=cfg.scale)
    torch.cuda.synchronize()
    bad_lens = sln.copy()
    bad_lens[1] = bad
    bad_d = torch.from_numpy(bad_lens).cuda()
    # without the check the call runs (the value is clamped into range)
    xa.attn_decode_splitkv(q, kc, vc, bad_d, 4, scale=cfg.scale)
    torch.cuda.synchronize()
    monkeypatch.setenv("ATTN_DEBUG", "1")
    o = torch.full_like(q, 7.0)
    with pytest.raises(xa.AttnError) as e:
        xa.attn_decode_splitkv(q, kc, vc, bad_d, 4, scale=cfg.scale, o=o)
    assert e.value.code == xa.ATTN_ERR_INVALID
    assert "seqlens[1]" in str(e.value)
    torch.cuda.synchronize()
    assert (o == 7.0).all()  # nothing was launched
    o2, lse2 = xa.attn_decode_splitkv(q, kc, vc, good, 4, scale=cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(lse2, lse_ref)


def test_kvcache_lengths_checked_under_debug(monkeypatch):
    say("case debug kvcache")
    B, Hq, Hkv, Sq, D, Smax = 2, 8, 2, 16, 64, 128
    rng = np.random.default_rng(92)

    def bf(shape):
        return W.to_device(W.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32)))
    q, kn, vn = bf((B, Sq, Hq, D)), bf((B, Sq, Hkv, D)), bf((B, Sq, Hkv, D))
    kc, vc = bf((B, Smax, Hkv, D)), bf((B, Smax, Hkv, D))
    ok = torch.tensor([0, Smax - Sq], dtype=torch.int32, device="cuda")
    bad = torch.tensor([0, Smax - Sq + 1], dtype=torch.int32, device="cuda")
    monkeypatch.setenv("ATTN_DEBUG", "1")
    kc0, vc0 = kc.clone(), vc.clone()
    o = torch.full_like(q, 7.0)
    with pytest.raises(xa.AttnError) as e:
        xa.attn_prefill_kvcache(q, kn, vn, kc, vc, bad, causal=True, rope_base=10000.0, o=o)
    assert e.value.code == xa.ATTN_ERR_INVALID
    assert "cache_lens[1]" in str(e.value)
    torch.cuda.synchronize()
    assert (o == 7.0).all()
    assert torch.equal(kc.view(torch.int16), kc0.view(torch.int16))  # no append either
    assert torch.equal(vc.view(torch.int16), vc0.view(torch.int16))
    o1, l1 = xa.attn_prefill_kvcache(q, kn, vn, kc, vc, ok, causal=True, rope_base=10000.0)
    torch.cuda.synchronize()
    monkeypatch.delenv("ATTN_DEBUG")
    kc2, vc2 = kc0.clone(), vc0.clone()
    o2, l2 = xa.attn_prefill_kvcache(q, kn, vn, kc2, vc2, ok, causal=True, rope_base=10000.0)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    assert torch.equal(kc.view(torch.int16), kc2.view(torch.int16))
