"""GPU checks of the chunked prefill against a KV cache (attn_prefill_kvcache).

A serving-loop sequence (prefix already cached for one sequence, chunks of
57, 100, 64, 1, 1 and 33 tokens) is compared chunk by chunk with the oracle's
exact attention over the whole sequence so far (queries at positions
L_b + i, keys at j, bottom-right causal), with the forward's bf16 bar; the
cache then holds the rotated keys (the oracle's rotation, rounded to bf16)
and the values, and nothing past the written rows.  At full size, the LFM2
prefill done as four 1024-token chunks reproduces the one-shot attn_fwd bit
for bit (each query row sees the same 64-key tiles in the same order).
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import exact_attention_28_amd as xa
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

NTHREADS = max(1, min(16, len(os.sched_getaffinity(0))))
CANARY = 0x7FC0  # bf16 quiet NaN in unwritten cache rows


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _bits(x):
    return W.f32_to_bf16_bits(x)


@pytest.mark.parametrize("D,Hq,Hkv,causal,rope,Smax", [
    (64, 8, 2, True, 10000.0, 320),
    (128, 4, 4, False, 0.0, 320),
    (64, 12, 4, True, 500.0, 320),
    # caches of >= 16 key tiles: one head per workgroup at D 64 takes four key
    # groups (sized by the cache, most of whose rows are not yet written)
    (64, 4, 4, False, 0.0, 1100),
    (64, 3, 3, True, 0.0, 1100)])
def test_chunked_prefill_serving_loop(D, Hq, Hkv, causal, rope, Smax):
    say("case kvcache", D, Hq, Hkv, causal, rope, Smax)
    B = 2
    chunks = [57, 100, 64, 1, 1, 33]
    prefix = [0, 20]
    total = [prefix[b] + sum(chunks) for b in range(B)]
    rng = np.random.default_rng(D * 7 + Hq)
    k_all = _bits(rng.standard_normal((B, Smax, Hkv, D), dtype=np.float32))
    v_all = _bits(rng.standard_normal((B, Smax, Hkv, D), dtype=np.float32))
    kc = torch.full((B, Smax, Hkv, D), CANARY, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    vc = torch.full((B, Smax, Hkv, D), CANARY, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    # the cached prefix of sequence 1: keys rotated at positions 0..19 by rope_apply
    for b in range(B):
        if prefix[b]:
            kp = W.to_device(k_all[b:b + 1, :prefix[b]]).clone()
            if rope > 0:
                xa.rope_apply(kp, 0, rope)
            kc[b:b + 1, :prefix[b]] = kp
            vc[b:b + 1, :prefix[b]] = W.to_device(v_all[b:b + 1, :prefix[b]])
    lens = torch.tensor(prefix, dtype=torch.int32, device="cuda")
    L = list(prefix)
    scale = float(np.float32(1 / math.sqrt(D)))
    for n in chunks:
        q = _bits(rng.standard_normal((B, n, Hq, D), dtype=np.float32))
        kn = np.stack([k_all[b, L[b]:L[b] + n] for b in range(B)])
        vn = np.stack([v_all[b, L[b]:L[b] + n] for b in range(B)])
        o, lse = xa.attn_prefill_kvcache(W.to_device(q), W.to_device(kn), W.to_device(vn), kc, vc,
                                         lens, causal=causal, scale=scale, rope_base=rope)
        torch.cuda.synchronize()
        og, lg = _np(o), _np(lse)
        for b in range(B):
            o_ref, lse_ref = oracle.attn_fwd(q[b:b + 1], k_all[b:b + 1, :L[b] + n],
                                             v_all[b:b + 1, :L[b] + n], causal=causal,
                                             scale=scale, rope_base=rope, nthreads=NTHREADS)
            err = np.abs(og[b:b + 1] - o_ref).max()
            rel = np.linalg.norm(og[b:b + 1] - o_ref) / np.linalg.norm(o_ref)
            lerr = np.abs(lg[b:b + 1] - lse_ref).max()
            assert err <= 2e-2 and rel <= 5e-3 and lerr <= 1e-3, (n, b, err, rel, lerr)
        lens += n
        L = [L[b] + n for b in range(B)]
    # cache contents: rotated keys (1 bf16 ulp of the oracle's rounded rotation),
    # values as given, canary past the written rows
    kg = kc.view(torch.int16).cpu().numpy().view(np.uint16)
    vg = vc.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(B):
        if rope > 0:
            kr = oracle.rope(k_all[b:b + 1, :total[b]], 0, rope)
            kgot = (kg[b:b + 1, :total[b]].astype(np.uint32) << 16).view(np.float32)
            np.testing.assert_allclose(kgot.astype(np.float64), kr, rtol=2.0 ** -8, atol=0)
        else:
            assert (kg[b, :total[b]] == k_all[b, :total[b]]).all()
        assert (vg[b, :total[b]] == v_all[b, :total[b]]).all()
        assert (kg[b, total[b]:] == CANARY).all() and (vg[b, total[b]:] == CANARY).all()


def test_lfm2_prefill_in_chunks_equals_one_shot():
    """Full-size LFM2 prefill (B4 Hq32 Hkv8 S4096 D64 causal RoPE) as four
    1024-token chunks through the cache gives the one-shot output bit for bit."""
    cfg = W.C4
    say("case", cfg.name, "in 4 chunks")
    q, k, v = W.prefill_inputs(cfg)
    qd, kd, vd = W.to_device(q), W.to_device(k), W.to_device(v)
    o1, l1 = xa.attn_fwd(qd, kd, vd, causal=True, scale=cfg.scale, rope_base=cfg.rope_base)
    kc = torch.empty_like(kd)
    vc = torch.empty_like(vd)
    lens = torch.zeros(cfg.B, dtype=torch.int32, device="cuda")
    C = 1024
    for c0 in range(0, cfg.Sq, C):
        o, lse = xa.attn_prefill_kvcache(qd[:, c0:c0 + C].contiguous(),
                                         kd[:, c0:c0 + C].contiguous(),
                                         vd[:, c0:c0 + C].contiguous(), kc, vc, lens, causal=True,
                                         scale=cfg.scale, rope_base=cfg.rope_base)
        assert torch.equal(o.view(torch.int16), o1[:, c0:c0 + C].contiguous().view(torch.int16))
        assert torch.equal(lse, l1[:, :, c0:c0 + C].contiguous())
        lens += C
    torch.cuda.synchronize()
