"""GPU parity of the attention backward (attn_bwd through the C ABI) against
the fp64 oracle's gradients, on the same seeded bf16 inputs.

The GPU pass takes the forward's own bf16 output O and fp32 LSE (as a training
step would); the oracle differentiates the exact attention of the same q, k, v
(with the rotated q, k rounded to bf16 as the forward does) for the same dO.

Bar per gradient tensor (dq, dk, dv): relative L2 error <= 1e-2 and max-abs
error <= 2e-2 * max |reference|.  Sources of error, all relative to the
quantities they touch: P and dS enter the MFMAs as bf16 (2^-9 each, random),
the outputs are stored as bf16 (2^-9), and D_i = rowsum(dO o O) uses the
forward's bf16 O (2^-9 per term); the fp32 accumulation and the lse from the
forward add ~1e-6.  These give a relative L2 error of a few 1e-3; the bar is
about three times that.
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


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_grad(g, ref, what):
    g = np.asarray(g, np.float64)
    assert np.isfinite(g).all(), f"{what}: non-finite gradient"
    scale = max(np.abs(ref).max(), 1e-30)
    rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
    err = np.abs(g - ref).max() / scale
    say(f"  {what}: rel-L2 {rel:.2e}, max-abs/max|ref| {err:.2e}")
    assert rel <= 1e-2, f"{what}: rel-L2 {rel:.3e}"
    assert err <= 2e-2, f"{what}: max-abs {err:.3e} of max |ref|"
    return rel, err


def _inputs(rng, B, Hq, Hkv, Sq, Skv, D, amp=1.0):
    f = [rng.standard_normal(s, dtype=np.float32) * np.float32(amp)
         for s in ((B, Sq, Hq, D), (B, Skv, Hkv, D), (B, Skv, Hkv, D), (B, Sq, Hq, D))]
    return [W.f32_to_bf16_bits(x) for x in f]


def run_bwd(q, k, v, do, causal, scale, rope):
    qd, kd, vd, dod = (W.to_device(x) for x in (q, k, v, do))
    o, lse = xa.attn_fwd(qd, kd, vd, causal=causal, scale=scale, rope_base=rope)
    dq, dk, dv = xa.attn_bwd(qd, kd, vd, o, dod, lse, causal=causal, scale=scale, rope_base=rope)
    torch.cuda.synchronize()
    return _np(dq), _np(dk), _np(dv)


BWD_CASES = [  # B, Hq, Hkv, Sq, Skv, causal, rope
    (2, 8, 2, 300, 300, True, 10000.0),    # ragged query and key tiles, GQA 4, RoPE
    (1, 4, 4, 200, 333, False, 0.0),       # MHA, Sq != Skv, no mask
    (1, 4, 1, 100, 260, True, 10000.0),    # bottom-right causal, Sq < Skv, RoPE
    (1, 2, 1, 70, 20, True, 0.0),          # rows with no visible key (Sq > Skv)
    (1, 16, 2, 129, 129, False, 500.0),    # 8 query heads per kv head
    (2, 6, 3, 64, 64, True, 0.0),          # exactly one tile
    (3, 3, 3, 1, 1, False, 0.0),           # single key: dq = dk = 0
    (1, 12, 4, 97, 150, True, 0.0),        # 3 query heads per kv head
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[str(c) for c in BWD_CASES])
def test_bwd_variants(case):
    B, Hq, Hkv, Sq, Skv, causal, rope = case
    D = 64
    say("case bwd", case)
    rng = np.random.default_rng(W.case_seed(case))
    q, k, v, do = _inputs(rng, B, Hq, Hkv, Sq, Skv, D)
    scale = float(np.float32(1 / math.sqrt(D)))
    got = run_bwd(q, k, v, do, causal, scale, rope)
    ref = oracle.attn_bwd(q, k, v, do, causal=causal, scale=scale, rope_base=rope,
                          nthreads=NTHREADS)
    if Skv == 1:
        # P = 1 and dP = D analytically (dq = dk = 0 in the oracle); on the GPU
        # dP (MFMA) and D (from O) are two fp32 sums of ~64 products of size ~1,
        # each within ~64 * 2^-24 * 8 of the exact value, so |dS| < 1e-4 and
        # |dq|, |dk| < scale * |dS| * |k| (< 1e-5 here)
        assert np.abs(got[0]).max() < 1e-5 and np.abs(got[1]).max() < 1e-5
        check_grad(got[2], ref[2], f"{case} dv")
        return
    for g, r, n in zip(got, ref, ("dq", "dk", "dv")):
        if Sq > Skv and n == "dq":  # rows without keys have dq = 0 exactly
            hidden = np.arange(Sq) < Sq - Skv
            assert (got[0][:, hidden] == 0).all()
        check_grad(g, r, f"{case} {n}")


def test_bwd_mha_1024_workload_full():
    """The 1024-token causal MHA workload (B2 H8 D64), every gradient in full."""
    cfg = W.C2C
    say("case", cfg.name, "backward")
    q, k, v = W.prefill_inputs(cfg)
    rng = np.random.default_rng(cfg.seed + 7)
    do = W.f32_to_bf16_bits(rng.standard_normal(q.shape, dtype=np.float32))
    got = run_bwd(q, k, v, do, cfg.causal, cfg.scale, cfg.rope_base)
    ref = oracle.attn_bwd(q, k, v, do, causal=cfg.causal, scale=cfg.scale,
                          rope_base=cfg.rope_base, nthreads=NTHREADS)
    for g, r, n in zip(got, ref, ("dq", "dk", "dv")):
        check_grad(g, r, f"{cfg.name} {n}")


def test_bwd_lfm2_workload_four_groups():
    """The LFM2 prefill workload at full size (B4 Hq32 Hkv8 S4096 causal RoPE),
    in the launch configuration the benchmark times; the oracle evaluates four
    (batch, kv head) units, the first and last batch with the first and last
    kv head, each with its 4 query heads: dk, dv of those kv heads and dq of
    their query heads, every element."""
    cfg = W.C4
    say("case", cfg.name, "backward")
    q, k, v = W.prefill_inputs(cfg)
    rng = np.random.default_rng(cfg.seed + 7)
    do = W.f32_to_bf16_bits(rng.standard_normal(q.shape, dtype=np.float32))
    dq, dk, dv = run_bwd(q, k, v, do, cfg.causal, cfg.scale, cfg.rope_base)
    G = cfg.Hq // cfg.Hkv
    pairs = [(0, 0), (0, cfg.Hkv - 1), (cfg.B - 1, 0), (cfg.B - 1, cfg.Hkv - 1)]
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, causal=cfg.causal, scale=cfg.scale,
                                 rope_base=cfg.rope_base, units=[b * cfg.Hkv + g for b, g in pairs],
                                 nthreads=min(4, NTHREADS))
    for b, g in pairs:
        say(f"  unit b={b} kv head {g}")
        check_grad(dq[b, :, g * G:(g + 1) * G], rq[b, :, g * G:(g + 1) * G],
                   f"{cfg.name} dq b{b} g{g}")
        check_grad(dk[b, :, g], rk[b, :, g], f"{cfg.name} dk b{b} g{g}")
        check_grad(dv[b, :, g], rv[b, :, g], f"{cfg.name} dv b{b} g{g}")


def test_bwd_deterministic_and_workspace():
    """Two calls give the same bits (no atomics); a caller workspace gives the
    same result as the library's; outputs outside the tensors are untouched."""
    B, Hq, Hkv, Sq, Skv, D = 2, 8, 2, 200, 200, 64
    rng = np.random.default_rng(5)
    q, k, v, do = (W.to_device(x) for x in _inputs(rng, B, Hq, Hkv, Sq, Skv, D))
    o, lse = xa.attn_fwd(q, k, v, causal=True, rope_base=10000.0)
    a = xa.attn_bwd(q, k, v, o, do, lse, causal=True, rope_base=10000.0)
    ws = torch.empty(xa.attn_bwd_workspace_bytes(B, Hq, Hkv, Sq, Skv, D, 10000.0),
                     dtype=torch.uint8, device="cuda")
    guard = torch.full((B * Sq * Hq * D + 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    dq = guard[1024:1024 + B * Sq * Hq * D].view(B, Sq, Hq, D)
    b2 = xa.attn_bwd(q, k, v, o, do, lse, causal=True, rope_base=10000.0, dq=dq, workspace=ws)
    torch.cuda.synchronize()
    for x, y in zip(a, b2):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert (guard[:1024] == 7.0).all() and (guard[1024 + B * Sq * Hq * D:] == 7.0).all()


def test_bwd_guard_regions():
    """Every input of the backward sits between NaN guard regions and every
    output between sentinel regions: a read past an input turns a gradient
    NaN, a write past an output changes a sentinel."""
    B, Hq, Hkv, S, D = 1, 4, 2, 190, 64
    rng = np.random.default_rng(13)
    q, k, v, do = _inputs(rng, B, Hq, Hkv, S, S, D)
    G = 1 << 14

    def guarded(t, fill):
        flat = torch.full((t.numel() + 2 * G,), fill, dtype=t.dtype, device="cuda")
        flat[G:G + t.numel()] = t.reshape(-1)
        return flat, flat[G:G + t.numel()].view(t.shape)

    qd, kd, vd, dod = (W.to_device(x) for x in (q, k, v, do))
    for causal, rope in ((True, 10000.0), (False, 0.0)):
        o, lse = xa.attn_fwd(qd, kd, vd, causal=causal, rope_base=rope)
        gq, gk, gv, go, gdo, gl = (guarded(t, float("nan"))[1] for t in (qd, kd, vd, o, dod, lse))
        outs = [guarded(torch.empty_like(t), 7.0) for t in (qd, kd, vd)]
        dq, dk, dv = xa.attn_bwd(gq, gk, gv, go, gdo, gl, causal=causal, rope_base=rope,
                                 dq=outs[0][1], dk=outs[1][1], dv=outs[2][1])
        torch.cuda.synchronize()
        ref = oracle.attn_bwd(q, k, v, do, causal=causal, scale=1 / math.sqrt(D),
                              rope_base=rope, nthreads=NTHREADS)
        for g, r, n in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
            check_grad(_np(g), r, f"guarded causal={causal} {n}")
        for flat, view in outs:
            assert (flat[:G] == 7.0).all() and (flat[G + view.numel():] == 7.0).all()
