"""GPU parity for IEEE binary16 (fp16) inputs: attn_fwd, attn_fwd_masked,
attn_bwd and rope_apply with dtype fp16, through the C ABI, against the fp64 oracle fed the
same fp16 values (widened exactly; rotated q and k rounded to fp16, as the
kernels do).

Bar (derived as for bf16, with fp16's 11 significant bits): P enters the PV
product as fp16 (relative 2^-11 per weight, averaging out) and O is stored as
fp16 (half an ulp, 2^-11 relative: <= 2e-3 at |O| <= 4), so O max-abs 5e-3
and rel-L2 2e-3; the LSE comes from fp32 m and l as in bf16 (~1e-6), with the
same 1e-3 bar.
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


def check_f16(o_gpu, lse_gpu, o_ref, lse_ref, what):
    o_gpu = np.asarray(o_gpu, np.float64)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite output"
    err = np.abs(o_gpu - o_ref)
    rel = np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-30)
    say(f"  {what}: O max-abs {err.max():.2e} rel-L2 {rel:.2e}")
    assert err.max() <= 5e-3, f"{what}: O max-abs {err.max():.3e}"
    assert rel <= 2e-3, f"{what}: O rel-L2 {rel:.3e}"
    fin = np.isfinite(lse_ref)
    assert (np.isfinite(lse_gpu) == fin).all(), f"{what}: LSE finiteness differs"
    if fin.any():
        lerr = np.abs(np.asarray(lse_gpu, np.float64)[fin] - lse_ref[fin]).max()
        assert lerr <= 1e-3, f"{what}: LSE max-abs {lerr:.3e}"
    assert (np.asarray(lse_gpu)[~fin] == -np.inf).all()


def _inputs(rng, B, Hq, Hkv, Sq, Skv, D):
    return (rng.standard_normal((B, Sq, Hq, D), dtype=np.float32).astype(np.float16),
            rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32).astype(np.float16),
            rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32).astype(np.float16))


F16_CASES = [  # B, Hq, Hkv, Sq, Skv, D, causal, rope
    (2, 8, 2, 300, 300, 64, True, 10000.0),   # GQA 4, RoPE, ragged tiles
    (1, 4, 4, 200, 333, 128, False, 0.0),     # D = 128, cross lengths
    (1, 4, 1, 100, 260, 64, True, 10000.0),   # bottom-right causal, Sq < Skv
    (1, 2, 1, 70, 20, 64, True, 0.0),         # rows with no visible key
    (1, 16, 2, 129, 129, 128, True, 500.0),   # 8 heads per kv head
    (2, 6, 3, 33, 90, 40, False, 10000.0),    # padded head dim
    (4, 4, 4, 600, 600, 64, False, 0.0),      # two query blocks per wave
    (1, 4, 2, 150, 1090, 64, True, 0.0),      # two key groups per workgroup
    (1, 3, 3, 150, 1090, 64, True, 0.0),      # four key groups of two waves
]


@pytest.mark.parametrize("case", F16_CASES, ids=[str(c) for c in F16_CASES])
def test_f16_variants(case):
    B, Hq, Hkv, Sq, Skv, D, causal, rope = case
    say("case f16", case)
    rng = np.random.default_rng(W.case_seed(case))
    q, k, v = _inputs(rng, B, Hq, Hkv, Sq, Skv, D)
    scale = float(np.float32(1 / math.sqrt(D)))
    o, lse = xa.attn_fwd(W.to_device(q), W.to_device(k), W.to_device(v), causal=causal,
                         scale=scale, rope_base=rope)
    assert o.dtype == torch.float16
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=causal, scale=scale, rope_base=rope,
                                     nthreads=NTHREADS)
    check_f16(_np(o), _np(lse), o_ref, lse_ref, f"f16 {case}")


@pytest.mark.parametrize("Skv", [211, 212])
def test_f16_masked(Skv):
    """fp16 with an additive mask: per (batch, head), -inf entries, RoPE; 211
    keys read the mask per lane, 212 stage it through LDS."""
    B, Hq, Hkv, Sq, D = 2, 8, 2, 150, 64
    say("case f16 masked", Skv)
    rng = np.random.default_rng(21)
    q, k, v = _inputs(rng, B, Hq, Hkv, Sq, Skv, D)
    m = (rng.standard_normal((B, Hq, Sq, Skv)) * 2.0).astype(np.float32)
    m[rng.random(m.shape) < 0.1] = -np.inf
    o, lse = xa.attn_fwd_masked(W.to_device(q), W.to_device(k), W.to_device(v),
                                torch.from_numpy(m).cuda(), causal=True, scale=0.125,
                                rope_base=10000.0)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=True, scale=0.125, rope_base=10000.0,
                                     mask=m.astype(np.float64), nthreads=NTHREADS)
    check_f16(_np(o), _np(lse), o_ref, lse_ref, "f16 masked")


def test_f16_lfm2_workload_full():
    """The LFM2 prefill shape (B4 Hq32 Hkv8 S4096 D64 causal RoPE) with the
    workload's fp32 draws rounded to fp16 instead of bf16, every element of
    every (batch, head)."""
    cfg = W.C4
    say("case", cfg.name, "fp16")
    rng = np.random.default_rng(cfg.seed)
    q, k, v = (rng.standard_normal(s, dtype=np.float32).astype(np.float16)
               for s in ((cfg.B, cfg.Sq, cfg.Hq, cfg.D), (cfg.B, cfg.Skv, cfg.Hkv, cfg.D),
                         (cfg.B, cfg.Skv, cfg.Hkv, cfg.D)))
    o, lse = xa.attn_fwd(W.to_device(q), W.to_device(k), W.to_device(v), causal=True,
                         scale=cfg.scale, rope_base=cfg.rope_base)
    torch.cuda.synchronize()
    o, lse = _np(o), _np(lse)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=True, scale=cfg.scale,
                                     rope_base=cfg.rope_base, nthreads=NTHREADS)
    check_f16(o, lse, o_ref, lse_ref, f"{cfg.name} fp16")


@pytest.mark.parametrize("D,off", [(64, 0), (128, 1000), (6, 3)])
def test_rope_apply_f16(D, off):
    """Both sides round an fp64-accurate rotation once to fp16 (subnormals
    included): equal except where the two fp64 values straddle a rounding
    boundary, and never more than one fp16 step apart."""
    say("case rope_apply f16", D, off)
    rng = np.random.default_rng(34)
    x = rng.standard_normal((2, 37, 3, D), dtype=np.float32).astype(np.float16)
    x[0, 5, 0, :2] = np.float16(3e-6)  # a subnormal pair
    xd = W.to_device(x)
    xa.rope_apply(xd, pos_offset=off, rope_base=10000.0)
    torch.cuda.synchronize()
    got = _np(xd)
    ref = oracle.rope(x, pos_offset=off, base=10000.0)
    step = np.maximum(np.abs(ref) * 2.0 ** -10, 2.0 ** -24)
    assert (np.abs(got - ref) <= step).all()
    assert (got == ref).mean() > 0.9999


BWD16_CASES = [  # B, Hq, Hkv, Sq, Skv, causal, rope
    (2, 8, 2, 300, 300, True, 10000.0),    # GQA 4, RoPE, ragged tiles
    (1, 4, 4, 200, 333, False, 0.0),       # MHA, Sq != Skv
    (1, 4, 1, 100, 260, True, 10000.0),    # bottom-right causal, Sq < Skv
    (1, 12, 4, 97, 150, True, 0.0),        # 3 query heads per kv head
]


@pytest.mark.parametrize("case", BWD16_CASES, ids=[str(c) for c in BWD16_CASES])
def test_f16_backward(case):
    """attn_bwd on fp16 inputs (P and dS enter the MFMAs as fp16) against the
    oracle's gradients of the same fp16 values, with the bf16 backward's bar:
    per tensor rel-L2 <= 1e-2 and max-abs <= 2e-2 max |ref| (fp16's rounding
    is 8 times finer, so this holds with a wide margin)."""
    from test_gpu_backward import check_grad
    B, Hq, Hkv, Sq, Skv, causal, rope = case
    D = 64
    say("case f16 bwd", case)
    rng = np.random.default_rng(W.case_seed(case))
    q, k, v = _inputs(rng, B, Hq, Hkv, Sq, Skv, D)
    do = rng.standard_normal((B, Sq, Hq, D), dtype=np.float32).astype(np.float16)
    scale = float(np.float32(1 / math.sqrt(D)))
    qd, kd, vd, dod = (W.to_device(x) for x in (q, k, v, do))
    o, lse = xa.attn_fwd(qd, kd, vd, causal=causal, scale=scale, rope_base=rope)
    dq, dk, dv = xa.attn_bwd(qd, kd, vd, o, dod, lse, causal=causal, scale=scale, rope_base=rope)
    assert dq.dtype == torch.float16
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(q, k, v, do, causal=causal, scale=scale, rope_base=rope,
                          nthreads=NTHREADS)
    for g, r, n in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
        check_grad(_np(g), r, f"f16 {case} {n}")


def test_f16_unsupported_paths():
    """fp32 and D = 128 have no backward: ATTN_ERR_UNSUPPORTED."""
    for dt, D in ((torch.float32, 64), (torch.float16, 128)):
        q = torch.zeros(1, 8, 4, D, dtype=dt, device="cuda")
        o, lse = xa.attn_fwd(q, q, q)
        with pytest.raises(xa.AttnError) as e:
            xa.attn_bwd(q, q, q, o, o, lse)
        assert e.value.code == xa.ATTN_ERR_UNSUPPORTED
