"""GPU parity of the forward with an additive float mask (attn_fwd_masked
through the C ABI) against the fp64 oracle given the same fp32 mask values.

The bars are those of the unmasked forward (bf16: O max-abs 2e-2, rel-L2
5e-3, LSE max-abs 1e-3; fp32: 1e-4).  Masks are standard normal values times
2 with about a tenth of the entries -inf; they are passed in every broadcast
form the entry point takes (one [Sq, Skv] mask, per head, per batch and head,
a per-key padding row), with row lengths that do and do not allow 16-byte
loads, together with the causal flag, RoPE, grouped heads and padded head
dims.  At D = 64, masks whose rows allow 16-byte loads and whose key count is
a multiple of 4 are staged through LDS by the kernel (per wave, or once per
workgroup when every head shares the mask); the others are read per lane: all
three paths are covered, and one test checks that they give the same bits.  Rows whose keys are all hidden give O = 0 and lse = -inf.
"""
import json
import math
import os
import sys

import numpy as np
import pytest
import torch

import exact_attention_28_amd as xa
import oracle
import workloads as W
from test_gpu_parity import check_bf16, check_f32

pytestmark = pytest.mark.gpu

NTHREADS = max(1, min(16, len(os.sched_getaffinity(0))))
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _mask(rng, shape, hide=0.1):
    m = (rng.standard_normal(shape) * 2.0).astype(np.float32)
    m[rng.random(shape) < hide] = -np.inf
    return m


def run_masked(q, k, v, mask, causal, scale, rope):
    o, lse = xa.attn_fwd_masked(W.to_device(q), W.to_device(k), W.to_device(v),
                                torch.from_numpy(mask).to("cuda"), causal=causal, scale=scale,
                                rope_base=rope)
    torch.cuda.synchronize()
    return _np(o), _np(lse)


def _oracle(q, k, v, mask, causal, scale, rope, B, Hq, Sq, Skv, **kw):
    """The oracle takes a [1 or B, 1 or Hq, Sq, Skv] mask: a mask broadcast over
    query rows is widened along that axis first."""
    m4 = mask.reshape((1,) * (4 - mask.ndim) + mask.shape).astype(np.float64)
    m4 = np.broadcast_to(m4, (m4.shape[0], m4.shape[1], Sq, Skv))
    return oracle.attn_fwd(q, k, v, causal=causal, scale=scale, rope_base=rope, mask=m4,
                           nthreads=NTHREADS, **kw)


def test_golden_explicit_mask():
    """The page's two-token example with its explicit [[0, -inf], [0, 0]] mask
    (head dim 4, through the padded path): output[0] = 1.0, and the derived
    O and LSE."""
    g = json.load(open(os.path.join(GOLDEN, "whisper_causal_mask_example.json")))
    mask = np.array([[float(x) for x in r] for r in g["mask"]], dtype=np.float32)
    for dt in ("f32", "bf16"):
        say("case golden mask", dt)
        q, k, v = (np.array(g[n], dtype=np.float32)[None, :, None, :] for n in ("q", "k", "v"))
        if dt == "bf16":
            q, k, v = (W.f32_to_bf16_bits(x) for x in (q, k, v))
        o, lse = run_masked(q, k, v, mask, False, g["scale"], 0.0)
        assert abs(o[0, 0, 0, 0] - g["printed"]["o[0][0]"]) < g["printed"]["tolerance"]
        np.testing.assert_allclose(o[0, :, 0, :], np.array(g["derived"]["o"]), atol=1e-6)
        np.testing.assert_allclose(lse[0, 0], np.array(g["derived"]["lse"]), atol=1e-6)


MASK_CASES = [  # B, Hq, Hkv, Sq, Skv, D, causal, rope, mask shape ('s' [Sq,Skv], 'h', 'bh', 'kp')
    (2, 8, 2, 200, 333, 64, False, 0.0, "s"),      # ragged keys: scalar mask loads
    (2, 8, 2, 256, 256, 64, True, 10000.0, "bh"),  # 16-byte loads, causal, RoPE
    (1, 4, 4, 130, 300, 128, True, 0.0, "h"),      # D = 128, per-head mask
    (3, 6, 3, 97, 160, 64, False, 500.0, "kp"),    # per-key padding row [B,1,1,Skv]
    (1, 16, 2, 129, 129, 128, False, 10000.0, "s"),  # 8 heads per kv head
    (1, 3, 3, 64, 64, 64, True, 0.0, "bh"),        # one tile
    (2, 4, 1, 1, 517, 64, False, 0.0, "bh"),       # one query row
    (1, 4, 2, 50, 90, 40, True, 10000.0, "s"),     # padded head dim
    (1, 16, 2, 96, 192, 64, False, 0.0, "h"),      # LDS-staged rows, a wave spans two heads
    (2, 4, 2, 130, 256, 64, True, 10000.0, "bh"),  # LDS-staged rows, two heads per workgroup
    (1, 16, 2, 100, 256, 64, True, 10000.0, "s"),  # rows shared by 8 heads of a workgroup
]


def _mask_shape(kind, B, Hq, Sq, Skv):
    return {"s": (Sq, Skv), "h": (1, Hq, Sq, Skv), "bh": (B, Hq, Sq, Skv),
            "kp": (B, 1, 1, Skv)}[kind]


@pytest.mark.parametrize("case", MASK_CASES, ids=[str(c) for c in MASK_CASES])
def test_masked_bf16(case):
    B, Hq, Hkv, Sq, Skv, D, causal, rope, kind = case
    say("case mask bf16", case)
    rng = np.random.default_rng(W.case_seed(case))
    q = W.f32_to_bf16_bits(rng.standard_normal((B, Sq, Hq, D), dtype=np.float32))
    k = W.f32_to_bf16_bits(rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32))
    v = W.f32_to_bf16_bits(rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32))
    mask = _mask(rng, _mask_shape(kind, B, Hq, Sq, Skv))
    scale = float(np.float32(1 / math.sqrt(D)))
    o, lse = run_masked(q, k, v, mask, causal, scale, rope)
    o_ref, lse_ref = _oracle(q, k, v, mask, causal, scale, rope, B, Hq, Sq, Skv)
    check_bf16(o, lse, o_ref, lse_ref, f"mask {case}")


@pytest.mark.parametrize("case", [(2, 4, 2, 100, 150, 64, True, 0.0, "bh"),
                                  (1, 2, 1, 33, 70, 128, False, 10000.0, "s"),
                                  (2, 2, 2, 45, 80, 24, False, 0.0, "kp"),
                                  # 16 lanes per row over five key blocks; 8 lanes;
                                  # 4 lanes, ragged rows and keys, at D 64 and 128
                                  (1, 1, 1, 100, 300, 64, False, 0.0, "s"),
                                  (1, 16, 16, 200, 300, 128, True, 10000.0, "h"),
                                  (2, 8, 2, 1000, 1111, 64, True, 10000.0, "bh"),
                                  (1, 16, 4, 1000, 300, 128, False, 0.0, "kp")],
                         ids=str)
def test_masked_f32(case):
    B, Hq, Hkv, Sq, Skv, D, causal, rope, kind = case
    say("case mask f32", case)
    rng = np.random.default_rng(W.case_seed(case))
    q = rng.standard_normal((B, Sq, Hq, D), dtype=np.float32)
    k = rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32)
    mask = _mask(rng, _mask_shape(kind, B, Hq, Sq, Skv))
    scale = float(np.float32(1 / math.sqrt(D)))
    o, lse = run_masked(q, k, v, mask, causal, scale, rope)
    o_ref, lse_ref = _oracle(q, k, v, mask, causal, scale, rope, B, Hq, Sq, Skv)
    check_f32(o, lse, o_ref, lse_ref, f"mask f32 {case}")


def test_fully_hidden_rows_and_strided_mask():
    """Rows whose keys are all -inf give O = 0 and lse = -inf; a mask that is a
    strided view (rows of a wider array, a row pitch that rules out 16-byte
    loads: read per lane) and one broadcast by expand() give the same bits as
    their contiguous copies (staged through LDS)."""
    B, Hq, Hkv, Sq, Skv, D = 2, 4, 2, 70, 100, 64
    rng = np.random.default_rng(11)
    q = W.f32_to_bf16_bits(rng.standard_normal((B, Sq, Hq, D), dtype=np.float32))
    k = W.f32_to_bf16_bits(rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32))
    v = W.f32_to_bf16_bits(rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32))
    mask = _mask(rng, (Sq, Skv))
    mask[[0, 5, 69]] = -np.inf
    o, lse = run_masked(q, k, v, mask, False, 0.125, 0.0)
    assert (o[:, [0, 5, 69]] == 0).all() and (lse[:, :, [0, 5, 69]] == -np.inf).all()
    o_ref, lse_ref = _oracle(q, k, v, mask, False, 0.125, 0.0, B, Hq, Sq, Skv)
    check_bf16(o, lse, o_ref, lse_ref, "hidden rows")
    qd, kd, vd = W.to_device(q), W.to_device(k), W.to_device(v)
    wide = torch.zeros(Sq, Skv + 27, device="cuda")
    wide[:, :Skv] = torch.from_numpy(mask).cuda()
    a, la = xa.attn_fwd_masked(qd, kd, vd, wide[:, :Skv], scale=0.125)
    b, lb = xa.attn_fwd_masked(qd, kd, vd, wide[:, :Skv].contiguous(), scale=0.125)
    c, lc = xa.attn_fwd_masked(qd, kd, vd, wide[:, :Skv].contiguous().expand(B, Hq, Sq, Skv),
                               scale=0.125)
    torch.cuda.synchronize()
    for x, y in ((a, b), (a, c)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert torch.equal(la, lb) and torch.equal(la, lc)


def test_lfm2_workload_with_mask_full():
    """The LFM2 prefill workload (B4 Hq32 Hkv8 S4096 D64, causal, RoPE) with a
    shared [4096, 4096] mask (a 1024-key sliding window plus random -inf and
    normal entries inside it), every element of every (batch, head)."""
    cfg = W.C4
    say("case", cfg.name, "masked")
    q, k, v = W.prefill_inputs(cfg)
    rng = np.random.default_rng(cfg.seed + 13)
    S = cfg.Sq
    mask = _mask(rng, (S, S), hide=0.05)
    i, j = np.arange(S)[:, None], np.arange(S)[None, :]
    mask[j < i - 1023] = -np.inf
    o, lse = run_masked(q, k, v, mask, cfg.causal, cfg.scale, cfg.rope_base)
    o_ref, lse_ref = _oracle(q, k, v, mask, cfg.causal, cfg.scale, cfg.rope_base, cfg.B, cfg.Hq,
                             S, S)
    check_bf16(o, lse, o_ref, lse_ref, f"{cfg.name} masked")


def test_mask_between_nan_guards():
    """The mask sits between NaN guard regions (16-byte aligned, 100 keys: the
    staged path, whose loads of the last row's chunks reach the range end);
    any value read past the mask's valid elements that reached a score would
    turn the output NaN."""
    B, Hq, Hkv, Sq, Skv, D = 1, 8, 2, 70, 100, 64
    rng = np.random.default_rng(12)
    q = W.f32_to_bf16_bits(rng.standard_normal((B, Sq, Hq, D), dtype=np.float32))
    k = W.f32_to_bf16_bits(rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32))
    v = W.f32_to_bf16_bits(rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32))
    mask = _mask(rng, (Sq, Skv))
    G = 1 << 14
    flat = torch.full((Sq * Skv + 2 * G,), float("nan"), dtype=torch.float32, device="cuda")
    flat[G:G + Sq * Skv] = torch.from_numpy(mask).cuda().reshape(-1)
    for causal in (True, False):
        o, lse = xa.attn_fwd_masked(W.to_device(q), W.to_device(k), W.to_device(v),
                                    flat[G:G + Sq * Skv].view(Sq, Skv), causal=causal,
                                    scale=0.125)
        torch.cuda.synchronize()
        o_ref, lse_ref = _oracle(q, k, v, mask, causal, 0.125, 0.0, B, Hq, Sq, Skv)
        check_bf16(_np(o), _np(lse), o_ref, lse_ref, f"mask guarded causal={causal}")
