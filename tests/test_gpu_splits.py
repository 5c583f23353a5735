"""GPU checks of the key splits of under-filled 16-bit forward launches.

A launch with fewer than two workgroups per CU splits each query tile's keys
into runs, one workgroup per run, and merges the runs' partial (O, LSE) by
log-sum-exp.  The split count comes from the shape, or from ATTN_FWD_SPLITS
(1 turns splitting off).  Each case below runs unsplit and at several forced
split counts (including more splits than some workgroups have key tiles, so
that some runs are empty): every result must meet the bf16 bar against the
oracle, and the split results must agree with the unsplit one to within the
same bar.  Short query runs against long keys (256 queries x 4096 keys over
8 heads) and a small-chunk step of a KV-cache serving loop split by
themselves; the 1024-token MHA shapes (16 key tiles per query tile) do not.
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
from test_gpu_parity import check_bf16

pytestmark = pytest.mark.gpu

NTHREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


CASES = [  # B, Hq, Hkv, Sq, Skv, D, causal, rope, dtype
    (2, 8, 8, 256, 256, 64, False, 0.0, "bf16"),       # MHA
    (2, 8, 2, 300, 300, 64, True, 10000.0, "bf16"),    # GQA 4, causal, RoPE, ragged
    (1, 4, 1, 100, 700, 64, True, 10000.0, "bf16"),    # bottom-right causal, Sq < Skv
    (1, 2, 1, 70, 20, 64, True, 0.0, "bf16"),          # rows with no visible key
    (1, 4, 4, 64, 1000, 128, False, 0.0, "bf16"),      # D = 128, long keys
    (2, 6, 3, 33, 500, 64, True, 0.0, "f16"),          # fp16, 2 heads per kv head
    (1, 1, 1, 1, 8192, 64, False, 0.0, "bf16"),        # one query row, long keys
    (1, 32, 2, 64, 3000, 64, True, 10000.0, "bf16"),   # 16 query heads per kv head
]


def _inputs(case):
    B, Hq, Hkv, Sq, Skv, D, causal, rope, dt = case
    rng = np.random.default_rng(W.case_seed(case))
    f = [rng.standard_normal(s, dtype=np.float32)
         for s in ((B, Sq, Hq, D), (B, Skv, Hkv, D), (B, Skv, Hkv, D))]
    if dt == "f16":
        return [x.astype(np.float16) for x in f]
    return [W.f32_to_bf16_bits(x) for x in f]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_forced_splits(monkeypatch, case):
    B, Hq, Hkv, Sq, Skv, D, causal, rope, dt = case
    say("case splits", case)
    q, k, v = _inputs(case)
    qd, kd, vd = (W.to_device(x) for x in (q, k, v))
    scale = float(np.float32(1 / math.sqrt(D)))
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=causal, scale=scale, rope_base=rope,
                                     nthreads=NTHREADS)
    results = {}
    for ns in ("1", "2", "3", "16"):
        monkeypatch.setenv("ATTN_FWD_SPLITS", ns)
        o, lse = xa.attn_fwd(qd, kd, vd, causal=causal, scale=scale, rope_base=rope)
        torch.cuda.synchronize()
        results[ns] = (_np(o), _np(lse))
        check_bf16(results[ns][0], results[ns][1], o_ref, lse_ref, f"{case} splits={ns}")
    o1, l1 = results["1"]
    for ns in ("2", "3", "16"):
        check_bf16(results[ns][0], results[ns][1], o1, l1, f"{case} splits={ns} vs unsplit")


@pytest.mark.parametrize("causal", [False, True])
def test_long_keys_split_by_themselves(monkeypatch, causal):
    """B1 H8, 256 queries over 4096 keys: 16 workgroups unsplit, 8 splits by
    themselves; every element against the oracle, and the whole output
    against the unsplit call."""
    B, H, Sq, Skv, D = 1, 8, 256, 4096, 64
    say("case long keys", causal)
    rng = np.random.default_rng(78 + causal)
    q, k, v = (W.f32_to_bf16_bits(rng.standard_normal(s, dtype=np.float32))
               for s in ((B, Sq, H, D), (B, Skv, H, D), (B, Skv, H, D)))
    qd, kd, vd = (W.to_device(x) for x in (q, k, v))
    monkeypatch.delenv("ATTN_FWD_SPLITS", raising=False)
    o, lse = xa.attn_fwd(qd, kd, vd, causal=causal, scale=0.125)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=causal, scale=0.125, nthreads=NTHREADS)
    check_bf16(_np(o), _np(lse), o_ref, lse_ref, f"long keys causal={causal}")
    monkeypatch.setenv("ATTN_FWD_SPLITS", "1")
    o1, l1 = xa.attn_fwd(qd, kd, vd, causal=causal, scale=0.125)
    torch.cuda.synchronize()
    check_bf16(_np(o), _np(lse), _np(o1), _np(l1), f"long keys causal={causal} vs unsplit")


def test_small_chunk_serving_step(monkeypatch):
    """A 16-token chunk over 2000 cached keys (32 workgroups unsplit, 4
    splits by itself) against the same call unsplit and against the oracle."""
    B, Hq, Hkv, Sq, D, Smax, L0 = 4, 32, 8, 16, 64, 2048, 2000
    rng = np.random.default_rng(77)
    kall = W.f32_to_bf16_bits(rng.standard_normal((B, Smax, Hkv, D), dtype=np.float32))
    vall = W.f32_to_bf16_bits(rng.standard_normal((B, Smax, Hkv, D), dtype=np.float32))
    q = W.f32_to_bf16_bits(rng.standard_normal((B, Sq, Hq, D), dtype=np.float32))
    lens = torch.full((B,), L0, dtype=torch.int32, device="cuda")
    outs = {}
    for ns in ("1", ""):
        if ns:
            monkeypatch.setenv("ATTN_FWD_SPLITS", ns)
        else:
            monkeypatch.delenv("ATTN_FWD_SPLITS", raising=False)
        kc, vc = W.to_device(kall), W.to_device(vall)
        o, lse = xa.attn_prefill_kvcache(W.to_device(q), W.to_device(kall[:, L0:L0 + Sq]),
                                         W.to_device(vall[:, L0:L0 + Sq]), kc, vc, lens,
                                         causal=True, scale=0.125)
        torch.cuda.synchronize()
        outs[ns] = (_np(o), _np(lse))
    # the cache rows before L0 are the (unrotated) keys themselves: no RoPE here
    o_ref, lse_ref = oracle.attn_fwd(q, kall[:, :L0 + Sq], vall[:, :L0 + Sq], causal=True,
                                     scale=0.125, nthreads=NTHREADS)
    for ns, (o, lse) in outs.items():
        check_bf16(o, lse, o_ref, lse_ref, f"chunk step splits={ns or 'auto'}")
    check_bf16(outs[""][0], outs[""][1], outs["1"][0], outs["1"][1], "auto vs unsplit")
