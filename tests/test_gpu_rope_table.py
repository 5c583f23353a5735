"""GPU checks of the library's cached RoPE table.

The (cos, sin) table is rebuilt only when a call needs other positions, another
head dim or base, or runs on another stream than the one that built it.  A
sequence of calls that changes each of these in turn (and interleaves
rope_apply at other position offsets) must give, at every step, what the
oracle gives for that call alone; repeating a call gives the same bits.
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


def _inputs(rng, B, Hq, Hkv, Sq, Skv, D):
    f = [rng.standard_normal(s, dtype=np.float32)
         for s in ((B, Sq, Hq, D), (B, Skv, Hkv, D), (B, Skv, Hkv, D))]
    return [W.f32_to_bf16_bits(x) for x in f]


def test_table_reuse_and_rebuild_sequence():
    rng = np.random.default_rng(41)
    steps = [  # D, base, Sq, Skv
        (64, 10000.0, 200, 300),
        (64, 10000.0, 100, 250),    # fewer positions: reused
        (128, 10000.0, 100, 250),   # another head dim: rebuilt
        (64, 500.0, 150, 300),      # another base: rebuilt
        (64, 500.0, 300, 700),      # more positions: grown and rebuilt
        (40, 10000.0, 60, 90),      # padded head dim, its own angles
        (64, 10000.0, 200, 300),    # back to the first configuration
    ]
    first = None
    for i, (D, base, Sq, Skv) in enumerate(steps):
        say("step", i, D, base, Sq, Skv)
        q, k, v = _inputs(rng if i < len(steps) - 1 else np.random.default_rng(41), 1, 4, 2,
                          Sq, Skv, D)
        scale = float(np.float32(1 / math.sqrt(D)))
        o, lse = xa.attn_fwd(W.to_device(q), W.to_device(k), W.to_device(v), causal=True,
                             scale=scale, rope_base=base)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=True, scale=scale, rope_base=base,
                                         nthreads=NTHREADS)
        check_bf16(_np(o), _np(lse), o_ref, lse_ref, f"step {i}")
        if i == 0:
            first = (o.clone(), lse.clone())
        # rope_apply at another offset between the attention calls
        x = W.f32_to_bf16_bits(rng.standard_normal((1, 9, 2, D), dtype=np.float32))
        xd = W.to_device(x)
        xa.rope_apply(xd, pos_offset=1000 + i, rope_base=base)
        torch.cuda.synchronize()
        ref = oracle.rope(x, pos_offset=1000 + i, base=base)
        assert (np.abs(_np(xd) - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-30).all()
    # the last step repeated the first configuration on the same inputs
    assert torch.equal(o.view(torch.int16), first[0].view(torch.int16))
    assert torch.equal(lse, first[1])


def test_table_on_a_second_stream():
    """A call on another stream builds its own table there (stream order
    covers only the stream that built it), and gets the same result."""
    rng = np.random.default_rng(42)
    q, k, v = (W.to_device(x) for x in _inputs(rng, 2, 8, 2, 256, 256, 64))
    o1, l1 = xa.attn_fwd(q, k, v, causal=True, rope_base=10000.0)
    torch.cuda.synchronize()
    s2 = torch.cuda.Stream()
    with torch.cuda.stream(s2):
        o2, l2 = xa.attn_fwd(q, k, v, causal=True, rope_base=10000.0)
    s2.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
