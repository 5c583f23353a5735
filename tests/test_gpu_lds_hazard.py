"""LDS double-buffer hazard check of the 16-bit forward and backward kernels.

Both 16-bit forwards and the backward's two streaming kernels keep two tile
buffers in LDS and load the next tile while the current one is read; the
only thing that keeps a load from overwriting a tile still being read, or a
wave from reading a tile before every wave's share of it has landed, is the
placement of their waits and barriers.  ATTN_LDS_SINGLE_BUFFER=1 routes the
same calls to instances with one buffer of each kind, refilled only after a
barrier behind the last read of it and waited for before the next read, so
no load is ever in flight while LDS is read.  The arithmetic and its order
do not change, so every output and LSE must equal the double-buffered call's
bit for bit; a missing or misplaced wait or barrier in the double-buffered
kernel shows up as a difference.

The shapes cover every instance family: the pipelined kernel with one and
two query blocks per wave, the shared RoPE table, two key groups per
workgroup, D = 128 and fp16; the masked kernel with all three mask staging
paths; key splits; the tile kernel for unmasked launches
(ATTN_FWD_PIPELINE=0); the chunked prefill against a KV cache; and the
backward (dK/dV and dQ kernels, with and without RoPE, GQA, ragged tiles).
"""
import sys

import numpy as np
import pytest
import torch

import exact_attention_28_amd as xa

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _rand(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype).cuda()


def _bits(t):
    t = t.contiguous()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


def _both(monkeypatch, call):
    """call() with two buffers, then with one; returns both result tuples."""
    monkeypatch.delenv("ATTN_LDS_SINGLE_BUFFER", raising=False)
    two = [_bits(t) for t in call()]
    monkeypatch.setenv("ATTN_LDS_SINGLE_BUFFER", "1")
    one = [_bits(t) for t in call()]
    monkeypatch.delenv("ATTN_LDS_SINGLE_BUFFER")
    torch.cuda.synchronize()
    return two, one


def _same(two, one, names):
    for a, b, n in zip(two, one, names):
        assert a.shape == b.shape
        diff = int(np.count_nonzero(a != b))
        assert diff == 0, f"{n}: {diff} of {a.size} elements differ with one LDS buffer"


UNMASKED = [  # B, Hq, Hkv, Sq, Skv, D, causal, rope, dtype, env
    (2, 32, 8, 2048, 2048, 64, True, 10000.0, torch.bfloat16, {}),   # 2 query blocks/wave, table in LDS
    (2, 8, 2, 300, 300, 64, True, 10000.0, torch.bfloat16, {}),      # 1 block/wave, ragged
    (1, 8, 1, 100, 777, 128, True, 10000.0, torch.bfloat16, {}),     # 8 heads/kv head, D 128
    (1, 4, 4, 200, 1100, 128, False, 0.0, torch.bfloat16, {}),       # two key groups
    (1, 4, 2, 150, 1090, 64, True, 0.0, torch.float16, {}),          # two key groups, causal, fp16
    (1, 6, 2, 77, 190, 64, False, 0.0, torch.float16, {}),           # 1 head per workgroup
    (1, 4, 4, 200, 1100, 64, False, 0.0, torch.bfloat16, {}),        # four key groups
    (1, 3, 1, 150, 1090, 64, True, 0.0, torch.float16, {}),          # four key groups, causal, fp16
    (2, 32, 8, 2048, 2048, 64, True, 10000.0, torch.bfloat16,        # tile kernel, 2 blocks/wave
     {"ATTN_FWD_PIPELINE": "0"}),
    (1, 8, 2, 160, 600, 128, False, 10000.0, torch.bfloat16,         # tile kernel, D 128
     {"ATTN_FWD_PIPELINE": "0"}),
    (1, 4, 2, 64, 2048, 64, True, 0.0, torch.bfloat16,               # key splits + merge
     {"ATTN_FWD_SPLITS": "3"}),
]


@pytest.mark.parametrize("case", UNMASKED, ids=[str(c[:9]) + str(c[9]) for c in UNMASKED])
def test_unmasked_one_vs_two_buffers(case, monkeypatch):
    B, Hq, Hkv, Sq, Skv, D, causal, rope, dt, env = case
    say("case lds-hazard", case)
    for key, val in env.items():
        monkeypatch.setenv(key, val)
    q, k, v = (_rand(s, dt, 71 + i) for i, s in
               enumerate(((B, Sq, Hq, D), (B, Skv, Hkv, D), (B, Skv, Hkv, D))))
    two, one = _both(monkeypatch, lambda: xa.attn_fwd(q, k, v, causal=causal, rope_base=rope))
    _same(two, one, ("o", "lse"))


MASKED = [  # B, Hq, Hkv, Sq, Skv, D, mask shape (None = [Sq, Skv]), staging path
    (1, 4, 2, 130, 256, 64, None),            # rows shared by the workgroup's heads
    (1, 4, 4, 100, 192, 64, None),            # one head per workgroup: per-wave rows
    (2, 4, 2, 90, 200, 64, "per_head"),       # per-head mask: per-wave rows
    (1, 4, 2, 70, 150, 128, None),            # D 128: per-lane loads
    (1, 4, 2, 70, 151, 64, None),             # Skv not a multiple of 4: per-lane loads
]


@pytest.mark.parametrize("case", MASKED, ids=[str(c) for c in MASKED])
def test_masked_one_vs_two_buffers(case, monkeypatch):
    B, Hq, Hkv, Sq, Skv, D, kind = case
    say("case lds-hazard masked", case)
    q, k, v = (_rand(s, torch.bfloat16, 81 + i) for i, s in
               enumerate(((B, Sq, Hq, D), (B, Skv, Hkv, D), (B, Skv, Hkv, D))))
    mshape = (B, Hq, Sq, Skv) if kind == "per_head" else (Sq, Skv)
    mask = _rand(mshape, torch.float32, 85)
    two, one = _both(monkeypatch,
                     lambda: xa.attn_fwd_masked(q, k, v, mask, causal=True, rope_base=10000.0))
    _same(two, one, ("o", "lse"))


def test_chunked_prefill_one_vs_two_buffers(monkeypatch):
    B, Hq, Hkv, Sq, D, Smax = 2, 8, 2, 200, 64, 900
    say("case lds-hazard kvcache", B, Hq, Hkv, Sq, D, Smax)
    lens = torch.tensor([0, 517], dtype=torch.int32).cuda()
    q = _rand((B, Sq, Hq, D), torch.bfloat16, 91)
    kn = _rand((B, Sq, Hkv, D), torch.bfloat16, 92)
    vn = _rand((B, Sq, Hkv, D), torch.bfloat16, 93)
    kc0 = _rand((B, Smax, Hkv, D), torch.bfloat16, 94)
    vc0 = _rand((B, Smax, Hkv, D), torch.bfloat16, 95)

    def call():
        kc, vc = kc0.clone(), vc0.clone()
        o, lse = xa.attn_prefill_kvcache(q, kn, vn, kc, vc, lens, causal=True, rope_base=10000.0)
        return o, lse, kc, vc

    two, one = _both(monkeypatch, call)
    _same(two, one, ("o", "lse", "kcache", "vcache"))


BACKWARD = [  # B, Hq, Hkv, Sq, Skv, causal, rope, dtype
    (1, 8, 2, 300, 300, True, 10000.0, torch.bfloat16),
    (2, 4, 4, 130, 257, False, 0.0, torch.float16),
    (1, 8, 1, 200, 450, True, 0.0, torch.bfloat16),
]


@pytest.mark.parametrize("case", BACKWARD, ids=[str(c) for c in BACKWARD])
def test_backward_one_vs_two_buffers(case, monkeypatch):
    B, Hq, Hkv, Sq, Skv, causal, rope, dt = case
    D = 64
    say("case lds-hazard backward", case)
    q, k, v, do = (_rand(s, dt, 101 + i) for i, s in
                   enumerate(((B, Sq, Hq, D), (B, Skv, Hkv, D), (B, Skv, Hkv, D), (B, Sq, Hq, D))))
    o, lse = xa.attn_fwd(q, k, v, causal=causal, rope_base=rope)
    two, one = _both(monkeypatch,
                     lambda: xa.attn_bwd(q, k, v, o, do, lse, causal=causal, rope_base=rope))
    _same(two, one, ("dq", "dk", "dv"))
