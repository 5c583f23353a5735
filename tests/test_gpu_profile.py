"""The kernel-timing session of the C ABI (attn_profile_begin / _end): each
forward call records one event pair around its attention kernel, on its own
stream, and the times are plausible (positive, within the caller's events
around the whole call, which also hold the key-rotation pass)."""
import sys

import numpy as np
import pytest
import torch

import exact_attention_28_amd as xa
import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def test_profile_session_times_the_attention_kernel():
    say("case profile session")
    rng = np.random.default_rng(41)
    B, Hq, Hkv, S, D = 2, 8, 2, 1024, 64
    q, k, v = (W.to_device(W.f32_to_bf16_bits(rng.standard_normal(s, dtype=np.float32)))
               for s in ((B, S, Hq, D), (B, S, Hkv, D), (B, S, Hkv, D)))
    o = torch.empty_like(q)
    xa.attn_fwd(q, k, v, causal=True, rope_base=10000.0, o=o)  # table and staging exist
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    calls = []
    xa.attn_profile_begin()
    for i in range(6):
        st = torch.cuda.current_stream() if i % 2 == 0 else side
        with torch.cuda.stream(st):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            xa.attn_fwd(q, k, v, causal=True, rope_base=10000.0, o=o)
            e1.record(st)
            calls.append((e0, e1))
        st.synchronize()
    kern = xa.attn_profile_end()
    assert len(kern) == 6
    for (e0, e1), t in zip(calls, kern):
        whole = e0.elapsed_time(e1)
        assert 0.0 < t <= whole + 1e-3, (t, whole)
    # a session that is closed records nothing
    xa.attn_fwd(q, k, v, causal=True, rope_base=10000.0, o=o)
    torch.cuda.synchronize()
    xa.attn_profile_begin()
    assert xa.attn_profile_end() == []
