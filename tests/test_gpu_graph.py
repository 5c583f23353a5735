"""Library calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

A decode step (caller-owned workspace), a forward with RoPE and a forward
whose keys are split over several workgroups (each after one eager call of
the same shape, so that the library's table, key-staging and split buffers
exist and nothing is allocated during capture) are captured once and
replayed with new input contents, with eager work and synchronisation between
the replays; every replay must give the eager call's bits.
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


def _bits_equal(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16)) if a.dtype != torch.float32 \
        else torch.equal(a, b)


def test_decode_step_in_a_graph():
    say("case graph decode")
    cfg = W.Decode("graph", 4, 16, 4, 128, 4096, 100, 4096, 77)
    qn, kcn, vcn, sln = W.decode_inputs(cfg)
    q, kc, vc = W.to_device(qn), W.to_device(kcn), W.to_device(vcn)
    sl = torch.from_numpy(sln).cuda()
    ns = 8
    ws = torch.empty(xa.attn_decode_workspace_bytes(cfg.B, cfg.Hq, cfg.D, ns), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((cfg.B, cfg.Hq), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up outside the capture
        xa.attn_decode_splitkv(q, kc, vc, sl, ns, scale=cfg.scale, o=o, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        xa.attn_decode_splitkv(q, kc, vc, sl, ns, scale=cfg.scale, o=o, lse=lse, workspace=ws)
    rng = np.random.default_rng(5)
    for rep in range(4):
        q.copy_(W.to_device(W.f32_to_bf16_bits(
            rng.standard_normal(tuple(q.shape), dtype=np.float32))))
        # new lengths within the filled rows (rows past the original ones hold NaN)
        sl.copy_(torch.from_numpy((rng.integers(1, sln.astype(np.int64) + 1)).astype(np.int32)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_ref, lse_ref = xa.attn_decode_splitkv(q, kc, vc, sl, ns, scale=cfg.scale)
        torch.cuda.synchronize()
        assert _bits_equal(o, o_ref) and torch.equal(lse, lse_ref), rep


def test_rope_forward_in_a_graph():
    say("case graph forward")
    B, Hq, Hkv, S, D = 2, 8, 2, 300, 64
    rng = np.random.default_rng(6)
    q, k, v = (W.to_device(W.f32_to_bf16_bits(rng.standard_normal(s, dtype=np.float32)))
               for s in ((B, S, Hq, D), (B, S, Hkv, D), (B, S, Hkv, D)))
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    xa.attn_fwd(q, k, v, causal=True, rope_base=10000.0, o=o, lse=lse)  # buffers exist now
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        xa.attn_fwd(q, k, v, causal=True, rope_base=10000.0, o=o, lse=lse)
    for rep in range(4):
        q.copy_(W.to_device(W.f32_to_bf16_bits(rng.standard_normal((B, S, Hq, D),
                                                                   dtype=np.float32))))
        k.copy_(W.to_device(W.f32_to_bf16_bits(rng.standard_normal((B, S, Hkv, D),
                                                                   dtype=np.float32))))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_ref, lse_ref = xa.attn_fwd(q, k, v, causal=True, rope_base=10000.0)
        torch.cuda.synchronize()
        assert _bits_equal(o, o_ref) and torch.equal(lse, lse_ref), rep


def test_split_forward_in_a_graph():
    """256 queries over 4096 keys on 8 heads: the forward splits the keys (8
    runs) and merges them with a second kernel; both are captured."""
    say("case graph split forward")
    B, H, Sq, Skv, D = 1, 8, 256, 4096, 64
    rng = np.random.default_rng(7)
    q, k, v = (W.to_device(W.f32_to_bf16_bits(rng.standard_normal(s, dtype=np.float32)))
               for s in ((B, Sq, H, D), (B, Skv, H, D), (B, Skv, H, D)))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    xa.attn_fwd(q, k, v, causal=True, o=o, lse=lse)  # buffers exist now
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        xa.attn_fwd(q, k, v, causal=True, o=o, lse=lse)
    for rep in range(4):
        q.copy_(W.to_device(W.f32_to_bf16_bits(rng.standard_normal((B, Sq, H, D),
                                                                   dtype=np.float32))))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_ref, lse_ref = xa.attn_fwd(q, k, v, causal=True)
        torch.cuda.synchronize()
        assert _bits_equal(o, o_ref) and torch.equal(lse, lse_ref), rep


def _rand16(rng, shape):
    return W.to_device(W.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32)))


def test_graph_survives_library_buffer_growth():
    """A captured RoPE forward (and a captured key-split forward) keep
    replaying correctly after eager calls of larger shapes made the library
    grow the buffers the graphs hold: the captured buffers are retired, not
    freed."""
    say("case graph buffer growth")
    rng = np.random.default_rng(8)
    B, Hq, Hkv, S, D = 1, 8, 2, 200, 64
    q, k, v = _rand16(rng, (B, S, Hq, D)), _rand16(rng, (B, S, Hkv, D)), _rand16(rng, (B, S, Hkv, D))
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    # a key-split launch: 256 queries x 2048 keys on 4 heads
    qs, ks, vs = (_rand16(rng, (1, 256, 4, D)), _rand16(rng, (1, 2048, 4, D)),
                  _rand16(rng, (1, 2048, 4, D)))
    os_ = torch.empty_like(qs)
    ls_ = torch.empty((1, 4, 256), dtype=torch.float32, device="cuda")
    xa.attn_fwd(q, k, v, causal=True, rope_base=10000.0, o=o, lse=lse)
    xa.attn_fwd(qs, ks, vs, causal=True, o=os_, lse=ls_)
    torch.cuda.synchronize()
    g1, g2 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        xa.attn_fwd(q, k, v, causal=True, rope_base=10000.0, o=o, lse=lse)
    with torch.cuda.graph(g2):
        xa.attn_fwd(qs, ks, vs, causal=True, o=os_, lse=ls_)
    for rep in range(3):
        # larger eager calls: more positions (table), more keys (staging), a
        # larger split launch (partials)
        Sb = 1000 * (rep + 2)
        qb, kb, vb = (_rand16(rng, (2, Sb, Hq, D)), _rand16(rng, (2, Sb, Hkv, D)),
                      _rand16(rng, (2, Sb, Hkv, D)))
        xa.attn_fwd(qb, kb, vb, causal=True, rope_base=10000.0)
        q2, k2, v2 = (_rand16(rng, (1, 512, 8, D)), _rand16(rng, (1, 8192, 8, D)),
                      _rand16(rng, (1, 8192, 8, D)))
        xa.attn_fwd(q2, k2, v2, causal=True)
        torch.cuda.synchronize()
        q.copy_(_rand16(rng, (B, S, Hq, D)))
        qs.copy_(_rand16(rng, (1, 256, 4, D)))
        torch.cuda.synchronize()
        g1.replay()
        g2.replay()
        torch.cuda.synchronize()
        o_ref, lse_ref = xa.attn_fwd(q, k, v, causal=True, rope_base=10000.0)
        os_ref, ls_ref = xa.attn_fwd(qs, ks, vs, causal=True)
        torch.cuda.synchronize()
        assert _bits_equal(o, o_ref) and torch.equal(lse, lse_ref), rep
        assert _bits_equal(os_, os_ref) and torch.equal(ls_, ls_ref), rep


def test_graph_replay_does_not_corrupt_the_table_cache():
    """An eager rope_apply after a capture, a replay in between, and the same
    rope_apply again: the second must rotate with its own angles (a replay
    rewrites the table buffer the capture recorded, so eager calls must not
    trust a cache that lives in that buffer)."""
    say("case graph table cache")
    rng = np.random.default_rng(9)
    B, Hq, Hkv, S, D = 1, 4, 2, 256, 64
    q, k, v = _rand16(rng, (B, S, Hq, D)), _rand16(rng, (B, S, Hkv, D)), _rand16(rng, (B, S, Hkv, D))
    o = torch.empty_like(q)
    xa.attn_fwd(q, k, v, causal=True, rope_base=10000.0, o=o, want_lse=False)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        xa.attn_fwd(q, k, v, causal=True, rope_base=10000.0, o=o, want_lse=False)
    x0 = _rand16(rng, (1, 200, 2, D))
    x1, x2 = x0.clone(), x0.clone()
    xa.rope_apply(x1, pos_offset=1000, rope_base=10000.0)  # table for 1000..1199
    torch.cuda.synchronize()
    g.replay()  # records a build of the table for positions 0..255
    torch.cuda.synchronize()
    xa.rope_apply(x2, pos_offset=1000, rope_base=10000.0)
    torch.cuda.synchronize()
    assert _bits_equal(x1, x2)
    # and against the oracle's rotation (both sides round an fp64-accurate
    # value once to bf16: equal except where the two straddle a rounding
    # boundary, which is vanishingly rare)
    import oracle
    ref = oracle.rope(x0.view(torch.int16).cpu().numpy().view(np.uint16), pos_offset=1000,
                      base=10000.0)
    got = x2.float().cpu().numpy().astype(np.float64)
    assert (np.abs(got - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-30).all()
    assert (got == ref).mean() > 0.999
