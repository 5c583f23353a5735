"""GPU check of attn_decode_splitkv_noalloc, the decode entry point that keeps
its per-split partials in the library's built-in scratch instead of a
workspace: two calls in a row through the C ABI (a larger decode, then a
smaller one with empty and short sequences, so stale partials of the first
call would show), each compared with attn_decode_splitkv on the same inputs
(same kernels: bit-identical o and lse); and a shape whose partials exceed
the scratch is refused without a launch.
"""
import sys

import numpy as np
import pytest
import torch

import exact_attention_28_amd as xa

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _inputs(B, Hq, Hkv, D, Smax, lens, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16).cuda()
    kc = torch.randn(B, Smax, Hkv, D, generator=g).to(torch.bfloat16).cuda()
    vc = torch.randn(B, Smax, Hkv, D, generator=g).to(torch.bfloat16).cuda()
    sl = torch.tensor(lens, dtype=torch.int32).cuda()
    return q, kc, vc, sl


CASES = [  # B, Hq, Hkv, D, Smax, seqlens, num_splits, seed
    (4, 32, 8, 128, 4096, [4096, 1, 2900, 1777], 32, 51),
    (3, 8, 2, 64, 700, [0, 700, 33], 8, 52),
]


def test_noalloc_matches_workspace_entry_point_twice():
    for B, Hq, Hkv, D, Smax, lens, ns, seed in CASES:
        say("case noalloc decode", B, Hq, Hkv, D, Smax, lens, ns, seed)
        q, kc, vc, sl = _inputs(B, Hq, Hkv, D, Smax, lens, seed)
        o_ref, lse_ref = xa.attn_decode_splitkv(q, kc, vc, sl, ns)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
        xa.attn_decode_splitkv_noalloc(q, kc, vc, sl, ns, o, lse)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(o.view(torch.int16).cpu().numpy(),
                                      o_ref.view(torch.int16).cpu().numpy())
        np.testing.assert_array_equal(lse.cpu().numpy(), lse_ref.cpu().numpy())
        if 0 in lens:
            b = lens.index(0)
            assert torch.all(o[b] == 0) and torch.all(torch.isneginf(lse[b]))


def test_noalloc_refuses_partials_beyond_the_scratch():
    # 64 * 64 * 16 = 65536 > 32513 (the most that fits at D = 128)
    B, Hq, Hkv, D, Smax = 64, 64, 8, 128, 16
    say("case noalloc oversize", B, Hq, D)
    q, kc, vc, sl = _inputs(B, Hq, Hkv, D, Smax, [Smax] * B, 53)
    o = torch.empty_like(q)
    with pytest.raises(xa.AttnError) as ei:
        xa.attn_decode_splitkv_noalloc(q, kc, vc, sl, 16, o)
    assert ei.value.code == xa.ATTN_ERR_UNSUPPORTED
    assert "scratch" in str(ei.value)
    # a fitting split count still runs
    o_ref, _ = xa.attn_decode_splitkv(q, kc, vc, sl, 4, want_lse=False)
    xa.attn_decode_splitkv_noalloc(q, kc, vc, sl, 4, o)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o.view(torch.int16).cpu().numpy(),
                                  o_ref.view(torch.int16).cpu().numpy())
