"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on
the same seeded inputs.

Tolerances: fp32 inputs max-abs 1e-4 on O and LSE; bf16 inputs max-abs 2e-2
and relative-L2 5e-3 on O, max-abs 1e-3 on LSE (the oracle is fed the same
bf16 values, widened exactly).  Every case, the full-size workloads included
(in the launch configuration the benchmark times), is compared element by
element in full.
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
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_bf16(o_gpu, lse_gpu, o_ref, lse_ref, what, out_quant=False):
    """bf16 bar: O max-abs 2e-2, O rel-L2 5e-3, LSE max-abs 1e-3.

    out_quant: for test inputs outside the workloads' value range (|O| can
    exceed 4), the bf16 rounding of the output alone is up to half an ulp,
    2^-8 |O|, which is added to the absolute bound.
    """
    o_gpu = np.asarray(o_gpu, np.float64)
    err = np.abs(o_gpu - o_ref)
    if out_quant:
        err = err - 2.0 ** -8 * np.abs(o_ref)
    rel = np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-30)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite output"
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= 2e-2, (f"{what}: O max-abs {err.max():.3e} at {worst} "
                               f"(got {o_gpu[worst]:.5f}, oracle {o_ref[worst]:.5f})")
    assert rel <= 5e-3, f"{what}: O rel-L2 {rel:.3e}"
    if lse_gpu is not None:
        fin = np.isfinite(lse_ref)
        assert (np.isfinite(lse_gpu) == fin).all(), f"{what}: LSE finiteness differs"
        if fin.any():
            lerr = np.abs(np.asarray(lse_gpu, np.float64)[fin] - lse_ref[fin]).max()
            assert lerr <= 1e-3, f"{what}: LSE max-abs {lerr:.3e}"
        assert (np.asarray(lse_gpu)[~fin] == -np.inf).all()
    return err.max(), rel


def check_f32(o_gpu, lse_gpu, o_ref, lse_ref, what):
    err = np.abs(np.asarray(o_gpu, np.float64) - o_ref).max()
    assert err <= 1e-4, f"{what}: O max-abs {err:.3e}"
    fin = np.isfinite(lse_ref)
    assert (np.isfinite(lse_gpu) == fin).all()
    if fin.any():
        lerr = np.abs(np.asarray(lse_gpu, np.float64)[fin] - lse_ref[fin]).max()
        assert lerr <= 1e-4, f"{what}: LSE max-abs {lerr:.3e}"


def run_fwd(q, k, v, causal, scale, rope):
    o, lse = xa.attn_fwd(W.to_device(q), W.to_device(k), W.to_device(v), causal=causal,
                         scale=scale, rope_base=rope)
    torch.cuda.synchronize()
    return _np(o), _np(lse)


# ------------------------------------------------------------------ fp32 --

def test_single_head_f32_workload():
    cfg = W.C1
    say("case", cfg.name)
    q, k, v = W.prefill_inputs(cfg)
    o, lse = run_fwd(q, k, v, cfg.causal, cfg.scale, cfg.rope_base)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=cfg.causal, scale=cfg.scale,
                                     rope_base=cfg.rope_base, nthreads=NTHREADS)
    check_f32(o, lse, o_ref, lse_ref, cfg.name)
    # the tiled algorithm with the workload's 64/64 blocks gives the same result
    ot, lt = oracle.attn_tiled_head(q[0, :, 0].astype(np.float64), k[0, :, 0].astype(np.float64),
                                    v[0, :, 0].astype(np.float64), scale=cfg.scale, block_q=64,
                                    block_kv=64)
    np.testing.assert_allclose(ot, o_ref[0, :, 0], atol=1e-12)
    np.testing.assert_allclose(lt, lse_ref[0, 0], atol=1e-12)


F32_CASES = [  # B, Hq, Hkv, Sq, Skv, D, causal, rope
    (2, 4, 2, 100, 100, 64, True, 0.0),
    (1, 3, 1, 77, 130, 128, True, 10000.0),
    (2, 2, 2, 65, 65, 128, False, 500.0),
    (1, 2, 1, 40, 20, 64, True, 0.0),  # rows with no visible key
    (1, 1, 1, 1, 1, 64, False, 0.0),
    # the cases above have fewer than 64 blocks of 64 rows (16 lanes per row);
    # 64 to 255 run 8 lanes per row, >= 256 four
    (1, 8, 8, 512, 256, 64, False, 0.0),
    (1, 12, 4, 700, 900, 128, True, 500.0),
    (2, 8, 2, 1024, 1024, 64, True, 10000.0),
    (1, 16, 16, 1000, 512, 128, False, 0.0),
    (1, 1, 1, 100, 333, 64, False, 0.0),  # 16 lanes, 6 key blocks, ragged tail
    (4, 8, 8, 1000, 777, 64, False, 0.0),  # four lanes, ragged rows and keys
    (2, 8, 4, 1024, 1100, 128, True, 10000.0),
    (1, 16, 2, 1100, 1, 64, False, 0.0),  # four lanes, one key
    (1, 16, 16, 1030, 1000, 128, True, 0.0),  # four lanes, first 30 rows see no key
]


@pytest.mark.parametrize("case", F32_CASES, ids=[str(c) for c in F32_CASES])
def test_f32_variants(case):
    B, Hq, Hkv, Sq, Skv, D, causal, rope = case
    say("case f32", case)
    rng = np.random.default_rng(W.case_seed(case))
    q = rng.standard_normal((B, Sq, Hq, D), dtype=np.float32)
    k = rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32)
    scale = float(np.float32(1 / math.sqrt(D)))
    o, lse = run_fwd(q, k, v, causal, scale, rope)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=causal, scale=scale, rope_base=rope,
                                     nthreads=NTHREADS)
    check_f32(o, lse, o_ref, lse_ref, str(case))


# ------------------------------------------------------------------ bf16 --

BF16_CASES = [  # B, Hq, Hkv, Sq, Skv, D, causal, rope, amplitude
    (2, 8, 2, 300, 300, 64, True, 10000.0, 1.0),
    (1, 4, 4, 333, 333, 128, False, 0.0, 1.0),
    (2, 6, 2, 200, 200, 128, True, 10000.0, 1.0),
    (1, 4, 1, 130, 257, 64, True, 0.0, 1.0),     # bottom-right causal, Sq < Skv
    (1, 8, 8, 65, 190, 64, False, 10000.0, 2.0),
    (1, 2, 1, 50, 20, 64, True, 0.0, 1.0),      # rows with no visible key
    (3, 3, 3, 1, 1, 64, False, 0.0, 1.0),
    (1, 16, 2, 129, 129, 64, True, 10000.0, 1.0),  # 8 query heads per kv head
    (2, 5, 5, 64, 64, 128, True, 0.0, 1.0),
    (1, 12, 4, 97, 97, 64, False, 0.0, 1.0),    # 3 query heads per kv head
    (2, 8, 2, 1, 777, 64, True, 10000.0, 1.0),  # one query row against every key
    (1, 4, 2, 256, 320, 64, True, 0.0, 4.0),    # scores up to ~±100: the running max moves often
    (64, 1, 1, 33, 33, 64, True, 0.0, 1.0),     # many small (batch, head) units
    (1, 12, 2, 100, 100, 128, True, 10000.0, 1.0),  # 6 query heads per kv head (pairs of heads)
    # under-filled launches with >= 16 key tiles: two key groups per workgroup
    # (four of two waves for one head per workgroup at D 64) merged through
    # LDS (tile counts that do not divide leave the last groups tiles past
    # the keys; causal rows see only part of the later groups' keys)
    (1, 4, 2, 200, 1100, 64, False, 0.0, 1.0),
    (1, 4, 4, 150, 1050, 64, True, 0.0, 1.0),     # four groups
    (2, 4, 4, 100, 1300, 128, False, 0.0, 1.0),
    (1, 4, 1, 64, 1024, 64, True, 0.0, 4.0),
    (1, 4, 4, 200, 1100, 64, False, 0.0, 1.0),    # four groups, 18 tiles
    (1, 3, 1, 100, 1500, 64, True, 0.0, 4.0),     # four groups, bottom-right causal
    (2, 2, 2, 1, 1025, 64, True, 0.0, 1.0),       # four groups, one query row
]


def _bf16_inputs(rng, B, Hq, Hkv, Sq, Skv, D, amp):
    f = [rng.standard_normal(s, dtype=np.float32) * np.float32(amp)
         for s in ((B, Sq, Hq, D), (B, Skv, Hkv, D), (B, Skv, Hkv, D))]
    return [W.f32_to_bf16_bits(x) for x in f]


@pytest.mark.parametrize("case", BF16_CASES, ids=[str(c) for c in BF16_CASES])
def test_bf16_variants(case):
    B, Hq, Hkv, Sq, Skv, D, causal, rope, amp = case
    say("case bf16", case)
    rng = np.random.default_rng(W.case_seed(case))
    q, k, v = _bf16_inputs(rng, B, Hq, Hkv, Sq, Skv, D, amp)
    scale = float(np.float32(1 / math.sqrt(D)))
    o, lse = run_fwd(q, k, v, causal, scale, rope)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=causal, scale=scale, rope_base=rope,
                                     nthreads=NTHREADS)
    check_bf16(o, lse, o_ref, lse_ref, str(case), out_quant=amp > 1.0)


@pytest.mark.parametrize("cfg", [W.C2N, W.C2C], ids=lambda c: c.name)
def test_mha_1024_workload_full(cfg):
    say("case", cfg.name)
    q, k, v = W.prefill_inputs(cfg)
    o, lse = run_fwd(q, k, v, cfg.causal, cfg.scale, cfg.rope_base)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=cfg.causal, scale=cfg.scale,
                                     nthreads=NTHREADS)
    e, r = check_bf16(o, lse, o_ref, lse_ref, cfg.name)
    say(f"  {cfg.name}: O max-abs {e:.3e} rel-L2 {r:.3e}")


@pytest.mark.parametrize("cfg", [W.C3, W.C4], ids=lambda c: c.name)
def test_large_workload_full(cfg):
    """The Whisper-encoder and LFM2-prefill workloads at full size, in the
    launch configuration the benchmark times, compared with the oracle on
    every element of O and LSE."""
    say("case", cfg.name)
    q, k, v = W.prefill_inputs(cfg)
    o, lse = run_fwd(q, k, v, cfg.causal, cfg.scale, cfg.rope_base)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=cfg.causal, scale=cfg.scale,
                                     rope_base=cfg.rope_base, nthreads=NTHREADS)
    e, r = check_bf16(o, lse, o_ref, lse_ref, cfg.name)
    say(f"  {cfg.name}: all {cfg.B * cfg.Hq} heads x {cfg.Sq} rows: "
        f"O max-abs {e:.3e} rel-L2 {r:.3e}")


def test_gqa_equals_mha_with_repeated_kv():
    """On the GPU path, GQA(G) gives the same bits as MHA with every kv head
    repeated over its group (and GQA(1) = MQA likewise)."""
    rng = np.random.default_rng(31)
    for Hkv in (4, 1):
        q, k, v = _bf16_inputs(rng, 2, 8, Hkv, 200, 200, 64, 1.0)
        G = 8 // Hkv
        o1, l1 = run_fwd(q, k, v, True, 0.125, 10000.0)
        o2, l2 = run_fwd(q, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2), True, 0.125,
                         10000.0)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_guard_regions_untouched_and_unread():
    """Inputs sit between NaN guard regions and outputs between sentinel
    regions: a read past an input turns the output NaN, a write past an
    output changes a sentinel."""
    rng = np.random.default_rng(32)
    B, Hq, Hkv, S, D = 1, 4, 2, 190, 64
    q, k, v = _bf16_inputs(rng, B, Hq, Hkv, S, S, D, 1.0)
    G = 1 << 14

    def guarded(a, fill):
        flat = torch.full((a.size + 2 * G,), fill, dtype=torch.bfloat16, device=DEV)
        flat[G:G + a.size] = W.to_device(a).reshape(-1)
        return flat, flat[G:G + a.size].view(a.shape)

    _, qd = guarded(q, float("nan"))
    _, kd = guarded(k, float("nan"))
    _, vd = guarded(v, float("nan"))
    of, od = guarded(np.zeros(q.shape, np.uint16), 7.0)
    lf = torch.full((B * Hq * S + 2 * G,), 7.0, dtype=torch.float32, device=DEV)
    ld = lf[G:G + B * Hq * S].view(B, Hq, S)
    for causal, rope in ((True, 10000.0), (False, 0.0)):
        xa.attn_fwd(qd, kd, vd, causal=causal, scale=0.125, rope_base=rope, o=od, lse=ld)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=causal, scale=0.125, rope_base=rope,
                                         nthreads=NTHREADS)
        check_bf16(_np(od), _np(ld), o_ref, lse_ref, f"guarded causal={causal}")
        assert (of[:G] == 7.0).all() and (of[G + q.size:] == 7.0).all()
        assert (lf[:G] == 7.0).all() and (lf[G + B * Hq * S:] == 7.0).all()


# ------------------------------------------------------------------ RoPE --

@pytest.mark.parametrize("dtype,D,off", [("bf16", 64, 0), ("bf16", 128, 1000), ("bf16", 6, 3),
                                         ("f32", 64, 17), ("f32", 10, 0)])
def test_rope_apply(dtype, D, off):
    say("case rope_apply", dtype, D, off)
    rng = np.random.default_rng(33)
    x32 = rng.standard_normal((2, 37, 3, D), dtype=np.float32)
    x = x32 if dtype == "f32" else W.f32_to_bf16_bits(x32)
    xd = W.to_device(x)
    xa.rope_apply(xd, pos_offset=off, rope_base=10000.0)
    torch.cuda.synchronize()
    got = _np(xd)
    ref = oracle.rope(x, pos_offset=off, base=10000.0)
    if dtype == "f32":
        np.testing.assert_allclose(got, ref, atol=1e-6, rtol=0)
        assert (got == ref).mean() > 0.999
    else:
        # both sides round an fp64-accurate value once to bf16: identical except
        # where the two fp64 values straddle a rounding boundary (vanishingly rare)
        ulp = np.abs(ref) * 2.0 ** -7
        assert (np.abs(got - ref) <= ulp + 1e-30).all()
        assert (got == ref).mean() > 0.9999


# ---------------------------------------------------------------- decode --

@pytest.fixture(scope="module")
def decode_workload():
    cfg = W.C5
    say("generating", cfg.name)
    q, kc, vc, sl = W.decode_inputs(cfg)
    ref = oracle.decode(q, kc, vc, sl, scale=cfg.scale, nthreads=NTHREADS)
    dev = (W.to_device(q), W.to_device(kc), W.to_device(vc), torch.from_numpy(sl).to(DEV))
    return cfg, ref, dev


@pytest.mark.parametrize("ns", W.C5.splits)
def test_decode_workload_full(decode_workload, ns):
    cfg, (o_ref, lse_ref), (q, kc, vc, sl) = decode_workload
    say("case", cfg.name, "splits", ns)
    o, lse = xa.attn_decode_splitkv(q, kc, vc, sl, ns, scale=cfg.scale)
    torch.cuda.synchronize()
    e, r = check_bf16(_np(o), _np(lse), o_ref, lse_ref, f"{cfg.name} ns={ns}")
    say(f"  ns={ns}: O max-abs {e:.3e} rel-L2 {r:.3e}")


DEC_CASES = [  # B, Hq, Hkv, D, Smax, lengths, splits
    (4, 8, 2, 128, 300, [0, 1, 300, 157], (1, 3, 64)),
    (2, 3, 3, 64, 1000, [999, 17], (1, 7, 64)),
    (1, 24, 3, 128, 4096, [4096], (2, 16)),
    (3, 6, 1, 64, 100, [100, 0, 33], (5,)),
    (2, 16, 16, 128, 64, [64, 63], (64,)),
]


@pytest.mark.parametrize("case", DEC_CASES, ids=[str(c[:5]) for c in DEC_CASES])
def test_decode_variants(case):
    B, Hq, Hkv, D, Smax, lens, splits = case
    say("case decode", case)
    cfg = W.Decode("t", B, Hq, Hkv, D, Smax, 1, Smax, 77)
    q, kc, vc, sl = W.decode_inputs(cfg, lengths=lens)
    o_ref, lse_ref = oracle.decode(q, kc, vc, sl, scale=cfg.scale, nthreads=NTHREADS)
    dq, dk, dv, dsl = W.to_device(q), W.to_device(kc), W.to_device(vc), torch.from_numpy(sl).to(DEV)
    for ns in splits:
        ws = torch.empty(xa.attn_decode_workspace_bytes(B, Hq, D, ns), dtype=torch.uint8,
                         device=DEV)
        outs = []  # library-owned and caller workspace: the same bits
        for workspace in (None, ws):
            o, lse = xa.attn_decode_splitkv(dq, dk, dv, dsl, ns, scale=cfg.scale,
                                            workspace=workspace)
            torch.cuda.synchronize()
            og, lg = _np(o), _np(lse)
            empty = sl == 0
            assert (og[empty] == 0).all() and np.isneginf(lg[empty]).all()
            check_bf16(og, lg, o_ref, lse_ref, f"{case} ns={ns}")
            outs.append((o.view(torch.int16).cpu().numpy(), lse.cpu().numpy()))
        np.testing.assert_array_equal(outs[0][0], outs[1][0])
        np.testing.assert_array_equal(outs[0][1].view(np.int32), outs[1][1].view(np.int32))


def test_decode_equals_last_prefill_row():
    """Decoding the last position against the cache of the same tokens matches
    row L-1 of causal prefill (both within tolerance of the oracle and of each
    other)."""
    rng = np.random.default_rng(34)
    B, Hq, Hkv, L, D = 2, 8, 2, 700, 128
    q, k, v = _bf16_inputs(rng, B, Hq, Hkv, L, L, D, 1.0)
    o, lse = run_fwd(q, k, v, True, float(np.float32(1 / math.sqrt(D))), 0.0)
    od, lsed = xa.attn_decode_splitkv(W.to_device(np.ascontiguousarray(q[:, -1])), W.to_device(k),
                                      W.to_device(v), torch.tensor([L, L], dtype=torch.int32,
                                                                   device=DEV), 8)
    torch.cuda.synchronize()
    np.testing.assert_allclose(_np(od), o[:, -1], atol=2e-2)
    np.testing.assert_allclose(_np(lsed), lse[:, :, -1], atol=1e-3)


# ------------------------------------------------- other head dims (padded) --

PAD_CASES = [  # dtype, B, Hq, Hkv, Sq, Skv, D, causal, rope
    ("bf16", 2, 8, 2, 3, 7, 36, False, 0.0),        # Moonshine-tiny cross-attention shape
    ("bf16", 2, 8, 2, 64, 1500, 36, False, 0.0),    # decoder queries against 1500 encoder frames
    ("bf16", 1, 8, 2, 130, 130, 36, True, 10000.0),  # decoder self-attention, RoPE at D = 36
    ("bf16", 1, 4, 4, 77, 200, 80, True, 10000.0),
    ("bf16", 2, 2, 1, 50, 50, 1, False, 0.0),
    ("bf16", 1, 3, 3, 65, 65, 127, True, 0.0),
    ("f32", 1, 8, 2, 40, 90, 36, False, 0.0),
    ("f32", 1, 4, 2, 70, 70, 100, True, 500.0),
]


@pytest.mark.parametrize("case", PAD_CASES, ids=[str(c) for c in PAD_CASES])
def test_padded_head_dims(case):
    """Head dims other than 64 and 128 run the kernels on zero-padded copies;
    the result must meet the same bars as the native dims."""
    dt, B, Hq, Hkv, Sq, Skv, D, causal, rope = case
    say("case padded", case)
    rng = np.random.default_rng(W.case_seed(case))
    f = [rng.standard_normal(s, dtype=np.float32)
         for s in ((B, Sq, Hq, D), (B, Skv, Hkv, D), (B, Skv, Hkv, D))]
    q, k, v = f if dt == "f32" else [W.f32_to_bf16_bits(x) for x in f]
    scale = float(np.float32(1 / math.sqrt(D)))
    o, lse = run_fwd(q, k, v, causal, scale, rope)
    assert o.shape == (B, Sq, Hq, D)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal=causal, scale=scale, rope_base=rope,
                                     nthreads=NTHREADS)
    if dt == "f32":
        check_f32(o, lse, o_ref, lse_ref, str(case))
    else:
        check_bf16(o, lse, o_ref, lse_ref, str(case))


def test_keys_up_to_the_32bit_offset_limit():
    """One batch of K and V just under 2 GiB each (7 999 488 keys, D = 128,
    one kv head): the 16-bit kernel's 32-bit buffer offsets reach their
    largest values.  The keys are one random 4096-key block repeated 1953
    times, so O equals the block's attention and the LSE is the block's plus
    ln 1953 (every weight repeated n times); the oracle evaluates the block."""
    reps, blk, D = 1953, 4096, 128
    say("case 32-bit offset limit", reps * blk)
    rng = np.random.default_rng(77)
    q = W.f32_to_bf16_bits(rng.standard_normal((1, 4, 2, D), dtype=np.float32))
    kb = W.f32_to_bf16_bits(rng.standard_normal((1, blk, 1, D), dtype=np.float32))
    vb = W.f32_to_bf16_bits(rng.standard_normal((1, blk, 1, D), dtype=np.float32))
    kd = W.to_device(kb).repeat(1, reps, 1, 1)
    vd = W.to_device(vb).repeat(1, reps, 1, 1)
    assert kd.numel() * 2 < 2 ** 31
    scale = float(np.float32(1 / math.sqrt(D)))
    o, lse = xa.attn_fwd(W.to_device(q), kd, vd, causal=False, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(q, kb, vb, causal=False, scale=scale)
    check_bf16(_np(o), _np(lse), o_ref, lse_ref + math.log(reps), "8M keys")
    del kd, vd
    torch.cuda.empty_cache()
