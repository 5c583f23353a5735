"""Pins of the fp64 oracle to facts fixed outside the oracle itself.

Each ``pin_*`` function takes a loaded oracle library and raises AssertionError
when the oracle disagrees with:
  * values the pages print for a worked example (fixtures in tests/golden/),
  * a library routine the definition reduces to (torch's fp64 CPU
    scaled_dot_product_attention, scipy's logsumexp, numpy complex arithmetic,
    numpy's binary32 and binary16 rounding, torch's bfloat16 rounding),
  * closed forms and invariants of the mathematics.
The same functions run against deliberately broken builds of the oracle in
test_oracle_mutations.py, which checks that every planted mistake is caught.
"""
import json
import math
import os

import numpy as np
import scipy.special
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bshd(x):
    return torch.from_numpy(np.ascontiguousarray(x)).permute(0, 2, 1, 3).contiguous()


def _torch_sdpa(q, k, v, causal, scale):
    """Library reference: fp64 CPU SDPA on [B,S,H,D] inputs, GQA by repeat of
    each kv head over its contiguous group, causal mask aligned bottom-right."""
    qt, kt, vt = _bshd(q), _bshd(k), _bshd(v)
    Sq, Skv = qt.shape[2], kt.shape[2]
    mask = None
    if causal:
        mask = torch.ones(Sq, Skv, dtype=torch.bool).tril(diagonal=Skv - Sq)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale, enable_gqa=True)
    return o.permute(0, 2, 1, 3).numpy()


def _scipy_lse(q, k, causal, scale):
    """Library reference for LSE: scipy logsumexp over numpy matmul scores."""
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    out = np.empty((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            s = scale * (q[b, :, h, :] @ k[b, :, h // G, :].T)
            if causal:
                s = np.where(np.tril(np.ones((Sq, Skv), bool), k=Skv - Sq), s, -np.inf)
            out[b, h] = scipy.special.logsumexp(s, axis=1)
    return out


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ------------------------------------------------------------ worked values --

def pin_golden_whisper_mask(lib):
    g = _golden("whisper_causal_mask_example.json")
    q = np.array(g["q"])[None, :, None, :]
    k = np.array(g["k"])[None, :, None, :]
    v = np.array(g["v"])[None, :, None, :]
    o, lse = oracle.attn_fwd(q, k, v, causal=g["causal"], scale=g["scale"], lib=lib)
    assert abs(o[0, 0, 0, 0] - g["printed"]["o[0][0]"]) < g["printed"]["tolerance"]
    np.testing.assert_allclose(o[0, :, 0, :], np.array(g["derived"]["o"]), atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.array(g["derived"]["lse"]), atol=1e-14)
    # the page's explicit additive mask, no causal flag
    m = np.array([[float(x) for x in row] for row in g["mask"]])[None, None]
    o2, lse2 = oracle.attn_fwd(q, k, v, causal=False, scale=g["scale"], mask=m, lib=lib)
    assert abs(o2[0, 0, 0, 0] - g["printed"]["o[0][0]"]) < g["printed"]["tolerance"]
    np.testing.assert_allclose(o2[0, :, 0, :], np.array(g["derived"]["o"]), atol=1e-14)
    np.testing.assert_allclose(lse2[0, 0], np.array(g["derived"]["lse"]), atol=1e-14)


def pin_golden_decode_single_token(lib):
    g = _golden("flash_decode_single_token.json")
    q = np.array(g["q"])[None, None, :]
    k = np.array(g["k"])[None, :, None, :]
    v = np.array(g["v"])[None, :, None, :]
    o, lse = oracle.decode(q, k, v, [1], scale=g["scale"], lib=lib)
    np.testing.assert_allclose(o[0, 0], g["printed"]["o"], atol=g["printed"]["tolerance"])
    assert abs(lse[0, 0] - g["derived"]["lse"]) < 1e-14
    o2, lse2 = oracle.flash_decode_head(g["q"], g["k"], g["v"], 4, scale=g["scale"], lib=lib)
    np.testing.assert_allclose(o2, g["printed"]["o"], atol=1e-14)
    assert abs(lse2 - g["derived"]["lse"]) < 1e-14


def pin_golden_decode_uniform_keys(lib):
    g = _golden("flash_decode_uniform_keys.json")
    q = np.array(g["q"])[None, None, :]
    k = np.array(g["k"])[None, :, None, :]
    v = np.array(g["v"])[None, :, None, :]
    o, lse = oracle.decode(q, k, v, [4], scale=g["scale"], lib=lib)
    np.testing.assert_allclose(o[0, 0], g["printed"]["o"], atol=g["printed"]["tolerance"])
    np.testing.assert_allclose(o[0, 0], g["printed"]["o"], atol=1e-13)
    assert abs(lse[0, 0] - g["derived"]["lse"]) < 1e-13
    for tiles in (1, 2, 3, 4, 9):
        o2, lse2 = oracle.flash_decode_head(g["q"], g["k"], g["v"], tiles, scale=g["scale"], lib=lib)
        np.testing.assert_allclose(o2, g["printed"]["o"], atol=1e-13)
        assert abs(lse2 - g["derived"]["lse"]) < 1e-13


def pin_golden_constant_inputs(lib):
    g = _golden("flash_constant_inputs.json")
    S, D = g["seq"], g["head_dim"]
    x = np.full((1, S, 1, D), g["fill"])
    o, lse = oracle.attn_fwd(x, x, x, causal=False, scale=g["scale"], lib=lib)
    np.testing.assert_allclose(o, g["derived"]["o_all"], atol=1e-14)
    np.testing.assert_allclose(lse, g["derived"]["lse_all"], atol=1e-14)
    ot, lt = oracle.attn_tiled_head(x[0, :, 0], x[0, :, 0], x[0, :, 0], scale=g["scale"],
                                    block_q=g["block"], block_kv=g["block"], lib=lib)
    np.testing.assert_allclose(ot, g["derived"]["o_all"], atol=1e-10)
    np.testing.assert_allclose(lt, g["derived"]["lse_all"], atol=1e-12)


# ---------------------------------------------------------- library routines --

def pin_library_sdpa(lib):
    rng = np.random.default_rng(7)
    cases = [  # (B, Hq, Hkv, Sq, Skv, D, causal)
        (2, 4, 4, 7, 7, 8, False), (2, 4, 4, 7, 7, 8, True), (1, 6, 2, 5, 9, 4, True),
        (1, 4, 1, 6, 6, 8, True), (2, 8, 2, 3, 11, 16, False), (1, 3, 3, 9, 9, 6, True),
    ]
    for B, Hq, Hkv, Sq, Skv, D, causal in cases:
        q, k, v = _rand(rng, B, Sq, Hq, D), _rand(rng, B, Skv, Hkv, D), _rand(rng, B, Skv, Hkv, D)
        scale = 0.37
        o, lse = oracle.attn_fwd(q, k, v, causal=causal, scale=scale, lib=lib)
        np.testing.assert_allclose(o, _torch_sdpa(q, k, v, causal, scale), atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse, _scipy_lse(q, k, causal, scale), atol=1e-12, rtol=0)


def pin_library_decode(lib):
    rng = np.random.default_rng(8)
    B, Hq, Hkv, D, Smax = 3, 8, 2, 16, 12
    q, kc, vc = _rand(rng, B, Hq, D), _rand(rng, B, Smax, Hkv, D), _rand(rng, B, Smax, Hkv, D)
    lens = [12, 5, 1]
    o, lse = oracle.decode(q, kc, vc, lens, scale=0.25, lib=lib)
    for b, L in enumerate(lens):
        ref = _torch_sdpa(q[b][None, None], kc[b:b + 1, :L], vc[b:b + 1, :L], False, 0.25)
        np.testing.assert_allclose(o[b], ref[0, 0], atol=1e-12)
        np.testing.assert_allclose(lse[b], _scipy_lse(q[b][None, None], kc[b:b + 1, :L],
                                                      False, 0.25)[0, :, 0], atol=1e-12)


def pin_rounding(lib):
    """Rounding of rotated values: binary32 against numpy, bf16 against torch,
    and the two tie cases of round-to-nearest-even at 1.0."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal(2000) * 10.0 ** rng.integers(-3, 4, 2000)
    for xi in x:
        assert oracle.round_sig(xi, 24, lib=lib) == float(np.float32(xi))
    xf = x.astype(np.float32)
    tb = torch.from_numpy(xf).to(torch.bfloat16).to(torch.float64).numpy()
    for xi, ti in zip(xf, tb):
        assert oracle.round_sig(float(xi), 8, lib=lib) == ti
    assert oracle.round_sig(1.0 + 2.0 ** -8, 8, lib=lib) == 1.0
    assert oracle.round_sig(1.0 + 3 * 2.0 ** -8, 8, lib=lib) == 1.0 + 2.0 ** -6
    assert oracle.round_sig(-(1.0 + 3 * 2.0 ** -8), 8, lib=lib) == -(1.0 + 2.0 ** -6)


def pin_f16(lib):
    """IEEE binary16 inputs and rounding: every finite bit pattern widens to
    numpy's float16 value (and a few to the values of the format's definition);
    rounding to 11 bits equals numpy's direct float64 -> float16 conversion,
    subnormals and overflow included, with hand-checked ties."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    pats = pats[((pats >> 10) & 31) != 31]                 # finite patterns only
    x16 = pats.view(np.float16).reshape(1, 1, -1, 64)
    # position 0 rotates by angle 0: the widened inputs come back unchanged
    w = oracle.rope(x16, 0, 10000.0, round_bits=0, lib=lib)
    np.testing.assert_array_equal(w.ravel(), x16.astype(np.float64).ravel())
    byp = dict(zip(pats.tolist(), w.ravel().tolist()))
    for bitsv, val in ((0x0001, 2.0 ** -24), (0x03FF, 1023 * 2.0 ** -24), (0x0400, 2.0 ** -14),
                       (0x3C00, 1.0), (0x3C01, 1.0 + 2.0 ** -10), (0xC000, -2.0),
                       (0x7BFF, 65504.0), (0x3555, 0.333251953125)):
        assert byp[bitsv] == val, (hex(bitsv), byp[bitsv], val)
    rng = np.random.default_rng(15)
    x = rng.standard_normal(3000) * 2.0 ** rng.integers(-30, 18, 3000).astype(np.float64)
    for xi in x:
        assert oracle.round_sig(xi, 11, lib=lib) == float(np.float16(xi)), xi
    for xi, want in ((1.0 + 2.0 ** -11, 1.0), (1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),
                     (2.0 ** -25, 0.0), (3 * 2.0 ** -25, 2.0 ** -23), (1.5 * 2.0 ** -24, 2.0 ** -23),
                     (65519.0, 65504.0), (65520.0, np.inf), (-65520.0, -np.inf)):
        assert oracle.round_sig(xi, 11, lib=lib) == want, (xi, want)
    # attention on fp16 inputs with RoPE: the rotated q, k rounded to fp16
    f = [rng.standard_normal(sh).astype(np.float16) for sh in ((1, 7, 2, 16), (1, 7, 1, 16),
                                                                (1, 7, 1, 16))]
    o, lse = oracle.attn_fwd(*f, causal=True, scale=0.25, rope_base=10000.0, lib=lib)
    q, k, v = (a.astype(np.float64) for a in f)
    qr = _rope_complex(q, 0, 10000.0).astype(np.float16).astype(np.float64)
    kr = _rope_complex(k, 0, 10000.0).astype(np.float16).astype(np.float64)
    np.testing.assert_allclose(o, _torch_sdpa(qr, kr, v, True, 0.25), atol=1e-12)
    np.testing.assert_allclose(lse, _scipy_lse(qr, kr, True, 0.25), atol=1e-12)


# ---------------------------------------------------------- RoPE --

def _rope_complex(x, pos0, base):
    """Rotation as complex multiplication: pair (x_2i, x_2i+1) is the complex
    number x_2i + i x_2i+1, multiplied by exp(i * pos * base^(-2i/D))."""
    B, S, H, D = x.shape
    z = x[..., 0::2] + 1j * x[..., 1::2]
    pos = (pos0 + np.arange(S, dtype=np.float64))[None, :, None, None]
    inv = base ** (-2.0 * np.arange(D // 2) / D)
    zr = z * np.exp(1j * pos * inv)
    out = np.empty_like(x)
    out[..., 0::2], out[..., 1::2] = zr.real, zr.imag
    return out


def pin_rope(lib):
    rng = np.random.default_rng(10)
    x = _rand(rng, 2, 9, 3, 16)
    for off in (0, 5, 4000):
        r = oracle.rope(x, pos_offset=off, base=10000.0, round_bits=0, lib=lib)
        np.testing.assert_allclose(r, _rope_complex(x, off, 10000.0), atol=1e-11, rtol=0)
        # pair norms preserved
        np.testing.assert_allclose(r[..., 0::2] ** 2 + r[..., 1::2] ** 2,
                                   x[..., 0::2] ** 2 + x[..., 1::2] ** 2, rtol=1e-12)
    # identity at position 0 (the first token at offset 0)
    r = oracle.rope(x, 0, 10000.0, 0, lib=lib)
    np.testing.assert_array_equal(r[:, 0], x[:, 0])
    # R(-p) undoes R(p), and rotations compose: R(b) R(a) = R(a + b)
    x1 = x[:, :1]
    for p in (1, 17, 3000):
        back = oracle.rope(oracle.rope(x1, p, 10000.0, 0, lib=lib), -p, 10000.0, 0, lib=lib)
        np.testing.assert_allclose(back, x1, atol=1e-12)
        two = oracle.rope(oracle.rope(x1, p, 500.0, 0, lib=lib), 7, 500.0, 0, lib=lib)
        np.testing.assert_allclose(two, oracle.rope(x1, p + 7, 500.0, 0, lib=lib), atol=1e-11)
    # the pages' checks: a constant row changes at position 1; offsets 0 and 2 differ
    ones = np.ones((1, 4, 2, 8))
    r1 = oracle.rope(ones, 0, 10000.0, 0, lib=lib)
    assert np.abs(r1[0, 1] - ones[0, 1]).max() > 1e-10
    half = np.full((1, 4, 1, 4), 0.5)
    assert np.abs(oracle.rope(half, 0, 10000.0, 0, lib=lib)
                  - oracle.rope(half, 2, 10000.0, 0, lib=lib)).max() > 1e-10
    # odd head dim rejected
    try:
        oracle.rope(np.ones((1, 2, 1, 7)), 0, 10000.0, 0, lib=lib)
    except ValueError:
        pass
    else:
        raise AssertionError("odd head dim accepted by RoPE")


def pin_rope_attention(lib):
    """Attention with RoPE equals attention (library SDPA) on inputs rotated by
    complex multiplication, queries at Skv - Sq + i and keys at j; a common
    shift of all positions leaves the scores unchanged."""
    rng = np.random.default_rng(11)
    for (B, Hq, Hkv, Sq, Skv, D, causal) in ((1, 4, 2, 6, 6, 8, True), (2, 2, 1, 3, 8, 16, True),
                                             (1, 2, 2, 5, 5, 8, False)):
        q, k, v = _rand(rng, B, Sq, Hq, D), _rand(rng, B, Skv, Hkv, D), _rand(rng, B, Skv, Hkv, D)
        o, lse = oracle.attn_fwd(q, k, v, causal=causal, scale=0.3, rope_base=100.0,
                                 round_bits=0, lib=lib)
        qr, kr = _rope_complex(q, Skv - Sq, 100.0), _rope_complex(k, 0, 100.0)
        np.testing.assert_allclose(o, _torch_sdpa(qr, kr, v, causal, 0.3), atol=1e-11)
        np.testing.assert_allclose(lse, _scipy_lse(qr, kr, causal, 0.3), atol=1e-11)
        qs, ks = _rope_complex(q, Skv - Sq + 37, 100.0), _rope_complex(k, 37, 100.0)
        np.testing.assert_allclose(lse, _scipy_lse(qs, ks, causal, 0.3), atol=1e-10)


def pin_rope_rounding_in_attention(lib):
    """bf16 inputs with RoPE: the rotated q/k are rounded to bf16 before the
    dot products.  Reproduce by rounding the complex-rotated values with torch."""
    rng = np.random.default_rng(12)
    B, Hq, Hkv, S, D = 1, 2, 1, 7, 16
    f = [rng.standard_normal(s).astype(np.float32) for s in
         ((B, S, Hq, D), (B, S, Hkv, D), (B, S, Hkv, D))]
    bits = [torch.from_numpy(a).to(torch.bfloat16) for a in f]
    q, k, v = [b.to(torch.float64).numpy() for b in bits]
    qb, kb, vb = [b.view(torch.int16).numpy().view(np.uint16) for b in bits]
    o, lse = oracle.attn_fwd(qb, kb, vb, causal=True, scale=0.25, rope_base=10000.0, lib=lib)

    def rb(x):  # via float32 first: exact when the fp64 value is not near a tie
        return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    qr, kr = rb(_rope_complex(q, 0, 10000.0)), rb(_rope_complex(k, 0, 10000.0))
    np.testing.assert_allclose(o, _torch_sdpa(qr, kr, v, True, 0.25), atol=1e-12)
    np.testing.assert_allclose(lse, _scipy_lse(qr, kr, True, 0.25), atol=1e-12)


# ---------------------------------------------------------- invariants --

def pin_softmax_rows(lib):
    """With V = I (Skv = D) the output rows are the softmax rows: non-negative,
    summing to 1, and equal to exp(s - LSE)."""
    rng = np.random.default_rng(13)
    S, D = 8, 8
    q, k = _rand(rng, 1, S, 1, D), _rand(rng, 1, S, 1, D)
    v = np.eye(D)[None, :, None, :]
    for causal in (False, True):
        o, lse = oracle.attn_fwd(q, k, v, causal=causal, scale=0.5, lib=lib)
        P = o[0, :, 0, :]
        assert (P >= 0).all()
        np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-14)
        s = 0.5 * (q[0, :, 0] @ k[0, :, 0].T)
        expected = np.exp(s - lse[0, 0][:, None])
        if causal:
            expected = np.tril(expected)
        np.testing.assert_allclose(P, expected, atol=1e-14)


def pin_special_cases(lib):
    rng = np.random.default_rng(14)
    q, k = _rand(rng, 2, 6, 2, 8), _rand(rng, 2, 6, 2, 8)
    # constant V gives that constant
    o, _ = oracle.attn_fwd(q, k, np.full((2, 6, 2, 8), -1.25), causal=True, scale=0.4, lib=lib)
    np.testing.assert_allclose(o, -1.25, atol=1e-14)
    # a single key returns its value, LSE is its score
    v1 = _rand(rng, 2, 1, 2, 8)
    o, lse = oracle.attn_fwd(q, k[:, :1], v1, scale=0.4, lib=lib)
    np.testing.assert_allclose(o, np.broadcast_to(v1, o.shape), atol=1e-14)
    np.testing.assert_allclose(lse, 0.4 * np.einsum("bihd,bjhd->bhi", q, k[:, :1]), atol=1e-13)
    # causal row 0 is v0, with LSE the score s00
    v = _rand(rng, 2, 6, 2, 8)
    o, lse = oracle.attn_fwd(q, k, v, causal=True, scale=0.4, lib=lib)
    np.testing.assert_allclose(o[:, 0], v[:, 0], atol=1e-14)
    np.testing.assert_allclose(lse[:, :, 0], 0.4 * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0]),
                               atol=1e-13)
    # rows with no visible key (causal, Sq > Skv): O = 0, LSE = -inf
    o, lse = oracle.attn_fwd(_rand(rng, 1, 5, 1, 4), k[:1, :2, :1, :4], v[:1, :2, :1, :4],
                             causal=True, scale=0.5, lib=lib)
    assert (o[0, :3] == 0).all() and np.isneginf(lse[0, 0, :3]).all()
    assert np.isfinite(lse[0, 0, 3:]).all()
    np.testing.assert_allclose(o[0, 3, 0], v[0, 0, 0, :4], atol=1e-14)


def pin_gqa(lib):
    """GQA(H) = MHA; GQA(1) = MQA = MHA with K/V replicated; GQA(G) = MHA with
    each kv head repeated over its contiguous group of G query heads."""
    rng = np.random.default_rng(15)
    B, Hq, S, D = 2, 8, 6, 8
    q = _rand(rng, B, S, Hq, D)
    for Hkv in (8, 4, 2, 1):
        k, v = _rand(rng, B, S, Hkv, D), _rand(rng, B, S, Hkv, D)
        G = Hq // Hkv
        o, lse = oracle.attn_fwd(q, k, v, causal=True, scale=0.3, lib=lib)
        o2, lse2 = oracle.attn_fwd(q, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2),
                                   causal=True, scale=0.3, lib=lib)
        np.testing.assert_array_equal(o, o2)
        np.testing.assert_array_equal(lse, lse2)
        for h in range(Hq):  # each head alone, against its own kv head
            oh, _ = oracle.attn_fwd(q[:, :, h:h + 1], k[:, :, h // G:h // G + 1],
                                    v[:, :, h // G:h // G + 1], causal=True, scale=0.3, lib=lib)
            np.testing.assert_array_equal(o[:, :, h:h + 1], oh)


def pin_permutation_and_scale(lib):
    rng = np.random.default_rng(16)
    q, k, v = _rand(rng, 1, 5, 2, 8), _rand(rng, 1, 9, 2, 8), _rand(rng, 1, 9, 2, 8)
    o, lse = oracle.attn_fwd(q, k, v, scale=0.3, lib=lib)
    perm = rng.permutation(9)
    o2, lse2 = oracle.attn_fwd(q, k[:, perm], v[:, perm], scale=0.3, lib=lib)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, atol=1e-13)
    o3, lse3 = oracle.attn_fwd(q * 4.0, k, v, scale=0.3 / 4.0, lib=lib)
    np.testing.assert_array_equal(o, o3)
    np.testing.assert_array_equal(lse, lse3)
    # a shift of all scores by c leaves O unchanged and moves LSE by c:
    # append a constant dimension to q and k
    qa = np.concatenate([q, np.ones((1, 5, 2, 1))], axis=3)
    ka = np.concatenate([k, np.full((1, 9, 2, 1), 2.0)], axis=3)
    va = np.concatenate([v, np.zeros((1, 9, 2, 1))], axis=3)
    o4, lse4 = oracle.attn_fwd(qa, ka, va, scale=0.3, lib=lib)
    np.testing.assert_allclose(o4[..., :8], o, atol=1e-13)
    np.testing.assert_allclose(lse4, lse + 0.6, atol=1e-13)


def pin_split_merge(lib):
    """Split-KV decode merged by LSE equals the monolithic result for every
    tile count (including more tiles than keys), and the merge ignores empty
    parts."""
    rng = np.random.default_rng(17)
    S, D = 13, 8
    q, k, v = _rand(rng, D), _rand(rng, S, D), _rand(rng, S, D)
    o_ref, lse_ref = oracle.decode(q[None, None], k[None, :, None], v[None, :, None], [S],
                                   scale=0.35, lib=lib)
    for n in range(1, S + 3):
        o, lse = oracle.flash_decode_head(q, k, v, n, scale=0.35, lib=lib)
        np.testing.assert_allclose(o, o_ref[0, 0], atol=1e-13)
        assert abs(lse - lse_ref[0, 0]) < 1e-13
    # arbitrary partition with empty parts, merged by the oracle's merge
    cuts = [0, 0, 4, 4, 11, 13, 13]
    parts, lses = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        if a == b:
            parts.append(np.zeros(D))
            lses.append(-np.inf)
            continue
        op, lp = oracle.decode(q[None, None], k[None, a:b, None], v[None, a:b, None], [b - a],
                               scale=0.35, lib=lib)
        parts.append(op[0, 0])
        lses.append(lp[0, 0])
    o, lse = oracle.lse_merge(np.array(parts), np.array(lses), lib=lib)
    np.testing.assert_allclose(o, o_ref[0, 0], atol=1e-13)
    assert abs(lse - lse_ref[0, 0]) < 1e-13
    o, lse = oracle.lse_merge(np.zeros((3, D)), np.full(3, -np.inf), lib=lib)
    assert (o == 0).all() and lse == -np.inf


def pin_decode_multi_head_page_example(lib):
    """The per-head comparison of the flash_decode_multi_head test of the
    flash-decoding page: deterministic ramps, 2 heads, 16 tokens, head dim 8."""
    H, D, S = 2, 8, 16
    qs = 0.1 * np.arange(H * D, dtype=np.float32)
    ks = (0.05 * (np.arange(S * H * D) % 17) + 0.01).astype(np.float32)
    vs = (0.02 * (np.arange(S * H * D) % 13) + 0.1).astype(np.float32)
    q = qs.reshape(1, H, D)
    kc = ks.reshape(1, S, H, D)
    vc = vs.reshape(1, S, H, D)
    o, _ = oracle.decode(q, kc, vc, [S], lib=lib)
    for h in range(H):
        o1, _ = oracle.flash_decode_head(q[0, h], kc[0, :, h], vc[0, :, h], 1, lib=lib)
        o4, _ = oracle.flash_decode_head(q[0, h], kc[0, :, h], vc[0, :, h], 4, lib=lib)
        assert np.abs(o[0, h] - o1).mean() < 1e-4
        np.testing.assert_allclose(o[0, h], o4, atol=1e-13)
    np.testing.assert_allclose(o, _torch_sdpa(q.astype(np.float64)[:, None],
                                              kc.astype(np.float64), vc.astype(np.float64),
                                              False, 1 / math.sqrt(D))[:, 0], atol=1e-12)


def pin_tiled_equals_definition(lib):
    """The tiled online-softmax forward (query blocks outside, kv blocks
    inside) equals the definition for every block size, causal or not."""
    rng = np.random.default_rng(18)
    for Sq, Skv, causal in ((7, 7, False), (7, 7, True), (4, 9, True), (9, 9, True)):
        q, k, v = _rand(rng, Sq, 8), _rand(rng, Skv, 8), _rand(rng, Skv, 8)
        o_ref, lse_ref = oracle.attn_fwd(q[None, :, None], k[None, :, None], v[None, :, None],
                                         causal=causal, scale=0.3, lib=lib)
        for bq in range(1, Sq + 2):
            for bk in (1, 2, 3, Skv, Skv + 5):
                o, lse = oracle.attn_tiled_head(q, k, v, causal=causal, scale=0.3, block_q=bq,
                                                block_kv=bk, lib=lib)
                np.testing.assert_allclose(o, o_ref[0, :, 0], atol=1e-13)
                np.testing.assert_allclose(lse, lse_ref[0, 0], atol=1e-13)


def pin_decode_is_last_prefill_row(lib):
    """Decoding the query at position L-1 against an L-token cache equals row
    L-1 of causal prefill over the same tokens."""
    rng = np.random.default_rng(19)
    B, Hq, Hkv, L, D = 2, 4, 2, 10, 8
    q, k, v = _rand(rng, B, L, Hq, D), _rand(rng, B, L, Hkv, D), _rand(rng, B, L, Hkv, D)
    o, lse = oracle.attn_fwd(q, k, v, causal=True, scale=0.3, lib=lib)
    od, lsed = oracle.decode(q[:, -1], k, v, [L, L], scale=0.3, lib=lib)
    np.testing.assert_allclose(od, o[:, -1], atol=1e-13)
    np.testing.assert_allclose(lsed, lse[:, :, -1], atol=1e-13)
    # a shorter cache length is the prefill of that prefix
    od, _ = oracle.decode(q[:, 5], k, v, [6, 6], scale=0.3, lib=lib)
    np.testing.assert_allclose(od, o[:, 5], atol=1e-13)


def pin_sampled_rows(lib):
    """Row/unit sampling returns exactly the corresponding full results."""
    rng = np.random.default_rng(20)
    q, k, v = _rand(rng, 2, 9, 4, 8), _rand(rng, 2, 9, 2, 8), _rand(rng, 2, 9, 2, 8)
    o, lse = oracle.attn_fwd(q, k, v, causal=True, scale=0.3, rope_base=50.0, lib=lib)
    rows, units = [0, 4, 8], [1, 6]
    os_, ls = oracle.attn_fwd(q, k, v, causal=True, scale=0.3, rope_base=50.0, rows=rows,
                              units=units, nthreads=2, lib=lib)
    for ui, u in enumerate(units):
        b, h = divmod(u, 4)
        np.testing.assert_array_equal(os_[ui], o[b, rows, h])
        np.testing.assert_array_equal(ls[ui], lse[b, h, rows])


def pin_padded_head_dim(lib):
    """Zero-padding the head dim (36 -> 40) and multiplying Q by sqrt(40/36)
    under the scale 1/sqrt(40) gives exact attention at D = 36 with the scale
    1/sqrt(36): zero columns add nothing to the scores, V's zero columns give
    zero output columns, and the two scales agree."""
    rng = np.random.default_rng(33)
    for (B, Hq, Hkv, Sq, Skv, causal) in ((1, 8, 2, 3, 7, False), (2, 4, 1, 6, 6, True)):
        D, Dp = 36, 40
        q, k, v = _rand(rng, B, Sq, Hq, D), _rand(rng, B, Skv, Hkv, D), _rand(rng, B, Skv, Hkv, D)
        o, lse = oracle.attn_fwd(q, k, v, causal=causal, scale=1 / math.sqrt(D), lib=lib)

        def pad(x):
            return np.concatenate([x, np.zeros(x.shape[:-1] + (Dp - D,))], axis=-1)
        op, lsep = oracle.attn_fwd(pad(q * math.sqrt(Dp / D)), pad(k), pad(v), causal=causal,
                                   scale=1 / math.sqrt(Dp), lib=lib)
        np.testing.assert_allclose(op[..., :D], o, atol=1e-12)
        assert (op[..., D:] == 0).all()
        np.testing.assert_allclose(lsep, lse, atol=1e-12)


def pin_additive_mask(lib):
    """Additive masks: torch fp64 SDPA with a float attn_mask (broadcast over
    batch, per head, and per batch and head; GQA); a mask of -inf above the
    bottom-right diagonal equals causal=True; a constant mask c leaves O and
    shifts the LSE by c."""
    rng = np.random.default_rng(34)
    B, Hq, Hkv, Sq, Skv, D = 2, 4, 2, 5, 9, 8
    q, k, v = _rand(rng, B, Sq, Hq, D), _rand(rng, B, Skv, Hkv, D), _rand(rng, B, Skv, Hkv, D)
    for shape in ((1, 1, Sq, Skv), (1, Hq, Sq, Skv), (B, Hq, Sq, Skv), (B, 1, Sq, Skv)):
        m = rng.standard_normal(shape)
        m[..., 1, 3] = -np.inf
        o, lse = oracle.attn_fwd(q, k, v, scale=0.35, mask=m, lib=lib)
        qt, kt, vt = (torch.tensor(_bshd(a)) for a in (q, k, v))
        mt = torch.tensor(np.broadcast_to(m, (B, Hq, Sq, Skv)).copy())
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt, scale=0.35,
                                             enable_gqa=True).permute(0, 2, 1, 3).numpy()
        np.testing.assert_allclose(o, ref, atol=1e-12)
        s = 0.35 * np.einsum("bihd,bjhd->bhij", q, np.repeat(k, Hq // Hkv, axis=2)) + \
            np.broadcast_to(m, (B, Hq, Sq, Skv))
        np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=-1), atol=1e-12)
    hide = np.where(np.arange(Skv)[None, :] > np.arange(Sq)[:, None] + (Skv - Sq), -np.inf, 0.0)
    o1, l1 = oracle.attn_fwd(q, k, v, scale=0.35, mask=hide[None, None], lib=lib)
    o2, l2 = oracle.attn_fwd(q, k, v, scale=0.35, causal=True, lib=lib)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)
    o3, l3 = oracle.attn_fwd(q, k, v, scale=0.35, mask=np.full((1, 1, Sq, Skv), 2.5), lib=lib)
    o4, l4 = oracle.attn_fwd(q, k, v, scale=0.35, lib=lib)
    np.testing.assert_allclose(o3, o4, atol=1e-13)
    np.testing.assert_allclose(l3, l4 + 2.5, atol=1e-13)


# ---------------------------------------------------------- backward --

def _torch_rope(x, pos0, base):
    """Differentiable pair rotation (the complex multiplication of _rope_complex)."""
    B, S, H, D = x.shape
    pos = pos0 + torch.arange(S, dtype=torch.float64)
    inv = base ** (-2.0 * torch.arange(D // 2, dtype=torch.float64) / D)
    ang = pos[:, None] * inv[None, :]
    c, s = torch.cos(ang)[None, :, None, :], torch.sin(ang)[None, :, None, :]
    x0, x1 = x[..., 0::2], x[..., 1::2]
    return torch.stack((x0 * c - x1 * s, x0 * s + x1 * c), dim=-1).reshape(B, S, H, D)


def _torch_grads(q, k, v, dout, causal, scale, rope_base):
    """Reverse-mode gradients of sum(O * dout) from a plain fp64 torch attention
    (GQA by repeating kv heads, bottom-right causal mask, RoPE as above)."""
    q, k, v = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    qr = _torch_rope(q, Skv - Sq, rope_base) if rope_base > 0 else q
    kr = _torch_rope(k, 0, rope_base) if rope_base > 0 else k
    kh = kr.permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    vh = v.permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    s = scale * qr.permute(0, 2, 1, 3) @ kh.transpose(-1, -2)
    if causal:
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Skv)[None, :]
        s = s.masked_fill(j > i + (Skv - Sq), float("-inf"))
    o = (torch.softmax(s, dim=-1) @ vh).permute(0, 2, 1, 3)
    (o * torch.tensor(dout, dtype=torch.float64)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def pin_bwd_autograd(lib):
    """Gradients equal reverse-mode differentiation of a plain torch fp64
    attention: GQA groups, causal (square and Sq < Skv), RoPE, no mask."""
    rng = np.random.default_rng(30)
    for (B, Hq, Hkv, Sq, Skv, D, causal, rope) in ((1, 4, 2, 6, 6, 8, True, 100.0),
                                                   (2, 2, 1, 3, 7, 8, True, 0.0),
                                                   (1, 3, 3, 5, 4, 4, False, 50.0),
                                                   (1, 6, 2, 4, 9, 6, True, 1000.0)):
        q, k, v = _rand(rng, B, Sq, Hq, D), _rand(rng, B, Skv, Hkv, D), _rand(rng, B, Skv, Hkv, D)
        do = _rand(rng, B, Sq, Hq, D)
        got = oracle.attn_bwd(q, k, v, do, causal=causal, scale=0.4, rope_base=rope,
                              round_bits=0, lib=lib)
        ref = _torch_grads(q, k, v, do, causal, 0.4, rope)
        for g, r in zip(got, ref):
            np.testing.assert_allclose(g, r, atol=1e-11, rtol=0)


def pin_bwd_finite_differences(lib):
    """Central differences of L = sum(O * G) through the forward oracle."""
    rng = np.random.default_rng(31)
    B, Hq, Hkv, Sq, Skv, D = 1, 2, 1, 3, 4, 4
    q, k, v = _rand(rng, B, Sq, Hq, D), _rand(rng, B, Skv, Hkv, D), _rand(rng, B, Skv, Hkv, D)
    G = _rand(rng, B, Sq, Hq, D)
    kw = dict(causal=True, scale=0.5, rope_base=30.0, round_bits=0, lib=lib)
    dq, dk, dv = oracle.attn_bwd(q, k, v, G, **kw)

    def loss(q_, k_, v_):
        return float((oracle.attn_fwd(q_, k_, v_, **kw)[0] * G).sum())
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": (q, k, v), "k": (q, k, v), "v": (q, k, v)}[name]
            a_p = [xp if n == name else a for n, a in zip("qkv", args)]
            a_m = [xm if n == name else a for n, a in zip("qkv", args)]
            num[idx] = (loss(*a_p) - loss(*a_m)) / (2 * h)
        np.testing.assert_allclose(g, num, atol=2e-8, rtol=0, err_msg=name)


def pin_bwd_invariants(lib):
    """Without RoPE the keys' gradients of a (batch, kv head) sum to zero
    (softmax is unchanged by adding one vector to every key); each row of P
    sums to one, so the values' gradients of a kv head sum to the summed dO of
    its query heads (every row sees at least one key here); with a single key
    P = 1, so dq = dk = 0 and dv = that sum."""
    rng = np.random.default_rng(32)
    B, Hq, Hkv, Sq, Skv, D = 2, 4, 2, 5, 7, 8
    q, k, v = _rand(rng, B, Sq, Hq, D), _rand(rng, B, Skv, Hkv, D), _rand(rng, B, Skv, Hkv, D)
    do = _rand(rng, B, Sq, Hq, D)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal=True, scale=0.3, round_bits=0, lib=lib)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    dsum = do.reshape(B, Sq, Hkv, Hq // Hkv, D).sum(axis=(1, 3))
    np.testing.assert_allclose(dv.sum(axis=1), dsum, atol=1e-12)
    k1, v1 = k[:, :1], v[:, :1]
    dq, dk, dv = oracle.attn_bwd(q, k1, v1, do, causal=False, scale=0.3, round_bits=0, lib=lib)
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    np.testing.assert_allclose(dv[:, 0], dsum, atol=1e-12)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
