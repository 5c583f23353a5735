"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no attention arithmetic: it only draws random numbers and
rounds them to the storage format.  The same bytes are handed to the HIP
library and to the fp64 oracle.

Recipe: numpy PCG64 (``default_rng(seed)``) draws float32 N(0, 1) values, in
the order Q, K, V, each a full contiguous [B, S, H, D] array; values are then
multiplied by ``amplitude`` and rounded to bf16 (nearest, ties to even) by
torch's float32 -> bfloat16 conversion when the workload is bf16.  Decode
workloads draw q [B, Hq, D], then the lengths L_b ~ U{lo..hi} (inclusive), then
for each sequence b its K rows [0, L_b) followed by its V rows [0, L_b); cache
rows at and beyond L_b hold a quiet-NaN canary so that any read past the length
shows up in the output.
"""
import zlib
from dataclasses import dataclass, field

import numpy as np
import torch

BF16_NAN = np.uint16(0x7FC0)


@dataclass(frozen=True)
class Prefill:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    D: int
    causal: bool
    rope_base: float
    dtype: str  # "f32" or "bf16"
    seed: int
    amplitude: float = 1.0

    @property
    def scale(self):
        return float(np.float32(1.0 / np.sqrt(self.D)))

    @property
    def flops(self):
        """Algorithmic flops 4*B*Hq*Sq*Skv*D, halved when causal."""
        f = 4 * self.B * self.Hq * self.Sq * self.Skv * self.D
        return f // 2 if self.causal else f

    @property
    def io_bytes(self):
        """Bytes of Q, K, V, O and the fp32 LSE."""
        es = 4 if self.dtype == "f32" else 2
        return (2 * self.B * self.Sq * self.Hq * self.D * es
                + 2 * self.B * self.Skv * self.Hkv * self.D * es
                + 4 * self.B * self.Hq * self.Sq)


@dataclass(frozen=True)
class Decode:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    Smax: int
    len_lo: int
    len_hi: int
    seed: int
    splits: tuple = field(default=(4, 8, 16, 32, 64))

    @property
    def scale(self):
        return float(np.float32(1.0 / np.sqrt(self.D)))


# The five workloads: a single fp32 head; multi-head attention at 1024 tokens
# (causal and not); a Whisper-encoder-shaped 1500-token self-attention (inputs
# x0.5); an LFM2-2.6B-shaped GQA prefill (32 query heads over 8 kv heads,
# causal, RoPE base 10000); a split-KV decode over a 32768-token bf16 cache.
C1 = Prefill("single_head_f32", 1, 1, 1, 128, 128, 64, False, 0.0, "f32", 1001)
C2N = Prefill("mha_s1024", 2, 8, 8, 1024, 1024, 64, False, 0.0, "bf16", 1002)
C2C = Prefill("mha_s1024_causal", 2, 8, 8, 1024, 1024, 64, True, 0.0, "bf16", 1002)
C3 = Prefill("whisper_encoder_s1500", 8, 20, 20, 1500, 1500, 64, False, 0.0, "bf16", 1003, 0.5)
C4 = Prefill("lfm2_gqa_prefill_s4096", 4, 32, 8, 4096, 4096, 64, True, 10000.0, "bf16", 1004)
C5 = Decode("splitkv_decode_s32768", 16, 32, 8, 128, 32768, 1024, 32768, 1005)
PREFILL = (C1, C2N, C2C, C3, C4)


def case_seed(case):
    """A seed for a test case's inputs that is the same in every process
    (Python's hash() of a string changes from one interpreter to the next)."""
    return zlib.crc32(repr(case).encode())


def f32_to_bf16_bits(x):
    """float32 array -> uint16 bf16 bit patterns (nearest, ties to even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits):
    """uint16 bf16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def prefill_inputs(cfg, seed=None):
    """(q, k, v) as numpy arrays: float32 for an f32 workload, uint16 bf16 bit
    patterns for a bf16 one.  Shapes [B,Sq,Hq,D] and [B,Skv,Hkv,D]."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    out = []
    for shape in ((cfg.B, cfg.Sq, cfg.Hq, cfg.D), (cfg.B, cfg.Skv, cfg.Hkv, cfg.D),
                  (cfg.B, cfg.Skv, cfg.Hkv, cfg.D)):
        x = rng.standard_normal(shape, dtype=np.float32)
        if cfg.amplitude != 1.0:
            x *= np.float32(cfg.amplitude)
        out.append(x if cfg.dtype == "f32" else f32_to_bf16_bits(x))
    return tuple(out)


def decode_lengths(cfg, seed=None):
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    rng.standard_normal((cfg.B, cfg.Hq, cfg.D), dtype=np.float32)
    return rng.integers(cfg.len_lo, cfg.len_hi, size=cfg.B, endpoint=True).astype(np.int32)


def decode_inputs(cfg, seed=None, lengths=None):
    """(q [B,Hq,D], kcache, vcache [B,Smax,Hkv,D], seqlens [B] int32), bf16 bits.

    `lengths` overrides the drawn lengths (edge-case tests)."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    q = f32_to_bf16_bits(rng.standard_normal((cfg.B, cfg.Hq, cfg.D), dtype=np.float32))
    drawn = rng.integers(cfg.len_lo, cfg.len_hi, size=cfg.B, endpoint=True).astype(np.int32)
    seqlens = drawn if lengths is None else np.asarray(lengths, dtype=np.int32)
    kc = np.full((cfg.B, cfg.Smax, cfg.Hkv, cfg.D), BF16_NAN, dtype=np.uint16)
    vc = np.full((cfg.B, cfg.Smax, cfg.Hkv, cfg.D), BF16_NAN, dtype=np.uint16)
    for b in range(cfg.B):
        L = int(seqlens[b])
        if L == 0:
            continue
        kc[b, :L] = f32_to_bf16_bits(rng.standard_normal((L, cfg.Hkv, cfg.D), dtype=np.float32))
        vc[b, :L] = f32_to_bf16_bits(rng.standard_normal((L, cfg.Hkv, cfg.D), dtype=np.float32))
    return q, kc, vc, seqlens


def to_device(bits_or_f32, device="cuda"):
    """numpy input -> torch tensor on `device` (uint16 bits become bfloat16)."""
    a = np.ascontiguousarray(bits_or_f32)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)
