"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the polynomial method: it draws numbers
and rounds them to the I/O formats.  Both the oracle side and the GPU side
consume exactly these arrays.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), counter based: output i of stream `seed` is
mix(seed + (i + 1) * 0x9E3779B97F4A7C15).  Uniforms take the top 53 bits;
normals use Box-Muller on consecutive uniform pairs, in FP64; values are then
rounded to nearest-even into FP16 or BF16.

Workloads (the paper's shapes; "Fast Polynomial Transcendentals for LLMs",
sections 4.2 and 4.3):
  cfg1  x ~ U(-8, 8), 4,194,304 FP16, plus all 65,536 FP16 bit patterns
  cfg2  x ~ clip(N(0, 3), +-12) FP16 (sd 3), grad ~ N(0, 1), 4,194,304 and
        268,435,456 elements
  cfg3  gate, up ~ N(0, 2), dh ~ N(0, 1), BF16 [8192 x 14336]
  cfg4  16,384 tokens routed top-8 over 64 experts (Zipf s = 1.1 popularity
        over a seeded permutation), expert-sorted rows [sum counts x 1408]
  cfg5  Q, K, V ~ N(0, 1) BF16 [1, 16, 8192, 128]
  rope  Q [1, 4096, 32, 128], K [1, 4096, 8, 128] ~ N(0, 1) FP16 (Appendix
        B.2's fused rotary embedding, Llama-3-8B-like heads)
Seeds: 1 = x / gate / Q, 2 = up / K, 3 = grad / dh / V, 4 = routing,
5 = attention dO, 9 / 10 = rotary Q / K.
"""
from __future__ import annotations

import numpy as np

try:   # optional: the same recipe on a GPU for the 268M-element arrays
    import torch
except ImportError:  # pragma: no cover
    torch = None

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)

SEED_X, SEED_U, SEED_G, SEED_ROUTE, SEED_DO = 1, 2, 3, 4, 5


def splitmix64(seed: int, n: int, offset: int = 0) -> np.ndarray:
    """Outputs offset .. offset + n - 1 of the SplitMix64 stream `seed`."""
    with np.errstate(over="ignore"):
        i = np.arange(offset + 1, offset + n + 1, dtype=np.uint64)
        z = np.uint64(seed) + i * GOLDEN
        z = (z ^ (z >> np.uint64(30))) * M1
        z = (z ^ (z >> np.uint64(27))) * M2
        return z ^ (z >> np.uint64(31))


def uniform01(seed: int, n: int, offset: int = 0) -> np.ndarray:
    """FP64 uniforms in [0, 1): top 53 bits times 2^-53."""
    return (splitmix64(seed, n, offset) >> np.uint64(11)).astype(np.float64) * 2.0 ** -53


def normal(seed: int, n: int, sd: float = 1.0, chunk: int = 1 << 24) -> np.ndarray:
    """FP64 N(0, sd^2) by Box-Muller: uniforms (u1, u2) = outputs (2k, 2k+1)
    give elements 2k (cosine) and 2k+1 (sine)."""
    out = np.empty(n, dtype=np.float64)
    npairs = (n + 1) // 2
    for p0 in range(0, npairs, chunk):
        p1 = min(npairs, p0 + chunk)
        u = uniform01(seed, 2 * (p1 - p0), 2 * p0).reshape(-1, 2)
        r = np.sqrt(-2.0 * np.log1p(-u[:, 0])) * sd
        a = 2.0 * np.pi * u[:, 1]
        z = np.empty(2 * (p1 - p0))
        z[0::2] = r * np.cos(a)
        z[1::2] = r * np.sin(a)
        e0 = 2 * p0
        e1 = min(n, 2 * p1)
        out[e0:e1] = z[: e1 - e0]
    return out


# ---- the same recipe in torch, on any device ---------------------------------
# The integer stream is bit-identical to splitmix64() (int64 arithmetic wraps
# modulo 2^64; logical shifts are masked).  The FP64 Box-Muller transcendentals
# of the device library may differ from numpy's in the last bit, so an array
# drawn on the GPU can differ in rare roundings from the numpy one; every
# consumer that compares two paths hands both the same drawn array.

def _t_splitmix64(seed: int, n: int, offset: int, device):
    def shr(z, k):
        return (z >> k) & ((1 << (64 - k)) - 1)
    g = int(GOLDEN) - (1 << 64)
    m1 = int(M1) - (1 << 64)
    m2 = int(M2) - (1 << 64)
    i = torch.arange(offset + 1, offset + n + 1, dtype=torch.int64, device=device)
    z = seed + i * g
    z = (z ^ shr(z, 30)) * m1
    z = (z ^ shr(z, 27)) * m2
    return z ^ shr(z, 31)


def t_uniform01(seed: int, n: int, offset: int = 0, device="cuda"):
    z = _t_splitmix64(seed, n, offset, device)
    return ((z >> 11) & ((1 << 53) - 1)).to(torch.float64) * 2.0 ** -53


def t_normal(seed: int, n: int, sd: float = 1.0, device="cuda", chunk: int = 1 << 25):
    out = torch.empty(n, dtype=torch.float64, device=device)
    npairs = (n + 1) // 2
    for p0 in range(0, npairs, chunk):
        p1 = min(npairs, p0 + chunk)
        u = t_uniform01(seed, 2 * (p1 - p0), 2 * p0, device).view(-1, 2)
        r = torch.sqrt(-2.0 * torch.log1p(-u[:, 0])) * sd
        a = 2.0 * np.pi * u[:, 1]
        z = torch.stack([r * torch.cos(a), r * torch.sin(a)], dim=1).view(-1)
        e1 = min(n, 2 * p1)
        out[2 * p0:e1] = z[: e1 - 2 * p0]
    return out


def t_cfg2(n: int, device="cuda"):
    """cfg2's x and grad as torch float16 tensors drawn on `device` (torch's
    FP64 -> FP16 conversion)."""
    x = torch.clamp(t_normal(SEED_X, n, 3.0, device), -12.0, 12.0).to(torch.float16)
    g = t_normal(SEED_G, n, 1.0, device).to(torch.float16)
    return x, g


def t_rope_inputs(B: int = 1, S: int = 4096, Hq: int = 32, Hkv: int = 8, D: int = 128, device="cuda"):
    """Q [B, S, Hq, D] and K [B, S, Hkv, D] ~ N(0, 1) as float16 (seeds 9, 10)."""
    q = t_normal(9, B * S * Hq * D, 1.0, device).to(torch.float16).view(B, S, Hq, D)
    k = t_normal(10, B * S * Hkv * D, 1.0, device).to(torch.float16).view(B, S, Hkv, D)
    return q, k


def t_bf16(v):
    """Round an FP64 tensor to BF16: round the FP64 significand at BF16's last
    bit (nearest even), then convert exactly (normal-range values)."""
    b = v.view(torch.int64)
    lsb = (b >> 45) & 1
    b = (b + ((1 << 44) - 1) + lsb) & ~((1 << 45) - 1)
    return b.view(torch.float64).to(torch.float32).to(torch.bfloat16)


def t_swiglu_inputs(rows: int, cols: int, device="cuda"):
    n = rows * cols
    g = t_bf16(t_normal(SEED_X, n, 2.0, device)).view(rows, cols)
    u = t_bf16(t_normal(SEED_U, n, 2.0, device)).view(rows, cols)
    d = t_bf16(t_normal(SEED_G, n, 1.0, device)).view(rows, cols)
    return g, u, d


def t_attn_inputs(B=1, H=16, S=8192, D=128, device="cuda", Hkv=None):
    """Q [B, H, S, D], K and V [B, Hkv, S, D] (Hkv = H by default), BF16 ~ N(0, 1)."""
    Hkv = H if Hkv is None else Hkv
    q = t_bf16(t_normal(SEED_X, B * H * S * D, 1.0, device)).view(B, H, S, D)
    k, v = (t_bf16(t_normal(s, B * Hkv * S * D, 1.0, device)).view(B, Hkv, S, D)
            for s in (SEED_U, SEED_G))
    return q, k, v


def t_attn_grad(B=1, H=16, S=8192, D=128, device="cuda"):
    """Upstream gradient dO [B, H, S, D], BF16 ~ N(0, 1)."""
    return t_bf16(t_normal(SEED_DO, B * H * S * D, 1.0, device)).view(B, H, S, D)


def to_f16_bits(v: np.ndarray) -> np.ndarray:
    """Round FP64 to FP16 (numpy's conversion rounds to nearest even)."""
    return v.astype(np.float16).view(np.uint16)


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round FP64 to BF16, nearest even, directly from the FP64 bits (one
    rounding).  Values below the BF16 normal range go through FP32 first."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    b = v.view(np.uint64).copy()
    lsb = (b >> np.uint64(45)) & np.uint64(1)
    b += np.uint64((1 << 44) - 1) + lsb
    b &= ~np.uint64((1 << 45) - 1)
    r = b.view(np.float64).astype(np.float32)     # exact: <= 8 significant bits
    small = np.abs(v) < 2.0 ** -126
    if small.any():
        r[small] = v[small].astype(np.float32)
    out = (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    if small.any():
        w = r[small].view(np.uint32)
        lsb = (w >> np.uint32(16)) & np.uint32(1)
        out[small] = ((w + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    return out


# ---- workloads ---------------------------------------------------------------

def cfg1_x(n: int = 4_194_304) -> np.ndarray:
    """U(-8, 8) FP16 followed by all 65,536 FP16 bit patterns."""
    u = uniform01(SEED_X, n) * 16.0 - 8.0
    return np.concatenate([to_f16_bits(u), np.arange(65536, dtype=np.uint16)])


def cfg2_x(n: int) -> np.ndarray:
    """clip(N(0, 3), -12, 12) in FP16 (3 is the standard deviation)."""
    return to_f16_bits(np.clip(normal(SEED_X, n, 3.0), -12.0, 12.0))


def cfg2_grad(n: int) -> np.ndarray:
    return to_f16_bits(normal(SEED_G, n, 1.0))


def swiglu_inputs(rows: int, cols: int):
    """gate, up ~ N(0, 2) (sd 2) and dh ~ N(0, 1), BF16 [rows x cols]."""
    n = rows * cols
    g = to_bf16_bits(normal(SEED_X, n, 2.0)).reshape(rows, cols)
    u = to_bf16_bits(normal(SEED_U, n, 2.0)).reshape(rows, cols)
    d = to_bf16_bits(normal(SEED_G, n, 1.0)).reshape(rows, cols)
    return g, u, d


def zipf_routing(tokens: int = 16384, experts: int = 64, top_k: int = 8, s: float = 1.1):
    """Expert offsets of an expert-sorted token-copy buffer.

    Expert popularity: the expert at rank k (1-based) of a seeded permutation
    has weight k^-s.  Each token draws top_k distinct experts, one after the
    other, each with probability proportional to the weights of the experts it
    has not drawn yet.  Returns (offsets int64[experts + 1], counts)."""
    perm = np.argsort(uniform01(SEED_ROUTE, experts), kind="stable")
    w_rank = np.arange(1, experts + 1, dtype=np.float64) ** (-s)
    w = np.empty(experts)
    w[perm] = w_rank
    avail = np.ones((tokens, experts), dtype=bool)
    picks = np.empty((tokens, top_k), dtype=np.int64)
    for d in range(top_k):
        u = uniform01(SEED_ROUTE, tokens, experts + d * tokens)
        ww = np.where(avail, w[None, :], 0.0)
        cum = np.cumsum(ww, axis=1)
        target = u * cum[:, -1]
        e = np.minimum((cum <= target[:, None]).sum(axis=1), experts - 1)
        # never pick an unavailable expert (zero-width bins)
        while True:
            bad = ~avail[np.arange(tokens), e]
            if not bad.any():
                break
            e[bad] = np.minimum(e[bad] + 1, experts - 1)
        picks[:, d] = e
        avail[np.arange(tokens), e] = False
    counts = np.bincount(picks.ravel(), minlength=experts).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return offsets, counts


def attn_inputs(B: int = 1, H: int = 16, S: int = 8192, D: int = 128, Hkv: int = None):
    Hkv = H if Hkv is None else Hkv
    q = to_bf16_bits(normal(SEED_X, B * H * S * D)).reshape(B, H, S, D)
    k = to_bf16_bits(normal(SEED_U, B * Hkv * S * D)).reshape(B, Hkv, S, D)
    v = to_bf16_bits(normal(SEED_G, B * Hkv * S * D)).reshape(B, Hkv, S, D)
    return q, k, v


def attn_grad(B: int = 1, H: int = 16, S: int = 8192, D: int = 128):
    return to_bf16_bits(normal(SEED_DO, B * H * S * D)).reshape(B, H, S, D)
