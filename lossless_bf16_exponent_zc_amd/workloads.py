"""Seeded synthetic BF16 workloads (inputs only -- none of the codec's math).

The pages evaluate on real training traffic that is not available here
(Qwen3 all-to-all tensors, DeepSeek-V3 / Qwen3-MoE / Llama3-8B runs).  Their
own data model is that LLM communication tensors are near-Gaussian or
log-normal (ZipCCL, "Introduction"), so these generators draw such tensors
with the shapes of the evaluated collectives:

* ``small``     -- 1,048,576 values ~ N(0, 0.02^2)
* ``gradient``  -- 67,108,864 gradient-like values: N(0, 1e-3^2), 1% outliers
                   x100, 0.5% exact zeros, 0.01% subnormals
* ``llama_mlp`` -- the three Llama3-8B MLP weight matrices, N(0, 0.02^2)
                   times a per-row LogNormal(0, 0.3) scale
* ``moe``       -- MoE all-to-all activations: 256 expert segments with
                   Zipf(1.2) token counts summing to 65,536 tokens, hidden
                   7168, N(0, 1) times a per-token LogNormal(0, 0.5) scale
* ``shards``    -- 8 reduce-scatter shards of 33,554,432 values ~ N(0, 1e-3^2)
* ``gaussian_device`` -- N(0, scale^2) of any size drawn on the GPU (for the
                   largest segment a plan accepts, 2^32 - 1 values)
* ``mixed``     -- a seeded mix for randomized tests: Gaussian of a random
                   binade of scale with zeros, subnormals, Inf and NaN
                   injected, or uniform bit patterns

Every draw uses ``torch.Generator(device="cpu")`` with a fixed seed, in fp32,
in the order written below, then rounds to BF16 (nearest even).  The result is
handed out as uint16 bit patterns, so the CPU oracle and the GPU library see
identical bits.  Each generator takes size arguments so tests can draw the
same distribution at a smaller scale.
"""
from __future__ import annotations

import numpy as np
import torch

CHUNK = 65536


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def to_bits(t: torch.Tensor) -> np.ndarray:
    """fp32 tensor -> BF16 (round to nearest even) -> flat uint16 bits."""
    b = t.to(torch.bfloat16).contiguous().view(torch.int16)
    return b.reshape(-1).numpy().view(np.uint16)


def small(n: int = 1 << 20, seed: int = 0) -> np.ndarray:
    g = _gen(seed)
    return to_bits(torch.randn(n, generator=g) * 0.02)


def gradient(n: int = 1 << 26, seed: int = 0) -> np.ndarray:
    """Draw order: z = randn(n); u = rand(n); then, for the subnormal slots in
    index order, a sign randint(0, 2) and a mantissa randint(1, 128)."""
    g = _gen(seed)
    z = torch.randn(n, generator=g) * 1e-3
    u = torch.rand(n, generator=g)
    z = torch.where(u < 0.01, z * 100.0, z)
    bits = to_bits(z)
    zero = ((u >= 0.01) & (u < 0.015)).numpy()
    sub = ((u >= 0.015) & (u < 0.0151)).numpy()
    nsub = int(sub.sum())
    sign = torch.randint(0, 2, (nsub,), generator=g).numpy().astype(np.uint16)
    mant = torch.randint(1, 128, (nsub,), generator=g).numpy().astype(np.uint16)
    bits[zero] = 0
    bits[sub] = (sign << 15) | mant
    return bits


LLAMA_MLP_SHAPES = ((4096, 14336), (14336, 4096), (4096, 14336))


def llama_mlp(shapes=LLAMA_MLP_SHAPES, seeds=(0, 1, 2)) -> list[np.ndarray]:
    """One matrix per seed.  Draw order: z = randn(r, c), then the row scale
    exp(0.3 * randn(r, 1)); entries are 0.02 * z * scale, row-major."""
    out = []
    for (r, c), s in zip(shapes, seeds):
        g = _gen(s)
        z = torch.randn(r, c, generator=g)
        scale = torch.exp(0.3 * torch.randn(r, 1, generator=g))
        out.append(to_bits(z * 0.02 * scale))
    return out


def zipf_counts(total: int = 65536, experts: int = 256,
                s: float = 1.2) -> list[int]:
    """Deterministic Zipf(s) split of `total` tokens over `experts` ranks:
    w_r proportional to r^-s, floor of the proportional share, then the
    remaining tokens one each by largest fractional part (ties to the lower
    rank).  Segment i is rank i + 1."""
    r = np.arange(1, experts + 1, dtype=np.float64)
    w = r ** (-s)
    share = total * w / w.sum()
    base = np.floor(share).astype(np.int64)
    left = total - int(base.sum())
    frac = share - base
    order = sorted(range(experts), key=lambda i: (-frac[i], i))
    for i in order[:left]:
        base[i] += 1
    return [int(v) for v in base]


def moe(tokens: int = 65536, hidden: int = 7168, experts: int = 256,
        seed: int = 0, device: str = "cpu"):
    """Returns (flat bits, per-segment value counts).  Draw order:
    z = randn(tokens, hidden), then the token scale exp(0.5 * randn(tokens, 1)).
    Rows are grouped into contiguous expert segments by ``zipf_counts``.
    device="cuda" draws the same recipe with torch's CUDA generator (seeded
    the same way; other values, same distribution), which is much faster for
    the full 469,762,048-value tensor."""
    if device == "cpu":
        g = _gen(seed)
    else:
        g = torch.Generator(device=device)
        g.manual_seed(seed)
    z = torch.randn(tokens, hidden, generator=g, device=device)
    scale = torch.exp(0.5 * torch.randn(tokens, 1, generator=g, device=device))
    bits = to_bits((z * scale).cpu() if device != "cpu" else z * scale)
    counts = zipf_counts(tokens, experts)
    return bits, [c * hidden for c in counts]


def shards(n: int = 1 << 25, nshards: int = 8) -> list[np.ndarray]:
    """Shard s uses seed s: randn(n) * 1e-3."""
    return [to_bits(torch.randn(n, generator=_gen(s)) * 1e-3)
            for s in range(nshards)]


def gaussian_device(n: int, seed: int = 0, scale: float = 1e-3, device: str = "cuda"):
    """randn(n) * scale drawn with torch's generator on `device` (seeded),
    rounded to BF16 there; returns the bits as a device int16 tensor."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    z = torch.randn(n, generator=g, device=device)
    z.mul_(scale)
    bits = z.to(torch.bfloat16).view(torch.int16)
    del z
    return bits


def mixed(n: int, seed: int) -> np.ndarray:
    """One of four kinds, drawn from `seed`: plain Gaussian times 2^k
    (k in -30..29); the same with about 1% of the positions replaced by
    specials (+-0, subnormals, +-Inf, NaNs with payloads); the same with about
    30% replaced; or uniform 16-bit patterns."""
    rng = np.random.default_rng(seed)
    kind = int(rng.integers(0, 4))
    if kind == 3:
        return rng.integers(0, 65536, n, dtype=np.uint16)
    scale = float(2.0 ** int(rng.integers(-30, 30)))
    z = torch.from_numpy((rng.standard_normal(n) * scale).astype(np.float32))
    bits = to_bits(z).copy()
    if kind > 0 and n:
        specials = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x0040, 0x7F80, 0xFF80,
                             0x7FC0, 0x7F81, 0xFFFF], dtype=np.uint16)
        frac = 0.01 if kind == 1 else 0.3
        pos = rng.random(n) < frac
        bits[pos] = specials[rng.integers(0, specials.size, int(pos.sum()))]
    return bits
