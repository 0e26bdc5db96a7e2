"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws inputs; it holds none of the quantization arithmetic.
Randomness is SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014) evaluated at a counter, so any slice of a stream
can be produced on its own, on the CPU or the GPU.  Values are drawn in float64,
rounded to float32 and then to bfloat16 (nearest-even, torch's conversion).

The workloads stand in for the activations the pages quantize (MoE expert inputs
in the TransformerEngine grouped NVFP4 PR; DeepSeek-V3.2 indexer Q/K heads in the
TensorRT-LLM DSA PR), which need model weights that are not available here.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

_GOLDEN = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB
_MASK64 = (1 << 64) - 1


def _to_i64(u: int) -> int:
    u &= _MASK64
    return u - (1 << 64) if u >= (1 << 63) else u


def _srl(z: torch.Tensor, k: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (z >> k) & ((1 << (64 - k)) - 1)


def splitmix64(seed: int, start: int, n: int, device="cpu") -> torch.Tensor:
    """Outputs start..start+n-1 of the SplitMix64 stream of `seed` (int64 bit patterns)."""
    i = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    z = i * _to_i64(_GOLDEN) + _to_i64(seed)
    z = (z ^ _srl(z, 30)) * _to_i64(_MIX1)
    z = (z ^ _srl(z, 27)) * _to_i64(_MIX2)
    return z ^ _srl(z, 31)


def _stream_seed(seed: int, stream: int) -> int:
    """A separate SplitMix64 seed per (seed, stream) pair."""
    z = (seed * 0x100000001B3 + stream * _GOLDEN + 0x632BE59BD9B4E019) & _MASK64
    z = ((z ^ (z >> 30)) * _MIX1) & _MASK64
    z = ((z ^ (z >> 27)) * _MIX2) & _MASK64
    return z ^ (z >> 31)


def uniform(seed: int, stream: int, n: int, device="cpu", start: int = 0) -> torch.Tensor:
    """float64 uniforms in [0, 1) with 53 random bits."""
    z = splitmix64(_stream_seed(seed, stream), start, n, device)
    return _srl(z, 11).to(torch.float64) * (2.0 ** -53)


def normal(seed: int, stream: int, n: int, device="cpu") -> torch.Tensor:
    """Standard normals by Box-Muller from pairs of uniforms."""
    half = (n + 1) // 2
    u = uniform(seed, stream, 2 * half, device).view(half, 2)
    u1 = 1.0 - u[:, 0]                    # (0, 1]
    rad = torch.sqrt(-2.0 * torch.log(u1))
    ang = 2.0 * math.pi * u[:, 1]
    z = torch.stack([rad * torch.cos(ang), rad * torch.sin(ang)], dim=1).reshape(-1)
    return z[:n]


def student_t3(seed: int, stream: int, n: int, device="cpu", chunk: int = 1 << 26) -> torch.Tensor:
    """Student-t with 3 degrees of freedom: z0 / sqrt((z1^2 + z2^2 + z3^2) / 3)."""
    out = torch.empty(n, dtype=torch.float64, device=device)
    for c0 in range(0, n, chunk):
        m = min(chunk, n - c0)
        z = torch.stack([_normal_slice(seed, stream, j, c0, m, device) for j in range(4)])
        out[c0:c0 + m] = z[0] / torch.sqrt((z[1] ** 2 + z[2] ** 2 + z[3] ** 2) / 3.0)
    return out


def _normal_slice(seed, stream, j, start, m, device):
    """Normals start..start+m-1 of sub-stream j (Box-Muller on an aligned pair range)."""
    s0 = start - (start % 2)
    cnt = (start + m) - s0
    cnt += cnt % 2
    u = uniform(seed, stream * 16 + j + 1, cnt, device, start=s0).view(-1, 2)
    rad = torch.sqrt(-2.0 * torch.log(1.0 - u[:, 0]))
    ang = 2.0 * math.pi * u[:, 1]
    z = torch.stack([rad * torch.cos(ang), rad * torch.sin(ang)], dim=1).reshape(-1)
    return z[start - s0:start - s0 + m]


def to_bf16(v64: torch.Tensor) -> torch.Tensor:
    """float64 -> float32 -> bfloat16, each nearest-even."""
    return v64.to(torch.float32).to(torch.bfloat16)


class Rng:
    """Small host-side SplitMix64 for structural choices (cut points, masks, channels)."""

    def __init__(self, seed: int):
        self.state = seed & _MASK64

    def next(self) -> int:
        self.state = (self.state + _GOLDEN) & _MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * _MIX1) & _MASK64
        z = ((z ^ (z >> 27)) * _MIX2) & _MASK64
        return z ^ (z >> 31)

    def below(self, n: int) -> int:
        return self.next() % n

    def sample_distinct(self, lo: int, hi: int, count: int) -> list:
        """count distinct integers in [lo, hi], sorted."""
        pool = list(range(lo, hi + 1))
        for i in range(count):
            j = i + self.below(len(pool) - i)
            pool[i], pool[j] = pool[j], pool[i]
        return sorted(pool[:count])


def _sections_from_cuts(units: int, cuts: list, unit_rows: int) -> list:
    pts = [0] + sorted(cuts) + [units]
    return [(pts[i + 1] - pts[i]) * unit_rows for i in range(len(pts) - 1)]


def split_distinct(rng: Rng, units: int, parts: int, unit_rows: int = 128) -> list:
    """`parts` non-empty sections: parts-1 distinct cut points in 1..units-1."""
    if not 1 <= parts <= units:
        raise ValueError(f"cannot cut {units} units into {parts} non-empty sections")
    return _sections_from_cuts(units, rng.sample_distinct(1, units - 1, parts - 1), unit_rows)


def split_with_empties(rng: Rng, units: int, parts: int, forced_empty: int,
                       unit_rows: int = 128) -> list:
    """`parts` sections, `forced_empty` of them chosen empty; the units go to the
    others through cut points drawn with replacement from 0..units (more empty
    sections are possible)."""
    empty = set(rng.sample_distinct(0, parts - 1, forced_empty))
    live = parts - forced_empty
    cuts = [rng.below(units + 1) for _ in range(live - 1)]
    sizes = iter(_sections_from_cuts(units, cuts, unit_rows))
    return [0 if s in empty else next(sizes) for s in range(parts)]


# ---------------------------------------------------------------------------
# The five workloads.  Each takes optional size overrides so the same recipe can
# be drawn at a size the oracle finishes in seconds.
# ---------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    tensors: dict
    params: dict = field(default_factory=dict)


def plain_fp8(m=256, k=1024, seed=1, device="cpu") -> Workload:
    """Plain FP8 1x128 quantization of one N(0,1) BF16 tensor [m][k]."""
    x = to_bf16(normal(seed, 0, m * k, device)).view(m, k)
    return Workload("fp8_1x128", {"x": x}, {"m": m, "k": k})


def swiglu_fp8(tokens=16384, n=4096, seed=6, device="cpu") -> Workload:
    """Fused SwiGLU input of a W8A8 MoE expert: one BF16 [tokens][2n] buffer, gate in
    the first half (N(0,1) * 2) and up in the second (N(0,1))."""
    gate = normal(seed, 0, tokens * n, device).view(tokens, n) * 2.0
    up = normal(seed, 1, tokens * n, device).view(tokens, n)
    gu = torch.cat([to_bf16(gate), to_bf16(up)], dim=1).contiguous()
    return Workload("swiglu_fp8", {"gate_up": gu}, {"tokens": tokens, "n": n})


def dsa_rotate_fp8(tokens=4096, heads=64, d_pe=64, seed=2, outlier_frac=0.02,
                   outlier_scale=20.0, device="cpu") -> Workload:
    """DSA-indexer Q: [tokens*heads] rows of cat[qk_pe(d_pe), qk_nope(128-d_pe)],
    N(0,1) with a seeded 2% of the (head, dim) channels scaled by 20."""
    rows = tokens * heads
    v = normal(seed, 0, rows * 128, device).view(tokens, heads, 128)
    rng = Rng(seed)
    n_out = round(outlier_frac * heads * 128)
    chans = rng.sample_distinct(0, heads * 128 - 1, n_out)
    scale = torch.ones(heads * 128, dtype=torch.float64, device=device)
    scale[torch.tensor(chans, dtype=torch.int64, device=device)] = outlier_scale
    v = v * scale.view(1, heads, 128)
    v = to_bf16(v).view(rows, 128)
    pe = v[:, :d_pe].contiguous()
    nope = v[:, d_pe:].contiguous()
    return Workload("dsa_rotate_fp8", {"pe": pe, "nope": nope},
                    {"rows": rows, "d_pe": d_pe, "outlier_channels": chans})


def grouped_nvfp4(total_rows=16384, k=4096, parts=8, seed=3, device="cpu") -> Workload:
    """Grouped NVFP4 with RHT: N(0,1) x, `parts` non-empty 128-aligned sections
    cut at distinct seeded points, a seeded 16-bit sign mask, RNE."""
    units = total_rows // 128
    rng = Rng(seed)
    sections = split_distinct(rng, units, parts)
    mask = rng.below(1 << 16)
    x = to_bf16(normal(seed, 0, total_rows * k, device)).view(total_rows, k)
    return Workload("grouped_nvfp4_rht", {"x": x},
                    {"split_sections": sections, "sign_mask": mask, "flags": 3,
                     "seed": None, "row_offsets": None, "col_offsets": None})


def grouped_nvfp4_sr(total_rows=16384, k=4096, parts=32, forced_empty=4, seed=4,
                     device="cpu") -> Workload:
    """As grouped_nvfp4 with 32 sections (some empty) and stochastic rounding in
    both directions: Philox keyed by a seed with distinct per-section offsets."""
    units = total_rows // 128
    rng = Rng(seed)
    sections = split_with_empties(rng, units, parts, forced_empty)
    mask = rng.below(1 << 16)
    sr_seed = rng.next()
    row_off = [rng.next() for _ in range(parts)]
    col_off = [rng.next() for _ in range(parts)]
    x = to_bf16(normal(seed, 0, total_rows * k, device)).view(total_rows, k)
    return Workload("grouped_nvfp4_rht_sr", {"x": x},
                    {"split_sections": sections, "sign_mask": mask, "flags": 3,
                     "seed": sr_seed, "row_offsets": row_off, "col_offsets": col_off})


def large_moe(total_rows=65536, k=7168, parts=32, forced_empty=3, seed=5,
              outlier_frac=0.01, outlier_scale=100.0, zero_block_p=0.005,
              device="cpu") -> Workload:
    """Large MoE activations: Student-t(3) x with a seeded 1% of channels x100 and
    each row-wise 1x16 block set to +0 with probability 0.005; 32 sections (some
    empty); NVFP4 row + column and FP8 1x128 row-wise in one call."""
    units = total_rows // 128
    rng = Rng(seed)
    sections = split_with_empties(rng, units, parts, forced_empty)
    mask = rng.below(1 << 16)
    n_out = round(outlier_frac * k)
    chans = rng.sample_distinct(0, k - 1, n_out)
    v = student_t3(seed, 0, total_rows * k, device).view(total_rows, k)
    scale = torch.ones(k, dtype=torch.float64, device=device)
    scale[torch.tensor(chans, dtype=torch.int64, device=device)] = outlier_scale
    v.mul_(scale.view(1, k))
    zb = uniform(seed, 99, total_rows * (k // 16), device).view(total_rows, k // 16) < zero_block_p
    v.view(total_rows, k // 16, 16).masked_fill_(zb.unsqueeze(-1), 0.0)
    x = to_bf16(v)
    del v
    return Workload("large_moe_nvfp4_fp8", {"x": x},
                    {"split_sections": sections, "sign_mask": mask, "flags": 7,
                     "seed": None, "row_offsets": None, "col_offsets": None,
                     "outlier_channels": chans})
