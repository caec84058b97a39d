"""Seeded synthetic workloads for the quantized-attention path.

This module only draws random numbers and lays them out.  It holds none of the
method's arithmetic (no quantization, no attention): both the HIP path (tests,
bench) and the CPU oracle (tests) take their inputs from here, so the two sides
see the same bytes.

Shapes follow the Wan2.1 video-DiT self-attention workloads that the
TurboDiffusion pages accelerate (1.3B and 14B models at 480p and 720p, see the
digipub.cc TurboDiffusion article, section on end-to-end results, and the
jefxiong.cn "AIGC weekend special 5.10" digest, section 1.4).  Head count, head
dimension and token grid are fixed by the table below; the pages give no
activations, so values are drawn from the stated distributions.

Recipe per (b, h) head, one PCG64 stream each
(``SeedSequence(config_index).spawn(B*H)`` in b-major order):
  1. Q  : N x d draws (standard normal, or Student-t with nu=3 for the
          heavy-tailed workload),
  2. K  : N x d draws of the same family,
  3. K offset : d draws from a normal with variance 2 (sigma = sqrt 2),
          added to every row of K (a per-channel bias, the outlier structure
          that K smoothing removes),
  4. V  : N x d standard normal draws,
  5. the checked query rows (see ``sample_rows``).
Every value is drawn in float64, cast to float32 and rounded to bfloat16
(round to nearest even); tensors are returned as uint16 bf16 bit patterns in
[B, H, N, d] row-major order.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "gen_head", "gen_inputs", "sample_rows",
           "f32_to_bf16_bits", "bf16_bits_to_f32", "gen_block_mask"]


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int            # seed of the SeedSequence
    name: str
    B: int
    H: int
    N: int
    d: int
    q_block: int
    k_block: int
    dist: str             # "normal" or "t3" (Q and K); V is always normal
    pv: str               # "bf16" or "fp8"
    checked_rows: int     # query rows per head that the oracle checks (0 = all)

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), as a float32 value."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def nq(self) -> int:
        return -(-self.N // self.q_block)

    @property
    def nk(self) -> int:
        return -(-self.N // self.k_block)

    @property
    def ops(self) -> int:
        """Operation count of one attention pass, 4*B*H*N^2*d."""
        return 4 * self.B * self.H * self.N * self.N * self.d


WORKLOADS = [
    Workload(0, "tiny-256x64", 1, 1, 256, 64, 64, 64, "normal", "bf16", 0),
    Workload(1, "wan1.3b-480p", 1, 12, 32760, 128, 128, 64, "normal", "bf16", 1024),
    Workload(2, "wan14b-480p", 1, 40, 32760, 128, 128, 64, "normal", "bf16", 1024),
    Workload(3, "wan14b-480p-fp8", 1, 40, 32760, 128, 128, 64, "t3", "fp8", 1024),
    Workload(4, "wan14b-720p", 1, 40, 75600, 128, 128, 64, "normal", "bf16", 1024),
]


def get(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    for w in WORKLOADS:
        if w.name == name_or_index:
            return w
    raise KeyError(name_or_index)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest even (inputs finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit pattern -> float32 (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(rng: np.random.Generator, dist: str, shape) -> np.ndarray:
    if dist == "normal":
        return rng.standard_normal(shape)
    if dist == "t3":
        return rng.standard_t(3.0, shape)
    raise ValueError(dist)


def sample_rows(rng: np.random.Generator, N: int, q_block: int, count: int) -> np.ndarray:
    """Checked query rows of one head, sorted.

    All rows of the last (possibly partial) Q block are always included so the
    tail is exercised; the rest are distinct rows drawn uniformly from the
    other blocks.  ``count == 0`` or ``count >= N`` selects every row."""
    if count <= 0 or count >= N:
        return np.arange(N, dtype=np.int64)
    tail_start = ((N - 1) // q_block) * q_block
    tail = np.arange(tail_start, N, dtype=np.int64)
    rest = max(0, count - tail.size)
    rest = min(rest, tail_start)
    others = rng.choice(tail_start, size=rest, replace=False).astype(np.int64)
    return np.sort(np.concatenate([others, tail]))


def _head_rng(w: Workload, i: int) -> np.random.Generator:
    """PCG64 stream of head i = b*H + h: child i of SeedSequence(index)."""
    ss = np.random.SeedSequence(w.index)
    return np.random.Generator(np.random.PCG64(ss.spawn(i + 1)[i]))


def _draw_head(w: Workload, rng: np.random.Generator, N: int, d: int):
    q = _draw(rng, w.dist, (N, d))
    k = _draw(rng, w.dist, (N, d))
    off = rng.normal(0.0, math.sqrt(2.0), d)
    v = rng.standard_normal((N, d))
    k += off[None, :]
    rows = sample_rows(rng, N, w.q_block, w.checked_rows)
    return (f32_to_bf16_bits(q.astype(np.float32)), f32_to_bf16_bits(k.astype(np.float32)),
            f32_to_bf16_bits(v.astype(np.float32)), rows)


def gen_head(w: Workload, b: int, h: int, N: int | None = None, d: int | None = None):
    """One head's inputs: (q, k, v, rows) with q/k/v uint16 bf16 bits [N, d].

    ``N``/``d`` override the workload's sizes for small test cases while keeping
    its distributions (the stream and draw order are unchanged)."""
    N = w.N if N is None else N
    d = w.d if d is None else d
    return _draw_head(w, _head_rng(w, b * w.H + h), N, d)


def gen_inputs(w: Workload, N: int | None = None, d: int | None = None, B: int | None = None,
               H: int | None = None, workers: int | None = None):
    """All heads: (q, k, v, rows) with q/k/v uint16 [B, H, N, d] and rows a list
    indexed [b*H + h] of checked row indices.  Head i = b*H + h uses child i of
    ``SeedSequence(index)``, the same stream as ``gen_head``."""
    N = w.N if N is None else N
    d = w.d if d is None else d
    B = w.B if B is None else B
    H = w.H if H is None else H
    q = np.empty((B, H, N, d), np.uint16)
    k = np.empty_like(q)
    v = np.empty_like(q)
    rows = [None] * (B * H)
    ss = np.random.SeedSequence(w.index)
    children = ss.spawn(B * H)

    def one(i):
        b, h = divmod(i, H)
        q[b, h], k[b, h], v[b, h], rows[i] = _draw_head(
            w, np.random.Generator(np.random.PCG64(children[i])), N, d)

    if workers is None:
        workers = min(16, len(os.sched_getaffinity(0)))
    if B * H == 1 or workers <= 1:
        for i in range(B * H):
            one(i)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, range(B * H)))
    return q, k, v, rows


def add_channel_offset(x_bits: np.ndarray, sigma: float, seed: int) -> np.ndarray:
    """x + o for uint16 bf16 bits x [..., N, d]: one offset vector o ~ N(0,
    sigma^2) per head (leading index), the same for every row, rounded back
    to bf16 -- the per-channel outliers of Q that Q smoothing targets (K gets
    such an offset in every workload already)."""
    x_bits = np.asarray(x_bits, np.uint16)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    lead = x_bits.shape[:-2]
    off = g.normal(0.0, sigma, lead + (1, x_bits.shape[-1]))
    return f32_to_bf16_bits((bf16_bits_to_f32(x_bits).astype(np.float64) + off).astype(np.float32))


def gen_block_mask(B: int, H: int, N: int, density: float, seed: int, band: int = 2) -> np.ndarray:
    """A block-sparse mask uint8 [B, H, ceil(N/128), ceil(N/64)] for 128-row
    query blocks x 64-key tiles: every query block keeps the key tiles within
    `band` query-block widths of its own rows (a local window), plus each
    other tile with probability `density` (one PCG64 stream from
    SeedSequence(seed)).  The pages give no mask; this stands in for a
    selector's output (locality plus scattered long-range blocks)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    mq, nt = -(-N // 128), -(-N // 64)
    m = (g.random((B, H, mq, nt)) < density)
    qi = np.arange(mq)[:, None] * 2          # first 64-key tile of each query block
    tj = np.arange(nt)[None, :]
    m |= (np.abs(tj - qi) < 2 * band)[None, None]
    return m.astype(np.uint8)
