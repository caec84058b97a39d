"""Seeded synthetic inputs of the W8A8 linear layers around attention.

Like the attention workloads, this module only draws random numbers and lays
them out (no quantization, no products).  The layers are the projections on
either side of the attention step of a Wan2.1 video-DiT block: the fused Q/K/V
projection (in-features H*d, out-features 3*H*d) and the output projection
(H*d -> H*d), over the same token counts as the attention workloads
(21x30x52 = 32760 tokens at 480p).  H and d are those of the attention
workloads (12 x 128 for 1.3B, 40 x 128 for 14B).

Recipe (the pages give no activations or weights, so values are drawn):
  * x [M, K]: standard normal, drawn 128 rows at a time; row block i uses
    child i of SeedSequence([index, 0]) (PCG64),
  * W [N, K]: normal with standard deviation 1/sqrt(K) (so y = x W^T has unit
    variance), 128 rows at a time from the children of SeedSequence([index, 1]),
  * b [N]: standard normal from SeedSequence([index, 2]) (when the workload has
    a bias),
  * the checked row blocks of x: the last (possibly partial) one and
    `checked_row_blocks - 1` others drawn from SeedSequence([index, 3]).
Every value is drawn in float64, cast to float32 and rounded to bfloat16 (x and
W, as uint16 bit patterns) or kept in float32 (b).  Drawing per 128-row block
lets a check regenerate just the blocks it needs.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import f32_to_bf16_bits

__all__ = ["LinearWorkload", "LINEAR_WORKLOADS", "get_linear", "gen_x_blocks", "gen_w_blocks",
           "gen_bias", "gen_x", "gen_w", "checked_row_blocks"]

ROWS = 128


@dataclasses.dataclass(frozen=True)
class LinearWorkload:
    index: int               # seed
    name: str
    M: int                   # tokens
    K: int                   # in-features
    N: int                   # out-features
    bias: bool
    checked_row_blocks: int  # row blocks of x the oracle checks (0 = all)

    @property
    def ops(self) -> int:
        """Operation count of one product, 2*M*N*K."""
        return 2 * self.M * self.N * self.K

    @property
    def mb(self) -> int:
        return -(-self.M // ROWS)


LINEAR_WORKLOADS = [
    LinearWorkload(100, "w8a8-tiny", 300, 384, 200, True, 0),
    LinearWorkload(101, "w8a8-qkv-wan1.3b-480p", 32760, 1536, 4608, True, 4),
    LinearWorkload(102, "w8a8-qkv-wan14b-480p", 32760, 5120, 15360, True, 4),
    LinearWorkload(103, "w8a8-out-wan14b-480p", 32760, 5120, 5120, True, 4),
]


def get_linear(name: str) -> LinearWorkload:
    for w in LINEAR_WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def _rows(total: int, i: int) -> int:
    return min(ROWS, total - i * ROWS)


def _gen_blocks(index, which, total, K, sigma, blocks, workers):
    blocks = list(blocks)
    out = np.empty((sum(_rows(total, i) for i in blocks), K), np.uint16)
    starts = np.cumsum([0] + [_rows(total, i) for i in blocks])
    ss = np.random.SeedSequence([index, which])
    children = ss.spawn(max(blocks) + 1) if blocks else []

    def one(t):
        i = blocks[t]
        g = np.random.Generator(np.random.PCG64(children[i]))
        v = g.standard_normal((_rows(total, i), K))
        if sigma != 1.0:
            v *= sigma
        out[starts[t]:starts[t + 1]] = f32_to_bf16_bits(v.astype(np.float32))

    if workers is None:
        workers = min(16, len(os.sched_getaffinity(0)))
    if len(blocks) <= 1 or workers <= 1:
        for t in range(len(blocks)):
            one(t)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, range(len(blocks))))
    return out


def gen_x_blocks(w: LinearWorkload, blocks, workers=None) -> np.ndarray:
    """Rows of x in the given 128-row blocks (in the order given), uint16 bf16 bits."""
    return _gen_blocks(w.index, 0, w.M, w.K, 1.0, blocks, workers)


def gen_w_blocks(w: LinearWorkload, blocks, workers=None) -> np.ndarray:
    """Rows of W in the given 128-row blocks, uint16 bf16 bits."""
    return _gen_blocks(w.index, 1, w.N, w.K, 1.0 / math.sqrt(w.K), blocks, workers)


def gen_x(w: LinearWorkload, workers=None) -> np.ndarray:
    """x [M, K] as uint16 bf16 bits."""
    return gen_x_blocks(w, range(-(-w.M // ROWS)), workers)


def gen_w(w: LinearWorkload, workers=None) -> np.ndarray:
    """W [N, K] as uint16 bf16 bits."""
    return gen_w_blocks(w, range(-(-w.N // ROWS)), workers)


def gen_bias(w: LinearWorkload):
    """b [N] float32, or None."""
    if not w.bias:
        return None
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.index, 2])))
    return g.standard_normal(w.N).astype(np.float32)


def checked_row_blocks(w: LinearWorkload) -> np.ndarray:
    """Row blocks of x whose outputs the oracle checks, sorted; always
    includes the last (possibly partial) block."""
    mb = w.mb
    if w.checked_row_blocks <= 0 or w.checked_row_blocks >= mb:
        return np.arange(mb, dtype=np.int64)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.index, 3])))
    others = g.choice(mb - 1, size=w.checked_row_blocks - 1, replace=False)
    return np.sort(np.concatenate([others, [mb - 1]])).astype(np.int64)
