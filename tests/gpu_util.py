"""Helpers of the GPU parity tests: device upload of the seeded inputs, the
oracle run over heads (threaded), and the comparison metrics."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import workloads as W

MAX_ABS = 1e-2
MIN_COS = 0.9999


def dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def oracle_heads(q, k, v, rows, q_block, scale, pv, heads=None, workers=None, smooth_q=False):
    """forward_head over the (b, h) heads; returns a list indexed by b*H + h."""
    B, H = q.shape[:2]
    idx = list(range(B * H)) if heads is None else list(heads)
    workers = workers or min(16, len(os.sched_getaffinity(0)))

    def one(i):
        b, h = divmod(i, H)
        return oracle.forward_head(q[b, h], k[b, h], v[b, h], rows[i], q_block, 64, scale, pv=pv,
                                   smooth_q=smooth_q)

    res = [None] * (B * H)
    with ThreadPoolExecutor(workers) as ex:
        for n, (i, r) in enumerate(zip(idx, ex.map(one, idx))):
            res[i] = r
            if len(idx) >= 8 and (n + 1) % 4 == 0:
                print(f"  oracle: {n + 1}/{len(idx)} heads", flush=True)
    return res


# FP8 P.V: the fraction of checked output elements' P operands that fall in the
# ambiguity band may not exceed this (heavy-tailed 14B-shaped data: ~7e-5)
MAX_ENV_HIT_FRAC = 1e-3


def check_fp8(m: dict, hits: int, elements: int, bound_hits: bool = True):
    """FP8 P.V bar: beyond the envelope-aware excess, the raw max-abs error
    itself is <= MAX_ABS, and (on workload-shaped data; crafted extreme logits
    widen the band by construction) ambiguous P elements stay rare."""
    frac = hits / max(elements, 1)
    print(f"  fp8: raw max_abs={m['max_abs']:.3e} envelope hits={hits} ({frac:.2e} of {elements} "
          f"P elements) env_max={m['env_max']:.2e}", flush=True)
    assert m["max_abs"] <= MAX_ABS, m
    if bound_hits:
        assert frac <= MAX_ENV_HIT_FRAC, (hits, elements)


def out_metrics(gpu_rows: list, ref_rows: list, env_rows: list | None = None):
    g = np.concatenate([x.reshape(-1) for x in gpu_rows]).astype(np.float64)
    r = np.concatenate([x.reshape(-1) for x in ref_rows]).astype(np.float64)
    err = np.abs(g - r)
    if env_rows is not None and all(e is not None for e in env_rows):
        env = np.concatenate([e.reshape(-1) for e in env_rows])
    else:
        env = np.zeros_like(err)
    cos = float(g @ r / (np.linalg.norm(g) * np.linalg.norm(r)))
    return {"max_abs": float(err.max()), "max_excess": float((err - env).max()), "cos": cos,
            "env_max": float(env.max())}
