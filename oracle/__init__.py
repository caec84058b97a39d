"""CPU oracle of the low-bit quantized attention step.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check of
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import or
run anything in this package.  It shares no code with the HIP path: it is a
plain, slow, obviously correct implementation written from the method's
definition (numpy, exact integer arithmetic for every quantization decision,
float64 for attention).

What it computes, per (b, h) head, following the quantized attention step that
TurboDiffusion uses (SageAttention2++: jefxiong.cn "AIGC weekend special 5.10",
section 1.2 item (1); digipub.cc TurboDiffusion article, attention-acceleration
paragraph; GVCLab research log 2026-09-02, section 5.5 table):

  quant.kmean_exact      per-channel K mean, exact sum rounded once
  quant.quantize_q       per-block INT8 codes + scales of Q
  quant.quantize_q_smoothed  the same after removing each block's mean (Q
                         smoothing, optional; the mean returns as a logit bias)
  quant.quantize_k       K smoothed by its mean, then per-block INT8
  quant.quantize_v_fp8   per-block E4M3 codes + scales of V (FP8 path)
  attention.attend_bf16  logits from the integer codes, exact softmax, P.V
  attention.attend_fp8   the same with the kernel's online FP8 P rounding
                         mirrored, plus an ambiguity envelope
  (both take an optional block mask: block-sparse attention over
  128-row x 64-key blocks)

and, for the W8A8 linear layers on either side of attention (jefxiong.cn
"AIGC weekend special 5.10", section 1.2 item (4); digipub.cc TurboDiffusion
article, linear-layer quantization paragraph):

  w8a8.quantize_blocks   INT8 codes + one scale per 128x128 block
  w8a8.linear            y = x W^T (+ b) from the block codes and scales
  norm.rmsnorm_quantize  RMSNorm (exact mean square, binary32 steps) fused
                         with that block quantization

Pins (what ties these functions to something other than themselves) live in
``tests/test_oracle_*.py``.  The end-to-end output against the pages is
"parity unpinned": the pages print no numerical example of the attention
step; the quantized-vs-exact gap is reported as a diagnostic only.
"""
from __future__ import annotations

from . import attention, fp, norm, quant, w8a8  # noqa: F401

__all__ = ["attention", "fp", "norm", "quant", "w8a8", "forward_head"]


def forward_head(q_bits, k_bits, v_bits, rows, q_block, k_block, scale, pv="bf16",
                 v_block=64, kv_tile=64, block_mask=None, smooth_q=False):
    """Run every step for one head; returns a dict of all intermediate results.

    q_bits/k_bits/v_bits: uint16 bf16 bits [N, d]; rows: checked query rows;
    block_mask: optional [ceil(N/128), ceil(N/64)] block-sparse mask;
    smooth_q: Q smoothing per Q block (quant.quantize_q_smoothed)."""
    qm = ks_ = None
    if smooth_q:
        qc, qs, qm = quant.quantize_q_smoothed(q_bits, q_block)
    else:
        qc, qs = quant.quantize_q(q_bits, q_block)
    kc, ks, mu = quant.quantize_k(k_bits, k_block)
    res = {"q_codes": qc, "q_scale": qs, "k_codes": kc, "k_scale": ks, "k_mean": mu}
    if smooth_q:
        ks_ = quant.smooth_k(k_bits, mu)
        res["q_mean"] = qm
    if pv == "bf16":
        res["out"] = attention.attend_bf16(qc, qs, kc, ks, v_bits, rows, q_block, k_block, scale,
                                           block_mask=block_mask, q_mean=qm, k_smooth=ks_)
        res["envelope"] = None
    elif pv == "fp8":
        vc, vs = quant.quantize_v_fp8(v_bits, v_block)
        res["v_codes"], res["v_scale"] = vc, vs
        o, e, hits = attention.attend_fp8(qc, qs, kc, ks, vc, vs, rows, q_block, k_block, scale,
                                          v_block=v_block, kv_tile=kv_tile, block_mask=block_mask,
                                          q_mean=qm, k_smooth=ks_)
        res["out"], res["envelope"], res["envelope_hits"] = o, e, hits
    else:
        raise ValueError(pv)
    return res
