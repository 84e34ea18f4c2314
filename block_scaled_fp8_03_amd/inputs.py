"""Seeded synthetic inputs for the block-scaled FP8 linear.

This module only draws random numbers and arranges them; it holds none of the
method's arithmetic (no quantisation, no scaling, no GEMM), so both the GPU
library's tests and the CPU oracle can take their inputs from it.

Recipe
------
* Base seed 965 (the seed the DeepSeek-V3 generate script fixes, per the
  "DeepSeek-V3 User Guide", FAQ).  Tensor ``t`` of the workload with seed id
  ``c`` uses ``seed = 965 * 1000 + 10 * c + t``; the ids are SEED_TINY (1),
  SEED_DECODE (2), SEED_PREFILL (3), SEED_MOE (4), SEED_UE8M0 (5) and
  SEED_MLA (6).
* Normals are drawn in float32 with numpy's PCG64 (``standard_normal``),
  multiplied by the standard deviation, optionally given outliers, and then
  rounded to bfloat16 (round-to-nearest-even, torch's CPU cast).
* Outliers (decode-shaped workload): each element independently with
  probability 0.01 (a uniform draw from the same generator) is multiplied by
  50 in float32 before the bf16 rounding.
* Very large weight stacks (the 256-expert MoE) are drawn on the device with
  torch's Philox generator seeded the same way, because drawing 7.5e9 normals
  on the host would take minutes; ``normal_bf16_device`` documents this.
* MoE routing: token t picks 8 distinct experts with probabilities
  p_e proportional to (e + 1)^-1.1 (a Zipf law, expert 0 hottest), drawn by
  the Gumbel-top-k trick: argtop8(log p_e + G_te) with G standard Gumbel.
  Rows are ordered by (expert, token) and ``offsets`` are the prefix sums of
  the per-expert counts.
"""
from __future__ import annotations

import numpy as np
import torch

BASE_SEED = 965


# Seed ids of the workloads (the c of the recipe above).
SEED_TINY, SEED_DECODE, SEED_PREFILL, SEED_MOE, SEED_UE8M0, SEED_MLA = 1, 2, 3, 4, 5, 6


def seed_for(workload: int, tensor: int) -> int:
    """Seed of tensor `tensor` of the workload with seed id `workload`."""
    return BASE_SEED * 1000 + 10 * int(workload) + int(tensor)


def normal_f32(shape, std: float, seed: int, outlier_frac: float = 0.0,
               outlier_mult: float = 1.0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    x *= np.float32(std)
    if outlier_frac > 0.0:
        mask = rng.random(size=shape, dtype=np.float32) < np.float32(outlier_frac)
        x[mask] *= np.float32(outlier_mult)
    return x


def normal_bf16(shape, std: float, seed: int, outlier_frac: float = 0.0,
                outlier_mult: float = 1.0) -> torch.Tensor:
    """CPU bf16 tensor (torch) drawn by the recipe above."""
    x = normal_f32(shape, std, seed, outlier_frac, outlier_mult)
    return torch.from_numpy(x).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a CPU bf16 tensor (for the oracle)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def normal_bf16_device(shape, std: float, seed: int, device) -> torch.Tensor:
    """bf16 normals drawn on ``device`` with torch's generator for that device."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, dtype=torch.float32, device=device, generator=g)
    x.mul_(std)
    return x.to(torch.bfloat16)


def zipf_topk_routing(tokens: int, experts: int, topk: int, s: float, seed: int):
    """Synthetic top-k expert routing, Zipf(s) over experts, no repeats per token.

    Returns dict with
      ``choice``  int64 [tokens, topk]  experts picked by each token,
      ``token``   int64 [tokens*topk]   token of each grouped row,
      ``offsets`` int32 [experts+1]     row range of each expert,
      ``counts``  int64 [experts].
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    logp = -s * np.log(np.arange(1, experts + 1, dtype=np.float64))
    g = rng.gumbel(size=(tokens, experts))
    choice = np.argsort(-(logp[None, :] + g), axis=1, kind="stable")[:, :topk]
    flat_e = choice.reshape(-1)
    flat_t = np.repeat(np.arange(tokens, dtype=np.int64), topk)
    order = np.lexsort((flat_t, flat_e))           # by expert, then token
    counts = np.bincount(flat_e, minlength=experts).astype(np.int64)
    offsets = np.zeros(experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return {"choice": choice.astype(np.int64), "token": flat_t[order], "offsets": offsets,
            "counts": counts}


def routing_weights(tokens: int, topk: int, seed: int) -> np.ndarray:
    """Synthetic routing weights float32 [tokens, topk]: uniform(0.05, 1)
    draws normalised to sum 1 per token (a stand-in for the gate's normalised
    scores, which the expert combine multiplies each expert output by)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    w = rng.uniform(0.05, 1.0, (tokens, topk))
    return (w / w.sum(axis=1, keepdims=True)).astype(np.float32)


# Workload shapes (rows of the hot-path scope table).  M, N, K follow
# nn.Linear: x [M, K], W [N, K] (out x in).
TINY = dict(name="tiny fp8 linear", seed_id=SEED_TINY, M=16, N=256, K=256, x_std=1.0, w_std=0.02,
            fmt="fp32")
DECODE = dict(name="decode weight-streaming fp8 linear", seed_id=SEED_DECODE, M=32, N=18432, K=7168,
              x_std=1.0, w_std=0.02, outlier_frac=0.01, outlier_mult=50.0, fmt="fp32")
PREFILL = dict(name="prefill fp8 linear (up and down)", seed_id=SEED_PREFILL, M=4096, N=18432, K=7168,
               x_std=1.0, w_std=0.02, down=dict(M=4096, N=7168, K=18432), fmt="fp32")
MOE = dict(name="grouped MoE expert GEMM", seed_id=SEED_MOE, tokens=4096, experts=256, topk=8,
           zipf_s=1.1, up=dict(N=2048, K=7168), down=dict(N=7168, K=2048), x_std=1.0, w_std=0.02,
           fmt="fp32")
UE8M0 = dict(name="ue8m0 act_quant, weight_dequant, small-N and small-K GEMMs", seed_id=SEED_UE8M0,
             M=1024, K=7168, dequant=dict(N=18432, K=7168),
             gemms=[dict(N=1536, K=7168), dict(N=16384, K=512)], x_std=1.0, w_std=0.02, fmt="ue8m0")

# The MLA absorb products (seed id SEED_MLA): the attention
# shape the pages' configurations share (qk_nope_head_dim 128, v_head_dim 128,
# kv_lora_rank 512) with the 671B model's 128 heads, wkv_b drawn like the other
# weights (std 0.02) and N(0, 1) activations, at a decode batch of 32 tokens and
# a 4096-token prefill.
MLA = dict(name="MLA absorb with an FP8 wkv_b", heads=128, dn=128, dv=128, R=512,
           decode_tokens=32, prefill_tokens=4096, x_std=1.0, w_std=0.02, seed_id=SEED_MLA)
