"""GPU parity of the BF16 path of the linear (gemm_impl "bf16": the FP8 weight
dequantised as weight_dequant does, then a bf16 GEMM) against the CPU oracle,
through the C ABI.  The kernel multiplies exact bf16 products and accumulates
in float32 (one fp32 addition per 32-wide MFMA step), so the bar is derived
from that: |gpu - ref| <= 2^-13 * S on the float32 output, S = sum_k |x w|,
plus 2^-8 |ref| for the bf16 store."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_03_amd as fp8bs
import oracle
from block_scaled_fp8_03_amd import inputs
from gpu_util import DEV, to_dev_f32, to_dev_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()


def operands(M, N, K, seed, w_std=0.02):
    x = inputs.normal_bf16((M, K), 1.0, seed)
    q, s = oracle.weight_quant(inputs.bf16_bits(inputs.normal_bf16((N, K), w_std, seed + 1)))
    return x, q, s


def run(x, q, s, dt):
    c = fp8bs.w8a16_gemm(x.to(DEV), to_dev_u8(q), to_dev_f32(s), dt)
    torch.cuda.synchronize()
    return c.float().cpu().numpy().astype(np.float64)


def check(got, ref, S, bf16, what):
    bar = 2.0 ** -13 * S + (2.0 ** -8 * np.abs(ref) if bf16 else 0.0) + 1e-30
    bad = np.abs(got - ref) > bar
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside, first {np.argwhere(bad)[:4].tolist()}"


@pytest.mark.parametrize("M,N,K", [
    (1, 1, 128), (16, 256, 256), (32, 200, 384),          # decode sizes, N <= 4096: split-K kernel
    (1, 1536, 7168), (17, 576, 2048), (32, 4096, 640),    # split-K: 56 / 16 / 5 K blocks
    (20, 4500, 384),                                      # decode sizes, N > 4096: streaming kernel
    (48, 300, 384), (64, 129, 256),                       # 64-row decode tiles
    (65, 200, 384), (257, 129, 256), (300, 520, 1024), (513, 300, 640),   # 64-row tiles (few 128 x 128)
    (100, 18000, 256),                                    # 128 x 128 tiles, one per CU (141)
    (500, 4000, 640),                                     # 64-row tiles in one round (512)
    (2050, 8200, 256),                                    # 256 x 256 tiles, ragged M and N
    (300, 12000, 640),                                    # 128 x 128, two per CU (282 tiles)
    (520, 14000, 256),                                    # 256 x 256 tiles, one partial round
])
def test_w8a16_small(M, N, K):
    x, q, s = operands(M, N, K, 7000 + M + N + K)
    xb = inputs.bf16_bits(x)
    ref = oracle.w8a16_gemm(xb, q, s)
    S = oracle.w8a16_gemm(xb & 0x7FFF, q & 0x7F, np.abs(s))
    check(run(x, q, s, torch.float32), ref, S, False, f"w8a16[{M}x{N}x{K}] f32")
    check(run(x, q, s, torch.bfloat16), ref, S, True, f"w8a16[{M}x{N}x{K}] bf16")


def test_w8a16_wide_scales():
    """Weight scales spread over 2^-20 .. 2^6 and activations with x50
    outliers: the dequantised values span a wide range and round in bf16."""
    M, N, K = 96, 384, 768
    rng = np.random.default_rng(71)
    x = inputs.normal_bf16((M, K), 1.0, 72, outlier_frac=0.01, outlier_mult=50.0)
    q = rng.integers(0, 256, (N, K), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x30                         # no NaN codes
    s = (2.0 ** rng.uniform(-20, 6, (N // 128, K // 128))).astype(np.float32)
    xb = inputs.bf16_bits(x)
    ref = oracle.w8a16_gemm(xb, q, s)
    S = oracle.w8a16_gemm(xb & 0x7FFF, q & 0x7F, s)
    check(run(x, q, s, torch.float32), ref, S, False, "w8a16 wide scales f32")


@pytest.mark.parametrize("sid,M,N,K", [
    (inputs.SEED_PREFILL, 4096, 18432, 7168),  # prefill up-projection shape
    (inputs.SEED_PREFILL, 4096, 7168, 18432),  # prefill down-projection shape
    (inputs.SEED_DECODE, 32, 18432, 7168),     # decode shape
    (inputs.SEED_PREFILL, 4000, 18000, 1024),  # ragged M and N, the launch split into 256x256 and 128x128 tiles
])
def test_w8a16_full_size_sampled(sid, M, N, K):
    """Full-size shapes (inputs drawn on the host and quantised by the oracle),
    checked at sampled points: whole rows, whole columns, tile corners and
    random points."""
    x, q, s = operands(M, N, K, inputs.seed_for(sid, 20))
    c = fp8bs.w8a16_gemm(x.to(DEV), to_dev_u8(q), to_dev_f32(s), torch.float32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(sid * 100 + N)
    rows = [0, M - 1, min(255, M - 1), min(256, M - 1)] + list(rng.integers(0, M, 2))
    # 16383 / 16384: the last column of the 256x256 launch and the first of the 128x128 one
    cols = [0, N - 1, 255, 256] + [c for c in (16383, 16384) if c < N] + list(rng.integers(0, N, 2))
    pr = np.concatenate([np.repeat(rows, N), np.tile(np.arange(M), len(cols)), rng.integers(0, M, 2000)])
    pc = np.concatenate([np.tile(np.arange(N), len(rows)), np.repeat(cols, M), rng.integers(0, N, 2000)])
    xb = inputs.bf16_bits(x)
    ref = oracle.w8a16_gemm_points(xb, q, s, pr, pc)
    S = oracle.w8a16_gemm_points(xb & 0x7FFF, q & 0x7F, np.abs(s), pr, pc)
    got = c.cpu().numpy().astype(np.float64)[pr, pc]
    check(got, ref, S, False, f"w8a16[{M}x{N}x{K}] sampled")
