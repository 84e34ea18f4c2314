"""GPU parity of the quantisation kernels against the CPU oracle, through the
C ABI: act_quant (fp32 and ue8m0 scales), weight_quant and weight_dequant must
be bit-exact -- every e4m3 byte, every float32 scale bit and every bf16 bit."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_03_amd as fp8bs
import oracle
from block_scaled_fp8_03_amd import inputs
from gpu_util import DEV, assert_bytes_equal, bf16_bits_dev, f32_bits, to_dev_f32, to_dev_u8, u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()


def check_act_quant(x_cpu: torch.Tensor, fmt: int, what: str):
    q, s = fp8bs.act_quant(x_cpu.to(DEV), fmt)
    torch.cuda.synchronize()
    qr, sr = oracle.act_quant(inputs.bf16_bits(x_cpu), fmt)
    assert_bytes_equal(f32_bits(s), sr.view(np.uint32), what + " scales")
    assert_bytes_equal(u8(q), qr, what + " codes")


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,K", [(16, 256), (1, 128), (7, 384), (129, 512), (37, 1024), (300, 7168)])
def test_act_quant_small(fmt, M, K):
    x = inputs.normal_bf16((M, K), 1.0, 1000 + M + K, outlier_frac=0.01, outlier_mult=50.0)
    check_act_quant(x, fmt, f"act_quant[{M}x{K}] fmt={fmt}")


def _special_blocks() -> torch.Tensor:
    """Blocks that pin the rounding: every e4m3 midpoint and its bf16
    neighbours at scale 1 (a block whose amax is 448), ties in the subnormal
    range, zero and negative-zero blocks, tiny blocks under the 1e-4 floor, a
    single outlier, all-negative blocks and power-of-two scales."""
    rows = []
    mags = [oracle.e4m3_decode(c) for c in range(127)]
    mids = [(a + b) / 2 for a, b in zip(mags[:-1], mags[1:])]
    vals = []
    for m in mids:
        mb = torch.tensor([m], dtype=torch.float32).to(torch.bfloat16)
        assert mb.item() == m                    # e4m3 midpoints are bf16 values
        vals += [m, -m]
        bits = mb.view(torch.int16).item()
        for d in (-1, 1):                        # bf16 neighbours of the midpoint
            nb = torch.tensor([bits + d], dtype=torch.int16).view(torch.bfloat16).item()
            vals += [nb, -nb]
    vals = [v for v in vals if abs(v) <= 448]
    for i in range(0, len(vals), 127):
        chunk = vals[i:i + 127]
        rows.append([448.0] + chunk + [0.0] * (127 - len(chunk)))
    rows.append([0.0] * 128)
    rows.append([-0.0] * 128)
    rows.append([1e-6 * (i - 64) for i in range(128)])                 # amax below the floor
    rows.append([1e-30] * 64 + [-1e-35] * 64)                          # far below the floor
    rows.append([0.001] * 127 + [3.0e4])                               # one outlier
    rows.append([-(i + 1) * 0.37 for i in range(128)])                 # all negative
    rows.append([2.0 ** (i % 40 - 20) * (-1) ** i for i in range(128)])
    rows.append([7.0] + [1.0, -0.5, 0.0078125, 3.0, -6.5] * 25 + [0.0, 0.0])   # s = 2^-6 exactly
    rows.append([448.0 * 2.0 ** -5] * 128)                             # s = 2^-5 exactly
    x = torch.tensor(rows, dtype=torch.float32).to(torch.bfloat16)
    return x.reshape(-1, 256) if x.shape[0] % 2 == 0 else torch.cat(
        [x, torch.zeros(1, 128, dtype=torch.bfloat16)]).reshape(-1, 256)


@pytest.mark.parametrize("fmt", [0, 1])
def test_act_quant_special_blocks(fmt):
    check_act_quant(_special_blocks(), fmt, f"act_quant special fmt={fmt}")


@pytest.mark.parametrize("sid,shape,fmt,outliers", [
    (inputs.SEED_DECODE, (32, 7168), 0, True),       # decode-shaped activations, 1% x50 outliers
    (inputs.SEED_PREFILL, (4096, 7168), 0, False),   # prefill up-proj input
    (inputs.SEED_PREFILL, (4096, 18432), 0, False),  # prefill down-proj input
    (inputs.SEED_MOE, (32768, 2048), 0, False),      # MoE down-proj input
    (inputs.SEED_UE8M0, (1024, 7168), 1, False),     # ue8m0
    (inputs.SEED_UE8M0, (1024, 512), 1, False),      # ue8m0, K = 512 GEMM input
])
def test_act_quant_full_size(sid, shape, fmt, outliers):
    x = inputs.normal_bf16(shape, 1.0, inputs.seed_for(sid, 0),
                           outlier_frac=0.01 if outliers else 0.0, outlier_mult=50.0)
    check_act_quant(x, fmt, f"act_quant{shape} fmt={fmt}")


def check_weight_quant(w_cpu: torch.Tensor, what: str):
    q, s = fp8bs.weight_quant(w_cpu.to(DEV))
    torch.cuda.synchronize()
    qr, sr = oracle.weight_quant(inputs.bf16_bits(w_cpu))
    assert_bytes_equal(f32_bits(s), sr.view(np.uint32), what + " scales")
    assert_bytes_equal(u8(q), qr, what + " codes")


@pytest.mark.parametrize("N,K", [(256, 256), (200, 300), (130, 200), (1, 1), (129, 128), (384, 1040)])
def test_weight_quant_small(N, K):
    w = inputs.normal_bf16((N, K), 0.02, 2000 + N + K)
    check_weight_quant(w, f"weight_quant[{N}x{K}]")


def test_weight_quant_full_size():
    w = inputs.normal_bf16((18432, 7168), 0.02, inputs.seed_for(inputs.SEED_PREFILL, 1))
    check_weight_quant(w, "weight_quant[18432x7168]")


def check_dequant(q: np.ndarray, s: np.ndarray, what: str):
    y = fp8bs.weight_dequant(to_dev_u8(q), to_dev_f32(s))
    torch.cuda.synchronize()
    ref = oracle.weight_dequant(q, s)
    got = bf16_bits_dev(y)
    nan_ref = (ref & 0x7FFF) > 0x7F80
    nan_got = (got & 0x7FFF) > 0x7F80
    assert np.array_equal(nan_ref, nan_got), what + " NaN positions"
    assert_bytes_equal(np.where(nan_ref, 0, got), np.where(nan_ref, 0, ref), what)


@pytest.mark.parametrize("N,K", [(256, 256), (257, 200), (130, 384), (131, 1040), (1, 16), (3, 5),
                                 (5, 1824), (9103, 14880)])
def test_weight_dequant_all_codes(N, K):
    """Every code (NaN included) against a spread of scales, ragged edges, both
    the vector path (K % 16 == 0) and the element path.  In the vector path a
    lane takes 8-column chunks c and c + 64 of a 1024-column span: K = 1040
    and 1824 leave a last span where only some lanes (or none) have the second
    chunk, and N not a multiple of 4 leaves idle waves in the last row group;
    9103 x 14880 has 15 spans."""
    rng = np.random.default_rng(N * 31 + K)
    q = rng.integers(0, 256, (N, K), dtype=np.uint8)
    q.reshape(-1)[:256] = np.arange(256, dtype=np.uint8)[: q.size]
    s = (2.0 ** rng.uniform(-20, 6, (-(-N // 128), -(-K // 128)))).astype(np.float32)
    check_dequant(q, s, f"weight_dequant[{N}x{K}]")


def test_weight_dequant_full_size():
    """The ue8m0/dequant workload: W [18432, 7168] drawn N(0, 0.02) and
    quantised by the oracle, then expanded to bf16."""
    w = inputs.normal_bf16((18432, 7168), 0.02, inputs.seed_for(inputs.SEED_UE8M0, 1))
    q, s = oracle.weight_quant(inputs.bf16_bits(w))
    check_dequant(q, s, "weight_dequant[18432x7168]")


def test_e4m3_encoder_exhaustive():
    """The hardware float32 -> e4m3 conversion used by act_quant and
    weight_quant (clamp to +-448, then round to nearest even), checked
    against the oracle's encoder on every float32 bit pattern of magnitude
    <= 464 (the midpoint above 448), both signs: about 2.3e9 values, in
    chunks of 2^28 generated on the device from their bit patterns."""
    top = int(np.float32(464.0).view(np.uint32))             # 0x43E80000
    chunk = 1 << 28
    x = torch.empty(chunk, dtype=torch.float32, device=DEV)
    q = torch.empty(chunk, dtype=torch.uint8, device=DEV)
    checked = 0
    for sign in (0, 0x80000000):
        for lo in range(0, top + 1, chunk):
            n = min(chunk, top + 1 - lo)
            bits = torch.arange(lo, lo + n, dtype=torch.int64, device=DEV) | sign
            x[:n] = bits.to(torch.int32).view(torch.float32) if sign == 0 else \
                (bits - (1 << 32)).to(torch.int32).view(torch.float32)
            del bits
            fp8bs.fp8bs_e4m3_encode(x[:n], q[:n])
            got = q[:n].cpu().numpy()
            ref_in = (np.arange(lo, lo + n, dtype=np.uint64) | sign).astype(np.uint32).view(np.float32)
            ref = oracle.e4m3_encode_f32(ref_in)
            if not np.array_equal(got, ref):
                bad = np.nonzero(got != ref)[0][:8]
                raise AssertionError(f"e4m3 encode differs at bit patterns "
                                     f"{[hex(int(ref_in[i].view(np.uint32))) for i in bad]}: gpu "
                                     f"{[hex(int(got[i])) for i in bad]} oracle {[hex(int(ref[i])) for i in bad]}")
            checked += n
    assert checked == 2 * (top + 1)
