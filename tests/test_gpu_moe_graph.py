"""Stream ordering of the grouped MoE GEMM.  The call is one launch on the
caller's stream that runs both expert classes (experts with more than 64 rows
and the others).  These tests check that from the outside: a consumer
enqueued on the caller's stream right after the call sees the whole output,
and a graph captured from the call replays to the same bytes as the eager
call, several times, with eager work and synchronisation between the
replays.  Outputs are also checked against the oracle (binary64) with the GEMM
bar |gpu - ref| <= 1e-2 |ref| + 1e-3."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_03_amd as fp8bs
import oracle
from block_scaled_fp8_03_amd import inputs
from gpu_util import DEV, assert_close, to_dev_f32, to_dev_u8

pytestmark = pytest.mark.gpu

# both expert classes present: <= 64 rows and > 64 rows
COUNTS = [3, 200, 64, 65, 0, 17, 300, 1, 40, 129]
N, K = 384, 512


@pytest.fixture(scope="module")
def operands():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()
    E = len(COUNTS)
    off = np.concatenate([[0], np.cumsum(COUNTS)]).astype(np.int32)
    R = int(off[-1])
    x = inputs.normal_bf16((R, K), 1.0, 7100)
    a, a_s = oracle.act_quant(inputs.bf16_bits(x), oracle.FMT_FP32)
    w = inputs.normal_bf16((E * N, K), 0.02, 7200)
    bq, bs = [], []
    for e in range(E):
        q, s = oracle.weight_quant(inputs.bf16_bits(w[e * N:(e + 1) * N]))
        bq.append(q)
        bs.append(s)
    b, b_s = np.stack(bq), np.stack(bs)
    ref = oracle.moe_gemm(a, a_s, b, b_s, off)
    dev = (to_dev_u8(a), to_dev_f32(a_s), to_dev_u8(b), to_dev_f32(b_s), torch.from_numpy(off).to(DEV))
    return dev, ref, R


def test_moe_consumer_on_caller_stream(operands):
    """A torch kernel enqueued on the caller's (non-default) stream right
    after the call reads the complete output."""
    (a, a_s, b, b_s, off), ref, R = operands
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y = torch.empty((R, N), dtype=torch.float32, device=DEV)
        for _ in range(3):
            y.fill_(float("nan"))
            fp8bs.fp8bs_moe_gemm(a, a_s, b, b_s, off, y)
            z = y * 2.0                      # consumer on the same stream
    s.synchronize()
    assert_close((z * 0.5).cpu().numpy(), ref, "moe consumer after the call")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_moe_graph_replays_match_eager(operands, out_dtype):
    """A graph captured from the call replays to the eager call's bytes,
    three times, with eager work and synchronisation between the replays."""
    (a, a_s, b, b_s, off), ref, R = operands
    y_ref = torch.empty((R, N), dtype=out_dtype, device=DEV)
    fp8bs.fp8bs_moe_gemm(a, a_s, b, b_s, off, y_ref)
    torch.cuda.synchronize()
    assert_close(y_ref.float().cpu().numpy(), ref, f"moe eager {out_dtype}")
    y = torch.empty_like(y_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                # warm-up outside the capture
        fp8bs.fp8bs_moe_gemm(a, a_s, b, b_s, off, y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp8bs.fp8bs_moe_gemm(a, a_s, b, b_s, off, y)
    torch.cuda.synchronize()
    other = torch.empty_like(y_ref)
    bits = torch.int32 if out_dtype == torch.float32 else torch.int16
    for i in range(3):
        y.fill_(float("nan"))                    # eager work between replays
        fp8bs.fp8bs_moe_gemm(a, a_s, b, b_s, off, other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(bits), y_ref.view(bits)), f"replay {i} differs from the eager call"
        assert torch.equal(other.view(bits), y_ref.view(bits)), f"eager call {i} differs"
