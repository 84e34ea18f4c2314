"""GPU parity of the MLA absorb products with an FP8 wkv_b (key side: q_nope
through the key rows; value side: the attention-weighted latent through the
value rows) against the CPU oracle, through the C ABI.  The kernels multiply
exact bf16 products (weight_dequant's rounding of the weight) and accumulate
in float32 on the bf16 MFMA, so the bar is the BF16 path's: |gpu - ref| <=
2^-13 * S on the float32 output, S = sum |input * weight|, plus 2^-8 |ref|
for the bf16 store.  Weights are host draws quantised by the oracle."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_03_amd as fp8bs
import oracle
from block_scaled_fp8_03_amd import inputs
from gpu_util import DEV, to_dev_f32, to_dev_u8

pytestmark = pytest.mark.gpu

KEY, VALUE = oracle.MLA_KEY, oracle.MLA_VALUE


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()


def wkv_b(H, dn, dv, R, seed):
    w = inputs.normal_bf16((H * (dn + dv), R), 0.02, seed)
    return oracle.weight_quant(inputs.bf16_bits(w))


def run(side, inp_dev, q, s, dn, dv, dt):
    fn = fp8bs.mla_absorb_key if side == KEY else fp8bs.mla_absorb_value
    out = fn(inp_dev, to_dev_u8(q), to_dev_f32(s), dn, dv, dt)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def check(got, ref, S, bf16, what):
    bar = 2.0 ** -13 * S + (2.0 ** -8 * np.abs(ref) if bf16 else 0.0) + 1e-30
    bad = np.abs(got - ref) > bar
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside, first {np.argwhere(bad)[:4].tolist()}"


def both_sides(T, H, dn, dv, R, seed, q, s):
    """Key and value sides on fresh N(0, 1) activations, both output types."""
    for side, width in ((KEY, dn), (VALUE, R)):
        x = inputs.normal_bf16((T, H, width), 1.0, seed + side)
        xb = inputs.bf16_bits(x)
        ref = oracle.mla_absorb(side, xb, q, s, dn, dv)
        S = oracle.mla_absorb(side, xb & 0x7FFF, q & 0x7F, np.abs(s), dn, dv)
        xd = x.to(DEV)
        name = "key" if side == KEY else "value"
        check(run(side, xd, q, s, dn, dv, torch.float32), ref, S, False, f"mla {name} [{T},{H},{dn},{dv},{R}] f32")
        check(run(side, xd, q, s, dn, dv, torch.bfloat16), ref, S, True, f"mla {name} [{T},{H},{dn},{dv},{R}] bf16")


@pytest.mark.parametrize("T,H,dn,dv,R", [
    (1, 1, 128, 128, 128), (5, 3, 128, 128, 512), (17, 2, 256, 128, 384),   # ragged token tiles
    (33, 4, 128, 256, 256), (64, 2, 128, 128, 512),
    (300, 3, 128, 128, 512),                                                # two token chunks, ragged
    (600, 2, 256, 256, 128),
])
def test_mla_small(T, H, dn, dv, R):
    q, s = wkv_b(H, dn, dv, R, 600 + T + H + dn + dv + R)
    both_sides(T, H, dn, dv, R, 610 + T, q, s)


@pytest.mark.parametrize("T", [72, 200])
def test_mla_mid_tokens_all_heads(T):
    """128 heads at token counts whose 256-token chunks would leave CUs idle:
    64-token chunks (the weight re-read per chunk, a ragged last chunk at
    200 tokens), compared in full."""
    H, dn, dv, R = 128, 128, 128, 512
    q, s = wkv_b(H, dn, dv, R, 640 + T)
    both_sides(T, H, dn, dv, R, 650 + T, q, s)


def test_mla_strided_inputs():
    """q_nope as the pages slice it: the first dn of each head's dn + 64 query
    values (head stride dn + 64, token stride H (dn + 64)); x as a view with a
    padded token stride."""
    T, H, dn, dv, R = 40, 6, 128, 128, 512
    q, s = wkv_b(H, dn, dv, R, 620)
    qfull = inputs.normal_bf16((T, H, dn + 64), 1.0, 621)
    qn = qfull[:, :, :dn]
    qb = inputs.bf16_bits(qn.contiguous())
    ref = oracle.mla_absorb(KEY, qb, q, s, dn, dv)
    S = oracle.mla_absorb(KEY, qb & 0x7FFF, q & 0x7F, np.abs(s), dn, dv)
    qd = qfull.to(DEV)[:, :, :dn]
    assert qd.stride() == (H * (dn + 64), dn + 64, 1)
    check(run(KEY, qd, q, s, dn, dv, torch.float32), ref, S, False, "mla key strided q")
    xpad = inputs.normal_bf16((T, H * R + 64), 1.0, 622)
    x = xpad[:, : H * R].reshape(T, H, R)
    xb = inputs.bf16_bits(x.contiguous())
    ref = oracle.mla_absorb(VALUE, xb, q, s, dn, dv)
    S = oracle.mla_absorb(VALUE, xb & 0x7FFF, q & 0x7F, np.abs(s), dn, dv)
    xd = xpad.to(DEV)[:, : H * R].view(T, H, R)
    assert xd.stride() == (H * R + 64, R, 1)
    check(run(VALUE, xd, q, s, dn, dv, torch.float32), ref, S, False, "mla value strided x")


def test_mla_wide_scales():
    """Random full-range codes (no NaN) with block scales over 2^-20 .. 2^6 and
    x50 outlier activations: every dequantised value takes its own bf16
    rounding, and each head's key and value blocks their own scales."""
    T, H, dn, dv, R = 48, 3, 128, 128, 512
    rng = np.random.default_rng(630)
    q = rng.integers(0, 256, (H * (dn + dv), R), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x30
    s = (2.0 ** rng.uniform(-20, 6, (H * (dn + dv) // 128, R // 128))).astype(np.float32)
    for side, width in ((KEY, dn), (VALUE, R)):
        x = inputs.normal_bf16((T, H, width), 1.0, 631 + side, outlier_frac=0.01, outlier_mult=50.0)
        xb = inputs.bf16_bits(x)
        ref = oracle.mla_absorb(side, xb, q, s, dn, dv)
        S = oracle.mla_absorb(side, xb & 0x7FFF, q & 0x7F, s, dn, dv)
        check(run(side, x.to(DEV), q, s, dn, dv, torch.float32), ref, S, False, f"mla wide scales side {side}")


def test_mla_decode_full():
    """The pages' attention shape (128 heads, dn = dv = 128, kv_lora_rank 512)
    at a decode batch of 32 tokens, compared in full."""
    m = inputs.MLA
    T, H, dn, dv, R = m["decode_tokens"], m["heads"], m["dn"], m["dv"], m["R"]
    q, s = wkv_b(H, dn, dv, R, inputs.seed_for(inputs.MLA["seed_id"], 1))
    both_sides(T, H, dn, dv, R, inputs.seed_for(inputs.MLA["seed_id"], 2), q, s)


def test_mla_prefill_sampled():
    """4096 tokens, 128 heads: whole (token, head) rows of both outputs at the
    chunk edges plus random points."""
    m = inputs.MLA
    T, H, dn, dv, R = m["prefill_tokens"], m["heads"], m["dn"], m["dv"], m["R"]
    q, s = wkv_b(H, dn, dv, R, inputs.seed_for(inputs.MLA["seed_id"], 1))
    rng = np.random.default_rng(640)
    for side, width, ncol in ((KEY, dn, R), (VALUE, R, dv)):
        x = inputs.normal_bf16((T, H, width), 1.0, inputs.seed_for(inputs.MLA["seed_id"], 3 + side))
        out = (fp8bs.mla_absorb_key if side == KEY else fp8bs.mla_absorb_value)(
            x.to(DEV), to_dev_u8(q), to_dev_f32(s), dn, dv, torch.float32)
        torch.cuda.synchronize()
        rows = [(0, 0), (255, 1), (256, 127), (T - 1, 64), (4000, 5)]
        ts = np.concatenate([np.repeat([r[0] for r in rows], ncol), rng.integers(0, T, 3000)])
        hs = np.concatenate([np.repeat([r[1] for r in rows], ncol), rng.integers(0, H, 3000)])
        cs = np.concatenate([np.tile(np.arange(ncol), len(rows)), rng.integers(0, ncol, 3000)])
        xb = inputs.bf16_bits(x)
        ref = oracle.mla_absorb_points(side, xb, q, s, dn, dv, ts, hs, cs)
        S = oracle.mla_absorb_points(side, xb & 0x7FFF, q & 0x7F, np.abs(s), dn, dv, ts, hs, cs)
        got = out[torch.from_numpy(ts).to(DEV), torch.from_numpy(hs).to(DEV),
                  torch.from_numpy(cs).to(DEV)].cpu().numpy().astype(np.float64)
        check(got, ref, S, False, f"mla prefill sampled side {side}")


@pytest.mark.parametrize("T,H,dn,R", [(100, 2, 128, 640), (200, 1, 256, 896), (70, 3, 128, 1152)])
def test_mla_key_partial_workgroup(T, H, dn, R):
    """Key side with R not a multiple of 512: the last workgroup of eight
    waves has idle waves, and its staged bf16 rows stop at R."""
    dv = 128
    q, s = wkv_b(H, dn, dv, R, 650 + T + R)
    x = inputs.normal_bf16((T, H, dn), 1.0, 660 + T)
    xb = inputs.bf16_bits(x)
    ref = oracle.mla_absorb(KEY, xb, q, s, dn, dv)
    S = oracle.mla_absorb(KEY, xb & 0x7FFF, q & 0x7F, np.abs(s), dn, dv)
    xd = x.to(DEV)
    check(run(KEY, xd, q, s, dn, dv, torch.float32), ref, S, False, f"mla key [{T},{H},{dn},{R}] f32")
    check(run(KEY, xd, q, s, dn, dv, torch.bfloat16), ref, S, True, f"mla key [{T},{H},{dn},{R}] bf16")


@pytest.mark.parametrize("T", [4096, 2048, 1000])
def test_mla_prefill_bf16_is_rounded_f32(T):
    """Both output types come from the same float32 accumulators, so every
    bf16 output must be the float32 output rounded to nearest even, bit for
    bit, over the whole tensor.  At 128 heads this covers the launches whose
    large stream (key output, value input) takes the non-temporal hint (4096
    and 2048 tokens) and those below the cut (1000 tokens), including the
    staged rows of the ragged last token tile; the float32 output itself is
    checked against the oracle at 4096 tokens by test_mla_prefill_sampled."""
    m = inputs.MLA
    H, dn, dv, R = m["heads"], m["dn"], m["dv"], m["R"]
    q, s = wkv_b(H, dn, dv, R, inputs.seed_for(inputs.MLA["seed_id"], 1))
    qd, sd = to_dev_u8(q), to_dev_f32(s)
    for side, width in ((KEY, dn), (VALUE, R)):
        fn = fp8bs.mla_absorb_key if side == KEY else fp8bs.mla_absorb_value
        x = inputs.normal_bf16_device((T, H, width), 1.0, 670 + side, DEV)
        o32 = fn(x, qd, sd, dn, dv, torch.float32)
        o16 = fn(x, qd, sd, dn, dv, torch.bfloat16)
        torch.cuda.synchronize()
        want = o32.to(torch.bfloat16)
        same = o16.view(torch.int16) == want.view(torch.int16)
        assert bool(same.all()), (f"side {side} T={T}: {int((~same).sum())} bf16 outputs differ, "
                                  f"first {torch.nonzero(~same)[:4].tolist()}")
        del x, o32, o16, want, same
