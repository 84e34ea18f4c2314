"""Helpers shared by the GPU parity tests: moving seeded inputs between torch
and the oracle's numpy arrays, and the element-wise comparisons."""
import numpy as np
import torch

DEV = "cuda"

# GEMM bar: |gpu - ref| <= REL * |ref| + ABS, element-wise, with the GPU value
# taken in float32 before the bf16 store (and also checked after it).
REL = 1e-2
ABS = 1e-3


def u8(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.uint8).cpu().numpy()


def f32_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy().view(np.uint32)


def bf16_bits_dev(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).view(torch.float8_e4m3fn)


def to_dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def assert_bytes_equal(got: np.ndarray, ref: np.ndarray, what: str):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    bad = np.nonzero(got != ref)
    n = bad[0].size
    if n:
        idx = list(zip(*[b[:8] for b in bad]))
        pairs = [(i, hex(int(got[i])), hex(int(ref[i]))) for i in idx]
        raise AssertionError(f"{what}: {n} of {got.size} differ; first (index, gpu, oracle): {pairs}")


def assert_close(got: np.ndarray, ref: np.ndarray, what: str):
    got = got.astype(np.float64)
    err = np.abs(got - ref)
    bound = REL * np.abs(ref) + ABS
    bad = np.nonzero(~(err <= bound))
    n = bad[0].size
    if n:
        idx = list(zip(*[b[:8] for b in bad]))
        pairs = [(i, float(got[i]), float(ref[i])) for i in idx]
        raise AssertionError(f"{what}: {n} of {got.size} outside {REL}|ref|+{ABS}; "
                             f"first (index, gpu, oracle): {pairs}")
