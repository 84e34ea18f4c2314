"""CPU oracle for the block-scaled FP8 linear -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct binary64 model of the DeepSeek-V3 block-scaled
FP8 linear ("DeepSeek-V3 Administrator & Developer Guide", sections 6.3, 6.4,
8.5.1-8.5.3; "DeepSeek-V3 User Guide", FAQ on ue8m0).  The arithmetic lives in
``fp8bs_oracle.c`` (plain C + OpenMP); this module only compiles it with gcc
and marshals numpy arrays through ctypes.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
and imports nothing from it.

Every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` against closed forms, invariants, torch/numpy
library routines and brute force; see the docstring of each test for which
mistake it would catch.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8bs_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_fp8bs.so")

FMT_FP32 = 0
FMT_UE8M0 = 1
BLOCK = 128

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (strict IEEE: no fast-math) and return the path."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_f32.restype = ctypes.c_float
    lib.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.orc_f32_to_bf16.restype = ctypes.c_uint16
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_e4m3_encode_f32_array.argtypes = [P, P, I64]
    lib.orc_e4m3_decode_array.argtypes = [P, P, I64]
    lib.orc_block_scale.argtypes = [ctypes.c_float, ctypes.c_int]
    lib.orc_block_scale.restype = ctypes.c_float
    lib.orc_act_quant.argtypes = [P, I64, I64, ctypes.c_int, P, P]
    lib.orc_weight_quant.argtypes = [P, I64, I64, P, P]
    lib.orc_weight_quant_fmt.argtypes = [P, I64, I64, ctypes.c_int, P, P]
    lib.orc_weight_dequant.argtypes = [P, P, I64, I64, P]
    lib.orc_gemm.argtypes = [P, P, P, P, I64, I64, I64, P]
    lib.orc_gemm_points.argtypes = [P, P, P, P, I64, P, P, I64, P]
    lib.orc_moe_gemm.argtypes = [P, P, P, P, P, I64, I64, I64, I64, P]
    lib.orc_moe_gemm_points.argtypes = [P, P, P, P, P, I64, I64, I64, P, P, I64, P]
    lib.orc_w8a16_gemm.argtypes = [P, P, P, I64, I64, I64, P]
    lib.orc_w8a16_gemm_points.argtypes = [P, P, P, I64, I64, P, P, I64, P]
    lib.orc_mla_absorb.argtypes = [ctypes.c_int, P, P, P, I64, I64, I64, I64, I64, P]
    lib.orc_mla_absorb_points.argtypes = [ctypes.c_int, P, P, P, I64, I64, I64, I64, P, P, P, I64, P]
    lib.orc_moe_route.argtypes = [P, I64, I64, I64, P, P, P, P]
    lib.orc_moe_route.restype = I64
    lib.orc_moe_quant_scatter.argtypes = [P, I64, I64, ctypes.c_int, P, I64, I64, P, P]
    lib.orc_moe_combine.argtypes = [P, P, P, I64, I64, I64, I64, P]
    lib.orc_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def num_threads() -> int:
    return int(_load().orc_num_threads())


# ---- scalar conversions -------------------------------------------------------

def e4m3_decode(code: int) -> float:
    """Value of one e4m3fn code (OCP E4M3, no infinities; 0x7F/0xFF are NaN)."""
    return float(_load().orc_e4m3_decode(int(code) & 0xFF))


def e4m3_encode(y: float) -> int:
    """e4m3fn code of a real number: nearest, ties to even, saturating at +-448."""
    return int(_load().orc_e4m3_encode(float(y)))


def e4m3_encode_f32(y: np.ndarray) -> np.ndarray:
    y = _c(np.asarray(y, dtype=np.float32), np.float32)
    q = np.empty(y.shape, dtype=np.uint8)
    _load().orc_e4m3_encode_f32_array(_ptr(y), _ptr(q), y.size)
    return q


def e4m3_decode_array(q: np.ndarray) -> np.ndarray:
    q = _c(q, np.uint8)
    out = np.empty(q.shape, dtype=np.float64)
    _load().orc_e4m3_decode_array(_ptr(q), _ptr(out), q.size)
    return out


def f32_to_bf16(f: float) -> int:
    return int(_load().orc_f32_to_bf16(float(np.float32(f))))


def block_scale(amax: float, fmt: int = FMT_FP32) -> float:
    """Block scale rule: RN32(max(amax, 1e-4) / 448), ue8m0 -> next power of two."""
    return float(_load().orc_block_scale(float(np.float32(amax)), int(fmt)))


# ---- the method's steps -----------------------------------------------------

def act_quant(x_bf16_bits: np.ndarray, fmt: int = FMT_FP32):
    """act_quant on bf16 bit patterns ``uint16 [M, K]`` (K % 128 == 0).

    Returns (q uint8 [M, K] e4m3 codes, s float32 [M, K/128]).
    Admin guide 8.5.1; User guide FAQ (ue8m0)."""
    x = _c(x_bf16_bits, np.uint16)
    if x.ndim != 2 or x.shape[1] % BLOCK:
        raise ValueError("x must be [M, K] with K % 128 == 0")
    M, K = x.shape
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // BLOCK), dtype=np.float32)
    _load().orc_act_quant(_ptr(x), M, K, int(fmt), _ptr(q), _ptr(s))
    return q, s


def weight_quant(w_bf16_bits: np.ndarray, fmt: int = FMT_FP32):
    """128x128 block quantisation of a bf16 weight ``uint16 [N, K]`` (any N, K)
    with act_quant's rule per block (fmt FMT_UE8M0: power-of-two scales, a
    harness option for the ue8m0 fast path).

    Returns (q uint8 [N, K], s float32 [ceil(N/128), ceil(K/128)])."""
    w = _c(w_bf16_bits, np.uint16)
    N, K = w.shape
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty(((N + BLOCK - 1) // BLOCK, (K + BLOCK - 1) // BLOCK), dtype=np.float32)
    _load().orc_weight_quant_fmt(_ptr(w), N, K, int(fmt), _ptr(q), _ptr(s))
    return q, s


def weight_dequant(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of RN32(decode(q) * s_block). Admin guide 8.5.2."""
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    N, K = q.shape
    assert s.shape == ((N + BLOCK - 1) // BLOCK, (K + BLOCK - 1) // BLOCK)
    out = np.empty((N, K), dtype=np.uint16)
    _load().orc_weight_dequant(_ptr(q), _ptr(s), N, K, _ptr(out))
    return out


def _check_gemm(a, a_s, b, b_s):
    M, K = a.shape
    N, K2 = b.shape
    if K != K2 or K % BLOCK:
        raise ValueError("A [M,K] and B [N,K] need the same K, a multiple of 128")
    assert a_s.shape == (M, K // BLOCK), a_s.shape
    assert b_s.shape == ((N + BLOCK - 1) // BLOCK, K // BLOCK), b_s.shape
    return M, N, K


def gemm(a, a_s, b, b_s) -> np.ndarray:
    """Block-scaled FP8 GEMM in binary64: C [M, N] = A . B^T with per-block
    scales folded once per 128-wide K block. Admin guide 8.5.3."""
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    a_s, b_s = _c(a_s, np.float32), _c(b_s, np.float32)
    M, N, K = _check_gemm(a, a_s, b, b_s)
    c = np.empty((M, N), dtype=np.float64)
    _load().orc_gemm(_ptr(a), _ptr(a_s), _ptr(b), _ptr(b_s), M, N, K, _ptr(c))
    return c


def gemm_points(a, a_s, b, b_s, rows, cols) -> np.ndarray:
    """Oracle GEMM evaluated only at the given (row, col) pairs."""
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    a_s, b_s = _c(a_s, np.float32), _c(b_s, np.float32)
    M, N, K = _check_gemm(a, a_s, b, b_s)
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    cols = _c(np.asarray(cols, dtype=np.int64), np.int64)
    assert rows.shape == cols.shape and rows.ndim == 1
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < M and cols.min() >= 0 and cols.max() < N)
    out = np.empty(rows.shape, dtype=np.float64)
    _load().orc_gemm_points(_ptr(a), _ptr(a_s), _ptr(b), _ptr(b_s), K, _ptr(rows), _ptr(cols),
                            rows.size, _ptr(out))
    return out


def _check_moe(a, a_s, b, b_s, offsets):
    R, K = a.shape
    E, N, K2 = b.shape
    if K != K2 or K % BLOCK:
        raise ValueError("bad K")
    assert a_s.shape == (R, K // BLOCK)
    assert b_s.shape == (E, (N + BLOCK - 1) // BLOCK, K // BLOCK)
    assert offsets.shape == (E + 1,) and offsets[0] == 0 and offsets[-1] == R
    assert np.all(np.diff(offsets) >= 0)
    return R, E, N, K


def moe_gemm(a, a_s, b, b_s, offsets) -> np.ndarray:
    """Grouped GEMM: rows [off[e], off[e+1]) of A use expert e's weight.
    Admin guide 6.4 (per-expert loop), each expert as in 8.5.3."""
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    a_s, b_s = _c(a_s, np.float32), _c(b_s, np.float32)
    offsets = _c(np.asarray(offsets, dtype=np.int32), np.int32)
    R, E, N, K = _check_moe(a, a_s, b, b_s, offsets)
    c = np.empty((R, N), dtype=np.float64)
    _load().orc_moe_gemm(_ptr(a), _ptr(a_s), _ptr(b), _ptr(b_s), _ptr(offsets), R, E, N, K, _ptr(c))
    return c


def moe_gemm_points(a, a_s, b, b_s, offsets, rows, cols) -> np.ndarray:
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    a_s, b_s = _c(a_s, np.float32), _c(b_s, np.float32)
    offsets = _c(np.asarray(offsets, dtype=np.int32), np.int32)
    R, E, N, K = _check_moe(a, a_s, b, b_s, offsets)
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    cols = _c(np.asarray(cols, dtype=np.int64), np.int64)
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < R and cols.min() >= 0 and cols.max() < N)
    out = np.empty(rows.shape, dtype=np.float64)
    _load().orc_moe_gemm_points(_ptr(a), _ptr(a_s), _ptr(b), _ptr(b_s), _ptr(offsets), E, N, K,
                                _ptr(rows), _ptr(cols), rows.size, _ptr(out))
    return out


# ------------------------------------------------------------ the BF16 path

def w8a16_gemm(x_bf16_bits: np.ndarray, q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """C = x . weight_dequant(q, s)^T in binary64: x bf16 bits uint16 [M, K],
    q e4m3 [N, K], s float32 [ceil(N/128), ceil(K/128)] (Admin guide 6.3, the
    gemm_impl "bf16" path: dequantise, then a BF16 linear)."""
    x = _c(x_bf16_bits, np.uint16)
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    M, K = x.shape
    N, K2 = q.shape
    if K != K2 or s.shape != (-(-N // BLOCK), -(-K // BLOCK)):
        raise ValueError("x [M, K], q [N, K], s [ceil(N/128), ceil(K/128)]")
    c = np.empty((M, N), dtype=np.float64)
    _load().orc_w8a16_gemm(_ptr(x), _ptr(q), _ptr(s), M, N, K, _ptr(c))
    return c


def w8a16_gemm_points(x_bf16_bits, q, s, rows, cols) -> np.ndarray:
    x = _c(x_bf16_bits, np.uint16)
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    M, K = x.shape
    N = q.shape[0]
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    cols = _c(np.asarray(cols, dtype=np.int64), np.int64)
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < M and cols.min() >= 0 and cols.max() < N)
    out = np.empty(rows.shape, dtype=np.float64)
    _load().orc_w8a16_gemm_points(_ptr(x), _ptr(q), _ptr(s), N, K, _ptr(rows), _ptr(cols), rows.size,
                                  _ptr(out))
    return out


# ------------------------------------------------------------------ MLA absorb

MLA_KEY, MLA_VALUE = 0, 1


def _mla_check(side, inp, w, s, dn, dv):
    inp = _c(inp, np.uint16)
    w = _c(w, np.uint8)
    s = _c(s, np.float32)
    T, H, width = inp.shape
    rows, R = w.shape
    if rows != H * (dn + dv) or width != (dn if side == MLA_KEY else R):
        raise ValueError("wkv_b must be [H*(dn+dv), R]; q [T, H, dn] or x [T, H, R]")
    if s.shape != (-(-rows // BLOCK), -(-R // BLOCK)):
        raise ValueError("scale shape")
    return inp, w, s, T, H, R


def mla_absorb(side: int, inp_bf16_bits: np.ndarray, w: np.ndarray, s: np.ndarray, dn: int,
               dv: int) -> np.ndarray:
    """MLA absorb with an FP8 wkv_b (Admin guide 8.3 steps 5 and 7, the weight
    dequantised as weight_dequant does), in binary64.

    side MLA_KEY:   q bf16 bits [T, H, dn] -> [T, H, R],
                    out[t,h,c] = sum_d q[t,h,d] Wd[h(dn+dv)+d, c]
    side MLA_VALUE: x bf16 bits [T, H, R] -> [T, H, dv],
                    out[t,h,d] = sum_c x[t,h,c] Wd[h(dn+dv)+dn+d, c]"""
    inp, w, s, T, H, R = _mla_check(side, inp_bf16_bits, w, s, dn, dv)
    ncol = R if side == MLA_KEY else dv
    out = np.empty((T, H, ncol), dtype=np.float64)
    _load().orc_mla_absorb(int(side), _ptr(inp), _ptr(w), _ptr(s), T, H, dn, dv, R, _ptr(out))
    return out


def mla_absorb_points(side: int, inp_bf16_bits, w, s, dn, dv, ts, hs, cols) -> np.ndarray:
    """mla_absorb at the points (ts[i], hs[i], cols[i])."""
    inp, w, s, T, H, R = _mla_check(side, inp_bf16_bits, w, s, dn, dv)
    ts, hs, cols = (_c(np.asarray(a, dtype=np.int64), np.int64) for a in (ts, hs, cols))
    ncol = R if side == MLA_KEY else dv
    assert ts.size == 0 or (0 <= ts.min() and ts.max() < T and 0 <= hs.min() and hs.max() < H
                            and 0 <= cols.min() and cols.max() < ncol)
    out = np.empty(ts.shape, dtype=np.float64)
    _load().orc_mla_absorb_points(int(side), _ptr(inp), _ptr(w), _ptr(s), H, dn, dv, R, _ptr(ts),
                                  _ptr(hs), _ptr(cols), ts.size, _ptr(out))
    return out


# --------------------------------------------------------------- MoE dispatch

def moe_route(indices: np.ndarray, E: int):
    """Stable counting sort of routed expert ids ``int32 [T, topk]`` by expert
    (Admin guide 6.4 / 8.4: bincount of the ids, then each expert's (token,
    slot) pairs in token order).  Returns dict with offsets int32 [E+1],
    row_token / row_slot int32 [R] and row_of int32 [T, topk] (-1 for ids
    outside [0, E))."""
    idx = _c(np.asarray(indices, dtype=np.int32), np.int32)
    if idx.ndim != 2:
        raise ValueError("indices must be [T, topk]")
    T, topk = idx.shape
    off = np.empty(E + 1, dtype=np.int32)
    row_token = np.empty(T * topk, dtype=np.int32)
    row_slot = np.empty(T * topk, dtype=np.int32)
    row_of = np.empty((T, topk), dtype=np.int32)
    R = _load().orc_moe_route(_ptr(idx), T, topk, E, _ptr(off), _ptr(row_token), _ptr(row_slot),
                              _ptr(row_of))
    return {"offsets": off, "row_token": row_token[:R].copy(), "row_slot": row_slot[:R].copy(),
            "row_of": row_of}


def moe_quant_scatter(x_bf16_bits: np.ndarray, row_of: np.ndarray, R: int, fmt: int = FMT_FP32):
    """act_quant of each token row of x ``uint16 [T, K]`` placed at the rows
    ``row_of [T, topk]`` names (rows no pair maps to are left zero).
    Returns (q uint8 [R, K], s float32 [R, K/128])."""
    x = _c(x_bf16_bits, np.uint16)
    row_of = _c(np.asarray(row_of, dtype=np.int32), np.int32)
    T, K = x.shape
    if K % BLOCK or row_of.shape[0] != T:
        raise ValueError("x must be [T, K] with K % 128 == 0 and row_of [T, topk]")
    q = np.zeros((R, K), dtype=np.uint8)
    s = np.zeros((R, K // BLOCK), dtype=np.float32)
    _load().orc_moe_quant_scatter(_ptr(x), T, K, int(fmt), _ptr(row_of), row_of.shape[1], R,
                                  _ptr(q), _ptr(s))
    return q, s


def moe_combine(out_bf16_bits: np.ndarray, weights: np.ndarray, row_of: np.ndarray) -> np.ndarray:
    """y[t] = sum_k weights[t, k] * out[row_of[t, k]] in binary64, with out the
    expert outputs as bf16 bit patterns ``uint16 [R, N]`` and weights float32
    [T, topk].  Returns float64 [T, N]."""
    out = _c(out_bf16_bits, np.uint16)
    w = _c(np.asarray(weights, dtype=np.float32), np.float32)
    row_of = _c(np.asarray(row_of, dtype=np.int32), np.int32)
    R, N = out.shape
    T, topk = w.shape
    if row_of.shape != (T, topk):
        raise ValueError("row_of must have the shape of weights")
    y = np.empty((T, N), dtype=np.float64)
    _load().orc_moe_combine(_ptr(out), _ptr(w), _ptr(row_of), T, topk, R, N, _ptr(y))
    return y
