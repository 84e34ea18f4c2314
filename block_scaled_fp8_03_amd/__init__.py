"""Block-scaled FP8 linear for AMD MI355X (gfx950): Python binding.

This module only marshals torch tensors into the C ABI of ``libfp8bs.so``
(declared in ``include/fp8bs.h``); every step of the computation runs in the
library's HIP kernels.  PyTorch provides device memory and streams.

Raw entry points carry the C names and take caller-allocated outputs:
``fp8bs_act_quant``, ``fp8bs_weight_quant``, ``fp8bs_weight_dequant``,
``fp8bs_gemm``, ``fp8bs_moe_gemm``, the BF16 path ``fp8bs_w8a16_gemm`` and
the MoE dispatch/combine steps
``fp8bs_moe_route``, ``fp8bs_moe_quant_scatter``, ``fp8bs_moe_combine``.
Allocating conveniences: ``act_quant``, ``weight_quant``, ``weight_dequant``,
``fp8_gemm``, ``moe_gemm``, ``linear``, ``w8a16_gemm``, ``moe_route``,
``moe_quant_scatter``, ``moe_combine``.

The operations follow the DeepSeek-V3 inference pages ("DeepSeek-V3
Administrator & Developer Guide", sections 6.3, 6.4, 8.5.1-8.5.3; "DeepSeek-V3
User Guide", FAQ on scale_fmt ue8m0).  If the library has not been built the
calls raise; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "SCALE_FP32", "SCALE_UE8M0", "OUT_BF16", "OUT_F32", "Fp8bsError", "library_path", "lib",
    "fp8bs_act_quant", "fp8bs_weight_quant", "fp8bs_weight_dequant", "fp8bs_gemm",
    "fp8bs_moe_gemm", "fp8bs_w8a16_gemm", "fp8bs_moe_route", "fp8bs_moe_quant_scatter",
    "fp8bs_moe_combine", "w8a16_gemm", "fp8bs_gemm_ue8m0", "fp8bs_weight_quant_ue8m0",
    "fp8_gemm_ue8m0", "fp8bs_mla_absorb_key", "fp8bs_mla_absorb_value", "mla_absorb_key",
    "mla_absorb_value", "act_quant", "weight_quant", "weight_dequant", "fp8_gemm", "moe_gemm", "linear", "moe_route",
    "moe_quant_scatter", "moe_combine",
]

SCALE_FP32 = 0
SCALE_UE8M0 = 1
OUT_BF16 = 0
OUT_F32 = 1
BLOCK = 128

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8bs.so")
_lib = None


class Fp8bsError(RuntimeError):
    """A non-zero status returned by the C ABI."""

    def __init__(self, fn: str, status: int):
        msg = lib().fp8bs_status_string(status).decode()
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded ``libfp8bs.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(f"{library_path} is missing: build it with "
                           "`python -m block_scaled_fp8_03_amd.build`")
    L = ctypes.CDLL(library_path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.fp8bs_status_string.argtypes = [I]
    L.fp8bs_status_string.restype = ctypes.c_char_p
    L.fp8bs_version.restype = I
    L.fp8bs_act_quant.argtypes = [P, P, P, I64, I64, I, P]
    L.fp8bs_e4m3_encode.argtypes = [P, P, I64, P]
    L.fp8bs_weight_quant.argtypes = [P, P, P, I64, I64, P]
    L.fp8bs_weight_dequant.argtypes = [P, P, P, I64, I64, P]
    L.fp8bs_gemm.argtypes = [P, P, P, P, P, I64, I64, I64, I, P]
    L.fp8bs_moe_gemm.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I, P]
    L.fp8bs_w8a16_gemm.argtypes = [P, P, P, P, I64, I64, I64, I, P]
    L.fp8bs_gemm_ue8m0.argtypes = [P, P, P, P, P, I64, I64, I64, I, P]
    L.fp8bs_weight_quant_ue8m0.argtypes = [P, P, P, I64, I64, P]
    L.fp8bs_moe_route_workspace_size.argtypes = [I64, I64, I64]
    L.fp8bs_moe_route_workspace_size.restype = I64
    L.fp8bs_moe_route.argtypes = [P, I64, I64, I64, P, P, P, P, I64, P]
    L.fp8bs_moe_route_noalloc.argtypes = [P, I64, I64, I64, P, P, P, P]
    L.fp8bs_moe_quant_scatter.argtypes = [P, P, P, P, I64, I64, I64, I64, I, P]
    L.fp8bs_moe_combine.argtypes = [P, P, P, P, I64, I64, I64, I64, I, P]
    L.fp8bs_mla_absorb_key.argtypes = [P, I64, I64, P, P, P, I64, I64, I64, I64, I64, I, P]
    L.fp8bs_mla_absorb_value.argtypes = [P, I64, I64, P, P, P, I64, I64, I64, I64, I64, I, P]
    for fn in ("fp8bs_act_quant", "fp8bs_weight_quant", "fp8bs_weight_dequant", "fp8bs_gemm",
               "fp8bs_moe_gemm", "fp8bs_w8a16_gemm", "fp8bs_moe_route", "fp8bs_moe_quant_scatter",
               "fp8bs_moe_combine", "fp8bs_gemm_ue8m0", "fp8bs_weight_quant_ue8m0",
               "fp8bs_mla_absorb_key", "fp8bs_mla_absorb_value"):
        getattr(L, fn).restype = I
    _lib = L
    return L


# ---------------------------------------------------------------- marshalling

_F8 = (torch.float8_e4m3fn, torch.uint8)


def _need(t: torch.Tensor, dtypes, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _call(fn: str, *args) -> None:
    st = getattr(lib(), fn)(*args)
    if st != 0:
        raise Fp8bsError(fn, st)


def _fmt(scale_fmt) -> int:
    if scale_fmt in (SCALE_FP32, "fp32", None):
        return SCALE_FP32
    if scale_fmt in (SCALE_UE8M0, "ue8m0"):
        return SCALE_UE8M0
    raise ValueError(f"unknown scale_fmt {scale_fmt!r}")


def _out_code(c: torch.Tensor) -> int:
    if c.dtype == torch.bfloat16:
        return OUT_BF16
    if c.dtype == torch.float32:
        return OUT_F32
    raise TypeError(f"output dtype {c.dtype} is neither bfloat16 nor float32")


# ------------------------------------------------------- raw C-named wrappers

def fp8bs_act_quant(x: torch.Tensor, q: torch.Tensor, s: torch.Tensor, scale_fmt=SCALE_FP32) -> None:
    """x bf16 [M, K] -> q e4m3 [M, K], s float32 [M, K/128] (outputs preallocated)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x.shape
    if tuple(q.shape) != (M, K) or tuple(s.shape) != (M, K // BLOCK if K % BLOCK == 0 else -1):
        raise ValueError("q must be [M, K] and s [M, K/128]")
    _call("fp8bs_act_quant", _need(x, (torch.bfloat16,), "x"), _need(q, _F8, "q"),
          _need(s, (torch.float32,), "s"), M, K, _fmt(scale_fmt), _stream(x))


def fp8bs_weight_quant(w: torch.Tensor, q: torch.Tensor, s: torch.Tensor, scale_fmt=SCALE_FP32) -> None:
    """w bf16 [N, K] -> q e4m3 [N, K], s float32 [ceil(N/128), ceil(K/128)]
    (scale_fmt "ue8m0": power-of-two block scales)."""
    N, K = w.shape
    if tuple(q.shape) != (N, K) or tuple(s.shape) != (-(-N // BLOCK), -(-K // BLOCK)):
        raise ValueError("q must be [N, K] and s [ceil(N/128), ceil(K/128)]")
    fn = "fp8bs_weight_quant_ue8m0" if _fmt(scale_fmt) == SCALE_UE8M0 else "fp8bs_weight_quant"
    _call(fn, _need(w, (torch.bfloat16,), "w"), _need(q, _F8, "q"), _need(s, (torch.float32,), "s"),
          N, K, _stream(w))


def fp8bs_weight_dequant(w: torch.Tensor, s: torch.Tensor, y: torch.Tensor) -> None:
    """w e4m3 [N, K], s float32 [ceil(N/128), ceil(K/128)] -> y bf16 [N, K]."""
    N, K = w.shape
    if tuple(s.shape) != (-(-N // BLOCK), -(-K // BLOCK)) or tuple(y.shape) != (N, K):
        raise ValueError("s must be [ceil(N/128), ceil(K/128)] and y [N, K]")
    _call("fp8bs_weight_dequant", _need(w, _F8, "w"), _need(s, (torch.float32,), "s"),
          _need(y, (torch.bfloat16,), "y"), N, K, _stream(w))


def fp8bs_gemm(a: torch.Tensor, a_s: torch.Tensor, b: torch.Tensor, b_s: torch.Tensor,
               c: torch.Tensor, ue8m0: bool = False) -> None:
    """C [M, N] (bf16 or float32, by c.dtype) = block-scaled A [M, K] . B [N, K]^T.
    ue8m0=True calls fp8bs_gemm_ue8m0 (all scales must be powers of two)."""
    M, K = a.shape
    N, K2 = b.shape
    if K != K2 or K % BLOCK:
        raise ValueError("A and B need the same K, a multiple of 128")
    if (tuple(a_s.shape) != (M, K // BLOCK) or tuple(b_s.shape) != (-(-N // BLOCK), K // BLOCK)
            or tuple(c.shape) != (M, N)):
        raise ValueError("scale or output shape mismatch")
    _call("fp8bs_gemm_ue8m0" if ue8m0 else "fp8bs_gemm", _need(a, _F8, "a"),
          _need(a_s, (torch.float32,), "a_s"),
          _need(b, _F8, "b"), _need(b_s, (torch.float32,), "b_s"),
          _need(c, (torch.bfloat16, torch.float32), "c"), M, N, K, _out_code(c), _stream(a))


def fp8bs_moe_gemm(a: torch.Tensor, a_s: torch.Tensor, b: torch.Tensor, b_s: torch.Tensor,
                   offsets: torch.Tensor, c: torch.Tensor) -> None:
    """Grouped GEMM: rows [offsets[e], offsets[e+1]) of A use expert e's B[e]."""
    R, K = a.shape
    E, N, K2 = b.shape
    if K != K2 or K % BLOCK:
        raise ValueError("A and B need the same K, a multiple of 128")
    if (tuple(a_s.shape) != (R, K // BLOCK) or tuple(b_s.shape) != (E, -(-N // BLOCK), K // BLOCK)
            or tuple(offsets.shape) != (E + 1,) or tuple(c.shape) != (R, N)):
        raise ValueError("scale, offsets or output shape mismatch")
    _call("fp8bs_moe_gemm", _need(a, _F8, "a"), _need(a_s, (torch.float32,), "a_s"),
          _need(b, _F8, "b"), _need(b_s, (torch.float32,), "b_s"),
          _need(offsets, (torch.int32,), "offsets"),
          _need(c, (torch.bfloat16, torch.float32), "c"), R, E, N, K, _out_code(c), _stream(a))


def fp8bs_w8a16_gemm(x: torch.Tensor, w: torch.Tensor, w_s: torch.Tensor, c: torch.Tensor) -> None:
    """The BF16 path: C [M, N] = x bf16 [M, K] . weight_dequant(w e4m3 [N, K], w_s)^T."""
    M, K = x.shape
    N, K2 = w.shape
    if K != K2 or K % BLOCK:
        raise ValueError("x and w need the same K, a multiple of 128")
    if tuple(w_s.shape) != (-(-N // BLOCK), K // BLOCK) or tuple(c.shape) != (M, N):
        raise ValueError("scale or output shape mismatch")
    _call("fp8bs_w8a16_gemm", _need(x, (torch.bfloat16,), "x"), _need(w, _F8, "w"),
          _need(w_s, (torch.float32,), "w_s"), _need(c, (torch.bfloat16, torch.float32), "c"),
          M, N, K, _out_code(c), _stream(x))


def fp8bs_moe_route(indices: torch.Tensor, E: int, offsets: torch.Tensor, row_token: torch.Tensor,
                    row_of: torch.Tensor, workspace: torch.Tensor) -> None:
    """Stable counting sort of routed expert ids int32 [T, topk] by expert:
    offsets [E+1], row_token [T*topk], row_of [T, topk] (see fp8bs.h)."""
    if indices.dim() != 2:
        raise ValueError("indices must be [T, topk]")
    T, topk = indices.shape
    need = lib().fp8bs_moe_route_workspace_size(T, topk, E)
    if need < 0:
        raise ValueError("sizes out of range")
    if (tuple(offsets.shape) != (E + 1,) or tuple(row_token.shape) != (T * topk,)
            or tuple(row_of.shape) != (T, topk)):
        raise ValueError("offsets must be [E+1], row_token [T*topk] and row_of [T, topk]")
    nbytes = workspace.numel() * workspace.element_size()
    ws = _need(workspace, (torch.uint8, torch.int32), "workspace") if nbytes else None
    _call("fp8bs_moe_route", _need(indices, (torch.int32,), "indices"), T, topk, E,
          _need(offsets, (torch.int32,), "offsets"), _need(row_token, (torch.int32,), "row_token"),
          _need(row_of, (torch.int32,), "row_of"), ws, nbytes, _stream(indices))


def fp8bs_e4m3_encode(x: torch.Tensor, q: torch.Tensor) -> None:
    """The float32 -> e4m3 conversion act_quant uses (RNE, saturating at 448):
    q e4m3 [n] from x float32 [n]."""
    if x.numel() != q.numel():
        raise ValueError("x and q need the same number of elements")
    _call("fp8bs_e4m3_encode", _need(x, (torch.float32,), "x"), _need(q, _F8, "q"),
          x.numel(), _stream(x))


def fp8bs_moe_route_noalloc(indices: torch.Tensor, E: int, offsets: torch.Tensor,
                            row_token: torch.Tensor, row_of: torch.Tensor) -> None:
    """fp8bs_moe_route without a workspace: the library's own device table
    (no allocation; calls overlapping on one GPU race, see fp8bs.h)."""
    if indices.dim() != 2:
        raise ValueError("indices must be [T, topk]")
    T, topk = indices.shape
    if (tuple(offsets.shape) != (E + 1,) or tuple(row_token.shape) != (T * topk,)
            or tuple(row_of.shape) != (T, topk)):
        raise ValueError("offsets must be [E+1], row_token [T*topk] and row_of [T, topk]")
    _call("fp8bs_moe_route_noalloc", _need(indices, (torch.int32,), "indices"), T, topk, E,
          _need(offsets, (torch.int32,), "offsets"), _need(row_token, (torch.int32,), "row_token"),
          _need(row_of, (torch.int32,), "row_of"), _stream(indices))


def fp8bs_moe_quant_scatter(x: torch.Tensor, row_of: torch.Tensor, q: torch.Tensor, s: torch.Tensor,
                            scale_fmt=SCALE_FP32) -> None:
    """act_quant of each token row of x bf16 [T, K] written to its routed rows
    of q e4m3 [R, K] and s float32 [R, K/128]."""
    T, K = x.shape
    R = q.shape[0]
    if row_of.dim() != 2 or row_of.shape[0] != T:
        raise ValueError("row_of must be [T, topk]")
    if tuple(q.shape) != (R, K) or K % BLOCK or tuple(s.shape) != (R, K // BLOCK):
        raise ValueError("q must be [R, K] and s [R, K/128], K a multiple of 128")
    _call("fp8bs_moe_quant_scatter", _need(x, (torch.bfloat16,), "x"),
          _need(row_of, (torch.int32,), "row_of"), _need(q, _F8, "q"),
          _need(s, (torch.float32,), "s"), T, row_of.shape[1], R, K, _fmt(scale_fmt), _stream(x))


def fp8bs_moe_combine(out: torch.Tensor, w: torch.Tensor, row_of: torch.Tensor, y: torch.Tensor) -> None:
    """y [T, N] = sum_k w[t, k] * out[row_of[t, k]] (out bf16 [R, N], y bf16 or float32)."""
    R, N = out.shape
    T, topk = w.shape
    if tuple(row_of.shape) != (T, topk) or tuple(y.shape) != (T, N):
        raise ValueError("row_of must be [T, topk] like w, and y [T, N]")
    _call("fp8bs_moe_combine", _need(out, (torch.bfloat16,), "out"), _need(w, (torch.float32,), "w"),
          _need(row_of, (torch.int32,), "row_of"), _need(y, (torch.bfloat16, torch.float32), "y"),
          T, topk, R, N, _out_code(y), _stream(out))


# ------------------------------------------------------ allocating wrappers

def act_quant(x: torch.Tensor, scale_fmt="fp32"):
    """x bf16 [..., K] -> (e4m3 [..., K], float32 [..., K/128])."""
    K = x.shape[-1]
    x2 = x.reshape(-1, K)
    q = torch.empty(x2.shape, dtype=torch.float8_e4m3fn, device=x.device)
    s = torch.empty((x2.shape[0], K // BLOCK), dtype=torch.float32, device=x.device)
    fp8bs_act_quant(x2, q, s, scale_fmt)
    return q.view(x.shape), s.view(*x.shape[:-1], K // BLOCK)


def weight_quant(w: torch.Tensor, scale_fmt="fp32"):
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.float8_e4m3fn, device=w.device)
    s = torch.empty((-(-N // BLOCK), -(-K // BLOCK)), dtype=torch.float32, device=w.device)
    fp8bs_weight_quant(w, q, s, scale_fmt)
    return q, s


def weight_dequant(w: torch.Tensor, s: torch.Tensor) -> torch.Tensor:
    y = torch.empty(w.shape, dtype=torch.bfloat16, device=w.device)
    fp8bs_weight_dequant(w, s, y)
    return y


def fp8_gemm(a, a_s, b, b_s, out_dtype=torch.bfloat16) -> torch.Tensor:
    c = torch.empty((a.shape[0], b.shape[0]), dtype=out_dtype, device=a.device)
    fp8bs_gemm(a, a_s, b, b_s, c)
    return c


def fp8_gemm_ue8m0(a, a_s, b, b_s, out_dtype=torch.bfloat16) -> torch.Tensor:
    """fp8_gemm for power-of-two scales, the scales applied by the MFMA."""
    c = torch.empty((a.shape[0], b.shape[0]), dtype=out_dtype, device=a.device)
    fp8bs_gemm(a, a_s, b, b_s, c, ue8m0=True)
    return c


def moe_gemm(a, a_s, b, b_s, offsets, out_dtype=torch.bfloat16) -> torch.Tensor:
    c = torch.empty((a.shape[0], b.shape[1]), dtype=out_dtype, device=a.device)
    fp8bs_moe_gemm(a, a_s, b, b_s, offsets, c)
    return c


def linear(x: torch.Tensor, w: torch.Tensor, w_s: torch.Tensor, scale_fmt="fp32",
           out_dtype=torch.bfloat16) -> torch.Tensor:
    """The FP8 linear: act_quant(x) then the block-scaled GEMM with W (Admin
    guide 6.3, gemm_impl = "fp8")."""
    K = x.shape[-1]
    q, s = act_quant(x.reshape(-1, K), scale_fmt)
    y = fp8_gemm(q, s, w, w_s, out_dtype)
    return y.view(*x.shape[:-1], w.shape[0])


def moe_route(indices: torch.Tensor, E: int):
    """Routed expert ids int32 [T, topk] -> (offsets [E+1], row_token [T*topk],
    row_of [T, topk]), all int32 on the device; no host synchronisation."""
    T, topk = indices.shape
    dev = indices.device
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(T * topk, dtype=torch.int32, device=dev)
    row_of = torch.empty((T, topk), dtype=torch.int32, device=dev)
    need = lib().fp8bs_moe_route_workspace_size(T, topk, E)
    if need < 0:
        raise ValueError("sizes out of range")
    ws = torch.empty(max(need, 0), dtype=torch.uint8, device=dev)
    fp8bs_moe_route(indices, E, offsets, row_token, row_of, ws)
    return offsets, row_token, row_of


def moe_quant_scatter(x: torch.Tensor, row_of: torch.Tensor, R: int, scale_fmt="fp32"):
    """The expert inputs: (q e4m3 [R, K], s float32 [R, K/128])."""
    K = x.shape[-1]
    q = torch.empty((R, K), dtype=torch.float8_e4m3fn, device=x.device)
    s = torch.empty((R, K // BLOCK), dtype=torch.float32, device=x.device)
    fp8bs_moe_quant_scatter(x, row_of, q, s, scale_fmt)
    return q, s


def moe_combine(out: torch.Tensor, w: torch.Tensor, row_of: torch.Tensor,
                out_dtype=torch.bfloat16) -> torch.Tensor:
    y = torch.empty((w.shape[0], out.shape[1]), dtype=out_dtype, device=out.device)
    fp8bs_moe_combine(out, w, row_of, y)
    return y


def _fp8bs_mla(fn: str, inp: torch.Tensor, w: torch.Tensor, w_s: torch.Tensor, out: torch.Tensor,
               dn: int, dv: int, value_side: bool) -> None:
    if inp.dim() != 3 or w.dim() != 2:
        raise ValueError("input must be [T, H, width] and wkv_b [H*(dn+dv), R]")
    T, H, width = inp.shape
    R = w.shape[1]
    if w.shape[0] != H * (dn + dv) or width != (R if value_side else dn):
        raise ValueError("wkv_b must be [H*(dn+dv), R]; q [T, H, dn] or x [T, H, R]")
    if tuple(w_s.shape) != (-(-w.shape[0] // BLOCK), -(-R // BLOCK)):
        raise ValueError("wkv_b_s must be [H*(dn+dv)/128, R/128]")
    if tuple(out.shape) != (T, H, dv if value_side else R):
        raise ValueError("out shape mismatch")
    if inp.dtype != torch.bfloat16 or not inp.is_cuda or (width > 1 and inp.stride(2) != 1):
        raise ValueError("input must be a bf16 device tensor with a contiguous last dimension")
    _call(fn, inp.data_ptr(), inp.stride(0), inp.stride(1), _need(w, _F8, "wkv_b"),
          _need(w_s, (torch.float32,), "wkv_b_s"), _need(out, (torch.bfloat16, torch.float32), "out"),
          T, H, dn, dv, R, _out_code(out), _stream(inp))


def fp8bs_mla_absorb_key(q: torch.Tensor, w: torch.Tensor, w_s: torch.Tensor, out: torch.Tensor,
                         dn: int, dv: int) -> None:
    """q bf16 [T, H, dn] (strided token/head dims allowed, e.g. the q_nope
    slice of q) -> out [T, H, R] = q_nope absorbed through the key rows of
    the FP8 wkv_b [H*(dn+dv), R]."""
    _fp8bs_mla("fp8bs_mla_absorb_key", q, w, w_s, out, dn, dv, False)


def fp8bs_mla_absorb_value(x: torch.Tensor, w: torch.Tensor, w_s: torch.Tensor, out: torch.Tensor,
                           dn: int, dv: int) -> None:
    """x bf16 [T, H, R] (the attention-weighted latent) -> out [T, H, dv]
    through the value rows of the FP8 wkv_b [H*(dn+dv), R]."""
    _fp8bs_mla("fp8bs_mla_absorb_value", x, w, w_s, out, dn, dv, True)


def mla_absorb_key(q, w, w_s, dn: int, dv: int, out_dtype=torch.bfloat16) -> torch.Tensor:
    out = torch.empty((q.shape[0], q.shape[1], w.shape[1]), dtype=out_dtype, device=q.device)
    fp8bs_mla_absorb_key(q, w, w_s, out, dn, dv)
    return out


def mla_absorb_value(x, w, w_s, dn: int, dv: int, out_dtype=torch.bfloat16) -> torch.Tensor:
    out = torch.empty((x.shape[0], x.shape[1], dv), dtype=out_dtype, device=x.device)
    fp8bs_mla_absorb_value(x, w, w_s, out, dn, dv)
    return out


def w8a16_gemm(x: torch.Tensor, w: torch.Tensor, w_s: torch.Tensor, out_dtype=torch.bfloat16) -> torch.Tensor:
    """x bf16 [..., K] times the dequantised FP8 weight [N, K]^T -> [..., N]."""
    K = x.shape[-1]
    x2 = x.reshape(-1, K)
    c = torch.empty((x2.shape[0], w.shape[0]), dtype=out_dtype, device=x.device)
    fp8bs_w8a16_gemm(x2, w, w_s, c)
    return c.view(*x.shape[:-1], w.shape[0])
