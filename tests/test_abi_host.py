"""Host-side checks of the C ABI: the library loads without a GPU, exports
every function include/fp8bs.h declares, and rejects bad arguments on the host
before any HIP call (the pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

import block_scaled_fp8_03_amd as fp8bs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bs.h")

OK, NULL, SHAPE, ALIGN, ENUM, HIP, ALIAS = 0, 1, 2, 3, 4, 5, 6
P0 = 0x100000        # fake, 16-byte aligned "device" addresses: only compared, never touched
P1 = 0x10000000
P2 = 0x20000000
P3 = 0x30000000
P4 = 0x40000000


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fp8bs.library_path):
        from block_scaled_fp8_03_amd import build
        build.build()
    return fp8bs.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(fp8bs_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("fp8bs_act_quant", "fp8bs_weight_dequant", "fp8bs_gemm", "fp8bs_moe_gemm",
              "fp8bs_weight_quant", "fp8bs_status_string", "fp8bs_version"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in range(0, 8):
        s = L.fp8bs_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert L.fp8bs_status_string(0) == b"ok"
    assert L.fp8bs_version() >= 10000


def test_act_quant_validation(L):
    f = L.fp8bs_act_quant
    assert f(P0, P1, P2, 4, 100, 0, None) == SHAPE            # K % 128
    assert f(P0, P1, P2, -1, 128, 0, None) == SHAPE
    assert f(P0, P1, P2, 4, 128, 7, None) == ENUM
    assert f(None, P1, P2, 4, 128, 0, None) == NULL
    assert f(P0, None, P2, 4, 128, 0, None) == NULL
    assert f(P0 + 8, P1, P2, 4, 128, 0, None) == ALIGN
    assert f(P0, P1 + 4, P2, 4, 128, 0, None) == ALIGN
    assert f(P0, P1, P2 + 2, 4, 128, 0, None) == ALIGN
    assert f(P0, P0 + 256, P2, 4, 128, 0, None) == ALIAS    # q inside x
    assert f(P0, P1, P1 + 64, 4, 128, 0, None) == ALIAS     # s inside q
    assert f(None, None, None, 0, 128, 0, None) == OK       # empty: no launch
    assert f(None, None, None, 5, 0, 1, None) == OK


def test_weight_quant_and_dequant_validation(L):
    for wq in (L.fp8bs_weight_quant, L.fp8bs_weight_quant_ue8m0):
        assert wq(P0, P1, P2, -3, 5, None) == SHAPE
        assert wq(None, P1, P2, 3, 5, None) == NULL
        assert wq(P0 + 2, P1, P2, 3, 5, None) == ALIGN
        assert wq(P0, P0, P2, 3, 5, None) == ALIAS
        assert wq(None, None, None, 0, 5, None) == OK
    assert L.fp8bs_weight_dequant(P0, P1, P2, 3, -5, None) == SHAPE
    assert L.fp8bs_weight_dequant(P0, None, P2, 3, 5, None) == NULL
    assert L.fp8bs_weight_dequant(P0, P1, P2 + 8, 3, 5, None) == ALIGN
    assert L.fp8bs_weight_dequant(P0, P1, P0, 3, 5, None) == ALIAS
    assert L.fp8bs_weight_dequant(None, None, None, 7, 0, None) == OK


def test_e4m3_encode_validation(L):
    f = L.fp8bs_e4m3_encode
    assert f(P0, P1, -1, None) == SHAPE
    assert f(None, None, 0, None) == OK
    assert f(None, P1, 8, None) == NULL
    assert f(P0 + 4, P1, 8, None) == ALIGN
    assert f(P0, P1 + 2, 8, None) == ALIGN
    assert f(P0, P0 + 16, 8, None) == ALIAS
    lim = ((2 ** 32 - 1) // 256) * 1024
    assert f(None, None, lim, None) == NULL
    assert f(P0, P1, lim + 1, None) == SHAPE


def test_act_quant_launch_limits(L):
    """One act_quant launch covers at most 2^32 - 1 threads: 256-thread
    workgroups of 32 blocks, so M * (K / 128) <= 16777215 * 32 = 536870880
    blocks.  Shapes just inside pass the shape check and stop at the null
    pointers; just outside they are rejected as shapes.  moe_quant_scatter
    has the same limit on its T token rows."""
    f = L.fp8bs_act_quant
    lim = ((2 ** 32 - 1) // 256) * 32
    assert f(None, None, None, lim, 128, 0, None) == NULL
    assert f(P0, P1, P2, lim + 1, 128, 0, None) == SHAPE
    assert f(None, None, None, lim // 56, 7168, 1, None) == NULL
    assert f(P0, P1, P2, lim // 56 + 1, 7168, 1, None) == SHAPE
    g = L.fp8bs_moe_quant_scatter
    assert g(None, None, None, None, lim // 2, 8, 64, 256, 0, None) == NULL
    assert g(P0, P1, P2, P3, lim // 2 + 1, 8, 64, 256, 0, None) == SHAPE


def test_route_noalloc_validation(L):
    """The workspace-free route: its table limit (1 MiB, i.e. ceil(T*topk/512)
    * E <= 262144) and the usual checks, all before any HIP call."""
    f = L.fp8bs_moe_route_noalloc
    assert f(P0, 1 << 15, 8, 1024, P1, P2, P3, None) == SHAPE      # 512 x 1024 entries
    assert f(P0, 1 << 14, 8, 1025, P1, P2, P3, None) == SHAPE      # 256 x 1025 entries
    assert f(None, 1 << 14, 8, 1024, None, None, None, None) == NULL  # 256 x 1024: fits
    assert f(P0, 4, 2, -1, P1, P2, P3, None) == SHAPE
    assert f(P0, 4, 2, 8, P1 + 2, P2, P3, None) == ALIGN
    assert f(P0, 4, 2, 8, P1, P1, P3, None) == ALIAS


def test_weight_dequant_launch_limits(L):
    """One launch covers at most 2^32 - 1 threads: N*K + 255 < 2^32 for
    K % 16 != 0, ceil(N/4) * ceil(K/1024) < 2^24 workgroups for K % 16 == 0.
    Shapes just inside pass the shape check and stop at the null pointers."""
    d = L.fp8bs_weight_dequant
    assert d(P0, P1, P2, 1 << 20, 4097, None) == SHAPE           # 4296015872 elements
    assert d(None, None, None, 1 << 20, 4095, None) == NULL      # 4293918720 + 255 < 2^32
    assert d(None, None, None, (2 ** 32 - 256) // 3, 3, None) == NULL
    assert d(P0, P1, P2, (2 ** 32 - 256) // 3 + 1, 3, None) == SHAPE
    assert d(P0, P1, P2, 1 << 26, 1024, None) == SHAPE           # 2^24 workgroups
    assert d(None, None, None, (1 << 26) - 4, 1024, None) == NULL  # 2^24 - 1
    assert d(P0, P1, P2, (1 << 26) - 3, 1024, None) == SHAPE     # ceil(N/4) = 2^24
    assert d(None, None, None, 1048592, 128, None) == NULL       # more than 2^20 rows
    assert d(None, None, None, (1 << 25) - 8, 1040, None) == NULL  # (2^23 - 2) x 2 spans
    assert d(P0, P1, P2, 1 << 25, 1040, None) == SHAPE           # 2^23 groups x 2 spans


@pytest.mark.parametrize("name", ["fp8bs_gemm", "fp8bs_gemm_ue8m0"])
def test_gemm_validation(L, name):
    g = getattr(L, name)
    assert g(P0, P1, P2, P3, P4, 4, 4, 100, 0, None) == SHAPE        # K % 128
    assert g(P0, P1, P2, P3, P4, 4, 4, 0, 0, None) == SHAPE          # K = 0
    assert g(P0, P1, P2, P3, P4, -4, 4, 128, 0, None) == SHAPE
    assert g(P0, P1, P2, P3, P4, 4, 4, 128, 2, None) == ENUM
    assert g(P0, P1, None, P3, P4, 4, 4, 128, 0, None) == NULL
    assert g(P0, P1, P2, P3, P4 + 4, 4, 4, 128, 1, None) == ALIGN
    assert g(P0, P1, P2, P3 + 1, P4, 4, 4, 128, 1, None) == ALIGN
    assert g(P0, P1, P2, P3, P0, 4, 4, 128, 1, None) == ALIAS         # C over A
    assert g(P0, P1, P2, P3, P3 - 16, 4, 4, 128, 1, None) == ALIAS    # C runs into b_s
    assert g(None, None, None, None, None, 0, 4, 128, 0, None) == OK  # M = 0
    assert g(None, None, None, None, None, 4, 0, 128, 0, None) == OK  # N = 0
    big = 1 << 25
    assert g(P0, P1, P2, P3, P4, big, 4, 128, 0, None) == SHAPE       # M*K >= 2^32


def test_moe_gemm_validation(L):
    m = L.fp8bs_moe_gemm
    assert m(P0, P1, P2, P3, P4, P4 + 4096, 8, 2, 4, 100, 0, None) == SHAPE
    assert m(P0, P1, P2, P3, P4, P4 + 4096, 8, -2, 4, 128, 0, None) == SHAPE
    assert m(P0, P1, P2, P3, P4, P4 + 4096, 8, 2, 4, 128, 9, None) == ENUM
    assert m(P0, P1, P2, P3, None, P4 + 4096, 8, 2, 4, 128, 0, None) == NULL
    assert m(P0, P1, P2, P3, P4 + 2, P4 + 4096, 8, 2, 4, 128, 0, None) == ALIGN
    assert m(P0, P1, P2, P3, P4, P0, 8, 2, 4, 128, 0, None) == ALIAS
    assert m(None, None, None, None, None, None, 0, 2, 4, 128, 0, None) == OK
    assert m(None, None, None, None, None, None, 8, 0, 4, 128, 0, None) == OK


def test_w8a16_gemm_validation(L):
    g = L.fp8bs_w8a16_gemm
    assert g(P0, P1, P2, P3, 4, 4, 100, 0, None) == SHAPE        # K % 128
    assert g(P0, P1, P2, P3, -1, 4, 128, 0, None) == SHAPE
    assert g(P0, P1, P2, P3, 4, 4, 128, 3, None) == ENUM
    assert g(P0, None, P2, P3, 4, 4, 128, 0, None) == NULL
    assert g(P0, P1, P2 + 2, P3, 4, 4, 128, 0, None) == ALIGN
    assert g(P0, P1, P2, P3 + 8, 4, 4, 128, 0, None) == ALIGN
    assert g(P0, P1, P2, P0, 4, 4, 128, 0, None) == ALIAS        # C over x
    assert g(None, None, None, None, 0, 4, 128, 0, None) == OK
    assert g(P0, P1, P2, P3, 1 << 24, 4, 128, 0, None) == SHAPE  # (M + 256) * 2K >= 2^32


def test_moe_route_validation(L):
    r = L.fp8bs_moe_route
    ws = L.fp8bs_moe_route_workspace_size
    assert ws(4096, 8, 256) == 4 * 64 * 256
    assert ws(0, 8, 256) == 0 and ws(3, 1, 5) == 4 * 1 * 5
    assert ws(-1, 8, 4) == -1 and ws(4, 0, 4) == -1 and ws(4, 8, 0) == -1 and ws(1 << 30, 8, 4) == -1
    need = ws(100, 8, 16)
    assert r(P0, 100, 8, 16, P1, P2, P3, P4, need - 4, None) == SHAPE      # workspace too small
    assert r(P0, 100, 0, 16, P1, P2, P3, P4, need, None) == SHAPE          # topk = 0
    assert r(P0, 100, 8, 16, None, P2, P3, P4, need, None) == NULL
    assert r(P0, 100, 8, 16, P1, P2, P3, None, need, None) == NULL
    assert r(P0, 100, 8, 16, P1 + 2, P2, P3, P4, need, None) == ALIGN
    assert r(P0, 100, 8, 16, P1, P2, P2 + 64, P4, need, None) == ALIAS     # row_of inside row_token
    assert r(P0, 100, 8, 16, P1, P2, P3, P0 + 64, need, None) == ALIAS     # workspace over indices


def test_moe_quant_scatter_and_combine_validation(L):
    q = L.fp8bs_moe_quant_scatter
    assert q(P0, P1, P2, P3, 4, 8, 32, 100, 0, None) == SHAPE             # K % 128
    assert q(P0, P1, P2, P3, 4, 0, 32, 128, 0, None) == SHAPE             # topk = 0
    assert q(P0, P1, P2, P3, 4, 8, 32, 128, 3, None) == ENUM
    assert q(P0, None, P2, P3, 4, 8, 32, 128, 0, None) == NULL
    assert q(P0, P1, P2 + 8, P3, 4, 8, 32, 128, 0, None) == ALIGN
    assert q(P0, P1, P1, P3, 4, 8, 32, 128, 0, None) == ALIAS             # q over row_of
    assert q(None, None, None, None, 0, 8, 32, 128, 0, None) == OK         # no tokens
    c = L.fp8bs_moe_combine
    assert c(P0, P1, P2, P3, 4, 8, 32, -1, 0, None) == SHAPE
    assert c(P0, P1, P2, P3, 4, 8, 32, 64, 5, None) == ENUM
    assert c(P0, None, P2, P3, 4, 8, 32, 64, 0, None) == NULL
    assert c(P0, P1, P2, P3 + 4, 4, 8, 32, 64, 1, None) == ALIGN
    assert c(P0, P1, P2, P0 + 128, 4, 8, 32, 64, 0, None) == ALIAS         # y inside out
    assert c(None, None, None, None, 0, 8, 32, 64, 0, None) == OK


def test_python_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises((ValueError, RuntimeError)):
        fp8bs.act_quant(x)


@pytest.mark.parametrize("name", ["fp8bs_mla_absorb_key", "fp8bs_mla_absorb_value"])
def test_mla_absorb_validation(L, name):
    f = getattr(L, name)
    H, dn, dv, R = 4, 128, 128, 512
    ld_t, ld_h = H * (R if name.endswith("value") else dn), (R if name.endswith("value") else dn)
    ok = (P0, ld_t, ld_h, P1, P2, P3, 8, H, dn, dv, R, 0, None)

    def call(**kw):
        names = ("inp", "ld_t", "ld_h", "w", "ws", "out", "T", "H", "dn", "dv", "R", "dt", "st")
        args = dict(zip(names, ok))
        args.update(kw)
        return f(*[args[n] for n in names])

    assert call(T=-1) == SHAPE
    assert call(dn=100) == SHAPE
    assert call(dv=0) == SHAPE
    assert call(R=0) == SHAPE
    assert call(ld_h=-8) == SHAPE
    if name.endswith("value"):
        assert call(R=640) == SHAPE                     # value side: R <= 512
    else:
        assert call(dn=384) == SHAPE                    # key side: dn is 128 or 256
    assert call(dt=2) == ENUM
    assert call(ld_t=ld_t + 4) == ALIGN
    assert call(ld_h=12) == ALIGN
    assert call(inp=P0 + 2) == ALIGN
    assert call(ws=P2 + 2) == ALIGN
    assert call(out=P3 + 8) == ALIGN
    assert call(w=None) == NULL
    assert call(out=P0) == ALIAS                        # out over the input
    assert call(out=P1 + 64) == ALIAS                   # out inside wkv_b
    assert call(inp=None, w=None, ws=None, out=None, T=0) == OK
    assert call(inp=None, w=None, ws=None, out=None, H=0) == OK
    assert call(H=1 << 20, T=1 << 12) == SHAPE          # output beyond 2^31 elements
