"""fp8bs_moe_route_noalloc (the route with its count table in the library's
own device array, for callers that cannot allocate) against fp8bs_moe_route
with a caller workspace: offsets, row_of and the used rows of row_token must
be identical (integer work, bit-exact).  Two calls in a row, the second with
a smaller input, so the second reads a table the first left behind."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_03_amd as fp8bs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ids(T, topk, E, seed):
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E, (T, topk)).astype(np.int32)
    idx[rng.random((T, topk)) < 0.01] = -1            # a few unrouted pairs
    idx[rng.random((T, topk)) < 0.01] = E + 3
    return torch.from_numpy(idx).to(DEV)


def _route(idx, E, noalloc):
    T, topk = idx.shape
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    row_token = torch.full((T * topk,), -7, dtype=torch.int32, device=DEV)
    row_of = torch.full((T, topk), -7, dtype=torch.int32, device=DEV)
    if noalloc:
        fp8bs.fp8bs_moe_route_noalloc(idx, E, offsets, row_token, row_of)
    else:
        ws = torch.empty(fp8bs.lib().fp8bs_moe_route_workspace_size(T, topk, E), dtype=torch.uint8,
                         device=DEV)
        fp8bs.fp8bs_moe_route(idx, E, offsets, row_token, row_of, ws)
    torch.cuda.synchronize()
    return offsets.cpu().numpy(), row_token.cpu().numpy(), row_of.cpu().numpy()


def test_route_noalloc_matches_workspace_route():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # first call: a count table of 64 x 2048 entries (512 KiB, the unfused
    # scan path); second: the 4096 x top-8 workload shape with 256 experts
    # (the fused path) and then a smaller one
    for (T, topk, E, seed) in [(4096, 8, 2048, 1), (4096, 8, 256, 2), (1000, 6, 100, 3)]:
        idx = _ids(T, topk, E, seed)
        o_ref, t_ref, r_ref = _route(idx, E, noalloc=False)
        o, t, r = _route(idx, E, noalloc=True)
        R = int(o_ref[-1])
        assert np.array_equal(o, o_ref), f"offsets T={T} E={E}"
        assert np.array_equal(r, r_ref), f"row_of T={T} E={E}"
        assert np.array_equal(t[:R], t_ref[:R]), f"row_token T={T} E={E}"
        assert np.all(t[R:] == -7), "row_token past R written"


def test_route_noalloc_rejects_oversize():
    """A table beyond the library's 1 MiB array is rejected before any launch."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    T, topk, E = 1 << 15, 8, 1024                       # 512 chunks x 1024 experts = 2 MiB
    idx = torch.zeros((T, topk), dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    row_token = torch.empty(T * topk, dtype=torch.int32, device=DEV)
    row_of = torch.empty((T, topk), dtype=torch.int32, device=DEV)
    with pytest.raises(fp8bs.Fp8bsError):
        fp8bs.fp8bs_moe_route_noalloc(idx, E, offsets, row_token, row_of)
