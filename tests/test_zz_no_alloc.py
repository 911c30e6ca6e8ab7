"""moe_permute_noalloc (no workspace: the library's static device scratch)
against moe_permute (caller's workspace) and the oracle, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input, for both
grouping paths (one workgroup up to 2048 routes; the chunked histogram
above), so the second call runs on the scratch the first one left behind.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _ids(T, K, E, seed, masked=0.0):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    if masked:
        ids[rng.random(ids.shape) < masked] = -1
    return ids


def _both(ids, offset, E_local):
    import mxfp8_mxfp4_experts_amd as m

    T, K = ids.shape
    idx = torch.from_numpy(ids).to(DEV)
    ws = torch.empty(m.moe_workspace_size(T, K, E_local, 128, 128), dtype=torch.uint8, device=DEV)
    ref = m.moe_permute(idx, offset, E_local, ws)
    got = m.moe_permute_noalloc(idx, offset, E_local)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in ref], [t.cpu().numpy() for t in got]


@pytest.mark.parametrize("first,second", [
    # (T, K, E, E_local, offset, masked fraction): chunked path (512-route
    # chunks), then one workgroup
    ((4096, 16, 896, 224, 0, 0.05), (100, 8, 64, 64, 0, 0.0)),
    # one workgroup, then a smaller one-workgroup call with an expert window
    ((120, 16, 896, 896, 0, 0.0), (7, 4, 32, 8, 8, 0.1)),
    # chunked (512-route chunks), then a smaller chunked call (256-route chunks)
    ((2048, 16, 896, 896, 0, 0.0), (300, 8, 128, 96, 16, 0.0)),
])
def test_noalloc_permute_matches_workspace_call(first, second):
    for i, (T, K, E, E_local, offset, masked) in enumerate((first, second)):
        print(f"[noalloc] call {i}: T={T} K={K} E={E} E_local={E_local} offset={offset}",
              flush=True)
        ids = _ids(T, K, E, 1000 + 7 * T + i, masked)
        ref, got = _both(ids, offset, E_local)
        for a, b, name in zip(ref, got, ("expert_offsets", "sorted_route", "route_row")):
            assert np.array_equal(a, b), name
        offs, sroute, rrow = oracle.permute(ids, offset, E_local)
        assert np.array_equal(got[0], offs)
        assert np.array_equal(got[1][:offs[-1]], sroute) and np.all(got[1][offs[-1]:] == -1)
        assert np.array_equal(got[2], rrow)


def test_noalloc_permute_rejects_sizes_past_its_scratch():
    import mxfp8_mxfp4_experts_amd as m

    # 2^18 routes over 4096 local experts: 512 chunks x 4096 experts x 4 B = 8 MiB > 4 MiB.
    idx = torch.zeros((16384, 16), dtype=torch.int32, device=DEV)
    with pytest.raises(m.MoEError) as ei:
        m.moe_permute_noalloc(idx, 0, 4096)
    assert ei.value.status == 8
