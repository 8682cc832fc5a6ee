"""GPU parity of the bias controller (moe_bias_update) against the oracle, and
the controller in a loop with the router and the permute."""

import numpy as np
import pytest
import torch

import routing_fp8_grouped_amd as moe
from oracle import balance as ob, permute as operm, route as oroute
from tests.gpu_util import DEV, log, to_np


def bf16_tensor(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("E,total,gamma,seed", [
    (256, 131072, 0.001, 0),      # V3: loads around 512
    (16, 1024, 0.05, 1),
    (1000, 8000, 0.3, 2),         # more experts than one workgroup
    (7, 21, 1e-3, 3),             # fractional mean
])
def test_bias_update_parity(E, total, gamma, seed):
    rng = np.random.default_rng(seed)
    mean = total // E                      # every case has total a multiple of E
    load = np.full(E, mean, np.int64)
    # move rows between random pairs past the first quarter (which stays at the mean)
    for _ in range(4 * E):
        i, j = rng.integers(E // 4, E, 2)
        dlt = int(rng.integers(0, load[j] // 2 + 1))
        load[i] += dlt
        load[j] -= dlt
    assert load.sum() == total and load.min() >= 0
    offsets = np.concatenate([[0], np.cumsum(load), [total + 5]]).astype(np.int32)
    bias = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    b_gpu = torch.from_numpy(bias).to(DEV)
    moe.moe_bias_update(torch.from_numpy(offsets).to(DEV), b_gpu, gamma)
    torch.cuda.synchronize()
    ref = ob.bias_update(bias, offsets, E, gamma)
    assert np.array_equal(to_np(b_gpu), ref)
    assert np.any(ref != bias)


def test_controller_loop_matches_oracle():
    """Ten steps of route -> permute -> bias update on a skewed router: the
    GPU and the oracle bias vectors stay bit-identical while no token is a
    near tie, and the load spread shrinks."""
    T, d, E, G, M, k, gamma = 256, 256, 16, 4, 2, 4, 0.02
    rng = np.random.default_rng(7)
    x = bf16_tensor(rng.standard_normal((T, d)))
    w = rng.standard_normal((E, d)) / np.sqrt(d)
    w += 1.5 * np.outer(np.linspace(1.0, -1.0, E), rng.standard_normal(d) / np.sqrt(d))
    wg = bf16_tensor(w)
    xg, wgg = x.to(DEV), wg.to(DEV)
    b_gpu = torch.zeros(E, dtype=torch.float32, device=DEV)
    b_ref = np.zeros(E, np.float32)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    wts = torch.empty(T, k, dtype=torch.float32, device=DEV)
    offsets = torch.empty(E + 2, dtype=torch.int32, device=DEV)
    pos = torch.empty(T, k, dtype=torch.int32, device=DEV)
    row_token = torch.empty(T * k + T, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(16, moe.moe_permute_workspace_bytes(T, k, E)), dtype=torch.uint8, device=DEV)
    spreads = []
    for step in range(10):
        r = oroute.route(x.float().numpy(), wg.float().numpy(), b_ref, G, M, k, 2.5)
        if r["near_tie"].any():
            log(f"  step {step}: near tie, comparison stops")
            break
        moe.moe_route(xg, wgg, b_gpu, G, M, k, 2.5, idx, wts)
        moe.moe_permute(idx, E, offsets, pos, row_token, ws)
        moe.moe_bias_update(offsets, b_gpu, gamma)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(idx), r["idx"])
        ro, _, _ = operm.permute(r["idx"], E)
        assert np.array_equal(to_np(offsets)[:E + 1], ro[:E + 1])
        load = np.diff(ro[:E + 1])
        spreads.append(int(load.max() - load.min()))
        b_ref = ob.bias_update(b_ref, ro, E, gamma)
        assert np.array_equal(to_np(b_gpu), b_ref), step
    log(f"  load spread by step: {spreads}")
    assert len(spreads) >= 3 and spreads[-1] < spreads[0]
