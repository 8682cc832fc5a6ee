"""moe_permute_noalloc, the allocation-free permute, against moe_permute with
its workspace (GPU).  The two must agree bit for bit (integer work): offsets,
pos, row_token and, with the dispatch copy, the grouped FP8 rows and scales.
Two calls in a row on one GPU, the second with a smaller input, so the
second runs on the static scratch the first left behind; the first result is
also checked against the oracle's stable grouping."""

import numpy as np
import pytest
import torch

import routing_fp8_grouped_amd as moe
from oracle import permute as operm

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def _idx(rng, T, k, E):
    """k distinct ascending experts per token, skewed toward low ids."""
    p = np.exp(-np.arange(E) / (E / 3.0))
    p /= p.sum()
    return np.stack([np.sort(rng.choice(E, k, replace=False, p=p)) for _ in range(T)]).astype(np.int32)


def _run(fn, idx, E, d, rng):
    T, k = idx.shape
    rows = T * k + T
    xq = torch.from_numpy(rng.integers(0, 256, (T, d), dtype=np.uint8)).to(DEV)
    xs = torch.from_numpy(rng.uniform(0.01, 1.0, (T, d // 128)).astype(np.float32)).to(DEV)
    out = dict(offsets=torch.full((E + 2,), -7, dtype=torch.int32, device=DEV),
               pos=torch.full((T, k), -7, dtype=torch.int32, device=DEV),
               row_token=torch.full((rows,), -7, dtype=torch.int32, device=DEV),
               xq_perm=torch.zeros(rows, d, dtype=torch.uint8, device=DEV),
               xs_perm=torch.zeros(rows, d // 128, dtype=torch.float32, device=DEV))
    fn(torch.from_numpy(idx).to(DEV), E, out, xq, xs)
    torch.cuda.synchronize()
    return {k_: v.cpu() for k_, v in out.items()}, xq, xs


def _with_workspace(idx_d, E, o, xq, xs):
    T, k = idx_d.shape
    ws = torch.empty(max(16, moe.moe_permute_workspace_bytes(T, k, E)), dtype=torch.uint8, device=DEV)
    moe.moe_permute(idx_d, E, o["offsets"], o["pos"], o["row_token"], ws, xq, xs, o["xq_perm"], o["xs_perm"])


def _noalloc(idx_d, E, o, xq, xs):
    moe.moe_permute_noalloc(idx_d, E, o["offsets"], o["pos"], o["row_token"], xq, xs, o["xq_perm"],
                            o["xs_perm"])


@pytest.mark.parametrize("first,second", [((16384, 8, 256, 256), (1000, 6, 64, 128)),
                                          ((4097, 8, 256, 128), (37, 4, 16, 128))])
def test_noalloc_matches_workspace_permute(first, second):
    for n, (T, k, E, d) in enumerate((first, second)):
        print(f"[no-alloc] call {n + 1}: T={T} k={k} E={E} d={d}", flush=True)
        idx = _idx(np.random.default_rng(T + 13 * k), T, k, E)
        a, _, _ = _run(_noalloc, idx, E, d, np.random.default_rng(5))
        b, _, _ = _run(_with_workspace, idx, E, d, np.random.default_rng(5))
        for name in ("offsets", "pos", "row_token", "xq_perm", "xs_perm"):
            assert torch.equal(a[name], b[name]), name
        if n == 0:
            ro, rp, rt = operm.permute(idx, E)
            assert np.array_equal(a["offsets"].numpy(), ro)
            assert np.array_equal(a["pos"].numpy(), rp)
            assert np.array_equal(a["row_token"].numpy()[:T * k], rt)
