"""The C ABI used from C alone (GPU): tests/c_abi_layer (tests/c_abi_layer.c,
compiled by __graft_entry__.build() against include/moe.h and libmoe.so)
runs a whole layer in a process with no Python in it: buffers from hipMalloc,
the stacked weights quantised by fp8_quant_128x128, moe_route,
fp8_quant_1x128, moe_permute with the FP8 rows copied into grouped order,
grouped_gemm_fp8_swiglu and moe_combine.  Its selection, gates and output
must equal byte for byte those of the Python binding's layer on the same
inputs (the binding gathers rows inside the GEMM and calls the two expert
GEMMs separately; both forms are tested elsewhere to give the same bytes, and
the binding's layer is held to the oracle by test_gpu_layer.py)."""

import os
import subprocess

import numpy as np
import pytest
import torch

from routing_fp8_grouped_amd import configs, inputs
from tests.gpu_util import DEV, log, to_np, device_weights, run_layer

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROG = os.path.join(ROOT, "tests", "c_abi_layer")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


CASES = {
    # the tiny layer (tiled GEMM), a wider one with 64 experts (tiled GEMM),
    # and a decode-sized batch of it (weight-streaming GEMM)
    "tiny": configs.get("tiny"),
    "e64": configs.MoEConfig("e64", T=600, d=1024, E=64, G=8, M=4, k=8, f=256, seed=11),
    "e64_decode": configs.MoEConfig("e64_decode", T=8, d=1024, E=64, G=8, M=4, k=8, f=256, seed=11),
}


def raw(t):
    """Bytes of a CPU tensor (BF16 as its 16-bit patterns)."""
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.numpy().tobytes()


@pytest.mark.parametrize("name", sorted(CASES))
def test_c_program_layer_matches_binding(name, tmp_path):
    cfg = CASES[name]
    assert os.path.exists(PROG), "tests/c_abi_layer is missing: run __graft_entry__.build()"
    log(f"C ABI layer {name}: T={cfg.T} d={cfg.d} E={cfg.E} G={cfg.G} M={cfg.M} k={cfg.k} f={cfg.f}")
    x, wg, b = inputs.host_inputs(cfg)
    # the binding's weights are drawn on the GPU: the same draws, copied to the host
    w13s, w2s = zip(*((a.cpu(), c.cpu()) for a, c in (inputs.expert_weights(cfg, e, DEV)
                                                      for e in range(cfg.E + 1))))
    files = {"x.bin": raw(x), "wg.bin": raw(wg), "bias.bin": raw(b),
             "w13.bin": raw(torch.stack(w13s)), "w2.bin": raw(torch.stack(w2s))}
    for fname, data in files.items():
        (tmp_path / fname).write_bytes(data)
    args = [PROG, str(tmp_path), str(cfg.T), str(cfg.d), str(cfg.E), str(cfg.G), str(cfg.M), str(cfg.k),
            str(cfg.f), repr(float(cfg.route_scale))]
    r = subprocess.run(args, capture_output=True, text=True, timeout=120)
    log("  " + (r.stdout.strip() or r.stderr.strip()))
    assert r.returncode == 0, r.stderr
    idx = np.fromfile(tmp_path / "idx.bin", np.int32).reshape(cfg.T, cfg.k)
    w = np.fromfile(tmp_path / "w.bin", np.float32).reshape(cfg.T, cfg.k)
    out = np.fromfile(tmp_path / "out.bin", np.uint16).reshape(cfg.T, cfg.d)
    # the binding's layer on the same inputs (its weights quantised on the
    # GPU from the same BF16 values, expert by expert)
    W = device_weights(cfg)
    L = run_layer(cfg, x, wg, b, W)
    assert np.array_equal(idx, to_np(L.idx))
    assert np.array_equal(w.view(np.uint32), to_np(L.w).view(np.uint32))
    assert np.array_equal(out, L.out.cpu().view(torch.int16).numpy().view(np.uint16))
    log(f"  selection, gates and {cfg.T} x {cfg.d} output equal byte for byte")
