"""The layer's forward captured in a HIP graph (through torch.cuda.CUDAGraph)
and replayed: every replay, with eager work of another layer in between and
with new input data written into the captured input buffer, gives the eager
result bit for bit.  The library allocates nothing and issues no memsets, so
its launches are capture-safe; this checks it on the tiled GEMM path (tiny),
on the weight-streaming path with the two-kernel router (decode_64), and with
the activation quantisation forked onto the layer's side stream (2048 tokens
and up)."""

import pytest
import torch

import routing_fp8_grouped_amd as moe
from routing_fp8_grouped_amd import configs, inputs
from tests.gpu_util import DEV, log, device_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def _layer(cfg):
    return moe.MoELayer(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.f, cfg.route_scale)


CASES = {"tiny": configs.get("tiny"), "decode_64": configs.get("decode_64"),
         "side_stream": configs.MoEConfig("side_stream", T=moe.OVERLAP_QUANT_T, d=256, E=16, G=4, M=2, k=4,
                                          f=128, seed=9)}


@pytest.mark.parametrize("name", sorted(CASES))
def test_forward_replays_in_a_graph(name):
    cfg = CASES[name]
    log(f"graph capture of the {name} forward")
    x, wg, b = inputs.host_inputs(cfg)
    W = device_weights(cfg)
    xd, wgd, bd = x.to(DEV), wg.to(DEV), b.to(DEV)
    gen = torch.Generator(device=DEV).manual_seed(5)
    x2 = torch.randn(cfg.T, cfg.d, generator=gen, device=DEV).to(torch.bfloat16)
    L, L2 = _layer(cfg), _layer(cfg)
    ref = L.forward(xd, wgd, bd, W).clone()
    ref2 = L2.forward(x2, wgd, bd, W).clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        L.forward(xd, wgd, bd, W)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.forward(xd, wgd, bd, W)
    for rep in range(3):
        L2.forward(x2, wgd, bd, W)     # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(L.out, ref), rep
        assert torch.equal(L2.out, ref2), rep
    xd.copy_(x2)                       # new data in the captured input buffer
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(L.out, ref2)
    assert torch.equal(L.idx, L2.idx) and torch.equal(L.w, L2.w)
    log("  4 replays equal to the eager results")
