"""Seeded synthetic inputs for the MoE layer.

This module only draws random numbers and rounds them to their storage type;
it holds none of the layer's arithmetic.  Both the GPU path and the CPU oracle
receive the very same tensors from it.

Recipe (per configuration, see ``configs.py``):
  * activations X [T, d]      : BF16(N(0, 1))                     numpy PCG64, host
  * router centroids Wg [E, d]: BF16(N(0, 1/d))                   numpy PCG64, host
    - Zipf-skewed variant: Wg + beta * a (x) v, v a seeded unit vector in R^d,
      a_e = r_e^-s - mean(r^-s) for a seeded permutation r of the ranks 1..E,
      added in float32 before the BF16 rounding
  * selection bias b [E]      : FP32 U(-0.05, 0.05), or zeros      numpy PCG64, host
  * expert weights, per expert e = 0..E (E = shared), each from its own seed
    derived from the configuration's expert seed (one set shared by the V3
    workloads, as the batches of a deployed layer share its resident weights):
      W13[e] [2f, d] = BF16(N(0, 1/d))  (rows [0, f) gate W1, [f, 2f) up W3)
      W2[e]  [d, f]  = BF16(N(0, 1/d))
    drawn with torch's generator on the device that will hold them (the GPU for
    the full V3 shapes: 257 experts are 22.6 GB of BF16 before quantisation).
"""

import numpy as np
import torch


def _rng(cfg, stream):
    return np.random.default_rng([cfg.seed, stream])


def _to_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def activations(cfg, T=None, offset=0):
    """X [T, d] BF16 (host).  ``T``/``offset`` select a contiguous token range
    of the configuration's full activation matrix without changing values."""
    T = cfg.T if T is None else T
    r = _rng(cfg, 1)
    full = r.standard_normal((cfg.T if offset + T <= cfg.T else offset + T, cfg.d), dtype=np.float32)
    return _to_bf16(full[offset:offset + T])


def router_weights(cfg):
    """Wg [E, d] BF16 (host), with the optional rank-1 Zipf component."""
    r = _rng(cfg, 2)
    wg = r.standard_normal((cfg.E, cfg.d), dtype=np.float32) * np.float32(1.0 / np.sqrt(cfg.d))
    if cfg.skew_beta:
        rs = _rng(cfg, 5)
        v = rs.standard_normal(cfg.d)
        v /= np.linalg.norm(v)
        ranks = rs.permutation(cfg.E) + 1
        a = ranks.astype(np.float64) ** (-cfg.zipf_s)
        a -= a.mean()
        wg = (wg.astype(np.float64) + cfg.skew_beta * np.outer(a, v)).astype(np.float32)
    return _to_bf16(wg)


def selection_bias(cfg):
    """b [E] float32 (host)."""
    if cfg.bias == "zero":
        return torch.zeros(cfg.E, dtype=torch.float32)
    r = _rng(cfg, 3)
    return torch.from_numpy(r.uniform(-0.05, 0.05, cfg.E).astype(np.float32))


def expert_weights(cfg, e, device="cpu"):
    """(W13[e] [2f, d], W2[e] [d, f]) BF16 on ``device``; e = E is the shared expert."""
    g = torch.Generator(device=device)
    g.manual_seed(cfg.expert_seed * 4096 + 17 + e)
    std = 1.0 / float(np.sqrt(cfg.d))
    w13 = (torch.randn(2 * cfg.f, cfg.d, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)
    w2 = (torch.randn(cfg.d, cfg.f, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)
    return w13, w2


def host_inputs(cfg):
    """X, Wg, b on the host (BF16, BF16, FP32)."""
    return activations(cfg), router_weights(cfg), selection_bias(cfg)
