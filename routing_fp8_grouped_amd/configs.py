"""Workload shapes for the DeepSeek-V3 MoE-layer forward.

The V3 layer shape (the "DeepSeek-V3" summary page, section 1: N_r = 256 routed
experts, N_s = 1 shared, K_r = 8, expert hidden size 2048; node-limited routing
with M = 4 of 8 nodes; d_model = 7168 from "DeepSeek-V3: the recipe, and the
interconnect that shaped it", "The constraint, counted"; routed scaling factor
2.5 from the book's chapter 7).  Each entry also fixes the seeded synthetic input
recipe (see ``inputs.py``).
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                 # tokens
    d: int                 # model width
    E: int                 # routed experts (the shared expert is index E)
    G: int                 # expert groups
    M: int                 # groups kept per token
    k: int                 # routed experts per token
    f: int                 # expert intermediate width
    route_scale: float = 2.5
    bias: str = "uniform"  # "uniform": U(-0.05, 0.05); "zero"
    skew_beta: float = 0.0  # rank-1 Zipf component added to the router weights
    zipf_s: float = 1.1
    seed: int = 20241227
    note: str = ""
    weight_seed: int = 0    # seed of the expert weights; 0: the workload's own seed

    @property
    def expert_seed(self):
        """Seed of the expert weights: the V3 workloads share one set, as the
        batches of a deployed layer run through the same resident weights."""
        return self.weight_seed or self.seed

    @property
    def rows(self):
        """Rows of the grouped GEMM: T*k routed assignments plus T shared rows."""
        return self.T * self.k + self.T

    def gemm_flops(self):
        """Useful grouped-GEMM FLOPs: 3 matrices of d x f per row, 2 per MAC."""
        return self.rows * 6 * self.d * self.f


V3 = dict(d=7168, E=256, G=8, M=4, k=8, f=2048, weight_seed=20241227)

# The skew strength is fixed offline by tests/calibrate_zipf_skew.py (bisection so
# that the busiest routed expert receives about 4000 of the 16384*8 assignments).
ZIPF_BETA = 2.885

CONFIGS = {
    "tiny": MoEConfig("tiny", T=256, d=256, E=16, G=4, M=2, k=4, f=128, seed=20241227,
                      note="tiny layer for CPU-speed checks"),
    "prefill_4k": MoEConfig("prefill_4k", T=4096, seed=20241228, **V3,
                            note="V3 layer, prefill batch of 4096 tokens"),
    "uniform_16k": MoEConfig("uniform_16k", T=16384, bias="zero", seed=20241229, **V3,
                             note="V3 layer, 16384 tokens, near-uniform load (bias 0)"),
    "zipf_16k": MoEConfig("zipf_16k", T=16384, skew_beta=ZIPF_BETA, seed=20241230, **V3,
                          note="V3 layer, 16384 tokens, Zipf-skewed router (s=1.1)"),
    "decode_64": MoEConfig("decode_64", T=64, seed=20241231, **V3,
                           note="V3 layer, 64-token decode step (memory bound)"),
}

# Order used by the tests (smallest first).
ORDER = ["tiny", "decode_64", "prefill_4k", "uniform_16k", "zipf_16k"]


def get(name):
    return CONFIGS[name]


def with_tokens(cfg, T, name=None):
    """Same layer with a different token count (for parity at reduced size)."""
    from dataclasses import replace
    return replace(cfg, T=T, name=name or f"{cfg.name}@T{T}")
