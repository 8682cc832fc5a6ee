"""Host-side logic (CPU): the workload table, the seeded input recipe, the
rocprofv3 summaries (kernel statistics, per-dispatch counters, the HBM-traffic
calibration) and the bench's reading of a committed traffic summary.

None of this is the layer's arithmetic; it decides what the tests feed the
kernels and what the bench reports, so it is pinned here on synthetic files
and closed forms.
"""

import csv
import dataclasses
import io
import os
import contextlib

import numpy as np
import pytest

from routing_fp8_grouped_amd import configs, inputs, profiling


# ---------------------------------------------------------------- workloads

def test_workloads_meet_the_abi_preconditions():
    assert sorted(configs.ORDER) == sorted(configs.CONFIGS)
    for name, c in configs.CONFIGS.items():
        assert c.name == name
        assert c.d % 128 == 0 and c.f % 128 == 0
        assert c.E % c.G == 0 and 1 <= c.M <= c.G
        assert 1 <= c.k <= min(c.M * c.E // c.G, 16)
        assert c.rows == c.T * c.k + c.T


def test_v3_shape_and_flop_count():
    """The V3 layer (256 routed experts in 8 groups, 4 groups and 8 experts per
    token, d 7168, f 2048) and its grouped-GEMM work at 16384 tokens:
    147456 rows x 3 matrices of d x f x 2 FLOP = 12.988 TFLOP."""
    c = configs.get("uniform_16k")
    assert (c.d, c.E, c.G, c.M, c.k, c.f, c.T) == (7168, 256, 8, 4, 8, 2048, 16384)
    assert c.rows == 147456
    assert c.gemm_flops() == 147456 * 6 * 7168 * 2048
    assert abs(c.gemm_flops() / 1e12 - 12.988) < 5e-4
    assert configs.with_tokens(c, 64).T == 64 and configs.with_tokens(c, 64).d == c.d


# ------------------------------------------------------------- input recipe

def test_inputs_are_seeded_and_sliceable():
    c = configs.get("tiny")
    x1, wg1, b1 = inputs.host_inputs(c)
    x2, wg2, b2 = inputs.host_inputs(c)
    assert x1.dtype == wg1.dtype == __import__("torch").bfloat16
    assert x1.shape == (c.T, c.d) and wg1.shape == (c.E, c.d) and b1.shape == (c.E,)
    assert x1.equal(x2) and wg1.equal(wg2) and b1.equal(b2)
    # a token range is a slice of the full matrix, values unchanged
    assert inputs.activations(c, T=17, offset=100).equal(x1[100:117])
    # experts are seeded one by one and differ from each other
    a13, a2 = inputs.expert_weights(c, 3)
    b13, b2_ = inputs.expert_weights(c, 3)
    c13, _ = inputs.expert_weights(c, c.E)          # the shared expert
    assert a13.equal(b13) and a2.equal(b2_)
    assert a13.shape == (2 * c.f, c.d) and a2.shape == (c.d, c.f)
    assert not a13.equal(c13)


def test_input_distributions():
    """X ~ N(0, 1), router and expert weights ~ N(0, 1/d), bias ~ U(-0.05, 0.05)
    or zero: moments within a few standard errors of the recipe's."""
    c = configs.get("prefill_4k")
    x = inputs.activations(c, T=512).float().numpy().astype(np.float64)
    n = x.size
    assert abs(x.mean()) < 5 / np.sqrt(n)
    assert abs(x.var() - 1.0) < 5 * np.sqrt(2.0 / n)
    wg = inputs.router_weights(c).float().numpy().astype(np.float64)
    assert abs(wg.var() * c.d - 1.0) < 5 * np.sqrt(2.0 / wg.size) + 1e-3
    b = inputs.selection_bias(c).numpy()
    assert b.min() >= -0.05 and b.max() < 0.05
    assert abs(b.mean()) < 5 * 0.1 / np.sqrt(12 * b.size)
    assert not inputs.selection_bias(configs.get("uniform_16k")).any()
    w13, w2 = inputs.expert_weights(configs.get("tiny"), 0)
    for w in (w13, w2):
        v = w.float().numpy().astype(np.float64)
        assert abs(v.var() * 256 - 1.0) < 5 * np.sqrt(2.0 / v.size) + 1e-3


def test_zipf_skew_is_a_rank_one_component():
    """The skewed router's centroids are the plain ones plus beta * a (x) v: the
    difference is rank one up to the BF16 rounding of both matrices, its
    expert factor has mean zero, and its size matches beta * |a|."""
    c = configs.get("zipf_16k")
    plain = dataclasses.replace(c, skew_beta=0.0)
    diff = (inputs.router_weights(c).double() - inputs.router_weights(plain).double()).numpy()
    u, s, _ = np.linalg.svd(diff, full_matrices=False)
    a = np.arange(1, c.E + 1, dtype=np.float64) ** (-c.zipf_s)
    a -= a.mean()
    assert abs(s[0] - c.skew_beta * np.linalg.norm(a)) < 0.01 * s[0]
    assert s[1] < 0.02 * s[0]                          # the rest is rounding noise
    u1 = u[:, 0]                                        # the expert factor, unit norm
    assert abs(u1.sum()) < 1e-2 * np.abs(u1).sum()
    # it is a permutation of the centred rank weights
    assert np.allclose(np.sort(np.abs(u1)), np.sort(np.abs(a)) / np.linalg.norm(a), atol=2e-3)


# ------------------------------------------------------- rocprofv3 summaries

GEMM = "void moe::grouped_gemm_kernel<true, false>(moe::GemmArgs, int const*)"
COPY = "void at::native::elementwise_kernel<128, 4>(int, F)"


def write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def counter_file(path, counter, dispatches):
    """dispatches: [(id, kernel name, [values of the counter's instances])]"""
    rows = []
    for disp, name, vals in dispatches:
        for v in vals:
            rows.append([disp, name, counter, v])
    write_csv(path, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)


def test_stats_table(tmp_path):
    write_csv(str(tmp_path / "run" / "x_kernel_stats.csv"),
              ["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"],
              [["void moe::combine_kernel<8>(...)", 4, 1_000_000, 250_000, 240_000, 260_000],
               [GEMM, 4, 3_000_000, 750_000, 700_000, 800_000],
               ["some_unknown_kernel", 1, 0, 0, 0, 0]])
    out = profiling.stats_table(str(tmp_path / "run"))
    assert out[0].startswith("grouped_gemm_fp8_up") and "avg      750.0 us" in out[0]
    assert out[1].startswith("moe_combine") and "share  25.0%" in out[1]
    assert out[2].startswith("some_unknown_kernel")


def test_counters_mean_per_dispatch(tmp_path):
    # one counter summed over its instances per dispatch, then averaged
    counter_file(str(tmp_path / "a" / "p_counter_collection.csv"), "SQ_WAVES",
                 [(1, GEMM, [10, 20]), (2, GEMM, [40]), (3, COPY, [999])])
    r = profiling.counters([str(tmp_path / "a")], ["grouped_gemm_kernel<true"])
    assert list(r) == ["grouped_gemm_fp8_up"]
    assert r["grouped_gemm_fp8_up"]["SQ_WAVES"] == (35.0, 2)


def traffic_dirs(tmp_path, fetch_gemm, write_gemm, copy_fetch=524288.0, copy_write=524288.0):
    f, w = str(tmp_path / "fetch"), str(tmp_path / "write")
    counter_file(os.path.join(f, "p_counter_collection.csv"), "FETCH_SIZE",
                 [(1, COPY, [copy_fetch / 2, copy_fetch / 2])]
                 + [(10 + i, GEMM, [v / 4] * 4) for i, v in enumerate(fetch_gemm)])
    counter_file(os.path.join(w, "p_counter_collection.csv"), "WRITE_SIZE",
                 [(1, COPY, [copy_write])] + [(10 + i, GEMM, [v]) for i, v in enumerate(write_gemm)])
    return f, w


def run_traffic(f, w, workload="uniform_16k"):
    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        profiling.main(["traffic", f, w, "--workload", workload, "--command-fetch", "cmd f",
                        "--command-write", "cmd w"])
    return buf.getvalue()


def test_traffic_calibration(tmp_path):
    """The copy of 1 GiB reads as 0.5 GiB of FETCH_SIZE: factor 2; the GEMM's
    KiB per launch (averaged over launches, instances summed) scale by it."""
    f, w = traffic_dirs(tmp_path, fetch_gemm=[4.0e6, 6.0e6], write_gemm=[1.0e5, 3.0e5],
                        copy_write=262144.0)
    text = run_traffic(f, w)
    vals = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line)
    assert float(vals["fetch_factor"]) == 2.0 and float(vals["write_factor"]) == 4.0
    assert float(vals["fetch_kib_per_launch"]) == 5.0e6
    assert float(vals["write_kib_per_launch"]) == 2.0e5
    want = (5.0e6 * 2.0 + 2.0e5 * 4.0) * 1024
    assert abs(float(vals["hbm_bytes_per_launch"]) - want) <= 1e-5 * want
    assert vals["kernel_source_sha256_16"] == profiling.gemm_source_hash()
    assert vals["launches"] == "2"


def test_traffic_needs_the_copy(tmp_path):
    f, w = str(tmp_path / "fetch"), str(tmp_path / "write")
    counter_file(os.path.join(f, "p_counter_collection.csv"), "FETCH_SIZE", [(10, GEMM, [1.0])])
    counter_file(os.path.join(w, "p_counter_collection.csv"), "WRITE_SIZE", [(10, GEMM, [1.0])])
    with pytest.raises(SystemExit):
        profiling.traffic(f, w)


def test_bench_reads_only_a_current_traffic_summary(tmp_path, monkeypatch):
    """bench.py reports the committed traffic figure only while the summary was
    taken on the kernel it names and on that kernel's current source."""
    import bench
    f, w = traffic_dirs(tmp_path, fetch_gemm=[1.0e6], write_gemm=[1.0e5])
    text = run_traffic(f, w, workload="synthetic_wl")
    prof = tmp_path / "root" / "profiles"
    prof.mkdir(parents=True)
    path = prof / "grouped_gemm_up_synthetic_wl_traffic.txt"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path / "root"))
    path.write_text(text)
    want = (1.0e6 * 2.0 + 1.0e5 * 2.0) * 1024
    got = bench.read_traffic("synthetic_wl", profiling.TILED)
    assert got is not None and abs(got - want) <= 1e-5 * want
    assert bench.read_traffic("synthetic_wl", profiling.STREAMING) is None      # other kernel
    assert bench.read_traffic("other_wl", profiling.TILED) is None              # no summary
    path.write_text(text.replace(profiling.gemm_source_hash(), "0" * 16))
    assert bench.read_traffic("synthetic_wl", profiling.TILED) is None          # stale source


def test_gini():
    import bench
    assert bench.gini([5, 5, 5, 5]) == 0.0
    assert abs(bench.gini([0, 0, 0, 12]) - 0.75) < 1e-12      # (n - 1) / n
    assert bench.gini([0, 0]) == 0.0
