"""The C ABI loads, exports every declared symbol, and rejects bad arguments
before touching a GPU (CPU only: nothing here launches a kernel)."""

import ctypes
import os
import subprocess

import pytest

from routing_fp8_grouped_amd import _lib

P = ctypes.c_void_p
A = P(0x1000)          # aligned fake device address: never dereferenced by validation
MIS = P(0x1004)        # misaligned for 16-byte matrices
MIS4 = P(0x1002)       # misaligned for FP32/int32 arrays


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def last(lib):
    return lib.moe_last_error().decode()


def test_exports_every_declared_symbol(lib):
    declared = _lib.header_symbols()
    assert set(declared) == {"moe_route", "moe_route_workspace_bytes", "moe_route_ws",
                             "fp8_quant_1x128", "fp8_quant_128x128",
                             "moe_permute_workspace_bytes", "moe_permute", "moe_permute_noalloc",
                             "grouped_gemm_fp8_swiglu", "grouped_gemm_fp8_up",
                             "grouped_gemm_fp8_down", "moe_combine", "moe_bias_update",
                             "fp8_quant_1x128_pow2", "fp8_quant_128x128_pow2",
                             "grouped_gemm_fp8_up_e8m0", "grouped_gemm_fp8_down_e8m0",
                             "grouped_gemm_fp8_up_train", "moe_transpose_fp8_blocks",
                             "moe_combine_backward", "moe_combine_backward_q",
                             "moe_wgrad_columns", "moe_regroup_128x1",
                             "moe_swiglu_backward", "grouped_gemm_fp8_wgrad",
                             "moe_roof_fp8_mfma", "moe_roof_hbm_read",
                             "moe_roof_dma_read", "moe_roof_hbm_latency",
                             "moe_status_string", "moe_last_error"}
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in declared:
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(3) == b"MOE_ERR_WORKSPACE"
    assert lib.moe_status_string(99) == b"MOE_ERR_UNKNOWN"


def rp(E=256, G=8, M=4, k=8, s=2.5):
    return _lib.RouteParams(E, G, M, k, s)


@pytest.mark.parametrize("params,d,code,msg", [
    (rp(E=0), 256, 1, "n_experts"),
    (rp(E=300), 256, 1, "n_experts"),
    (rp(E=250, G=8), 256, 1, "multiple of n_groups"),
    (rp(M=0), 256, 1, "topk_groups"),
    (rp(M=9), 256, 1, "topk_groups"),
    (rp(k=6), 256, 1, "multiple of topk_groups"),
    (rp(E=16, G=8, M=4, k=12), 256, 1, "exceeds the 2 experts of a group"),
    (rp(s=float("inf")), 256, 1, "route_scale"),
    (rp(k=0), 256, 1, "topk"),
    (rp(E=256, G=1, M=1, k=17), 256, 2, "not implemented"),
    (rp(), 100, 1, "d=100"),
    (rp(), 0, 1, "d=0"),
])
def test_route_validation(lib, params, d, code, msg):
    st = lib.moe_route(A, A, None, 10, d, params, A, A, None)
    assert st == code and msg in last(lib)


def test_route_null_and_alignment(lib):
    assert lib.moe_route(None, A, None, 10, 256, rp(), A, A, None) == 1 and "x is NULL" in last(lib)
    assert lib.moe_route(A, A, MIS4, 10, 256, rp(), A, A, None) == 1 and "bias" in last(lib)
    assert lib.moe_route(MIS, A, MIS, 10, 256, rp(), A, A, None) == 1 and "x is not 16" in last(lib)
    assert lib.moe_route(A, A, None, -1, 256, rp(), A, A, None) == 1
    # T = 0: successful no-op even with null pointers
    assert lib.moe_route(None, None, None, 0, 256, rp(), None, None, None) == 0


def test_route_ws_workspace(lib):
    assert lib.moe_route_workspace_bytes(64, 256) == 64 * 256 * 4
    assert lib.moe_route_workspace_bytes(100, 16) == 6400 + 0   # 100*16*4 rounded up to 256
    assert lib.moe_route_workspace_bytes(8192, 256) == 8192 * 256 * 4
    assert lib.moe_route_workspace_bytes(8193, 256) == 0          # single-kernel form
    assert lib.moe_route_workspace_bytes(0, 256) == 0
    assert lib.moe_route_workspace_bytes(64, 300) == 0
    # a workspace is required where the two-kernel form runs
    st = lib.moe_route_ws(A, A, None, 10, 256, rp(), A, A, None, 0, None)
    assert st == 3 and "workspace" in last(lib)
    st = lib.moe_route_ws(A, A, None, 10, 256, rp(), A, A, A, 100, None)
    assert st == 3 and "workspace" in last(lib)
    st = lib.moe_route_ws(A, A, None, 10, 256, rp(), A, A, MIS4, 1 << 20, None)
    assert st == 3 and "aligned" in last(lib)
    # the same argument checks as moe_route
    assert lib.moe_route_ws(None, A, None, 10, 256, rp(), A, A, A, 1 << 20, None) == 1
    assert lib.moe_route_ws(A, A, None, 10, 100, rp(), A, A, A, 1 << 20, None) == 1 and "d=100" in last(lib)
    assert lib.moe_route_ws(None, None, None, 0, 256, rp(), None, None, None, 0, None) == 0


def test_quant_validation(lib):
    assert lib.fp8_quant_1x128(A, 4, 100, A, A, None) == 1 and "cols=100" in last(lib)
    assert lib.fp8_quant_1x128(A, -1, 128, A, A, None) == 1
    assert lib.fp8_quant_1x128(MIS, 4, 128, A, A, None) == 1 and "aligned" in last(lib)
    assert lib.fp8_quant_1x128(None, 0, 128, None, None, None) == 0
    assert lib.fp8_quant_128x128(A, 100, 128, A, A, None) == 1 and "N=100" in last(lib)
    assert lib.fp8_quant_128x128(A, 128, 0, A, A, None) == 1
    assert lib.fp8_quant_128x128(A, 128 * 70000, 128, A, A, None) == 2
    assert lib.fp8_quant_128x128(None, 0, 128, None, None, None) == 0
    # the power-of-two variants validate the same way and name themselves
    assert lib.fp8_quant_1x128_pow2(A, 4, 100, A, A, None) == 1 and "cols=100" in last(lib)
    assert lib.fp8_quant_1x128_pow2(None, 0, 128, None, None, None) == 0
    assert lib.fp8_quant_128x128_pow2(A, 100, 128, A, A, None) == 1 and "N=100" in last(lib)
    assert lib.fp8_quant_128x128_pow2(A, 128 * 70000, 128, A, A, None) == 2


def test_permute_validation_and_workspace(lib):
    need = lib.moe_permute_workspace_bytes(1000, 8, 256)
    assert need == 4 * 256 * 4          # ceil(1000/256) blocks x E int32
    assert lib.moe_permute_workspace_bytes(0, 8, 256) == 0
    args = lambda T=1000, k=8, E=256, ws=A, wsb=need, xq_perm=None: (
        A, T, k, E, None, None, 0, A, A, A, xq_perm, None, ws, wsb, None)
    assert lib.moe_permute(*args(E=0)) == 1
    assert lib.moe_permute(*args(k=17)) == 1
    assert lib.moe_permute(*args(k=9, E=8)) == 1
    assert lib.moe_permute(*args(ws=None)) == 3 and "needed" in last(lib)
    assert lib.moe_permute(*args(wsb=need - 4)) == 3
    # asking for the row copy requires the quantised inputs and d
    assert lib.moe_permute(*args(xq_perm=A)) == 1
    assert lib.moe_permute(*args(T=0, ws=None, wsb=0)) == 0


def test_gemm_validation(lib):
    def call(n_groups=257, rows=100, d=256, f=128, a_rows=10, row_src=A, h=A):
        return lib.grouped_gemm_fp8_swiglu(A, A, a_rows, row_src, A, n_groups, rows, d, f,
                                           A, A, A, A, h, A, A, None)
    assert call(n_groups=0) == 1
    assert call(n_groups=2000) == 2
    assert call(d=100) == 1 and "d=100" in last(lib)
    assert call(f=64) == 1
    assert call(rows=-1) == 1
    assert call(a_rows=10, row_src=None) == 1 and "row_src" in last(lib)
    assert call(h=None) == 1 and "h is NULL" in last(lib)
    assert call(h=MIS) == 1
    assert call(rows=0, h=None) == 0
    # the kernels address rows and one expert's weights with 32-bit byte
    # offsets: rows x max(d, f) and 2f x d must stay below 4 GiB
    assert call(rows=599187, d=7168) == 2 and "4 GiB" in last(lib)
    assert call(rows=100, d=65536, f=32768) == 2 and "4 GiB" in last(lib)
    # the two stages validate the same way
    up = lambda rows=100, d=256, h=A, row_src=A: lib.grouped_gemm_fp8_up(
        A, A, 10, row_src, A, 257, rows, d, 128, A, A, h, A, None)
    assert up(d=100) == 1 and up(h=None) == 1 and up(row_src=None) == 1
    assert up(rows=0, h=None) == 0
    down = lambda rows=100, f=128, y=A: lib.grouped_gemm_fp8_down(
        A, A, A, 257, rows, 256, f, A, A, y, None)
    assert down(f=100) == 1 and down(y=MIS) == 1 and "y is not 16" in last(lib)
    assert down(rows=0, y=None) == 0
    up8 = lambda rows=100, d=256, h=A, row_src=A: lib.grouped_gemm_fp8_up_e8m0(
        A, A, 10, row_src, A, 257, rows, d, 128, A, A, h, A, None)
    assert up8(d=100) == 1 and up8(h=None) == 1 and up8(row_src=None) == 1
    assert up8(rows=0, h=None) == 0
    down8 = lambda rows=100, f=128, y=A: lib.grouped_gemm_fp8_down_e8m0(
        A, A, A, 257, rows, 256, f, A, A, y, None)
    assert down8(f=100) == 1 and down8(y=MIS) == 1 and "y is not 16" in last(lib)
    assert lib.grouped_gemm_fp8_up_e8m0(A, A, 10, A, A, 2000, 100, 256, 128, A, A, A, A, None) == 2


def test_combine_validation(lib):
    assert lib.moe_combine(A, A, A, 10, 0, 256, 80, None, A, None) == 1
    assert lib.moe_combine(A, A, A, 10, 8, 100, 80, None, A, None) == 1
    assert lib.moe_combine(A, A, A, 10, 8, 256, -2, None, A, None) == 1
    assert lib.moe_combine(A, None, A, 10, 8, 256, 80, None, A, None) == 1 and "pos is NULL" in last(lib)
    assert lib.moe_combine(A, A, A, 10, 8, 256, 80, MIS, A, None) == 1 and "residual" in last(lib)
    assert lib.moe_combine(None, None, None, 0, 8, 256, 0, None, None, None) == 0


def test_bias_update_validation(lib):
    assert lib.moe_bias_update(A, 0, 0.001, A, None) == 1
    assert lib.moe_bias_update(A, 256, float("inf"), A, None) == 1 and "gamma" in last(lib)
    assert lib.moe_bias_update(None, 256, 0.001, A, None) == 1 and "offsets is NULL" in last(lib)
    assert lib.moe_bias_update(A, 256, 0.001, MIS4, None) == 1


def test_error_is_thread_local(lib):
    import threading
    lib.fp8_quant_1x128(A, 4, 100, A, A, None)
    seen = {}

    def other():
        seen["msg"] = lib.moe_last_error().decode()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "cols=100" in last(lib)


def test_python_binding_requires_gpu_tensors():
    import torch
    import routing_fp8_grouped_amd as moe
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        moe.fp8_quant_1x128(x, torch.zeros(4, 128, dtype=torch.uint8), torch.zeros(4, 1))


def test_backward_validation(lib):
    assert lib.moe_wgrad_columns(1000, 3) == 128 * (1000 // 128 + 3)
    assert lib.moe_wgrad_columns(-1, 3) == 0 and lib.moe_wgrad_columns(10, 0) == 0
    assert lib.moe_transpose_fp8_blocks(A, A, 2, 100, 128, A, A, None) == 1 and "N=100" in last(lib)
    assert lib.moe_transpose_fp8_blocks(A, A, 2, 128, 128, A, A, None) == 1 and "in-place" in last(lib)
    assert lib.moe_transpose_fp8_blocks(None, None, 0, 128, 128, None, None, None) == 0
    assert lib.moe_combine_backward(A, A, A, A, 10, 0, 256, 80, A, A, None) == 1
    assert lib.moe_combine_backward(A, A, A, MIS4, 10, 8, 256, 80, A, A, None) == 1
    assert lib.moe_combine_backward(None, None, None, None, 0, 8, 256, 0, None, None, None) == 0
    # the quantising form: its two extra outputs are checked like the others
    assert lib.moe_combine_backward_q(A, A, A, A, 10, 8, 256, 80, A, A, None, A, None) == 1 \
        and "dyq is NULL" in last(lib)
    assert lib.moe_combine_backward_q(A, A, A, A, 10, 8, 256, 80, A, A, A, MIS4, None) == 1
    assert lib.moe_combine_backward_q(A, A, A, A, 10, 8, 100, 80, A, A, A, A, None) == 1 and "d=100" in last(lib)
    assert lib.moe_combine_backward_q(None, None, None, None, 0, 8, 256, 0, None, None, None, None, None) == 0
    # exactly one source for the regrouping
    assert lib.moe_regroup_128x1(A, A, A, None, A, 3, 100, 256, A, A, None) == 1 and "exactly one" in last(lib)
    assert lib.moe_regroup_128x1(None, None, A, A, A, 3, 100, 256, A, A, None) == 1 and "row_src" in last(lib)
    assert lib.moe_regroup_128x1(A, A, None, None, A, 3, 100, 100, A, A, None) == 1
    assert lib.moe_regroup_128x1(A, A, None, None, A, 2000, 100, 256, A, A, None) == 2
    assert lib.moe_swiglu_backward(A, A, A, A, 3, 100, 100, A, A, A, A, A, A, None) == 1
    assert lib.moe_swiglu_backward(A, A, None, A, 3, 100, 128, A, A, A, A, A, A, None) == 1 and "dh is NULL" in last(lib)
    assert lib.grouped_gemm_fp8_wgrad(A, A, A, A, A, 3, 100, 256, 100, A, None) == 1 and "N=100" in last(lib)
    assert lib.grouped_gemm_fp8_wgrad(A, A, A, A, A, 3, 100, 256, 256, MIS, None) == 1
    up = lambda gu=A: lib.grouped_gemm_fp8_up_train(A, A, 10, A, A, 257, 100, 256, 128, A, A, A, A, gu, A, None)
    assert up(gu=None) == 1 and "gu is NULL" in last(lib)


def test_permute_noalloc_validation(lib):
    """The allocation-free permute validates like moe_permute and refuses
    sizes beyond its static scratch (1 MiB: ceil(T/256) * E <= 262144) before
    any GPU call."""
    # T = 262145 at E = 256: 1025 blocks of histograms, 1,049,600 bytes
    st = lib.moe_permute_noalloc(A, 262145, 8, 256, None, None, 0, A, A, A, None, None, None)
    assert st == 2 and "moe_permute with a workspace" in last(lib)
    st = lib.moe_permute_noalloc(A, 100000, 8, 300, None, None, 0, A, A, A, None, None, None)
    assert st == 1 and "E=300" in last(lib)
    st = lib.moe_permute_noalloc(None, 16, 8, 256, None, None, 0, A, A, A, None, None, None)
    assert st == 1 and "idx" in last(lib)
    st = lib.moe_permute_noalloc(A, 16, 8, 256, None, None, 0, A, A, MIS4, None, None, None)
    assert st == 1 and "row_token" in last(lib)
    assert lib.moe_permute_noalloc(A, 0, 8, 256, None, None, 0, None, None, None, None, None, None) == 0


def test_roof_validation(lib):
    assert lib.moe_roof_fp8_mfma(0, 10, A, None) == 1
    assert lib.moe_roof_fp8_mfma(4, 0, A, None) == 1
    assert lib.moe_roof_fp8_mfma(4, 10, None, None) == 1 and "sink" in last(lib)
    assert lib.moe_roof_hbm_read(A, 24, 4, A, None) == 1 and "bytes" in last(lib)
    assert lib.moe_roof_hbm_read(MIS, 32, 4, A, None) == 1 and "buf" in last(lib)
    big = 32 * 7168
    assert lib.moe_roof_dma_read(A, big, 7168, 3, 4, A, None) == 1 and "ahead" in last(lib)
    assert lib.moe_roof_dma_read(A, big, 7000, 1, 4, A, None) == 1 and "K=" in last(lib)
    assert lib.moe_roof_dma_read(A, big - 1, 7168, 1, 4, A, None) == 1 and "bytes" in last(lib)
    assert lib.moe_roof_dma_read(A, big, 7168, 1, 0, A, None) == 1 and "workgroups" in last(lib)
    assert lib.moe_roof_dma_read(None, big, 7168, 1, 4, A, None) == 1 and "buf" in last(lib)
    assert lib.moe_roof_hbm_latency(A, 0, 0, 10, A, None) == 1 and "n=" in last(lib)
    assert lib.moe_roof_hbm_latency(A, 64, 64, 10, A, None) == 1 and "start" in last(lib)
    assert lib.moe_roof_hbm_latency(A, 64, 0, 0, A, None) == 1 and "steps" in last(lib)
    assert lib.moe_roof_hbm_latency(MIS4, 64, 0, 10, A, None) == 1 and "next" in last(lib)


def test_header_is_c(tmp_path, lib):
    """include/moe.h is a C header: a C11 program using every call of the
    layer (tests/c_abi_layer.c) compiles with -Wall -Wextra -Werror and links
    against libmoe.so (the GPU tier runs it)."""
    from routing_fp8_grouped_amd import build as b
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_layer.c")
    out = b.build_c_program(src, str(tmp_path / "c_abi_layer"))
    assert os.path.getsize(out) > 0
