"""ctypes loader for libmoe.so (built in-tree by ``routing_fp8_grouped_amd.build``).

The library is loaded on first use.  A missing library raises immediately:
there is no fallback implementation of any step.
"""

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "moe.h")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)


class MoEError(RuntimeError):
    def __init__(self, fn, status, msg):
        self.status = status
        super().__init__(f"{fn} failed: {_STATUS_NAMES.get(status, status)}: {msg}")


_STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED",
                 3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_HIP"}


class RouteParams(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int), ("n_groups", ctypes.c_int),
                ("topk_groups", ctypes.c_int), ("topk", ctypes.c_int),
                ("route_scale", ctypes.c_float)]


P = ctypes.c_void_p
I = ctypes.c_int
SZ = ctypes.c_size_t

SIGNATURES = {
    "moe_route": (I, [P, P, P, I, I, RouteParams, P, P, P]),
    "moe_route_workspace_bytes": (SZ, [I, I]),
    "moe_route_ws": (I, [P, P, P, I, I, RouteParams, P, P, P, SZ, P]),
    "fp8_quant_1x128": (I, [P, I, I, P, P, P]),
    "fp8_quant_128x128": (I, [P, I, I, P, P, P]),
    "moe_permute_workspace_bytes": (SZ, [I, I, I]),
    "moe_permute": (I, [P, I, I, I, P, P, I, P, P, P, P, P, P, SZ, P]),
    "moe_permute_noalloc": (I, [P, I, I, I, P, P, I, P, P, P, P, P, P]),
    "moe_roof_fp8_mfma": (I, [I, I, P, P]),
    "moe_roof_hbm_read": (I, [P, SZ, I, P, P]),
    "moe_roof_dma_read": (I, [P, SZ, I, I, I, P, P]),
    "moe_roof_hbm_latency": (I, [P, SZ, ctypes.c_uint32, I, P, P]),
    "grouped_gemm_fp8_swiglu": (I, [P, P, I, P, P, I, I, I, I, P, P, P, P, P, P, P, P]),
    "grouped_gemm_fp8_up": (I, [P, P, I, P, P, I, I, I, I, P, P, P, P, P]),
    "grouped_gemm_fp8_down": (I, [P, P, P, I, I, I, I, P, P, P, P]),
    "moe_combine": (I, [P, P, P, I, I, I, ctypes.c_int32, P, P, P]),
    "moe_bias_update": (I, [P, I, ctypes.c_float, P, P]),
    "fp8_quant_1x128_pow2": (I, [P, I, I, P, P, P]),
    "fp8_quant_128x128_pow2": (I, [P, I, I, P, P, P]),
    "grouped_gemm_fp8_up_e8m0": (I, [P, P, I, P, P, I, I, I, I, P, P, P, P, P]),
    "grouped_gemm_fp8_down_e8m0": (I, [P, P, P, I, I, I, I, P, P, P, P]),
    "moe_transpose_fp8_blocks": (I, [P, P, I, I, I, P, P, P]),
    "moe_combine_backward": (I, [P, P, P, P, I, I, I, ctypes.c_int32, P, P, P]),
    "moe_combine_backward_q": (I, [P, P, P, P, I, I, I, ctypes.c_int32, P, P, P, P, P]),
    "moe_wgrad_columns": (I, [I, I]),
    "moe_regroup_128x1": (I, [P, P, P, P, P, I, I, I, P, P, P]),
    "moe_swiglu_backward": (I, [P, P, P, P, I, I, I, P, P, P, P, P, P, P]),
    "grouped_gemm_fp8_wgrad": (I, [P, P, P, P, P, I, I, I, I, P, P]),
    "grouped_gemm_fp8_up_train": (I, [P, P, I, P, P, I, I, I, I, P, P, P, P, P, P, P]),
    "moe_status_string": (ctypes.c_char_p, [I]),
    "moe_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load():
    """Load libmoe.so once and attach the C signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m routing_fp8_grouped_amd.build` "
                               "(there is no fallback path)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(fn_name, status):
    if status != MOE_OK:
        msg = load().moe_last_error().decode(errors="replace")
        raise MoEError(fn_name, status, msg)


def header_symbols():
    """Function names declared in include/moe.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(?:moe_status|size_t|int|const char\*)\s+(\w+)\s*\(", text)))
