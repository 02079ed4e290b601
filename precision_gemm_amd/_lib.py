"""ctypes loader for liblora_lowp.so (argument marshalling only).

The library is built in-tree by ``precision_gemm_amd.build``.  If it is missing the
loader raises: there is no fallback implementation of any step.
"""

from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblora_lowp.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "lora_lowp.h")

_lib = None

c_i32, c_u32, c_size, c_vp = ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_void_p

_SIGNATURES = {
    "lora_status_string": (ctypes.c_char_p, [c_i32]),
    "lora_version": (ctypes.c_char_p, []),
    "lora_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32, c_i32]),
    "lora_workspace_init": (c_i32, [c_vp, c_size, c_vp]),
    "lora_workspace_status": (c_i32, [c_vp, c_vp, c_vp]),
    "lora_workspace_segment_error": (c_i32, [c_vp, c_vp, c_vp]),
    "lora_build_segments": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "lora_quant_act_mxfp8": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_vp, c_vp]),
    "lora_shrink": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_vp, c_vp, c_size, c_vp]),
    "lora_expand": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_vp, c_vp]),
    "gemm_lowp_lora_epilogue": (c_i32, [c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                        c_vp, c_vp, c_vp, c_i32, c_i32, c_vp, c_u32, c_vp, c_size, c_vp]),
    "gemm_lowp_lora_epilogue_noalloc": (c_i32, [c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp,
                                                c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_vp, c_u32, c_vp]),
    "lora_pack_weight": (c_i32, [c_i32, c_vp, c_vp, c_i32, c_i32, c_vp, c_vp, c_vp]),
    "lora_shrink_configured": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_vp,
                                       ctypes.POINTER(c_i32), c_vp]),
    "lora_pack_weight_t": (c_i32, [c_i32, c_vp, c_i32, c_i32, c_vp, c_vp]),
    "lora_pack_adapter_bwd": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]),
    "lora_backward": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                              c_vp, c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "lora_backward_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32, c_i32]),
    "lora_shrink_config_info": (c_i32, [c_i32, c_i32, c_i32, ctypes.POINTER(c_i32)]),
    "lora_shrink_bgmv_info": (c_i32, [c_i32, c_i32, c_i32, ctypes.POINTER(c_i32)]),
    "lora_merged_layer": (c_i32, [c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32,
                                  c_i32, c_vp, c_vp]),
    "lora_pack_adapter": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]),
    "lora_plan_info": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(c_i32), c_i32]),
}


def header_functions() -> list[str]:
    """Names of the functions declared in include/lora_lowp.h."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m precision_gemm_amd.build` "
                               "(there is no non-HIP implementation)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class LoraError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().lora_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != 0:
        raise LoraError(fn, status)
