"""ctypes handle on libmoe_route.so (the C ABI of include/moe_route.h).

There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_route.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, 1, 2, 3, 4

SYMBOLS = ("moe_status_string", "moe_workspace_bytes", "moe_expand_workspace_bytes",
           "moe_route_topk", "moe_send_counts", "moe_dispatch_permute",
           "moe_dispatch_permute_dedup", "moe_combine", "moe_coselect_counts",
           "moe_expand_counts", "moe_expand_permute", "moe_expand_reduce",
           "moe_placement_search", "moe_route_topk_softmax_all", "moe_shuffle_fit",
           "moe_shuffle_predict", "moe_shuffle_assign", "moe_route_plan",
           "moe_dispatch_permute_noalloc", "moe_route_dispatch", "moe_combine_route",
           "moe_dispatch_routed")

_lib = None


class MoeError(RuntimeError):
    def __init__(self, code: int, name: str):
        self.code = code
        super().__init__(f"{name}: {status_string(code)} (code {code})")


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m combine_top_router_select_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        L.moe_status_string.argtypes = [i32]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_workspace_bytes.argtypes = [i64, i32, i32, i32, i32]
        L.moe_workspace_bytes.restype = sz
        L.moe_route_topk.argtypes = [P, i64, i32, i32, P, P, P]
        L.moe_route_topk_softmax_all.argtypes = [P, i64, i32, i32, P, P, P]
        L.moe_send_counts.argtypes = [P, i64, i32, i32, i32, P, i32, P, P, P, P, P, sz, P]
        L.moe_route_plan.argtypes = [P, i64, i32, i32, i32, i32, P, i32, P, P, P, P, P, P, i64,
                                     P, P, sz, P]
        L.moe_dispatch_permute.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, P, sz, P, P,
                                           P, P, P, i64, P, P]
        L.moe_dispatch_permute_dedup.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, P, sz,
                                                 P, P, P, P, P, P, P, i64, P, P]
        L.moe_dispatch_permute_noalloc.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, i32, P,
                                                   P, P, P, P, P, P, P, P, P]
        L.moe_route_dispatch.argtypes = [P, P, i64, i32, i32, i32, i32, i32, P, i32, i32,
                                         P, P, P, P, P, P, P, P, P, P, P, P, P, i64, P, P, sz,
                                         P]
        L.moe_combine.argtypes = [P, P, P, i64, i32, i32, i32, P, P]
        L.moe_combine_route.argtypes = [P, P, P, i64, i32, i32, i32, P, P, i64, i32, i32, i32,
                                        i32, P, i32, P, P, P, sz, P]
        L.moe_dispatch_routed.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, i32, i32, P, P,
                                          P, P, P, P, P, P, P, P, P, i64, P, P, sz, P]
        L.moe_coselect_counts.argtypes = [P, i64, i32, i32, P, P]
        L.moe_expand_workspace_bytes.argtypes = [i64, i32, i32, i32]
        L.moe_expand_workspace_bytes.restype = sz
        L.moe_expand_counts.argtypes = [P, P, i64, i32, i32, i32, P, P, P, P, P, P, sz, P]
        L.moe_expand_permute.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, P, sz, P, i64,
                                         P, P, P, P, P]
        L.moe_expand_reduce.argtypes = [P, P, P, P, i64, i32, i32, i32, P, P]
        L.moe_placement_search.argtypes = [P, i32, i32, P, i32, P, P, P]
        L.moe_shuffle_fit.argtypes = [P, P, P, i64, i32, i32, i32, P, P, P, P]
        L.moe_shuffle_predict.argtypes = [P, P, i64, i32, i32, i32, P, P, i32, P, P]
        L.moe_shuffle_assign.argtypes = [P, i64, i32, P]
        for s in SYMBOLS[3:]:
            getattr(L, s).restype = i32
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().moe_status_string(int(code)).decode()


def check(code: int, name: str) -> None:
    if code != MOE_OK:
        raise MoeError(code, name)
