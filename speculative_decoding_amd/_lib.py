"""ctypes loader for libmedusa.so (built in-tree by ``speculative_decoding_amd.build``)."""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmedusa.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "medusa.h")

_lib = None

c_int, c_float, c_double, c_size_t = ctypes.c_int, ctypes.c_float, ctypes.c_double, ctypes.c_size_t
c_void_p = ctypes.c_void_p
c_char_p = ctypes.c_char_p
P_i32 = ctypes.POINTER(ctypes.c_int32)
P_u64 = ctypes.POINTER(ctypes.c_uint64)
P_f64 = ctypes.POINTER(ctypes.c_double)
PP = ctypes.POINTER(c_void_p)

# name -> (restype, argtypes); device pointers and the stream are passed as void*
_SIGS = {
    "medusa_tree_plan_create": (c_int, [P_i32, c_int, c_int, PP]),
    "medusa_tree_plan_full": (c_int, [P_i32, c_int, PP]),
    "medusa_tree_plan_from_accuracy": (c_int, [P_f64, c_int, P_i32, c_int, c_int, PP]),
    "medusa_tree_plan_info": (c_int, [c_void_p, ctypes.POINTER(c_int), ctypes.POINTER(c_int),
                                      ctypes.POINTER(c_int)]),
    "medusa_tree_plan_arrays": (c_int, [c_void_p, P_i32, P_i32, P_i32, P_u64]),
    "medusa_tree_plan_expected_accept": (c_int, [c_void_p, P_f64, c_int, c_int, P_f64]),
    "medusa_tree_plan_device_bytes": (c_size_t, [c_void_p]),
    "medusa_tree_plan_upload": (c_int, [c_void_p, c_void_p, c_size_t, c_void_p]),
    "medusa_tree_plan_destroy": (None, [c_void_p]),
    "medusa_heads_forward": (c_int, [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p, P_i32, c_int, c_void_p,
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_size_t, c_void_p]),
    "medusa_heads_workspace": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int]),
    "medusa_build_tree": (c_int, [c_void_p, c_int, c_int, c_int, P_i32, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_void_p, c_void_p]),
    "medusa_tree_attention": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_int, c_int,
                                      c_float, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                      c_void_p]),
    "medusa_attention_workspace": (c_size_t, [c_void_p, c_int, c_int, c_int, c_int, c_int,
                                              c_int]),
    "medusa_verify_accept": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_size_t, c_void_p]),
    "medusa_verify_workspace": (c_size_t, [c_void_p, c_int, c_int, c_int, c_int]),
    "medusa_verify_accept_noalloc": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_void_p,
                                             c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                             c_void_p, c_void_p, c_void_p]),
    "medusa_verify_accept_typical": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_void_p,
                                             c_void_p, c_void_p, ctypes.c_float, ctypes.c_float,
                                             ctypes.c_float, c_void_p, c_void_p, c_void_p,
                                             c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                             c_size_t, c_void_p]),
    "medusa_verify_typical_workspace": (c_size_t, [c_void_p, c_int, c_int, c_int, c_int]),
    "medusa_hbm_probe_bytes": (c_size_t, [c_size_t]),
    "medusa_hbm_read_probe": (c_int, [c_void_p, c_size_t, c_void_p, c_void_p]),
    "medusa_clock_probe": (c_int, [c_void_p, c_void_p, c_void_p]),
    "medusa_rope": (c_int, [c_int, c_int, c_int, c_int, c_int, c_void_p, ctypes.c_float, c_void_p,
                            c_void_p, c_void_p]),
    "medusa_advance": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_int, c_int, c_void_p,
                               c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                               c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "medusa_proxy_workspace": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int]),
    "medusa_proxy_qkv": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_size_t, c_void_p]),
    "medusa_proxy_out": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "medusa_status_string": (c_char_p, [c_int]),
    "medusa_last_hip_error": (c_int, []),
    "medusa_version": (c_int, []),
    "medusa_profile_enable": (c_int, [c_int]),
    "medusa_profile_reset": (c_int, []),
    "medusa_profile_only": (c_int, [c_char_p]),
    "medusa_profile_query": (c_int, [c_char_p, P_f64, ctypes.POINTER(c_int)]),
}


def header_functions():
    """Names of every function declared in include/medusa.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(medusa_[a-z0-9_]+)\s*\(", text)))


_LENIENT = False


def use_library(path: str) -> None:
    """Load `path` instead of the in-tree build, e.g. a build of an earlier revision for a
    before / after measurement; entry points that build lacks are left unbound.  Must be
    called before the first lib()."""
    global LIB_PATH, _LENIENT
    if _lib is not None:
        raise RuntimeError("the library is already loaded")
    LIB_PATH = os.path.abspath(path)
    _LENIENT = True


def lib() -> ctypes.CDLL:
    """Load libmedusa.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m speculative_decoding_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            if _LENIENT and not hasattr(L, name):
                continue
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib
