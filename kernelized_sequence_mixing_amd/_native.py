"""ctypes view of liblinattn.so: struct layouts, prototypes, and loading.

The shared library is loaded from this package directory (built in-tree by
``kernelized_sequence_mixing_amd.build``). There is no fallback: if it is
missing or fails to load, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblinattn.so")

LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_WORKSPACE, LA_ERR_ALIAS, LA_ERR_HIP = range(6)
LA_F32, LA_BF16 = 0, 1
LA_FMAP_ELU1, LA_FMAP_FAVOR, LA_FMAP_IDENTITY = 0, 1, 2
LA_GATE_NONE, LA_GATE_DECAY, LA_GATE_GLA, LA_GATE_SEL, LA_GATE_OUTER = 0, 1, 2, 3, 4
LA_SLOT_READ, LA_SLOT_WRITE = 1, 2

EXPORTED = ("la_abi_version", "la_status_str", "la_forward_workspace_size", "la_forward_segments",
            "la_forward", "la_forward_batch_workspace_size", "la_forward_batch", "la_backward_workspace_size",
            "la_backward", "la_decode_step", "la_feature_map_apply", "la_timing_begin", "la_timing_end",
            "la_forward_noalloc", "la_softmax_attention")
LA_NOALLOC_SCRATCH_BYTES = 32 << 20


class LaProblem(ctypes.Structure):
    _fields_ = [("B", c_int32), ("H", c_int32), ("n", c_int32), ("d_k", c_int32), ("d_v", c_int32),
                ("in_dtype", c_int32), ("out_dtype", c_int32), ("eps", c_float)]


class LaFeatureMap(ctypes.Structure):
    _fields_ = [("kind", c_int32), ("r", c_int32), ("omega", c_void_p)]


class LaGate(ctypes.Structure):
    _fields_ = [("kind", c_int32), ("tau", c_float), ("gamma", c_void_p), ("g", c_void_p), ("gv", c_void_p)]


class LaBatch(ctypes.Structure):
    _fields_ = [("cu_seqlens", c_void_p), ("num_seqs", c_int32), ("max_seqlen", c_int32), ("S", c_void_p),
                ("z", c_void_p), ("slot_ids", c_void_p), ("num_slots", c_int32), ("flags", c_int32)]


class LinattnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed: {status_name(status)} ({status})")


_lib = None


def lib():
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m kernelized_sequence_mixing_amd.build` "
                           "(the HIP library is required; there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    L.la_abi_version.restype = c_int32
    L.la_abi_version.argtypes = []
    L.la_status_str.restype = c_char_p
    L.la_status_str.argtypes = [c_int32]
    L.la_forward_workspace_size.restype = c_int32
    L.la_forward_workspace_size.argtypes = [POINTER(LaProblem), POINTER(LaFeatureMap), c_int32, POINTER(LaGate),
                                            POINTER(c_size_t)]
    L.la_forward_segments.restype = c_int32
    L.la_forward_segments.argtypes = [POINTER(LaProblem), POINTER(LaFeatureMap), c_int32, POINTER(LaGate),
                                      POINTER(c_int32), POINTER(c_int32)]
    L.la_forward.restype = c_int32
    L.la_forward.argtypes = [POINTER(LaProblem), c_void_p, c_void_p, c_void_p, POINTER(LaFeatureMap), c_int32,
                             POINTER(LaGate), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                             c_size_t, c_void_p]
    L.la_forward_batch_workspace_size.restype = c_int32
    L.la_forward_batch_workspace_size.argtypes = [POINTER(LaProblem), POINTER(LaBatch), POINTER(LaFeatureMap),
                                                  POINTER(LaGate), POINTER(c_size_t)]
    L.la_forward_batch.restype = c_int32
    L.la_forward_batch.argtypes = [POINTER(LaProblem), POINTER(LaBatch), c_void_p, c_void_p, c_void_p,
                                   POINTER(LaFeatureMap), POINTER(LaGate), c_void_p, c_void_p, c_size_t, c_void_p]
    L.la_backward_workspace_size.restype = c_int32
    L.la_backward_workspace_size.argtypes = [POINTER(LaProblem), POINTER(LaFeatureMap), c_int32, POINTER(LaGate),
                                             POINTER(c_size_t)]
    L.la_backward.restype = c_int32
    L.la_backward.argtypes = [POINTER(LaProblem), c_void_p, c_void_p, c_void_p, c_void_p, POINTER(LaFeatureMap),
                              c_int32, POINTER(LaGate), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_void_p, c_size_t, c_void_p]
    L.la_decode_step.restype = c_int32
    L.la_decode_step.argtypes = [POINTER(LaProblem), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 POINTER(LaFeatureMap), POINTER(LaGate), c_void_p, c_void_p]
    L.la_feature_map_apply.restype = c_int32
    L.la_feature_map_apply.argtypes = [POINTER(LaFeatureMap), c_int64, c_int32, c_int32, c_void_p, c_void_p,
                                       c_void_p]
    L.la_forward_noalloc.restype = c_int32
    L.la_forward_noalloc.argtypes = [POINTER(LaProblem), c_void_p, c_void_p, c_void_p, POINTER(LaFeatureMap),
                                     c_int32, POINTER(LaGate), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p]
    L.la_softmax_attention.restype = c_int32
    L.la_softmax_attention.argtypes = [POINTER(LaProblem), c_void_p, c_void_p, c_void_p, c_int32, c_float, c_void_p,
                                       c_void_p]
    L.la_timing_begin.restype = c_int32
    L.la_timing_begin.argtypes = [POINTER(c_void_p), c_int32]
    L.la_timing_end.restype = c_int32
    L.la_timing_end.argtypes = [c_void_p, POINTER(c_int32)]
    _lib = L
    return L


def status_name(status: int) -> str:
    try:
        return lib().la_status_str(status).decode()
    except Exception:  # noqa: BLE001 - naming a status must never mask the original error
        return str(status)


def check(status: int, where: str):
    if status != LA_OK:
        raise LinattnError(status, where)
