"""ctypes declarations of libw2v2.so (include/w2v2.h).

The library must be the in-tree build next to this file.  torch is imported
first so that the library binds to the HIP runtime torch already loaded
(both carry the soname libamdhip64.so.7): device pointers and streams
handed over from torch then belong to the same runtime.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (load torch's HIP runtime before the library)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw2v2.so")

ABI_VERSION = 2
MAX_CONV = 8

OK, E_ARG, E_CONFIG, E_WEIGHTS, E_NOMEM, E_DEVICE = range(6)
STATUS_NAMES = {OK: "OK", E_ARG: "E_ARG", E_CONFIG: "E_CONFIG", E_WEIGHTS: "E_WEIGHTS",
                E_NOMEM: "E_NOMEM", E_DEVICE: "E_DEVICE"}


class Config(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32),
        ("sample_rate", ctypes.c_int32),
        ("n_conv", ctypes.c_int32),
        ("conv_dim", ctypes.c_int32 * MAX_CONV),
        ("conv_kernel", ctypes.c_int32 * MAX_CONV),
        ("conv_stride", ctypes.c_int32 * MAX_CONV),
        ("conv_bias", ctypes.c_int32),
        ("feat_norm", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("ffn", ctypes.c_int32),
        ("layers", ctypes.c_int32),
        ("pos_kernel", ctypes.c_int32),
        ("pos_groups", ctypes.c_int32),
        ("stable_layer_norm", ctypes.c_int32),
        ("vocab", ctypes.c_int32),
        ("blank_id", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("precision", ctypes.c_int32),
        ("max_batch", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("gelu_kind", ctypes.c_int32),
    ]


class Tensor(ctypes.Structure):
    _fields_ = [
        ("name", ctypes.c_char_p),
        ("data", ctypes.POINTER(ctypes.c_float)),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
    ]


class LibraryMissing(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises LibraryMissing if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(f"{LIB_PATH} is missing: build it with "
                             "`python -m wav2vec2_ctc_encoder_amd.build` (there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.w2v2_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Tensor), i32, i32, ctypes.POINTER(vp)]
    L.w2v2_create.restype = i32
    L.w2v2_destroy.argtypes = [vp]
    L.w2v2_destroy.restype = None
    L.w2v2_num_frames.argtypes = [vp, i64, ctypes.POINTER(i32)]
    L.w2v2_num_frames.restype = i32
    L.w2v2_model_info.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i64)]
    L.w2v2_model_info.restype = i32
    L.w2v2_forward.argtypes = [vp, vp, vp, i32, vp, vp, vp]
    L.w2v2_forward.restype = i32
    L.w2v2_forward_greedy.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, vp]
    L.w2v2_forward_greedy.restype = i32
    L.w2v2_forward_greedy_noalloc.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, vp]
    L.w2v2_forward_greedy_noalloc.restype = i32
    L.w2v2_calibrate.argtypes = [vp, vp, vp, i32, vp, vp, vp]
    L.w2v2_calibrate.restype = i32
    L.w2v2_forward_true_length.argtypes = [vp, vp, vp, i32, vp, vp, vp]
    L.w2v2_forward_true_length.restype = i32
    L.w2v2_forward_frontend.argtypes = [vp, vp, vp, i32, vp, vp]
    L.w2v2_forward_frontend.restype = i32
    L.w2v2_forward_encoder.argtypes = [vp, vp, i32, vp, vp]
    L.w2v2_forward_encoder.restype = i32
    L.w2v2_ctc_greedy.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp]
    L.w2v2_ctc_greedy.restype = i32
    L.w2v2_profile_enable.argtypes = [vp, i32, ctypes.c_char_p]
    L.w2v2_profile_enable.restype = i32
    L.w2v2_profile_read.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(i64), ctypes.POINTER(i32)]
    L.w2v2_profile_read.restype = i32
    L.w2v2_last_error.argtypes = []
    L.w2v2_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


EXPORTED = ("w2v2_create", "w2v2_destroy", "w2v2_num_frames", "w2v2_model_info", "w2v2_forward",
            "w2v2_forward_greedy", "w2v2_forward_greedy_noalloc", "w2v2_calibrate", "w2v2_forward_true_length", "w2v2_forward_frontend", "w2v2_forward_encoder",
            "w2v2_ctc_greedy", "w2v2_profile_enable", "w2v2_profile_read", "w2v2_last_error")


class W2V2Error(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {message}")


def check(status: int, where: str) -> None:
    if status != OK:
        msg = lib().w2v2_last_error().decode(errors="replace")
        raise W2V2Error(status, where, msg)
