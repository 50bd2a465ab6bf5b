"""ctypes declarations of the C-ABI in include/recurrent_nn_amd.h.

Argument marshalling only: every step of the operator runs in the HIP
library.  The library must be built (recurrent_nn_amd/build.py); there is no
fallback, and loading fails loudly when it is missing.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# RNN_AMD_LIB names another build of the same library (the host-sanitizer
# build of the CPU test suite); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("RNN_AMD_LIB") or os.path.join(HERE, "librecurrent_nn_amd.so")

RNN_OK, RNN_ERR_INVALID_INPUT, RNN_ERR_UNSUPPORTED, RNN_ERR_DEVICE, RNN_ERR_OUT_OF_MEMORY = range(5)
RNN_OP_RNN, RNN_OP_GRU, RNN_OP_LSTM = 0, 1, 2
RNN_PROJ_F32, RNN_PROJ_BF16 = 0, 1
RNN_PATH_AUTO, RNN_PATH_PERSISTENT, RNN_PATH_PER_STEP = 0, 1, 2
RNN_NOALLOC_SCRATCH_BYTES = 64 << 20     # include/recurrent_nn_amd.h
RNN_NOALLOC_MAX_LENS_BATCH = 256

STATUS_NAMES = {0: "RNN_OK", 1: "RNN_ERR_INVALID_INPUT", 2: "RNN_ERR_UNSUPPORTED",
                3: "RNN_ERR_DEVICE", 4: "RNN_ERR_OUT_OF_MEMORY"}

EXPORTED = ["rnn_plan_create", "rnn_plan_workspace_size", "rnn_run", "rnn_cell_run",
            "rnn_run_noalloc", "rnn_workspace_check",
            "rnn_plan_enable_timing", "rnn_plan_last_timings", "rnn_plan_describe",
            "rnn_plan_destroy", "rnn_last_error"]


class rnn_attrs(ctypes.Structure):
    _fields_ = [
        ("op", ctypes.c_int32),
        ("direction", ctypes.c_char_p),
        ("hidden_size", ctypes.c_int64),
        ("layout", ctypes.c_int32),
        ("n_activations", ctypes.c_int32),
        ("activations", ctypes.POINTER(ctypes.c_char_p)),
        ("n_alpha", ctypes.c_int32),
        ("activation_alpha", ctypes.POINTER(ctypes.c_float)),
        ("n_beta", ctypes.c_int32),
        ("activation_beta", ctypes.POINTER(ctypes.c_float)),
        ("has_clip", ctypes.c_int32),
        ("clip", ctypes.c_float),
        ("input_forget", ctypes.c_int32),
        ("linear_before_reset", ctypes.c_int32),
        ("proj_dtype", ctypes.c_int32),
        ("constant_weights", ctypes.c_int32),
        ("kernel_path", ctypes.c_int32),
        ("units_per_block", ctypes.c_int32),
        ("batch_tile", ctypes.c_int32),
        ("waves_per_block", ctypes.c_int32),
        ("barrier_spin_limit", ctypes.c_int32),
        ("batch_halves", ctypes.c_int32),
        ("time_chunk", ctypes.c_int32),
        ("exact", ctypes.c_int32),
        ("fuse_projection", ctypes.c_int32),
    ]


class rnn_dims(ctypes.Structure):
    _fields_ = [
        ("seq_length", ctypes.c_int64),
        ("batch_size", ctypes.c_int64),
        ("input_size", ctypes.c_int64),
        ("hidden", ctypes.c_int64),
        ("num_directions", ctypes.c_int64),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python recurrent_nn_amd/build.py` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    L.rnn_plan_create.restype = i32
    L.rnn_plan_create.argtypes = [ctypes.POINTER(rnn_attrs), ctypes.POINTER(rnn_dims),
                                  ctypes.POINTER(vp)]
    L.rnn_plan_workspace_size.restype = i32
    L.rnn_plan_workspace_size.argtypes = [vp, ctypes.POINTER(sz)]
    L.rnn_run.restype = i32
    L.rnn_run.argtypes = [vp, vp, vp, sz, vp, vp, vp, vp, ctypes.POINTER(ctypes.c_int32),
                          vp, vp, vp, vp, vp, vp]
    L.rnn_cell_run.restype = i32
    L.rnn_cell_run.argtypes = [vp, vp, vp, sz, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.rnn_run_noalloc.restype = i32
    L.rnn_run_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(ctypes.c_int32),
                                  vp, vp, vp, vp, vp, vp]
    L.rnn_workspace_check.restype = i32
    L.rnn_workspace_check.argtypes = [vp, vp, vp]
    L.rnn_plan_enable_timing.restype = i32
    L.rnn_plan_enable_timing.argtypes = [vp, i32]
    L.rnn_plan_last_timings.restype = i32
    L.rnn_plan_last_timings.argtypes = [vp, ctypes.POINTER(ctypes.c_float), i32]
    L.rnn_plan_describe.restype = i32
    L.rnn_plan_describe.argtypes = [vp, ctypes.c_char_p, sz]
    L.rnn_plan_destroy.restype = None
    L.rnn_plan_destroy.argtypes = [vp]
    L.rnn_last_error.restype = ctypes.c_char_p
    L.rnn_last_error.argtypes = []
    _lib = L
    return L
