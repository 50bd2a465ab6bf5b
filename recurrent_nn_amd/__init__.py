"""MI355X (gfx950) implementation of the ONNX recurrent operators RNN, GRU and
LSTM behind a C-ABI (include/recurrent_nn_amd.h).

This module is the thin binding: the functions named like the C entry points
marshal arguments and call them; :class:`RNNPlan` adds torch-allocated
outputs and workspace on the current device and stream.  Every step of the
operator runs in the HIP library; if the library is missing, nothing runs.
"""
from __future__ import annotations

import ctypes
import sys
from typing import Optional, Sequence, Tuple

from . import _lib
from ._lib import (RNN_OK, RNN_ERR_INVALID_INPUT, RNN_ERR_UNSUPPORTED, RNN_ERR_DEVICE,  # noqa: F401
                   RNN_ERR_OUT_OF_MEMORY, RNN_OP_RNN, RNN_OP_GRU, RNN_OP_LSTM, RNN_PROJ_F32,
                   RNN_PROJ_BF16, RNN_PATH_AUTO, RNN_PATH_PERSISTENT, RNN_PATH_PER_STEP,
                   RNN_NOALLOC_SCRATCH_BYTES, RNN_NOALLOC_MAX_LENS_BATCH, STATUS_NAMES,
                   rnn_attrs, rnn_dims)

OPS = {"RNN": RNN_OP_RNN, "GRU": RNN_OP_GRU, "LSTM": RNN_OP_LSTM}
STAGES = ("pack", "projection", "recurrence", "other")


class RNNError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = rnn_last_error()
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def _check(st: int, where: str):
    if st != RNN_OK:
        raise RNNError(st, where)


# --------------------------------------------------------------------------
# The C entry points, one Python function each (same names, same arguments).
# --------------------------------------------------------------------------

def rnn_last_error() -> str:
    return _lib.load().rnn_last_error().decode()


def rnn_plan_create(attrs: rnn_attrs, dims: rnn_dims) -> Tuple[int, Optional[int]]:
    plan = ctypes.c_void_p()
    st = _lib.load().rnn_plan_create(ctypes.byref(attrs), ctypes.byref(dims), ctypes.byref(plan))
    return st, plan.value


def rnn_plan_workspace_size(plan: int) -> Tuple[int, int]:
    n = ctypes.c_size_t()
    st = _lib.load().rnn_plan_workspace_size(plan, ctypes.byref(n))
    return st, n.value


def rnn_run(plan: int, stream: int, workspace: int, workspace_bytes: int, X: int, W: int, R: int,
            B: int = 0, sequence_lens=None, initial_h: int = 0, initial_c: int = 0, P: int = 0,
            Y: int = 0, Y_h: int = 0, Y_c: int = 0) -> int:
    """Device pointers as ints (0 = NULL); sequence_lens a host int32 array
    object exposing ctypes (numpy array, ctypes array) or None."""
    return _lib.load().rnn_run(plan, stream, workspace, workspace_bytes, X, W, R, B,
                               _lens_ptr(sequence_lens), initial_h, initial_c, P, Y, Y_h, Y_c)


def _lens_ptr(sequence_lens):
    lens_p = ctypes.POINTER(ctypes.c_int32)()
    if sequence_lens is not None:
        if hasattr(sequence_lens, "ctypes"):
            lens_p = sequence_lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        else:
            lens_p = ctypes.cast(sequence_lens, ctypes.POINTER(ctypes.c_int32))
    return lens_p


def rnn_run_noalloc(plan: int, stream: int, X: int, W: int, R: int, B: int = 0,
                    sequence_lens=None, initial_h: int = 0, initial_c: int = 0, P: int = 0,
                    Y: int = 0, Y_h: int = 0, Y_c: int = 0) -> int:
    """rnn_run without a workspace (the library's own per-GPU scratch)."""
    return _lib.load().rnn_run_noalloc(plan, stream, X, W, R, B, _lens_ptr(sequence_lens),
                                       initial_h, initial_c, P, Y, Y_h, Y_c)


def rnn_cell_run(plan: int, stream: int, workspace: int, workspace_bytes: int, X: int, H: int,
                 C: int, W: int, R: int, B_sum: int, P: int, H_out: int, C_out: int) -> int:
    """Device pointers as ints (0 = NULL)."""
    return _lib.load().rnn_cell_run(plan, stream, workspace, workspace_bytes, X, H, C, W, R, B_sum,
                                    P, H_out, C_out)


def rnn_workspace_check(plan: int, stream: int, workspace: int) -> int:
    return _lib.load().rnn_workspace_check(plan, stream, workspace)


def rnn_plan_enable_timing(plan: int, enable: bool) -> int:
    return _lib.load().rnn_plan_enable_timing(plan, 1 if enable else 0)


def rnn_plan_last_timings(plan: int, n: int = 4) -> Tuple[int, list]:
    buf = (ctypes.c_float * n)()
    st = _lib.load().rnn_plan_last_timings(plan, buf, n)
    return st, list(buf)


def rnn_plan_describe(plan: int) -> str:
    buf = ctypes.create_string_buffer(512)
    _check(_lib.load().rnn_plan_describe(plan, buf, 512), "rnn_plan_describe")
    return buf.value.decode()


def rnn_plan_destroy(plan: Optional[int]) -> None:
    if plan:
        _lib.load().rnn_plan_destroy(plan)


# --------------------------------------------------------------------------
# Convenience: attributes from Python values, torch-managed memory.
# --------------------------------------------------------------------------

def make_attrs(op: str, direction: str = "forward", hidden_size: int = 0, layout: int = 0,
               activations: Optional[Sequence[str]] = None,
               activation_alpha: Optional[Sequence[float]] = None,
               activation_beta: Optional[Sequence[float]] = None, clip: Optional[float] = None,
               input_forget: int = 0, linear_before_reset: int = 0, proj_bf16: bool = False,
               constant_weights: bool = False, kernel_path: int = RNN_PATH_AUTO,
               units_per_block: int = 0, batch_tile: int = 0, waves_per_block: int = 0,
               barrier_spin_limit: int = 0, batch_halves: int = 0, time_chunk: int = 0,
               exact: bool = False, fuse_projection: int = 0):
    """Returns (attrs, keepalive); keep `keepalive` alive while attrs is used."""
    keep = []
    a = rnn_attrs()
    a.op = OPS[op]
    a.direction = direction.encode() if direction is not None else None
    keep.append(a.direction)
    a.hidden_size = hidden_size
    a.layout = layout
    if activations:
        arr = (ctypes.c_char_p * len(activations))(*[s.encode() for s in activations])
        keep.append(arr)
        a.n_activations = len(activations)
        a.activations = ctypes.cast(arr, ctypes.POINTER(ctypes.c_char_p))
    if activation_alpha:
        arr = (ctypes.c_float * len(activation_alpha))(*activation_alpha)
        keep.append(arr)
        a.n_alpha = len(activation_alpha)
        a.activation_alpha = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
    if activation_beta:
        arr = (ctypes.c_float * len(activation_beta))(*activation_beta)
        keep.append(arr)
        a.n_beta = len(activation_beta)
        a.activation_beta = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
    a.has_clip = 1 if clip is not None else 0
    a.clip = float(clip) if clip is not None else 0.0
    a.input_forget = input_forget
    a.linear_before_reset = linear_before_reset
    a.proj_dtype = RNN_PROJ_BF16 if proj_bf16 else RNN_PROJ_F32
    a.constant_weights = 1 if constant_weights else 0
    a.kernel_path = kernel_path
    a.units_per_block = units_per_block
    a.batch_tile = batch_tile
    a.waves_per_block = waves_per_block
    a.barrier_spin_limit = barrier_spin_limit
    a.batch_halves = batch_halves
    a.time_chunk = time_chunk
    a.exact = 1 if exact else 0
    a.fuse_projection = fuse_projection
    return a, keep


class RNNPlan:
    """A plan for one operator configuration.  ``run`` takes torch tensors on
    the current HIP device and returns (Y, Y_h, Y_c) as new torch tensors."""

    def __init__(self, op: str, seq: int, batch: int, input_size: int, hidden: int,
                 num_directions: Optional[int] = None, direction: str = "forward", **attrs):
        self.op = op
        self.direction = direction
        self.layout = attrs.get("layout", 0)
        D = num_directions if num_directions is not None else (2 if direction == "bidirectional" else 1)
        self.dims = rnn_dims(seq, batch, input_size, hidden, D)
        self.attrs, self._keep = make_attrs(op, direction, **attrs)
        st, plan = rnn_plan_create(self.attrs, self.dims)
        _check(st, "rnn_plan_create")
        self.plan = plan
        st, self.workspace_bytes = rnn_plan_workspace_size(plan)
        _check(st, "rnn_plan_workspace_size")
        self._ws = None

    def close(self) -> None:
        """Release the plan (rnn_plan_destroy) and drop the workspace tensor.
        Idempotent.  Call it, or use the plan as a context manager, before the
        process exits: the library's HIP objects (timing events, the pinned
        staging of sequence_lens) are then released while the HIP runtime is
        still fully alive."""
        plan, self.plan = getattr(self, "plan", None), None
        self._ws = None
        if plan:
            rnn_plan_destroy(plan)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
        return False

    def __del__(self, _finalizing=sys.is_finalizing):
        # During interpreter shutdown the HIP runtime and the profiler hooks
        # that wrap it may already be torn down (and this module's globals
        # cleared): make no library call then; the process is ending and its
        # memory goes with it.
        if getattr(self, "plan", None) is None or _finalizing():
            return
        try:
            self.close()
        except Exception:
            pass

    def describe(self) -> str:
        return rnn_plan_describe(self.plan)

    def workspace(self, device=None):
        import torch
        if self._ws is None and self.workspace_bytes > 0:
            self._ws = torch.empty(self.workspace_bytes, dtype=torch.uint8,
                                   device=device if device is not None else "cuda")
        return self._ws

    def output_shapes(self):
        S, Bt, _, H, D = (self.dims.seq_length, self.dims.batch_size, self.dims.input_size,
                          self.dims.hidden, self.dims.num_directions)
        if self.layout == 0:
            return (S, D, Bt, H), (D, Bt, H)
        return (Bt, S, D, H), (Bt, D, H)

    def enable_timing(self, on: bool = True):
        _check(rnn_plan_enable_timing(self.plan, on), "rnn_plan_enable_timing")

    def last_timings(self) -> dict:
        st, v = rnn_plan_last_timings(self.plan, len(STAGES))
        _check(st, "rnn_plan_last_timings")
        return dict(zip(STAGES, v))

    def check(self, stream=None):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        _check(rnn_workspace_check(self.plan, s.cuda_stream, self._ptr(self._ws)),
               "rnn_workspace_check")

    @staticmethod
    def _ptr(t) -> int:
        return 0 if t is None else t.data_ptr()

    def run(self, X, W, R, B=None, sequence_lens=None, initial_h=None, initial_c=None, P=None,
            want_y: bool = True, want_yh: bool = True, want_yc: Optional[bool] = None,
            out=None, stream=None, noalloc: bool = False):
        """Enqueue one invocation on `stream` (default: torch's current stream).
        sequence_lens: host int32 tensor/array or None.  `out` may supply
        preallocated (Y, Y_h, Y_c).  noalloc: through rnn_run_noalloc (no
        workspace; with `out` given, nothing is allocated at all)."""
        import numpy as np
        import torch
        for name, t in (("X", X), ("W", W), ("R", R), ("B", B), ("initial_h", initial_h),
                        ("initial_c", initial_c), ("P", P)):
            if t is not None:
                if t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
                    raise ValueError(f"{name} must be a contiguous float32 device tensor")
        if want_yc is None:
            want_yc = self.op == "LSTM"
        dev = X.device
        ysh, ssh = self.output_shapes()
        if out is not None:
            Y, Yh, Yc = out
        else:
            Y = torch.empty(ysh, dtype=torch.float32, device=dev) if want_y else None
            Yh = torch.empty(ssh, dtype=torch.float32, device=dev) if want_yh else None
            Yc = torch.empty(ssh, dtype=torch.float32, device=dev) if want_yc else None
        lens = None
        if sequence_lens is not None:
            if hasattr(sequence_lens, "numpy"):
                sequence_lens = sequence_lens.cpu().numpy()
            lens = np.ascontiguousarray(sequence_lens, dtype=np.int32)
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        if noalloc:
            st = rnn_run_noalloc(self.plan, s.cuda_stream, self._ptr(X), self._ptr(W),
                                 self._ptr(R), self._ptr(B), lens, self._ptr(initial_h),
                                 self._ptr(initial_c), self._ptr(P), self._ptr(Y), self._ptr(Yh),
                                 self._ptr(Yc))
            _check(st, "rnn_run_noalloc")
            return Y, Yh, Yc
        ws = self.workspace(dev)
        st = rnn_run(self.plan, s.cuda_stream, self._ptr(ws), self.workspace_bytes,
                     self._ptr(X), self._ptr(W), self._ptr(R), self._ptr(B), lens,
                     self._ptr(initial_h), self._ptr(initial_c), self._ptr(P),
                     self._ptr(Y), self._ptr(Yh), self._ptr(Yc))
        _check(st, "rnn_run")
        return Y, Yh, Yc


class RNNCell(RNNPlan):
    """One step in the single-cell convention (rnn_cell_run): summed bias,
    new state only.  ``op`` "RNN", "GRU" or "LSTM"; attributes as RNNPlan."""

    def __init__(self, op: str, batch: int, input_size: int, hidden: int, **attrs):
        super().__init__(op, 1, batch, input_size, hidden, num_directions=1, direction="forward",
                         **attrs)

    def step(self, X, W, R, B_sum=None, H=None, C=None, P=None, out=None, stream=None):
        """X [batch, input], W [G*hidden, input], R [G*hidden, hidden],
        B_sum [G*hidden], H / C [batch, hidden] (torch device tensors);
        returns (H_out, C_out or None)."""
        import torch
        for name, t in (("X", X), ("W", W), ("R", R), ("B_sum", B_sum), ("H", H), ("C", C),
                        ("P", P)):
            if t is not None:
                if t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
                    raise ValueError(f"{name} must be a contiguous float32 device tensor")
        dev = X.device
        Bt, Hd = self.dims.batch_size, self.dims.hidden
        if out is not None:
            Ho, Co = out
        else:
            Ho = torch.empty((Bt, Hd), dtype=torch.float32, device=dev)
            Co = torch.empty((Bt, Hd), dtype=torch.float32, device=dev) if self.op == "LSTM" else None
        ws = self.workspace(dev)
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        p = self._ptr
        st = rnn_cell_run(self.plan, s.cuda_stream, p(ws), self.workspace_bytes, p(X), p(H), p(C),
                          p(W), p(R), p(B_sum), p(P), p(Ho), p(Co))
        _check(st, "rnn_cell_run")
        return Ho, Co


def plan_for_case(case, **extra) -> RNNPlan:
    """An RNNPlan for a ``workloads.Case``-like object (attribute names as there)."""
    return RNNPlan(case.op, case.seq, case.batch, case.input, case.hidden,
                   num_directions=int(case.W.shape[0]), direction=case.direction,
                   hidden_size=case.hidden_size_attr, layout=case.layout,
                   activations=case.activations, activation_alpha=case.alpha,
                   activation_beta=case.beta, clip=case.clip, input_forget=case.input_forget,
                   linear_before_reset=case.linear_before_reset, proj_bf16=case.proj_bf16,
                   **extra)


def run_case(case, plan: Optional[RNNPlan] = None, device="cuda", **extra):
    """Copy a CPU case to the device, run it, return (Y, Y_h, Y_c) device tensors."""
    own = plan is None
    p = plan_for_case(case, **extra) if own else plan
    t = {k: (v.to(device) if v is not None and k != "sequence_lens" else v)
         for k, v in case.tensors().items()}
    try:
        return p.run(t["X"], t["W"], t["R"], t["B"], t["sequence_lens"], t["initial_h"],
                     t["initial_c"], t["P"])
    finally:
        if own:
            # (torch's allocator keeps the workspace for work already enqueued
            # on this stream; the plan's own staging is waited for on release)
            p.close()
