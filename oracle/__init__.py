"""ctypes wrapper of the CPU oracle (librnn_oracle.so, built from rnn_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg.  The HIP library never imports or links it and
this module imports nothing from the HIP library.  It takes numpy / torch CPU
arrays and returns numpy float32 arrays.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# RNN_ORACLE_LIB lets the mutation test load a deliberately broken build.
_LIB_PATH = os.environ.get("RNN_ORACLE_LIB") or os.path.join(_HERE, "librnn_oracle.so")

OK, INVALID_INPUT, UNSUPPORTED, NO_MEMORY = 0, 1, 2, 4
OPS = {"RNN": 0, "GRU": 1, "LSTM": 2}
ACT_KINDS = ["Sigmoid", "Tanh", "Relu", "Affine", "LeakyRelu", "ThresholdedRelu",
             "ScaledTanh", "HardSigmoid", "Elu", "Softsign", "Softplus"]


class OracleError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"oracle status {status}: {msg}")
        self.status = status


class _Attrs(ctypes.Structure):
    _fields_ = [
        ("op", ctypes.c_int32),
        ("direction", ctypes.c_char_p),
        ("hidden_size", ctypes.c_int64),
        ("layout", ctypes.c_int32),
        ("n_activations", ctypes.c_int32),
        ("activations", ctypes.POINTER(ctypes.c_char_p)),
        ("n_alpha", ctypes.c_int32),
        ("alpha", ctypes.POINTER(ctypes.c_float)),
        ("n_beta", ctypes.c_int32),
        ("beta", ctypes.POINTER(ctypes.c_float)),
        ("has_clip", ctypes.c_int32),
        ("clip", ctypes.c_float),
        ("input_forget", ctypes.c_int32),
        ("linear_before_reset", ctypes.c_int32),
        ("proj_bf16", ctypes.c_int32),
        ("constant_weights", ctypes.c_int32),
    ]


class _Act(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("alpha", ctypes.c_float), ("beta", ctypes.c_float)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b  # noqa: F401  (oracle/build.py)
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        fp = ctypes.POINTER(ctypes.c_float)
        L.orc_run.restype = ctypes.c_int32
        L.orc_run.argtypes = [ctypes.POINTER(_Attrs), ctypes.c_int64, ctypes.c_int64,
                              ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                              fp, fp, fp, fp, ctypes.POINTER(ctypes.c_int32), fp, fp, fp,
                              fp, fp, fp, ctypes.c_int32, ctypes.c_char_p, ctypes.c_size_t]
        L.orc_activation.restype = ctypes.c_float
        L.orc_activation.argtypes = [ctypes.c_int32, ctypes.c_float, ctypes.c_float, ctypes.c_float]
        L.orc_round_bf16.restype = ctypes.c_float
        L.orc_round_bf16.argtypes = [ctypes.c_float]
        L.orc_parse_activations.restype = ctypes.c_int32
        L.orc_parse_activations.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_char_p), ctypes.c_int32, fp,
                                            ctypes.c_int32, fp, ctypes.POINTER(_Act),
                                            ctypes.c_char_p, ctypes.c_size_t]
        L.orc_projection.restype = ctypes.c_int32
        L.orc_projection.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, fp, fp,
                                     ctypes.c_int32, fp, ctypes.c_int32]
        _lib = L
    return _lib


def _np32(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.float32)


def _fptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_float)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _names(names):
    if not names:
        return 0, ctypes.POINTER(ctypes.c_char_p)(), None
    arr = (ctypes.c_char_p * len(names))(*[n.encode() for n in names])
    return len(names), ctypes.cast(arr, ctypes.POINTER(ctypes.c_char_p)), arr


def _floats(vals):
    if not vals:
        return 0, ctypes.POINTER(ctypes.c_float)(), None
    arr = (ctypes.c_float * len(vals))(*vals)
    return len(vals), ctypes.cast(arr, ctypes.POINTER(ctypes.c_float)), arr


def default_threads() -> int:
    """Threads the oracle uses by default: the CPUs this process may run on,
    at most 16 (a one-GPU share of a GPU host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def run(case, n_threads: Optional[int] = None, want_y: bool = True,
        want_yh: bool = True, want_yc: Optional[bool] = None,
        constant_weights: bool = False, raise_on_error: bool = True):
    """Run the oracle on a ``workloads.Case``.  Returns (status, Y, Y_h, Y_c);
    absent outputs are None."""
    L = lib()
    D = int(case.W.shape[0])            # num_directions is W's first dimension
    S, Bt, I, H = case.seq, case.batch, case.input, case.hidden
    if want_yc is None:
        want_yc = case.op == "LSTM"
    X, W, R, B, P = (_np32(case.X), _np32(case.W), _np32(case.R), _np32(case.B), _np32(case.P))
    h0, c0 = _np32(case.initial_h), _np32(case.initial_c)
    lens = None
    if case.sequence_lens is not None:
        lens = np.ascontiguousarray(np.asarray(case.sequence_lens), dtype=np.int32)
    if case.layout == 0:
        yshape, sshape = (S, D, Bt, H), (D, Bt, H)
    else:
        yshape, sshape = (Bt, S, D, H), (Bt, D, H)
    Y = np.full(yshape, np.nan, np.float32) if want_y else None
    Yh = np.full(sshape, np.nan, np.float32) if want_yh else None
    Yc = np.full(sshape, np.nan, np.float32) if want_yc else None

    na, names_p, _keep1 = _names(case.activations)
    nal, alpha_p, _keep2 = _floats(case.alpha)
    nbe, beta_p, _keep3 = _floats(case.beta)
    at = _Attrs(OPS[case.op], case.direction.encode(), case.hidden_size_attr, case.layout,
                na, names_p, nal, alpha_p, nbe, beta_p,
                1 if case.clip is not None else 0,
                float(case.clip) if case.clip is not None else 0.0,
                int(case.input_forget), int(case.linear_before_reset),
                1 if case.proj_bf16 else 0, 1 if constant_weights else 0)
    err = ctypes.create_string_buffer(256)
    nt = default_threads() if n_threads is None else n_threads
    st = L.orc_run(ctypes.byref(at), S, Bt, I, H, D, _fptr(X), _fptr(W), _fptr(R), _fptr(B),
                   lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if lens is not None
                   else ctypes.POINTER(ctypes.c_int32)(),
                   _fptr(h0), _fptr(c0), _fptr(P), _fptr(Y), _fptr(Yh), _fptr(Yc),
                   nt, err, 256)
    if st != OK and raise_on_error:
        raise OracleError(st, err.value.decode())
    return st, Y, Yh, Yc


def run_cell(op: str, X, W, R, B_sum=None, H=None, C=None, P=None,
             activations: Optional[Sequence[str]] = None,
             alpha: Optional[Sequence[float]] = None, beta: Optional[Sequence[float]] = None,
             clip: Optional[float] = None, input_forget: int = 0, linear_before_reset: int = 0,
             n_threads: Optional[int] = None):
    """One step in the single-cell convention of the OpenVINO page "RNNCell-3"
    ("Inputs": X [batch, input], H [batch, hidden], W, R, and B the SUM of the
    W and R biases; "Outputs": the new hidden state only).  Reading: the summed
    bias is the ONNX B with Wb = B and Rb = 0 (so the pre-activation is
    (X Wi^T + H Ri^T) + B), applied to the gates of any operator; for GRU with
    linear_before_reset = 1 the recurrent candidate bias is scaled by the reset
    gate, so a sum cannot carry it and B_sum is refused.
    Returns (H_out [batch, hidden], C_out [batch, hidden] or None)."""
    from types import SimpleNamespace
    X, W, R = _np32(X), _np32(W), _np32(R)
    Bs, H0, C0, P0 = _np32(B_sum), _np32(H), _np32(C), _np32(P)
    if Bs is not None and op == "GRU" and linear_before_reset:
        raise ValueError("a summed bias cannot express GRU with linear_before_reset = 1")
    Bt, I = X.shape
    Hd = R.shape[1]
    B = None if Bs is None else np.concatenate([Bs, np.zeros_like(Bs)])[None]
    case = SimpleNamespace(
        op=op, direction="forward", seq=1, batch=Bt, input=I, hidden=Hd, layout=0,
        activations=activations, alpha=alpha, beta=beta, clip=clip, input_forget=input_forget,
        linear_before_reset=linear_before_reset, proj_bf16=False, hidden_size_attr=0,
        X=X[None], W=W[None], R=R[None], B=B, P=None if P0 is None else P0[None],
        initial_h=None if H0 is None else H0[None],
        initial_c=None if C0 is None else C0[None], sequence_lens=None)
    _, _, Yh, Yc = run(case, n_threads=n_threads, want_y=False)
    return Yh[0], (Yc[0] if Yc is not None else None)


def activation(name: str, x, alpha: float = 0.0, beta: float = 0.0) -> np.ndarray:
    """One activation over an array, through the oracle's scalar function."""
    L = lib()
    k = ACT_KINDS.index(name)
    xs = np.asarray(x, dtype=np.float32).ravel()
    out = np.empty_like(xs)
    for i, v in enumerate(xs):
        out[i] = L.orc_activation(k, alpha, beta, float(v))
    return out.reshape(np.shape(x))


def parse_activations(op: str, dirs: int, names: Optional[Sequence[str]],
                      alpha: Optional[Sequence[float]] = None,
                      beta: Optional[Sequence[float]] = None):
    """(status, [[(kind name, alpha, beta) per activation] per direction])."""
    L = lib()
    n, p, _k1 = _names(list(names) if names else None)
    nal, ap, _k2 = _floats(list(alpha) if alpha else None)
    nbe, bp, _k3 = _floats(list(beta) if beta else None)
    out = (_Act * 6)()
    err = ctypes.create_string_buffer(256)
    st = L.orc_parse_activations(OPS[op], dirs, n, p, nal, ap, nbe, bp, out, err, 256)
    na = {"RNN": 1, "GRU": 2, "LSTM": 3}[op]
    res = [[(ACT_KINDS[out[d * 3 + j].kind], out[d * 3 + j].alpha, out[d * 3 + j].beta)
            for j in range(na)] for d in range(dirs)]
    return st, res


def round_bf16(x) -> np.ndarray:
    L = lib()
    xs = np.asarray(x, dtype=np.float32).ravel()
    out = np.array([L.orc_round_bf16(float(v)) for v in xs], dtype=np.float32)
    return out.reshape(np.shape(x))


def projection(X, W, bf16: bool = False, n_threads: Optional[int] = None) -> np.ndarray:
    """XW = X . W^T for X [M, I], W [N, I] with the oracle's accumulation rule."""
    L = lib()
    X, W = _np32(X), _np32(W)
    M, I = X.shape
    N = W.shape[0]
    out = np.empty((M, N), np.float32)
    nt = default_threads() if n_threads is None else n_threads
    st = L.orc_projection(M, I, N, _fptr(X), _fptr(W), 1 if bf16 else 0, _fptr(out), nt)
    if st != OK:
        raise OracleError(st, "projection")
    return out
