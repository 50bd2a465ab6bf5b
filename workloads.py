"""Seeded synthetic inputs for the ONNX recurrent operators (RNN, GRU, LSTM).

This module only draws random tensors and slices them; it holds none of the
operators' arithmetic.  Both the CPU oracle (``oracle/``) and the HIP library
(``recurrent_nn_amd``) are fed from here, by the tests, the smoke check and
the benchmark, and neither of them imports this module.

Shapes follow the ONNX input tables of the recurrent operators (onemodel
"Recurrent operators" page, section *Support*; WebGPU ``ai.onnx.RNN`` README,
*Inputs*): X is [seq, batch, input] for layout 0 and [batch, seq, input] for
layout 1, W is [dirs, G*H, input], R is [dirs, G*H, H], B is [dirs, 2*G*H],
P is [dirs, 3*H], initial states are [dirs, batch, H] (layout 0) or
[batch, dirs, H] (layout 1), sequence_lens is int32 [batch].

Recipe: one CPU ``torch.Generator`` per workload, seeded once, drawing in the
order X, W, R, B, P, initial_h, initial_c, sequence_lens and skipping absent
tensors.  ``U(a, b)`` is ``a + (b - a) * rand``, ``N(0,1)`` is ``randn`` and
lengths are ``randint(lo, hi + 1)``.  No public dataset is involved: the pages
benchmark none, so these synthetic tensors are the workloads.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, List, Optional, Sequence, Tuple

import torch

GATES = {"RNN": 1, "GRU": 3, "LSTM": 4}


@dataclasses.dataclass
class Case:
    """One operator invocation: attributes, dimensions and host tensors."""

    op: str
    direction: str
    seq: int
    batch: int
    input: int
    hidden: int
    layout: int = 0
    activations: Optional[List[str]] = None
    alpha: Optional[List[float]] = None
    beta: Optional[List[float]] = None
    clip: Optional[float] = None
    input_forget: int = 0
    linear_before_reset: int = 0
    proj_bf16: bool = False
    hidden_size_attr: int = 0
    # tensors (CPU, float32 / int32); None = omitted input
    X: Optional[torch.Tensor] = None
    W: Optional[torch.Tensor] = None
    R: Optional[torch.Tensor] = None
    B: Optional[torch.Tensor] = None
    P: Optional[torch.Tensor] = None
    initial_h: Optional[torch.Tensor] = None
    initial_c: Optional[torch.Tensor] = None
    sequence_lens: Optional[torch.Tensor] = None
    name: str = ""

    @property
    def dirs(self) -> int:
        return 2 if self.direction == "bidirectional" else 1

    @property
    def gates(self) -> int:
        return GATES[self.op]

    def cell_updates(self) -> int:
        """Nominal cell-updates of one run: seq * batch * dirs."""
        return self.seq * self.batch * self.dirs

    def valid_cell_updates(self) -> int:
        if self.sequence_lens is None:
            return self.cell_updates()
        return int(self.sequence_lens.sum()) * self.dirs

    def tensors(self) -> Dict[str, Optional[torch.Tensor]]:
        return {k: getattr(self, k) for k in
                ("X", "W", "R", "B", "P", "initial_h", "initial_c", "sequence_lens")}

    def digests(self) -> Dict[str, str]:
        out = {}
        for k, v in self.tensors().items():
            if v is not None:
                out[k] = hashlib.sha256(v.contiguous().numpy().tobytes()).hexdigest()[:16]
        return out


def _u(gen, shape, lo, hi):
    return lo + (hi - lo) * torch.rand(shape, generator=gen, dtype=torch.float32)


def _n(gen, shape):
    return torch.randn(shape, generator=gen, dtype=torch.float32)


def _state_shape(layout, dirs, batch, hidden):
    return (dirs, batch, hidden) if layout == 0 else (batch, dirs, hidden)


def _x_shape(layout, seq, batch, inp):
    return (seq, batch, inp) if layout == 0 else (batch, seq, inp)


# --------------------------------------------------------------------------
# The five named workloads.  Sizes and distributions are those of the
# workload list; where a distribution is unstated the reading is noted.
# --------------------------------------------------------------------------

WORKLOADS = {
    "rnn_fwd_s4_b2_i3_h5": dict(seed=1001),
    "lstm_bidir_s16_b4_i32_h64": dict(seed=1002),
    "gru_fwd_s128_b32_i256_h512_lbr0": dict(seed=1003),
    "gru_fwd_s128_b32_i256_h512_lbr1": dict(seed=1003),
    "lstm_bidir_s512_b64_i1024_h1024": dict(seed=1004),
    "gru_rev_s256_b256_i2048_h2048_bf16": dict(seed=1005),
}


def workload(name: str, batch_rows: Optional[Sequence[int]] = None) -> Case:
    """Build a named workload on the CPU.  ``batch_rows`` keeps only those rows
    (pure indexing; rows of a recurrent layer are independent)."""
    seed = WORKLOADS[name]["seed"]
    g = torch.Generator().manual_seed(seed)
    if name == "rnn_fwd_s4_b2_i3_h5":
        S, Bt, I, H, D = 4, 2, 3, 5, 1
        c = Case("RNN", "forward", S, Bt, I, H, layout=0, activations=["Tanh"])
        c.X = _u(g, (S, Bt, I), -0.5, 0.5)
        c.W = _u(g, (D, H, I), -0.5, 0.5)
        c.R = _u(g, (D, H, H), -0.5, 0.5)
        c.B = _u(g, (D, 2 * H), -0.5, 0.5)
        c.initial_h = _u(g, (D, Bt, H), -0.5, 0.5)
    elif name == "lstm_bidir_s16_b4_i32_h64":
        S, Bt, I, H, D, G = 16, 4, 32, 64, 2, 4
        c = Case("LSTM", "bidirectional", S, Bt, I, H, layout=0, clip=3.0)
        # W, R, B distribution unstated: the U(-0.5, 0.5) of the small RNN
        # workload is used (it also drives some pre-activations past clip).
        c.X = _u(g, (S, Bt, I), -0.5, 0.5)
        c.W = _u(g, (D, G * H, I), -0.5, 0.5)
        c.R = _u(g, (D, G * H, H), -0.5, 0.5)
        c.B = _u(g, (D, 2 * G * H), -0.5, 0.5)
        c.P = _u(g, (D, 3 * H), -0.1, 0.1)
        c.initial_h = _u(g, (D, Bt, H), -0.5, 0.5)
        c.initial_c = _u(g, (D, Bt, H), -0.5, 0.5)
        c.sequence_lens = torch.tensor([16, 9, 1, 0], dtype=torch.int32)
    elif name.startswith("gru_fwd_s128_b32_i256_h512"):
        S, Bt, I, H, D, G = 128, 32, 256, 512, 1, 3
        lbr = 1 if name.endswith("lbr1") else 0
        c = Case("GRU", "forward", S, Bt, I, H, layout=1, linear_before_reset=lbr)
        a = 1.0 / math.sqrt(H)
        c.X = _n(g, (Bt, S, I))
        c.W = _u(g, (D, G * H, I), -a, a)
        c.R = _u(g, (D, G * H, H), -a, a)
        c.B = _u(g, (D, 2 * G * H), -a, a)  # B read as one of the "weights"
        c.sequence_lens = torch.randint(1, S + 1, (Bt,), generator=g, dtype=torch.int32)
    elif name == "lstm_bidir_s512_b64_i1024_h1024":
        S, Bt, I, H, D, G = 512, 64, 1024, 1024, 2, 4
        c = Case("LSTM", "bidirectional", S, Bt, I, H, layout=0)
        a = 1.0 / 32.0
        c.X = _n(g, (S, Bt, I))
        c.W = _u(g, (D, G * H, I), -a, a)
        c.R = _u(g, (D, G * H, H), -a, a)
        c.B = _u(g, (D, 2 * G * H), -a, a)
    elif name == "gru_rev_s256_b256_i2048_h2048_bf16":
        S, Bt, I, H, D, G = 256, 256, 2048, 2048, 1, 3
        c = Case("GRU", "reverse", S, Bt, I, H, layout=0, linear_before_reset=1,
                 activations=["HardSigmoid", "Tanh"], alpha=[0.2], beta=[0.5],
                 proj_bf16=True)
        a = 1.0 / math.sqrt(H)
        c.X = _n(g, (S, Bt, I))
        c.W = _u(g, (D, G * H, I), -a, a)
        c.R = _u(g, (D, G * H, H), -a, a)
        c.B = _u(g, (D, 2 * G * H), -a, a)
        c.sequence_lens = torch.randint(64, S + 1, (Bt,), generator=g, dtype=torch.int32)
    else:
        raise KeyError(name)
    c.name = name
    if batch_rows is not None:
        c = select_rows(c, batch_rows)
    return c


def select_rows(c: Case, rows: Sequence[int]) -> Case:
    """The same case restricted to the given batch rows (indexing only)."""
    idx = torch.as_tensor(list(rows), dtype=torch.long)
    n = dataclasses.replace(c)
    n.batch = len(idx)
    bx = 1 if c.layout == 0 else 0     # batch axis of X
    bs = 1 if c.layout == 0 else 0     # batch axis of the states
    n.X = c.X.index_select(bx, idx).contiguous()
    if c.initial_h is not None:
        n.initial_h = c.initial_h.index_select(bs, idx).contiguous()
    if c.initial_c is not None:
        n.initial_c = c.initial_c.index_select(bs, idx).contiguous()
    if c.sequence_lens is not None:
        n.sequence_lens = c.sequence_lens.index_select(0, idx).contiguous()
    n.name = f"{c.name}[rows={list(rows)[:4]}{'...' if len(idx) > 4 else ''}]"
    return n


def random_case(op: str, direction: str, seq: int, batch: int, inp: int, hidden: int,
                seed: int, layout: int = 0, with_bias: bool = True,
                with_lens: bool = False, lens: Optional[Sequence[int]] = None,
                with_h0: bool = False, with_c0: bool = False, with_p: bool = False,
                scale: float = 0.5, x_scale: float = 1.0, **attrs) -> Case:
    """A generic seeded case for tests: every tensor U(-scale, scale) (X is
    U(-x_scale, x_scale)), lengths randint(0, seq) when requested."""
    G = GATES[op]
    D = 2 if direction == "bidirectional" else 1
    g = torch.Generator().manual_seed(seed)
    c = Case(op, direction, seq, batch, inp, hidden, layout=layout, **attrs)
    c.X = _u(g, _x_shape(layout, seq, batch, inp), -x_scale, x_scale)
    c.W = _u(g, (D, G * hidden, inp), -scale, scale)
    c.R = _u(g, (D, G * hidden, hidden), -scale, scale)
    if with_bias:
        c.B = _u(g, (D, 2 * G * hidden), -scale, scale)
    if with_p:
        c.P = _u(g, (D, 3 * hidden), -scale, scale)
    if with_h0:
        c.initial_h = _u(g, _state_shape(layout, D, batch, hidden), -scale, scale)
    if with_c0:
        c.initial_c = _u(g, _state_shape(layout, D, batch, hidden), -scale, scale)
    if lens is not None:
        c.sequence_lens = torch.as_tensor(list(lens), dtype=torch.int32)
    elif with_lens:
        c.sequence_lens = torch.randint(0, seq + 1, (batch,), generator=g, dtype=torch.int32)
    c.name = f"{op}-{direction}-S{seq}-B{batch}-I{inp}-H{hidden}-L{layout}-seed{seed}"
    return c


def output_shapes(c: Case) -> Tuple[Tuple[int, ...], Tuple[int, ...]]:
    """(Y shape, Y_h / Y_c shape) per the ONNX output table."""
    D = c.dirs
    if c.layout == 0:
        return (c.seq, D, c.batch, c.hidden), (D, c.batch, c.hidden)
    return (c.batch, c.seq, D, c.hidden), (c.batch, D, c.hidden)
