"""Pins of the CPU oracle to things other than itself: hand-computed closed
forms, operation-order cases whose answer depends on the written order,
torch's fp64 RNN/GRU/LSTM modules, an fp64 brute force, library activation
functions and the parameter assignment printed on the onemodel page."""
import json
import math
import os
import struct

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import brute64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
f32 = np.float32


def bits(x):
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


def case_from(op, direction, X, W, R, B=None, **kw):
    """A Case built from explicit float64 lists (layout 0)."""
    X = torch.tensor(X, dtype=torch.float32)
    W = torch.tensor(W, dtype=torch.float32)
    R = torch.tensor(R, dtype=torch.float32)
    S, Bt, I = X.shape
    H = R.shape[-1]
    c = workloads.Case(op, direction, S, Bt, I, H,
                       **{k: v for k, v in kw.items() if k in
                          ("layout", "activations", "alpha", "beta", "clip",
                           "input_forget", "linear_before_reset")})
    c.X, c.W, c.R = X, W, R
    c.B = None if B is None else torch.tensor(B, dtype=torch.float32)
    for k in ("P", "initial_h", "initial_c"):
        if k in kw and kw[k] is not None:
            setattr(c, k, torch.tensor(kw[k], dtype=torch.float32))
    if "sequence_lens" in kw:
        c.sequence_lens = torch.tensor(kw["sequence_lens"], dtype=torch.int32)
    return c


# ---------------------------------------------------------------------------
# Closed forms (hand-computed values of one- and two-step cells)
# ---------------------------------------------------------------------------

def test_rnn_two_steps_hand_values():
    # I = H = 1, x = (1, -1), w = 0.5, r = 0.25, h0 = 1, Wb = 0.125, Rb = -0.375
    c = case_from("RNN", "forward", [[[1.0]], [[-1.0]]], [[[0.5]]], [[[0.25]]],
                  B=[[0.125, -0.375]], initial_h=[[[1.0]]])
    _, Y, Yh, _ = oracle.run(c)
    h1 = math.tanh(0.5)                              # pre = 0.5 + 0.25 + 0.125 - 0.375
    pre2 = 0.25 * float(f32(h1)) - 0.75
    h2 = math.tanh(pre2)
    assert abs(Y[0, 0, 0, 0] - h1) < 1e-7
    assert abs(Y[1, 0, 0, 0] - h2) < 1e-7
    assert abs(h1 - 0.462117157) < 1e-9 and abs(h2 - (-0.561122966)) < 1e-8
    assert Yh[0, 0, 0] == Y[1, 0, 0, 0]


def test_lstm_zero_weights_closed_form():
    # zero W, R, B; c0 = 1: every gate pre-activation is 0, so i = f = o = 1/2
    # and ct = 0: c1 = 1/2, h1 = tanh(1/2)/2, c2 = 1/4, h2 = tanh(1/4)/2.
    H = 3
    c = case_from("LSTM", "forward", np.random.RandomState(0).randn(2, 2, 4).tolist(),
                  np.zeros((1, 4 * H, 4)).tolist(), np.zeros((1, 4 * H, H)).tolist(),
                  B=np.zeros((1, 8 * H)).tolist(),
                  initial_h=np.random.RandomState(1).randn(1, 2, H).tolist(),
                  initial_c=np.ones((1, 2, H)).tolist())
    _, Y, Yh, Yc = oracle.run(c)
    assert np.all(Y[0] == f32(0.5 * math.tanh(0.5)))
    assert np.all(Y[1] == f32(0.5 * math.tanh(0.25)))
    assert np.all(Yc == 0.25)
    assert abs(0.5 * math.tanh(0.5) - 0.231058579) < 1e-9


def test_lstm_peephole_closed_form():
    # zero W, R, B; Pi = 0.5, Po = 1, Pf = -1, c0 = 2: the output gate sees the
    # NEW cell, the input and forget gates the previous one.
    c = case_from("LSTM", "forward", [[[0.0]]], np.zeros((1, 4, 1)).tolist(),
                  np.zeros((1, 4, 1)).tolist(), B=np.zeros((1, 8)).tolist(),
                  P=[[0.5, 1.0, -1.0]], initial_c=[[[2.0]]])
    _, Y, Yh, Yc = oracle.run(c)
    sig = lambda v: 1 / (1 + math.exp(-v))
    i, f = sig(1.0), sig(-2.0)
    c1 = f * 2.0                                          # ct = tanh(0) = 0
    o = sig(c1)
    h1 = o * math.tanh(c1)
    assert abs(Yc[0, 0, 0] - c1) < 2e-7 and abs(c1 - 0.238405844) < 1e-8
    assert abs(Y[0, 0, 0, 0] - h1) < 2e-7 and abs(h1 - 0.130875150) < 1e-8
    # with the old cell in the output gate the value would be different
    assert abs(sig(2.0) * math.tanh(c1) - h1) > 0.05


def test_lstm_clip_closed_form():
    # zero W / R, Wb_c = 10, clip = 3, c0 = 1: ct = tanh(3) instead of tanh(10)
    B = np.zeros((1, 8))
    B[0, 3] = 10.0
    kw = dict(B=B.tolist(), initial_c=[[[1.0]]])
    c = case_from("LSTM", "forward", [[[0.0]]], np.zeros((1, 4, 1)).tolist(),
                  np.zeros((1, 4, 1)).tolist(), clip=3.0, **kw)
    _, _, _, Yc = oracle.run(c)
    assert abs(Yc[0, 0, 0] - (0.5 + 0.5 * math.tanh(3.0))) < 1e-7
    assert abs(Yc[0, 0, 0] - 0.997527377) < 1e-7
    c.clip = None
    _, _, _, Yc2 = oracle.run(c)
    assert abs(Yc2[0, 0, 0] - (0.5 + 0.5 * math.tanh(10.0))) < 1e-7
    # clip <= 0 is not "present and positive": nothing is clamped
    c.clip = 0.0
    _, _, _, Yc3 = oracle.run(c)
    assert Yc3[0, 0, 0] == Yc2[0, 0, 0]


def test_clip_on_output_gate_and_nan_passes():
    B = np.zeros((1, 8))
    B[0, 1] = 10.0                                        # o gate
    c = case_from("LSTM", "forward", [[[0.0]]], np.zeros((1, 4, 1)).tolist(),
                  np.zeros((1, 4, 1)).tolist(), B=B.tolist(), clip=3.0,
                  initial_c=[[[1.0]]])
    _, Y, _, Yc = oracle.run(c)
    expect = (1 / (1 + math.exp(-3.0))) * math.tanh(float(Yc[0, 0, 0]))
    assert abs(Y[0, 0, 0, 0] - expect) < 1e-7


def test_gru_zero_weights_halves_state():
    for lbr in (0, 1):
        H = 4
        h0 = np.random.RandomState(3).randn(1, 2, H).astype(np.float32)
        c = case_from("GRU", "forward", np.random.RandomState(2).randn(2, 2, 3).tolist(),
                      np.zeros((1, 3 * H, 3)).tolist(), np.zeros((1, 3 * H, H)).tolist(),
                      B=np.zeros((1, 6 * H)).tolist(), initial_h=h0.tolist(),
                      linear_before_reset=lbr)
        _, Y, Yh, _ = oracle.run(c)
        assert np.array_equal(Y[0, 0], h0[0] * f32(0.5))   # exact in fp32
        assert np.array_equal(Y[1, 0], h0[0] * f32(0.25))


def test_gru_lbr0_equals_lbr1_when_reset_gate_is_one():
    c = workloads.random_case("GRU", "forward", 5, 3, 4, 6, seed=11, with_h0=True)
    B = c.B.clone()
    H = c.hidden
    B[0, H:2 * H] = 100.0                 # Wb_r: sigmoid(~100) == 1.0f exactly
    B[0, 2 * H:3 * H] = 0.0               # Wb_h
    B[0, 5 * H:6 * H] = 0.0               # Rb_h
    c.B = B
    c.linear_before_reset = 0
    _, Y0, H0, _ = oracle.run(c)
    c.linear_before_reset = 1
    _, Y1, H1, _ = oracle.run(c)
    assert np.array_equal(Y0.view(np.uint32), Y1.view(np.uint32))
    # and with an ordinary reset gate the two forms differ
    c2 = workloads.random_case("GRU", "forward", 5, 3, 4, 6, seed=11, with_h0=True)
    c2.linear_before_reset = 0
    a = oracle.run(c2)[1]
    c2.linear_before_reset = 1
    b = oracle.run(c2)[1]
    assert np.abs(a - b).max() > 1e-3


def test_rnn_single_step_is_the_rnncell_formula():
    # OpenVINO RNNCell-3: Ht = f(Xt Wi^T + Ht-1 Ri^T + Wbi + Rbi) with B the sum
    # of the biases; shapes of its IR example (batch 1, input 16, hidden 128).
    g = json.load(open(os.path.join(GOLDEN, "rnncell_ir_example.json")))
    Bn, I, H = g["batch"], g["input_size"], g["hidden_size"]
    rs = np.random.RandomState(5)
    x = rs.uniform(-1, 1, (Bn, I)).astype(np.float32)
    h = rs.uniform(-1, 1, (Bn, H)).astype(np.float32)
    W = rs.uniform(-0.1, 0.1, (H, I)).astype(np.float32)
    R = rs.uniform(-0.1, 0.1, (H, H)).astype(np.float32)
    Bsum = rs.uniform(-0.1, 0.1, (H,)).astype(np.float32)
    ho = np.tanh(x.astype(np.float64) @ W.T.astype(np.float64)
                 + h.astype(np.float64) @ R.T.astype(np.float64) + Bsum)
    c = case_from("RNN", "forward", x[None].tolist(), W[None].tolist(), R[None].tolist(),
                  B=np.concatenate([Bsum, np.zeros(H, np.float32)])[None].tolist(),
                  initial_h=h[None].tolist())
    _, Y, Yh, _ = oracle.run(c)
    assert Yh.shape == (1, Bn, H)
    assert np.abs(Yh[0] - ho).max() < 2e-6


@pytest.mark.parametrize("act", ["Tanh", "Relu", "Sigmoid"])
def test_cell_convention_matches_the_rnncell_closed_form(act):
    # OpenVINO RNNCell-3: Ho = f(X Wi^T + H Ri^T + B), B the summed bias,
    # f one of relu / sigmoid / tanh ("Attributes"); written out in fp64.
    rs = np.random.RandomState(7)
    Bn, I, H = 3, 5, 4
    x = rs.uniform(-1, 1, (Bn, I)).astype(np.float32)
    h = rs.uniform(-1, 1, (Bn, H)).astype(np.float32)
    W = rs.uniform(-0.5, 0.5, (H, I)).astype(np.float32)
    R = rs.uniform(-0.5, 0.5, (H, H)).astype(np.float32)
    Bs = rs.uniform(-0.5, 0.5, (H,)).astype(np.float32)
    pre = (x.astype(np.float64) @ W.T.astype(np.float64) + h.astype(np.float64) @ R.T.astype(np.float64)
           + Bs.astype(np.float64))
    f = {"Tanh": np.tanh, "Relu": lambda v: np.maximum(v, 0.0),
         "Sigmoid": lambda v: 1.0 / (1.0 + np.exp(-v))}[act]
    ho, co = oracle.run_cell("RNN", x, W, R, Bs, H=h, activations=[act])
    assert co is None and ho.shape == (Bn, H)
    assert np.abs(ho - f(pre)).max() < 2e-6
    # no H: the previous state is zero; no B: no bias
    ho0, _ = oracle.run_cell("RNN", x, W, R, None, activations=[act])
    assert np.abs(ho0 - f(x.astype(np.float64) @ W.T.astype(np.float64))).max() < 2e-6


@pytest.mark.parametrize("op,attrs", [("GRU", dict(linear_before_reset=0)), ("LSTM", {}),
                                      ("LSTM", dict(with_p=True))])
def test_cell_convention_of_gru_and_lstm_matches_fp64_brute_force(op, attrs):
    # the summed bias on every gate: Wb = B_sum, Rb = 0 in the operator's
    # formulas, checked against the fp64 restatement at seq 1
    a = dict(attrs)
    with_p = a.pop("with_p", False)
    c = workloads.random_case(op, "forward", 1, 4, 6, 5, seed=31, with_h0=True,
                              with_c0=(op == "LSTM"), with_p=with_p, **a)
    G = {"GRU": 3, "LSTM": 4}[op]
    Bs = c.B[0, :G * 5].clone()
    c.B = torch.cat([Bs, torch.zeros(G * 5)])[None]
    ref = brute64.run(c)
    ho, co = oracle.run_cell(op, c.X[0], c.W[0], c.R[0], Bs, H=c.initial_h[0],
                             C=None if c.initial_c is None else c.initial_c[0],
                             P=None if c.P is None else c.P[0], **a)
    assert np.abs(ho - ref[1][0]).max() < 3e-6
    if op == "LSTM":
        assert np.abs(co - ref[2][0]).max() < 3e-6


def test_cell_convention_refuses_a_summed_bias_for_gru_reset_after_product():
    x = np.zeros((1, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.run_cell("GRU", x, np.zeros((9, 2), np.float32), np.zeros((9, 3), np.float32),
                        np.zeros(9, np.float32), linear_before_reset=1)


# ---------------------------------------------------------------------------
# Operation order: cases whose answer depends on the written order
# ---------------------------------------------------------------------------

IDENT = dict(activations=["Affine"], alpha=[1.0], beta=[0.0])


def test_projection_accumulates_k_increasing_from_plus_zero():
    # ((0 + 1) + 1e8) + (-1e8) = 0 in binary32; k descending gives 1
    c = case_from("RNN", "forward", [[[1.0, 1e8, -1e8]]], [[[1.0, 1.0, 1.0]]], [[[0.0]]],
                  **IDENT)
    _, Y, _, _ = oracle.run(c)
    assert Y[0, 0, 0, 0] == 0.0
    # the accumulator starts at +0: the sum of -0 products is +0
    c = case_from("RNN", "forward", [[[-0.0]]], [[[1.0]]], [[[0.0]]], **IDENT)
    _, Y, _, _ = oracle.run(c)
    assert bits(Y[0, 0, 0, 0]) == 0x00000000
    # direct check of the exported projection on the same vectors
    out = oracle.projection(np.array([[1.0, 1e8, -1e8]], np.float32),
                            np.array([[1.0, 1.0, 1.0], [1.0, -1.0, 1.0]], np.float32))
    assert out[0, 0] == 0.0 and out[0, 1] == f32(-2e8)


def test_recurrent_product_accumulates_k_increasing():
    c = case_from("RNN", "forward", [[[0.0]]], [[[0.0], [0.0], [0.0]]],
                  [[[1.0, 1.0, 1.0], [0.0, 0.0, 0.0], [0.0, 0.0, 0.0]]],
                  initial_h=[[[1.0, 1e8, -1e8]]], **IDENT)
    _, Y, _, _ = oracle.run(c)
    assert Y[0, 0, 0, 0] == 0.0


def test_pre_activation_order():
    # pre = ((xw + rec) + Wb) + Rb: ((1e8 + 1) - 1e8) + 1 = 1 in binary32,
    # where (xw + Wb) + rec + Rb would give 2.
    c = case_from("RNN", "forward", [[[1.0]]], [[[1e8]]], [[[1.0]]], B=[[-1e8, 1.0]],
                  initial_h=[[[1.0]]], **IDENT)
    _, Y, _, _ = oracle.run(c)
    assert Y[0, 0, 0, 0] == 1.0


def test_lstm_cell_update_is_two_products_and_one_sum():
    # identity activations: i, fg, ct are the pre-activations themselves.
    # fg * c_prev = (1+2^-12)^2 rounds to 1+2^-11 (the 2^-24 is a tie to even);
    # adding i*ct = -(1+2^-11) gives exactly 0, a fused form would give 2^-24.
    e = 2.0 ** -12
    Wg = [[[-(1 + 2 * e)]], [[1.0]], [[1 + e]], [[1.0]]]     # i, o, f, c
    c = case_from("LSTM", "forward", [[[1.0]]], [[w[0] for w in Wg]],
                  np.zeros((1, 4, 1)).tolist(), initial_c=[[[1 + e]]],
                  activations=["Affine", "Affine", "Affine"], alpha=[1.0, 1.0, 1.0],
                  beta=[0.0, 0.0, 0.0])
    _, Y, _, Yc = oracle.run(c)
    assert Yc[0, 0, 0] == 0.0
    assert Y[0, 0, 0, 0] == 0.0


def test_gru_update_is_separately_rounded():
    # identity activations: z and ht are pre-activations; H = ((1-z)*ht) + (z*H).
    # z = -e so 1 - z = 1 + e; ht = 1 + e; H_prev = 2^12 + 2 so z*H_prev is
    # exactly -(1 + 2e).  (1+e)^2 rounds (tie to even) to 1 + 2e, so the
    # separately rounded update is 0 where a fused one would leave 2^-24.
    e = 2.0 ** -12
    W = [[[-e], [0.0], [1 + e]]]
    c = case_from("GRU", "forward", [[[1.0]]], W, np.zeros((1, 3, 1)).tolist(),
                  initial_h=[[[4098.0]]], activations=["Affine", "Affine"],
                  alpha=[1.0, 1.0], beta=[0.0, 0.0], linear_before_reset=1)
    _, Y, _, _ = oracle.run(c)
    assert Y[0, 0, 0, 0] == 0.0


# ---------------------------------------------------------------------------
# torch's fp64 modules (an independent library)
# ---------------------------------------------------------------------------

def _torch_reorder(w, op, H):
    """ONNX gate blocks -> torch order (LSTM i,o,f,c -> i,f,g,o; GRU z,r,h -> r,z,n)."""
    blocks = [w[k * H:(k + 1) * H] for k in range(w.shape[0] // H)]
    if op == "LSTM":
        return torch.cat([blocks[0], blocks[2], blocks[3], blocks[1]])
    if op == "GRU":
        return torch.cat([blocks[1], blocks[0], blocks[2]])
    return w


def _torch_run(c):
    """torch fp64 module with the case's weights.  A reverse-only layer is the
    reverse half of a bidirectional module (its forward half is ignored)."""
    H, I, G = c.hidden, c.input, c.gates
    rev_only = c.direction == "reverse"
    mod = {"RNN": torch.nn.RNN, "GRU": torch.nn.GRU, "LSTM": torch.nn.LSTM}[c.op]
    kw = dict(nonlinearity="tanh") if c.op == "RNN" else {}
    m = mod(I, H, bidirectional=True, **kw).double()
    tdirs = [0, 0] if rev_only else ([0, 1] if c.dirs == 2 else [0, 0])
    with torch.no_grad():
        for td in range(2):
            d = tdirs[td]
            sfx = "_l0" + ("_reverse" if td == 1 else "")
            getattr(m, "weight_ih" + sfx).copy_(_torch_reorder(c.W[d].double(), c.op, H))
            getattr(m, "weight_hh" + sfx).copy_(_torch_reorder(c.R[d].double(), c.op, H))
            B = c.B[d].double() if c.B is not None else torch.zeros(2 * G * H, dtype=torch.float64)
            getattr(m, "bias_ih" + sfx).copy_(_torch_reorder(B[:G * H], c.op, H))
            getattr(m, "bias_hh" + sfx).copy_(_torch_reorder(B[G * H:], c.op, H))
        X = c.X.double()
        h0 = (c.initial_h.double() if c.initial_h is not None
              else torch.zeros(c.dirs, c.batch, H, dtype=torch.float64))
        c0 = (c.initial_c.double() if c.initial_c is not None else torch.zeros_like(h0))
        h0 = h0[tdirs].contiguous()
        c0 = c0[tdirs].contiguous()
        hx = (h0, c0) if c.op == "LSTM" else h0
        if c.sequence_lens is not None:
            pk = torch.nn.utils.rnn.pack_padded_sequence(X, c.sequence_lens.long(), enforce_sorted=False)
            y, hn = m(pk, hx)
            y, _ = torch.nn.utils.rnn.pad_packed_sequence(y, total_length=c.seq)
        else:
            y, hn = m(X, hx)
    y = y.view(c.seq, c.batch, 2, H).permute(0, 2, 1, 3)
    keep = [1] if rev_only else ([0, 1] if c.dirs == 2 else [0])
    y = y[:, keep]
    if c.op == "LSTM":
        hn = (hn[0][keep], hn[1][keep])
    else:
        hn = hn[keep]
    return y.numpy(), hn


@pytest.mark.parametrize("op,direction,lens", [
    ("RNN", "forward", None), ("RNN", "bidirectional", [5, 3, 1]),
    ("GRU", "forward", None), ("GRU", "reverse", [2, 5, 4]), ("GRU", "bidirectional", [5, 1, 3]),
    ("LSTM", "forward", None), ("LSTM", "bidirectional", None), ("LSTM", "reverse", [4, 5, 1])])
def test_oracle_matches_torch_fp64(op, direction, lens):
    c = workloads.random_case(op, direction, 5, 3, 7, 6, seed=21, lens=lens,
                              with_h0=True, with_c0=(op == "LSTM"),
                              linear_before_reset=1 if op == "GRU" else 0)
    _, Y, Yh, Yc = oracle.run(c)
    y, hn = _torch_run(c)
    assert np.abs(Y - y).max() < 5e-6
    if op == "LSTM":
        assert np.abs(Yh - hn[0].numpy()).max() < 5e-6
        assert np.abs(Yc - hn[1].numpy()).max() < 5e-6
    else:
        assert np.abs(Yh - hn.numpy()).max() < 5e-6


def test_oracle_matches_torch_on_gru_workload_rows():
    c = workloads.workload("gru_fwd_s128_b32_i256_h512_lbr1", batch_rows=[0, 7, 19])
    c.X = c.X.transpose(0, 1).contiguous()
    c.layout = 0                      # torch takes seq-first input
    _, Y, Yh, _ = oracle.run(c)
    y, hn = _torch_run(c)
    assert np.abs(Y - y).max() < 2e-5
    assert np.abs(Yh - hn.numpy()).max() < 2e-5


# ---------------------------------------------------------------------------
# fp64 brute force on tiny shapes (every feature)
# ---------------------------------------------------------------------------

BRUTE_CASES = [
    dict(op="RNN", direction="forward", activations=["Relu"]),
    dict(op="RNN", direction="bidirectional", activations=["Tanh", "Affine"], alpha=[0.7], beta=[0.1],
         with_lens=True, layout=1),
    dict(op="GRU", direction="forward", linear_before_reset=0, with_lens=True),
    dict(op="GRU", direction="reverse", linear_before_reset=0, clip=0.6),
    dict(op="GRU", direction="bidirectional", linear_before_reset=1, layout=1,
         activations=["HardSigmoid", "Softsign", "Sigmoid", "Elu"], alpha=[0.3, 0.8], beta=[0.45]),
    dict(op="LSTM", direction="forward", with_p=True, clip=0.8),
    dict(op="LSTM", direction="bidirectional", with_p=True, with_lens=True, input_forget=1),
    dict(op="LSTM", direction="reverse", activations=["HardSigmoid", "LeakyRelu", "ScaledTanh"],
         alpha=[0.3, 0.2, 1.2], beta=[0.4, 0.7], with_lens=True),
    dict(op="LSTM", direction="forward", activations=["Sigmoid", "Softplus", "ThresholdedRelu"],
         alpha=[0.1]),
    dict(op="RNN", direction="forward", with_bias=False, activations=["Elu"], alpha=[0.5]),
]


@pytest.mark.parametrize("k", range(len(BRUTE_CASES)))
def test_oracle_matches_fp64_brute_force(k):
    spec = dict(BRUTE_CASES[k])
    op, direction = spec.pop("op"), spec.pop("direction")
    lay = spec.pop("layout", 0)
    kw = {key: spec.pop(key) for key in ("with_lens", "with_p", "with_bias") if key in spec}
    c = workloads.random_case(op, direction, 6, 4, 5, 7, seed=100 + k, layout=lay,
                              with_h0=True, with_c0=(op == "LSTM"), scale=0.6, **kw, **spec)
    _, Y, Yh, Yc = oracle.run(c)
    y, yh, yc = brute64.run(c)
    assert np.abs(Y - y).max() < 1e-5
    assert np.abs(Yh - yh).max() < 1e-5
    if op == "LSTM":
        assert np.abs(Yc - yc).max() < 1e-5


def test_bf16_projection_matches_brute_force_on_rounded_inputs():
    c = workloads.random_case("GRU", "reverse", 5, 3, 9, 6, seed=77, linear_before_reset=1,
                              with_lens=True, proj_bf16=True)
    _, Y, _, _ = oracle.run(c)
    rnd = lambda a: torch.from_numpy(np.asarray(a, np.float32)).bfloat16().double().numpy()
    y, _, _ = brute64.run(c, bf16_round=rnd)
    assert np.abs(Y - y).max() < 1e-5
    c.proj_bf16 = False
    _, Yf, _, _ = oracle.run(c)
    assert np.abs(Y - Yf).max() > 1e-5      # the rounding is really applied


# ---------------------------------------------------------------------------
# Projection on exactly-summable operands
# ---------------------------------------------------------------------------

def test_projection_integer_operands_exact():
    rs = np.random.RandomState(9)
    X = rs.randint(-8, 9, (37, 70)).astype(np.float32)
    W = rs.randint(-8, 9, (45, 70)).astype(np.float32)
    got = oracle.projection(X, W)
    ref = X.astype(np.int64) @ W.astype(np.int64).T
    assert np.array_equal(got, ref.astype(np.float32))


def test_projection_vs_fp64_matmul():
    rs = np.random.RandomState(10)
    X = rs.randn(33, 129).astype(np.float32)
    W = rs.randn(65, 129).astype(np.float32)
    got = oracle.projection(X, W)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.abs(got - ref).max() < 1e-4
    gb = oracle.projection(X, W, bf16=True)
    xb = torch.from_numpy(X).bfloat16().double().numpy()
    wb = torch.from_numpy(W).bfloat16().double().numpy()
    assert np.abs(gb - xb @ wb.T).max() < 1e-4


# ---------------------------------------------------------------------------
# Activations
# ---------------------------------------------------------------------------

SWEEP = np.array([-30, -20.5, -7, -3, -1, -0.5, -1e-3, -1e-30, -0.0, 0.0, 1e-30, 1e-3, 0.25,
                  0.5, 1, 2.5, 7, 19.9, 20, 20.5, 60], dtype=np.float32)


def _close_f32(got, ref64, ulps=1):
    ref = ref64.astype(np.float32)
    for g, r, r64 in zip(got, ref, ref64):
        if np.isnan(r64):
            assert np.isnan(g)
            continue
        sp = np.spacing(np.float32(abs(r))) if r != 0 else np.float32(1e-38)
        assert abs(float(g) - float(r64)) <= ulps * float(sp) + 1e-45, (g, r64)


def test_transcendental_activations_vs_torch_fp64():
    x = torch.from_numpy(SWEEP.astype(np.float64))
    _close_f32(oracle.activation("Sigmoid", SWEEP), torch.sigmoid(x).numpy())
    _close_f32(oracle.activation("Tanh", SWEEP), torch.tanh(x).numpy())
    _close_f32(oracle.activation("Elu", SWEEP, alpha=1.0),
               torch.nn.functional.elu(x, alpha=1.0).numpy())
    _close_f32(oracle.activation("Elu", SWEEP, alpha=0.5),
               torch.nn.functional.elu(x, alpha=0.5).numpy())
    _close_f32(oracle.activation("Softplus", SWEEP),
               torch.nn.functional.softplus(x, beta=1.0, threshold=20.0).numpy())
    a32, b32 = float(f32(1.7)), float(f32(0.66))
    _close_f32(oracle.activation("ScaledTanh", SWEEP, alpha=a32, beta=b32),
               (a32 * torch.tanh(b32 * x)).numpy())


def test_ieee_activations_special_values():
    nan, inf = float("nan"), float("inf")
    A = oracle.activation
    # Relu keeps a NaN; ThresholdedRelu's compare sends NaN to 0
    assert np.isnan(A("Relu", [nan])[0])
    assert A("Relu", [-2.0])[0] == 0.0 and A("Relu", [3.5])[0] == 3.5
    assert bits(A("Relu", [-0.0])[0]) == 0x80000000
    assert A("ThresholdedRelu", [nan], alpha=1.0)[0] == 0.0
    assert list(A("ThresholdedRelu", [0.5, 1.0, 1.5], alpha=1.0)) == [0.0, 0.0, 1.5]
    assert list(A("LeakyRelu", [-2.0, 3.0], alpha=0.25)) == [-0.5, 3.0]
    assert A("Affine", [2.0], alpha=3.0, beta=-1.0)[0] == 5.0
    hs = A("HardSigmoid", [-10.0, 0.0, 1.0, 10.0, nan], alpha=0.2, beta=0.5)
    assert list(hs[:4]) == [0.0, 0.5, f32(0.2) * f32(1.0) + f32(0.5), 1.0] and np.isnan(hs[4])
    assert A("Softsign", [1.0])[0] == 0.5 and A("Softsign", [-3.0])[0] == -0.75
    assert A("Softsign", [inf])[0] == 1.0 or np.isnan(A("Softsign", [inf])[0])
    assert A("Softplus", [0.0])[0] == f32(math.log(2.0))
    assert A("Softplus", [21.0])[0] == 21.0
    assert A("Sigmoid", [100.0])[0] == 1.0 and A("Sigmoid", [0.0])[0] == 0.5
    assert A("Tanh", [inf])[0] == 1.0 and A("Tanh", [-inf])[0] == -1.0
    for name in ("Sigmoid", "Tanh", "Elu", "Softplus", "Softsign", "Affine", "LeakyRelu",
                 "ScaledTanh", "HardSigmoid"):
        assert np.isnan(A(name, [nan], alpha=1.0, beta=1.0)[0]), name


def test_hardsigmoid_and_torch_library():
    x = torch.linspace(-5, 5, 41, dtype=torch.float64)
    # torch's hardsigmoid is x/6 + 1/2 clamped: HardSigmoid(alpha=1/6, beta=1/2)
    got = oracle.activation("HardSigmoid", x.numpy().astype(np.float32), alpha=float(f32(1 / 6)), beta=0.5)
    assert np.abs(got - torch.nn.functional.hardsigmoid(x).numpy()).max() < 1e-6


def test_activation_cursor_assignment_printed_on_the_page():
    g = json.load(open(os.path.join(GOLDEN, "activation_cursor_example.json")))
    st, sets = oracle.parse_activations(g["op"], 1, g["activations"],
                                        g["activation_alpha"], g["activation_beta"])
    assert st == 0
    for (name, a, b), e in zip(sets[0], g["expected"]):
        assert name == e["name"]
        assert a == f32(e["alpha"])
        if "beta" in e:
            assert b == f32(e["beta"])


def test_activation_defaults_and_case_insensitivity():
    g = json.load(open(os.path.join(GOLDEN, "activation_defaults.json")))
    for op, names in g["default_sets"].items():
        st, sets = oracle.parse_activations(op, 2, None)
        assert st == 0 and [s[0] for s in sets[0]] == names and [s[0] for s in sets[1]] == names
    for name, p in g["parameter_defaults"].items():
        st, sets = oracle.parse_activations("RNN", 1, [name.upper()])
        assert st == 0 and sets[0][0][0] == name
        assert sets[0][0][1] == f32(p["alpha"])
        if "beta" in p:
            assert sets[0][0][2] == f32(p["beta"])
    # two sets for a bidirectional layer, cursors across the whole list
    st, sets = oracle.parse_activations("GRU", 2, ["hardsigmoid", "AFFINE", "LeakyRelu", "elu"],
                                        [0.1, 0.2, 0.3], [0.9])
    assert st == 0
    assert sets[0] == [("HardSigmoid", f32(0.1), f32(0.9)), ("Affine", f32(0.2), f32(0.0))]
    assert sets[1][0] == ("LeakyRelu", f32(0.3), f32(0.0)) and sets[1][1][0] == "Elu"
    assert sets[1][1][1] == 1.0
    # wrong counts and unknown names are InvalidInput
    assert oracle.parse_activations("GRU", 1, ["Sigmoid"])[0] == oracle.INVALID_INPUT
    assert oracle.parse_activations("GRU", 1, ["Sigmoid", "Tanh", "Tanh", "Tanh"])[0] == oracle.INVALID_INPUT
    assert oracle.parse_activations("RNN", 1, ["Swish"])[0] == oracle.INVALID_INPUT


def test_bf16_rounding_matches_torch():
    rs = np.random.RandomState(4)
    x = np.concatenate([rs.randn(2000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 3.0e38, -3.4e38, 1e-40, 1.00390625,
                                  1.01171875, np.inf, -np.inf], np.float32)])
    got = oracle.round_bf16(x)
    ref = torch.from_numpy(x).bfloat16().float().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(oracle.round_bf16([np.nan])[0])
