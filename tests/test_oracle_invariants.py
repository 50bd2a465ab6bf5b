"""Bit-exact invariants of the CPU oracle that follow from the onemodel page's
rules (section "Choices the specification leaves open", "Exact mode",
"Limits"): sequence_lens masking, reverse as a flipped forward run,
bidirectional as two stacked runs, layout 1 as transposed layout 0, state
carry, thread-count independence, NaN canonicalisation, zero-size inputs and
the error classes."""
import dataclasses
import hashlib

import numpy as np
import pytest
import torch

import oracle
import workloads

u32 = lambda a: np.ascontiguousarray(a).view(np.uint32)


def same(a, b):
    return a.shape == b.shape and np.array_equal(u32(a), u32(b))


OPS = [("RNN", {}), ("GRU", {"linear_before_reset": 0}), ("GRU", {"linear_before_reset": 1}),
       ("LSTM", {}), ("LSTM", {"input_forget": 1})]


def _case(op, attrs, direction="forward", lens=None, seed=3, layout=0, S=7, Bt=5, **kw):
    return workloads.random_case(op, direction, S, Bt, 6, 8, seed=seed, layout=layout,
                                 lens=lens, with_h0=True, with_c0=(op == "LSTM"),
                                 with_p=(op == "LSTM"), **attrs, **kw)


@pytest.mark.parametrize("op,attrs", OPS)
@pytest.mark.parametrize("direction", ["forward", "reverse"])
def test_sequence_lens_masking(op, attrs, direction):
    lens = [7, 3, 0, 1, 5]
    c = _case(op, attrs, direction, lens)
    _, Y, Yh, Yc = oracle.run(c)
    for b, L in enumerate(lens):
        assert np.all(u32(Y[L:, 0, b]) == 0)             # +0.0 past the length
        if L == 0:
            assert np.all(u32(Yh[0, b]) == 0)             # zero, not initial_h
            if op == "LSTM":
                assert np.all(u32(Yc[0, b]) == 0)
        else:
            last = L - 1 if direction == "forward" else 0
            assert same(Yh[0, b], Y[last, 0, b])
    # each row equals a standalone run of its own length
    for b, L in enumerate(lens):
        if L == 0:
            continue
        r = workloads.select_rows(c, [b])
        r.X = r.X[:L].contiguous()
        r.seq = L
        r.sequence_lens = None
        _, Yr, Yhr, Ycr = oracle.run(r)
        assert same(Yr[:, 0, 0], Y[:L, 0, b])
        assert same(Yhr[0, 0], Yh[0, b])
        if op == "LSTM":
            assert same(Ycr[0, 0], Yc[0, b])


@pytest.mark.parametrize("op,attrs", OPS)
def test_full_lengths_equal_absent_lengths(op, attrs):
    c = _case(op, attrs, "bidirectional", lens=[7] * 5)
    a = oracle.run(c)
    c.sequence_lens = None
    b = oracle.run(c)
    for x, y in zip(a[1:], b[1:]):
        if x is not None:
            assert same(x, y)


@pytest.mark.parametrize("op,attrs", OPS)
def test_reverse_is_forward_on_flipped_rows(op, attrs):
    lens = [7, 4, 1, 6, 2]
    c = _case(op, attrs, "reverse", lens)
    _, Y, Yh, Yc = oracle.run(c)
    f = dataclasses.replace(c, direction="forward")
    X = c.X.clone()
    for b, L in enumerate(lens):
        X[:L, b] = c.X[:L, b].flip(0)
    f.X = X
    _, Yf, Yhf, Ycf = oracle.run(f)
    for b, L in enumerate(lens):
        assert same(Y[:L, 0, b], Yf[:L, 0, b][::-1])
    assert same(Yh, Yhf)
    if op == "LSTM":
        assert same(Yc, Ycf)


@pytest.mark.parametrize("op,attrs", OPS)
def test_bidirectional_is_two_stacked_runs(op, attrs):
    lens = [7, 2, 0, 5, 6]
    c = _case(op, attrs, "bidirectional", lens)
    na = {"RNN": 1, "GRU": 2, "LSTM": 3}[op]
    # two activation sets with parameters, consumed with the cursors
    if op == "RNN":
        c.activations, c.alpha, c.beta = ["LeakyRelu", "Affine"], [0.3, 0.9], [0.2]
        sets = [(["LeakyRelu"], [0.3], None), (["Affine"], [0.9], [0.2])]
    elif op == "GRU":
        c.activations, c.alpha, c.beta = ["HardSigmoid", "Tanh", "Sigmoid", "Elu"], [0.25, 0.7], [0.45]
        sets = [(["HardSigmoid", "Tanh"], [0.25], [0.45]), (["Sigmoid", "Elu"], [0.7], None)]
    else:
        c.activations = ["Sigmoid", "Tanh", "Tanh", "HardSigmoid", "ScaledTanh", "Softsign"]
        c.alpha, c.beta = [0.3, 1.1], [0.6, 0.8]
        sets = [(["Sigmoid", "Tanh", "Tanh"], None, None),
                (["HardSigmoid", "ScaledTanh", "Softsign"], [0.3, 1.1], [0.6, 0.8])]
    assert len(c.activations) == 2 * na
    _, Y, Yh, Yc = oracle.run(c)
    for d, dirn in enumerate(["forward", "reverse"]):
        s = dataclasses.replace(c, direction=dirn, activations=sets[d][0],
                                alpha=sets[d][1], beta=sets[d][2])
        s.W, s.R = c.W[d:d + 1].contiguous(), c.R[d:d + 1].contiguous()
        s.B = c.B[d:d + 1].contiguous()
        s.P = None if c.P is None else c.P[d:d + 1].contiguous()
        s.initial_h = c.initial_h[d:d + 1].contiguous()
        s.initial_c = None if c.initial_c is None else c.initial_c[d:d + 1].contiguous()
        _, Ys, Yhs, Ycs = oracle.run(s)
        assert same(Y[:, d], Ys[:, 0])
        assert same(Yh[d], Yhs[0])
        if op == "LSTM":
            assert same(Yc[d], Ycs[0])


@pytest.mark.parametrize("op,attrs", OPS)
def test_layout1_is_transposed_layout0(op, attrs):
    c = _case(op, attrs, "bidirectional", lens=[7, 3, 0, 1, 5])
    _, Y, Yh, Yc = oracle.run(c)
    t = dataclasses.replace(c, layout=1)
    t.X = c.X.transpose(0, 1).contiguous()
    t.initial_h = c.initial_h.transpose(0, 1).contiguous()
    t.initial_c = None if c.initial_c is None else c.initial_c.transpose(0, 1).contiguous()
    _, Y1, Yh1, Yc1 = oracle.run(t)
    assert same(Y1, np.ascontiguousarray(Y.transpose(2, 0, 1, 3)))
    assert same(Yh1, np.ascontiguousarray(Yh.transpose(1, 0, 2)))
    if op == "LSTM":
        assert same(Yc1, np.ascontiguousarray(Yc.transpose(1, 0, 2)))


@pytest.mark.parametrize("op,attrs", OPS)
def test_state_carry_splits_a_sequence(op, attrs):
    c = _case(op, attrs, "forward", S=9)
    _, Y, Yh, Yc = oracle.run(c)
    a = dataclasses.replace(c, seq=4)
    a.X = c.X[:4].contiguous()
    _, Ya, Yha, Yca = oracle.run(a)
    b = dataclasses.replace(c, seq=5)
    b.X = c.X[4:].contiguous()
    b.initial_h = torch.from_numpy(Yha)
    if op == "LSTM":
        b.initial_c = torch.from_numpy(Yca)
    _, Yb, Yhb, Ycb = oracle.run(b)
    assert same(Y, np.concatenate([Ya, Yb]))
    assert same(Yh, Yhb)
    if op == "LSTM":
        assert same(Yc, Ycb)


def test_thread_count_does_not_change_results():
    c = workloads.workload("gru_fwd_s128_b32_i256_h512_lbr0", batch_rows=range(12))
    digests = set()
    for nt in (1, 3, 8):
        _, Y, Yh, _ = oracle.run(c, n_threads=nt)
        digests.add(hashlib.sha256(Y.tobytes() + Yh.tobytes()).hexdigest())
    assert len(digests) == 1


@pytest.mark.parametrize("op,attrs", OPS)
def test_nan_is_written_canonically(op, attrs):
    c = _case(op, attrs, "bidirectional", lens=[7, 3, 0, 1, 5])
    X = c.X.numpy().copy()
    X.view(np.uint32)[2, 0, 1] = 0xFFC00123          # a negative NaN with payload
    c.X = torch.from_numpy(X)
    _, Y, Yh, Yc = oracle.run(c)
    for a in (Y, Yh) + ((Yc,) if op == "LSTM" else ()):
        n = np.isnan(a)
        assert n.any()
        assert np.all(u32(a)[n] == 0x7FC00000)


@pytest.mark.parametrize("op", ["RNN", "GRU", "LSTM"])
def test_zero_size(op):
    # seq = 0: nothing runs, the final states are the initial states
    c = workloads.random_case(op, "bidirectional", 0, 3, 4, 5, seed=1, with_h0=True,
                              with_c0=(op == "LSTM"))
    st, Y, Yh, Yc = oracle.run(c)
    assert st == 0 and Y.size == 0
    assert same(Yh, c.initial_h.numpy())
    if op == "LSTM":
        assert same(Yc, c.initial_c.numpy())
    # absent initial states give zeros
    c.initial_h = None
    c.initial_c = None
    _, _, Yh, Yc = oracle.run(c)
    assert np.all(u32(Yh) == 0)
    # batch = 0
    c = workloads.random_case(op, "forward", 4, 0, 4, 5, seed=1)
    st, Y, Yh, _ = oracle.run(c)
    assert st == 0 and Y.size == 0 and Yh.size == 0


def _err(c, **kw):
    return oracle.run(c, raise_on_error=False, **kw)[0]


def test_error_classes():
    base = lambda op="LSTM": workloads.random_case(op, "forward", 4, 3, 4, 5, seed=2)
    c = base()
    c.sequence_lens = torch.tensor([1, 5, 2], dtype=torch.int32)       # > seq
    assert _err(c) == oracle.INVALID_INPUT
    c.sequence_lens = torch.tensor([1, -1, 2], dtype=torch.int32)
    assert _err(c) == oracle.INVALID_INPUT
    c = base()
    c.hidden_size_attr = 6
    assert _err(c) == oracle.INVALID_INPUT
    c.hidden_size_attr = 5
    assert _err(c) == oracle.OK
    c = base()
    c.activations = ["Sigmoid", "Tanh"]
    assert _err(c) == oracle.INVALID_INPUT
    c.activations = ["Sigmoid", "Tanh", "Gelu"]
    assert _err(c) == oracle.INVALID_INPUT
    c = base()
    c.direction = "bidirectional"                                      # W has 1 direction
    assert _err(c) == oracle.INVALID_INPUT
    c = base("GRU")
    assert oracle.run(c, raise_on_error=False, want_yc=True)[0] == oracle.INVALID_INPUT
    c = base("GRU")
    c.input_forget = 1
    assert _err(c) == oracle.INVALID_INPUT
    c = base("LSTM")
    c.linear_before_reset = 1
    assert _err(c) == oracle.INVALID_INPUT
    c = base()
    c.layout = 2
    assert _err(c) == oracle.INVALID_INPUT


def test_zero_hidden_is_an_error():
    c = workloads.random_case("RNN", "forward", 2, 2, 3, 1, seed=2)
    c.hidden = 0
    c.R = torch.zeros(1, 0, 0)
    c.W = torch.zeros(1, 0, 3)
    c.B = None
    assert _err(c, want_y=False, want_yh=False) == oracle.INVALID_INPUT


def test_scratch_limit_is_unsupported():
    # per direction: seq*batch*G*H + 4*batch*H (+ G*H*(I+H) unless the weights
    # are constant) must stay below 2^30 floats, else Unsupported at plan time.
    no_out = dict(want_y=False, want_yh=False, want_yc=False)
    c = workloads.random_case("LSTM", "forward", 2, 2, 3, 4, seed=2)
    c.seq, c.batch = 2 ** 16, 2 ** 10                 # 2^16 * 2^10 * 4 * 4 = 2^30
    assert _err(c, **no_out) == oracle.UNSUPPORTED
    # 16 * batch * (seq + 1) = 2^30 - 16: below the limit with constant weights,
    # above it once the transposed weights (16 * 7 floats) are counted.
    c.seq, c.batch = 2 ** 26 - 2, 1
    c.sequence_lens = torch.tensor([-1], dtype=torch.int32)   # stops the run right after
    assert _err(c, **no_out) == oracle.UNSUPPORTED
    assert _err(c, constant_weights=True, **no_out) == oracle.INVALID_INPUT
