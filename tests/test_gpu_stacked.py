"""Stacked layers: one layer's Y is the next layer's X.  In layout 1, Y
[batch, seq, dirs, hidden] is already X [batch, seq, dirs * hidden] for any
number of directions; in layout 0 with one direction, Y [seq, 1, batch,
hidden] is X [seq, batch, hidden].  Either way the second layer reads the
first layer's output in place (a view, no copy).  The oracle runs the same
two layers on its own first-layer output; the second layer's outputs must
agree within the parity tolerance, and Y's zero positions stay bit-exact."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import recurrent_nn_amd as ra
import workloads
from tests.test_gpu_parity import compare, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ra._lib.load()
    yield


def _dev(c):
    return {k: (v.cuda() if v is not None and k != "sequence_lens" else v)
            for k, v in c.tensors().items()}


CASES = [
    # layout 1, bidirectional GRU into a forward LSTM
    (dict(op="GRU", direction="bidirectional", linear_before_reset=1, layout=1),
     dict(op="LSTM", direction="forward", layout=1, with_p=True)),
    # layout 0, one direction: reverse LSTM into a forward RNN
    (dict(op="LSTM", direction="reverse", layout=0),
     dict(op="RNN", direction="forward", layout=0)),
]


@pytest.mark.parametrize("k", range(len(CASES)))
def test_second_layer_reads_the_first_layers_y_in_place(k):
    s1, s2 = (dict(x) for x in CASES[k])
    S, Bt, I, H1, H2 = 9, 11, 12, 24, 20
    op1, dir1, lay = s1.pop("op"), s1.pop("direction"), s1.pop("layout")
    op2, dir2 = s2.pop("op"), s2.pop("direction")
    s2.pop("layout")
    D1 = 2 if dir1 == "bidirectional" else 1
    c1 = workloads.random_case(op1, dir1, S, Bt, I, H1, seed=1600 + k, layout=lay, with_lens=True,
                               with_h0=True, with_c0=(op1 == "LSTM"), scale=0.3, **s1)
    c2 = workloads.random_case(op2, dir2, S, Bt, D1 * H1, H2, seed=1700 + k, layout=lay,
                               with_h0=True, with_c0=(op2 == "LSTM"), scale=0.3, **s2)
    c2.sequence_lens = c1.sequence_lens
    say(f"case {c1.name} -> {c2.name}")

    # GPU: layer 1, then layer 2 on a view of layer 1's Y
    t1 = _dev(c1)
    p1, p2 = ra.plan_for_case(c1), ra.plan_for_case(c2)
    Y1, _, _ = p1.run(t1["X"], t1["W"], t1["R"], t1["B"], t1["sequence_lens"], t1["initial_h"],
                      t1["initial_c"], t1["P"])
    x2_shape = (Bt, S, D1 * H1) if lay == 1 else (S, Bt, H1)
    X2 = Y1.view(x2_shape)
    assert X2.data_ptr() == Y1.data_ptr()
    t2 = _dev(c2)
    got = p2.run(X2, t2["W"], t2["R"], t2["B"], t2["sequence_lens"], t2["initial_h"],
                 t2["initial_c"], t2["P"])
    torch.cuda.synchronize()
    got = tuple(to_np(t) for t in got)

    # oracle: the same two layers, the second on the oracle's first-layer Y
    _, Y1o, _, _ = oracle.run(c1)
    c2o = dataclasses.replace(c2, X=torch.from_numpy(np.ascontiguousarray(Y1o).reshape(x2_shape)))
    compare(c2o, got)
