"""Parity of rnn_cell_run (one step, summed bias, new state only; the
single-cell convention of the OpenVINO page "RNNCell-3") with the oracle's
run_cell, element by element: |gpu - oracle| <= 2e-5 + 1e-4 |oracle|."""
import numpy as np
import pytest
import torch

import oracle
import recurrent_nn_amd as ra

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-5, 1e-4
G = {"RNN": 1, "GRU": 3, "LSTM": 4}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ra._lib.load()
    yield


CASES = [
    dict(op="RNN", Bt=5, I=12, H=40, with_h=True, with_b=True),
    dict(op="RNN", Bt=3, I=7, H=9, with_h=False, with_b=False, activations=["Relu"]),
    dict(op="GRU", Bt=33, I=20, H=96, with_h=True, with_b=True, clip=0.6),
    dict(op="GRU", Bt=8, I=16, H=64, with_h=True, with_b=False, linear_before_reset=1),
    dict(op="LSTM", Bt=17, I=24, H=130, with_h=True, with_b=True, with_p=True, with_c=True),
    dict(op="LSTM", Bt=64, I=40, H=512, with_h=True, with_b=True, with_c=True),
    dict(op="LSTM", Bt=64, I=64, H=1024, with_h=True, with_b=True, with_c=True, no_cout=True),
]


@pytest.mark.parametrize("k", range(len(CASES)))
def test_cell_run_matches_the_oracle(k):
    spec = dict(CASES[k])
    op, Bt, I, H = spec.pop("op"), spec.pop("Bt"), spec.pop("I"), spec.pop("H")
    with_h, with_b = spec.pop("with_h"), spec.pop("with_b")
    with_p, with_c = spec.pop("with_p", False), spec.pop("with_c", False)
    no_cout = spec.pop("no_cout", False)
    g = torch.Generator().manual_seed(900 + k)
    s = min(0.6, 1.5 / H ** 0.5)
    u = lambda *shape, a=1.0: (torch.rand(shape, generator=g) * 2 - 1) * a
    X, W, R = u(Bt, I), u(G[op] * H, I, a=s), u(G[op] * H, H, a=s)
    Bs = u(G[op] * H, a=0.3) if with_b else None
    Hp = u(Bt, H, a=0.5) if with_h else None
    Cp = u(Bt, H, a=0.5) if with_c else None
    P = u(3 * H, a=0.1) if with_p else None
    print(f"case {k}: {CASES[k]}", flush=True)
    ref_h, ref_c = oracle.run_cell(op, X, W, R, Bs, H=Hp, C=Cp, P=P, **spec)
    cell = ra.RNNCell(op, Bt, I, H, **spec)
    d = lambda t: None if t is None else t.cuda()
    ho, co = cell.step(d(X), d(W), d(R), d(Bs), d(Hp), d(Cp), d(P))
    if no_cout:
        ho2 = torch.empty_like(ho)
        cell.step(d(X), d(W), d(R), d(Bs), d(Hp), d(Cp), d(P), out=(ho2, None))
        torch.cuda.synchronize()
        assert torch.equal(ho2, ho)
    torch.cuda.synchronize()
    got = ho.cpu().numpy()
    assert np.all(np.abs(got - ref_h) <= ATOL + RTOL * np.abs(ref_h)), np.abs(got - ref_h).max()
    if op == "LSTM":
        gc = co.cpu().numpy()
        assert np.all(np.abs(gc - ref_c) <= ATOL + RTOL * np.abs(ref_c))


def test_cell_step_equals_a_one_step_sequence_with_split_bias():
    # the summed bias as ONNX B = [B_sum, 0] through rnn_run gives the same bits
    g = torch.Generator().manual_seed(77)
    Bt, I, H = 20, 16, 96
    X = torch.rand(Bt, I, generator=g) - 0.5
    W = (torch.rand(4 * H, I, generator=g) - 0.5) * 0.2
    R = (torch.rand(4 * H, H, generator=g) - 0.5) * 0.2
    Bs = torch.rand(4 * H, generator=g) - 0.5
    Hp, Cp = torch.rand(Bt, H, generator=g) - 0.5, torch.rand(Bt, H, generator=g) - 0.5
    cell = ra.RNNCell("LSTM", Bt, I, H)
    ho, co = cell.step(X.cuda(), W.cuda(), R.cuda(), Bs.cuda(), Hp.cuda(), Cp.cuda())
    seq = ra.RNNPlan("LSTM", 1, Bt, I, H)
    B = torch.cat([Bs, torch.zeros(4 * H)])[None]
    Y, Yh, Yc = seq.run(X[None].cuda(), W[None].cuda(), R[None].cuda(), B.cuda(), None,
                        Hp[None].cuda(), Cp[None].cuda())
    torch.cuda.synchronize()
    assert torch.equal(ho.view(torch.int32), Yh[0].view(torch.int32))
    assert torch.equal(co.view(torch.int32), Yc[0].view(torch.int32))
    assert torch.equal(Y[0, 0].view(torch.int32), Yh[0].view(torch.int32))
