"""Pins of the oracle's binary64 elementary functions (the written method in
oracle/rnn_oracle.c, "Binary64 elementary functions"), through the
activations that use them: against numpy's binary64 exp / tanh / expm1 /
logaddexp rounded once to binary32.  The method is accurate to far below a
binary32 ulp, so the two must agree within one ulp everywhere and exactly on
all but a vanishing share of points (only where the binary64 value sits
within ~1e-16 of a binary32 rounding boundary can they differ)."""
import numpy as np
import pytest

import oracle


def _samples():
    rs = np.random.RandomState(123)
    x = np.concatenate([
        np.linspace(-30, 30, 20001),
        rs.uniform(-100, 100, 5000),
        rs.normal(0, 1, 5000),
        rs.uniform(-1e-3, 1e-3, 2000),
        [0.0, -0.0, 1e-30, -1e-30, 0.5, -0.5, 0.25, 20.0, -20.0, 22.0, -22.0, 11.0, -11.0,
         87.0, -87.0, 88.7, -88.7, 103.0, -103.0, 1e6, -1e6],
    ]).astype(np.float32)
    return x


def _ulp_diff(a, b):
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


REFS = {
    "Sigmoid": (lambda x, a, b: 1.0 / (1.0 + np.exp(-x)), 0.0, 0.0),
    "Tanh": (lambda x, a, b: np.tanh(x), 0.0, 0.0),
    "ScaledTanh": (lambda x, a, b: a * np.tanh(b * x), 1.7, 0.6),
    "Elu": (lambda x, a, b: np.where(x >= 0, x, a * np.expm1(np.minimum(x, 0))), 0.8, 0.0),
    "Softplus": (lambda x, a, b: np.logaddexp(0.0, x), 0.0, 0.0),
}


@pytest.mark.parametrize("name", sorted(REFS))
def test_transcendental_activations_are_correctly_rounded_binary64(name):
    f, alpha, beta = REFS[name]
    x = _samples()
    got = oracle.activation(name, x, alpha, beta)
    with np.errstate(over="ignore"):
        ref = f(x.astype(np.float64), np.float64(np.float32(alpha)),
                np.float64(np.float32(beta))).astype(np.float32)
    if name == "Elu":
        ref = np.where(x >= 0, x, ref)          # the positive branch is x itself
    d = _ulp_diff(got, ref)
    assert d.max() <= 1, (name, x[np.argmax(d)], got[np.argmax(d)], ref[np.argmax(d)])
    assert np.count_nonzero(d) <= 3, (name, np.count_nonzero(d), x[d > 0][:5])


@pytest.mark.parametrize("name", sorted(REFS))
def test_transcendental_activations_special_values(name):
    _, alpha, beta = REFS[name]
    nan = oracle.activation(name, np.array([np.nan], np.float32), alpha, beta)
    assert np.isnan(nan).all()
    big = oracle.activation(name, np.array([np.inf, -np.inf], np.float32), alpha, beta)
    expect = {"Sigmoid": [1.0, 0.0], "Tanh": [1.0, -1.0], "ScaledTanh": [alpha, -alpha],
              "Elu": [np.inf, -alpha], "Softplus": [np.inf, 0.0]}[name]
    assert np.array_equal(big, np.array(expect, np.float32))
