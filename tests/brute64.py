"""fp64 brute force of the ONNX recurrent operators, for tiny shapes.

An independent restatement (numpy, float64, whole-batch vector form) of the
formulas on the onemodel page "Recurrent operators: RNN, GRU, LSTM"
(sections "Support", "Computation", "Activations" and "Choices the
specification leaves open").  It pins the fp32 oracle: the two are written
differently (loops in C vs. vectorised numpy) and agree only to fp32 rounding.
It shares nothing with the oracle or with the HIP library.
"""
from __future__ import annotations

import numpy as np

_NA = {"RNN": 1, "GRU": 2, "LSTM": 3}
_DEFAULTS = {"RNN": ["tanh"], "GRU": ["sigmoid", "tanh"], "LSTM": ["sigmoid", "tanh", "tanh"]}
_ALPHA0 = {"leakyrelu": 0.01, "thresholdedrelu": 1.0, "elu": 1.0, "hardsigmoid": 0.2,
           "affine": 1.0, "scaledtanh": 1.0}
_BETA0 = {"hardsigmoid": 0.5, "affine": 0.0, "scaledtanh": 0.0}


def _act(name, a, b):
    n = name.lower()
    if n == "sigmoid":
        return lambda x: 1.0 / (1.0 + np.exp(-x))
    if n == "tanh":
        return np.tanh
    if n == "relu":
        return lambda x: np.where(x < 0, 0.0, x)
    if n == "affine":
        return lambda x: a * x + b
    if n == "leakyrelu":
        return lambda x: np.where(x < 0, a * x, x)
    if n == "thresholdedrelu":
        return lambda x: np.where(x > a, x, 0.0)
    if n == "scaledtanh":
        return lambda x: a * np.tanh(b * x)
    if n == "hardsigmoid":
        return lambda x: np.minimum(1.0, np.maximum(0.0, a * x + b))
    if n == "elu":
        return lambda x: np.where(x >= 0, x, a * np.expm1(np.minimum(x, 0.0)))
    if n == "softsign":
        return lambda x: x / (1.0 + np.abs(x))
    if n == "softplus":
        return lambda x: np.where(x > 20, x, np.log1p(np.exp(np.minimum(x, 20.0))))
    raise ValueError(name)


def _functions(case, dirs):
    na = _NA[case.op]
    names = [s.lower() for s in (case.activations or _DEFAULTS[case.op])]
    alpha = list(case.alpha or [])
    beta = list(case.beta or [])
    fs = []
    for n in names:
        a = alpha.pop(0) if (n in _ALPHA0 and alpha) else _ALPHA0.get(n, 0.0)
        b = beta.pop(0) if (n in _BETA0 and beta) else _BETA0.get(n, 0.0)
        # parameters are float32 values
        fs.append(_act(n, float(np.float32(a)), float(np.float32(b))))
    if len(fs) == na:
        return [fs] * dirs
    return [fs[d * na:(d + 1) * na] for d in range(dirs)]


def run(case, bf16_round=None):
    """Returns (Y, Y_h, Y_c) as float64 arrays in the case's layout."""
    op, S, Bt, I, H = case.op, case.seq, case.batch, case.input, case.hidden
    D = case.dirs
    G = {"RNN": 1, "GRU": 3, "LSTM": 4}[op]
    X = case.X.double().numpy()
    if case.layout == 1:
        X = X.transpose(1, 0, 2)                           # -> [S, Bt, I]
    if bf16_round is not None:
        X = bf16_round(X)
    W = case.W.double().numpy()
    if bf16_round is not None:
        W = bf16_round(W)
    R = case.R.double().numpy()
    B = None if case.B is None else case.B.double().numpy()
    P = None if case.P is None else case.P.double().numpy()

    def state(t):
        if t is None:
            return np.zeros((D, Bt, H))
        a = t.double().numpy()
        return a.transpose(1, 0, 2) if case.layout == 1 else a

    h0, c0 = state(case.initial_h), state(case.initial_c)
    lens = (np.full(Bt, S) if case.sequence_lens is None
            else np.asarray(case.sequence_lens, dtype=np.int64))
    clip = case.clip if (case.clip is not None and case.clip > 0) else None
    cl = (lambda v: np.clip(v, -clip, clip)) if clip is not None else (lambda v: v)
    fsets = _functions(case, D)

    Y = np.zeros((S, D, Bt, H))
    Yh = np.zeros((D, Bt, H))
    Yc = np.zeros((D, Bt, H))
    for d in range(D):
        rev = case.direction == "reverse" or d == 1
        f = fsets[d]
        Wd, Rd = W[d], R[d]
        wb = np.zeros(G * H) if B is None else B[d, :G * H]
        rb = np.zeros(G * H) if B is None else B[d, G * H:]
        h = h0[d].copy()
        c = c0[d].copy()
        for j in range(S):
            act = j < lens                                  # [Bt]
            t = np.where(rev, lens - 1 - j, j)
            t = np.clip(t, 0, S - 1)
            x = X[t, np.arange(Bt)]                         # [Bt, I]
            xw = x @ Wd.T
            if op == "RNN":
                hn = f[0](cl(xw + h @ Rd.T + wb + rb))
                cn = c
            elif op == "GRU":
                gz = slice(0, H)
                gr = slice(H, 2 * H)
                gh = slice(2 * H, 3 * H)
                z = f[0](cl(xw[:, gz] + h @ Rd[gz].T + wb[gz] + rb[gz]))
                r = f[0](cl(xw[:, gr] + h @ Rd[gr].T + wb[gr] + rb[gr]))
                if case.linear_before_reset:
                    ph = xw[:, gh] + r * (h @ Rd[gh].T + rb[gh]) + wb[gh]
                else:
                    ph = xw[:, gh] + (r * h) @ Rd[gh].T + wb[gh] + rb[gh]
                ht = f[1](cl(ph))
                hn = (1 - z) * ht + z * h
                cn = c
            else:
                gi, go, gf, gc = (slice(k * H, (k + 1) * H) for k in range(4))
                pre = xw + h @ Rd.T + wb + rb
                pi, po, pf, pc = pre[:, gi], pre[:, go], pre[:, gf], pre[:, gc]
                if P is not None:
                    pi = pi + P[d, 0:H] * c
                    pf = pf + P[d, 2 * H:3 * H] * c
                i = f[0](cl(pi))
                fg = (1 - i) if case.input_forget else f[0](cl(pf))
                ct = f[1](cl(pc))
                cn = fg * c + i * ct
                if P is not None:
                    po = po + P[d, H:2 * H] * cn
                o = f[0](cl(po))
                hn = o * f[2](cn)
            m = act[:, None]
            h = np.where(m, hn, h)
            c = np.where(m, cn, c)
            for b in range(Bt):
                if act[b]:
                    Y[t[b], d, b] = hn[b]
        Yh[d] = np.where((lens > 0)[:, None], h, 0.0)
        Yc[d] = np.where((lens > 0)[:, None], c, 0.0)
    if case.layout == 1:
        return Y.transpose(2, 0, 1, 3), Yh.transpose(1, 0, 2), Yc.transpose(1, 0, 2)
    return Y, Yh, Yc
