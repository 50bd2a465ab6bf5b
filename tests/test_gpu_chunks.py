"""Time-chunked execution (rnn_attrs.time_chunk): the projections and the H
history are held for one chunk of steps at a time and the states carry over
between chunks.  The arithmetic per element is unchanged, so every output
must be bit-identical to the unchunked run, and within the parity tolerance
of the oracle."""
import hashlib

import numpy as np
import pytest
import torch

import recurrent_nn_amd as ra
import workloads
from tests.test_gpu_parity import compare, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ra._lib.load()
    yield


def _digest(out):
    h = hashlib.sha256()
    for a in out:
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


CASES = [
    # reverse with ragged lengths: each chunk gathers per-row time windows
    dict(op="GRU", direction="reverse", S=23, Bt=37, I=24, H=96, with_lens=True,
         linear_before_reset=1, layout=1, chunks=[1, 5, 8]),
    # bidirectional LSTM, peepholes, the pipelined kernel (hidden 512)
    dict(op="LSTM", direction="bidirectional", S=17, Bt=40, I=32, H=512, with_lens=True,
         with_p=True, chunks=[4, 6]),
    # GRU with two phases per step; 16 columns of H per wave, so that a wave's
    # k range is part of a cache line that other unit blocks also write (the
    # step hand-over must wait for all of them)
    dict(op="GRU", direction="bidirectional", S=13, Bt=20, I=16, H=64, with_lens=True,
         linear_before_reset=0, chunks=[2, 5]),
    # RNN, full lengths, layout 1
    dict(op="RNN", direction="forward", S=30, Bt=9, I=11, H=33, layout=1, chunks=[7]),
]


@pytest.mark.parametrize("k", range(len(CASES)))
def test_chunked_runs_are_bit_identical_to_unchunked(k):
    spec = dict(CASES[k])
    chunks = spec.pop("chunks")
    op, direction = spec.pop("op"), spec.pop("direction")
    S, Bt, I, H = spec.pop("S"), spec.pop("Bt"), spec.pop("I"), spec.pop("H")
    lay = spec.pop("layout", 0)
    kw = {key: spec.pop(key) for key in ("with_lens", "with_p") if key in spec}
    c = workloads.random_case(op, direction, S, Bt, I, H, seed=1100 + k, layout=lay,
                              with_h0=True, with_c0=(op == "LSTM"),
                              scale=min(0.6, 1.5 / H ** 0.5), **kw, **spec)
    say(f"case {c.name} {CASES[k]}")
    full = run_gpu(c)
    compare(c, full)
    for ch in chunks:
        got = run_gpu(c, time_chunk=ch)
        assert _digest(got) == _digest(full), f"time_chunk={ch}"
    # the per-step launch form with chunks too
    got = run_gpu(c, time_chunk=chunks[0], kernel_path=ra.RNN_PATH_PER_STEP)
    assert _digest(got) == _digest(full)


def test_chunked_bench_shape_sampled():
    # the bidirectional LSTM workload's shape in chunks of 64 steps, on a few
    # batch rows: same bits as unchunked
    c = workloads.workload("lstm_bidir_s512_b64_i1024_h1024", batch_rows=list(range(16)))
    say(f"case {c.name} (16 rows) in chunks of 64 steps")
    assert _digest(run_gpu(c, time_chunk=64)) == _digest(run_gpu(c))
