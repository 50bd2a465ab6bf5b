"""Exact mode (rnn_attrs.exact; onemodel "Recurrent operators", section
"Exact mode"): every output of the HIP path must equal the oracle's BIT FOR
BIT -- the products are one binary32 accumulator per value over k in
increasing order from +0 with each multiply and add rounded on its own, the
gate arithmetic is the written order, and the transcendental activations
follow the same binary64 method on both sides (written twice, sharing no
code).  The results must not depend on the tiling, the launch form or time
chunks."""
import numpy as np
import pytest
import torch

import oracle
import recurrent_nn_amd as ra
import workloads
from tests.test_gpu_parity import FEATURES, check_masks, oracle_outputs, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ra._lib.load()
    yield


def u32(a):
    return np.ascontiguousarray(a).view(np.uint32)


def assert_bit_exact(c, gpu, ref=None):
    ref = ref if ref is not None else oracle.run(c)[1:]
    for what, g, r in zip(("Y", "Y_h", "Y_c"), gpu, ref):
        if r is None:
            continue
        assert g.shape == r.shape, (what, g.shape, r.shape)
        diff = u32(g) != u32(r)
        if diff.any():
            i = np.argwhere(diff)[0]
            raise AssertionError(f"{what}: {int(diff.sum())} of {diff.size} values differ; first at "
                                 f"{tuple(i)}: gpu {g[tuple(i)]!r} oracle {r[tuple(i)]!r}")
    check_masks(c, *gpu)


@pytest.mark.parametrize("name", ["rnn_fwd_s4_b2_i3_h5", "lstm_bidir_s16_b4_i32_h64",
                                  "gru_fwd_s128_b32_i256_h512_lbr0",
                                  "gru_fwd_s128_b32_i256_h512_lbr1"])
def test_named_workloads_are_bit_exact(name):
    c = workloads.workload(name)
    say(f"case {c.name} exact")
    assert_bit_exact(c, run_gpu(c, exact=True))


@pytest.mark.parametrize("k", range(len(FEATURES)))
def test_feature_cases_are_bit_exact(k):
    spec = dict(FEATURES[k])
    op, direction = spec.pop("op"), spec.pop("direction")
    S, Bt, I, H = spec.pop("S"), spec.pop("Bt"), spec.pop("I"), spec.pop("H")
    lay = spec.pop("layout", 0)
    kw = {key: spec.pop(key) for key in ("with_lens", "with_p", "with_bias", "with_h0") if key in spec}
    kw.setdefault("with_h0", True)
    c = workloads.random_case(op, direction, S, Bt, I, H, seed=500 + k, layout=lay,
                              with_c0=(op == "LSTM"), scale=min(0.6, 1.5 / H ** 0.5),
                              **kw, **spec)
    say(f"case {c.name} exact {FEATURES[k]}")
    assert_bit_exact(c, run_gpu(c, exact=True))


def test_exact_results_do_not_depend_on_tiling_launch_or_chunks():
    c = workloads.random_case("LSTM", "bidirectional", 9, 50, 24, 128, seed=17, with_lens=True,
                              with_h0=True, with_c0=True, with_p=True, clip=1.5,
                              scale=1.5 / 128 ** 0.5)
    say(f"case {c.name} exact, several tilings")
    ref = oracle.run(c)[1:]
    for extra in [dict(), dict(units_per_block=3, batch_tile=16), dict(units_per_block=8, batch_tile=64),
                  dict(kernel_path=ra.RNN_PATH_PER_STEP), dict(time_chunk=4),
                  dict(time_chunk=1, batch_tile=32)]:
        assert_bit_exact(c, run_gpu(c, exact=True, **extra), ref)


def test_lstm_bench_workload_bit_exact_every_element():
    name = "lstm_bidir_s512_b64_i1024_h1024"
    c = workloads.workload(name)
    say(f"case {name} exact, every element")
    assert_bit_exact(c, run_gpu(c, exact=True), oracle_outputs(c, name))


def test_gru_bf16_workload_bit_exact_every_element():
    name = "gru_rev_s256_b256_i2048_h2048_bf16"
    c = workloads.workload(name)
    say(f"case {name} exact, every element")
    assert_bit_exact(c, run_gpu(c, exact=True), oracle_outputs(c, name))
