"""Parity of the HIP path (through the C-ABI) with the CPU oracle.

Floating point: |gpu - oracle| <= 2e-5 + 1e-4 * |oracle| element by element
(fp32 projection); on the named workloads also max |gpu - oracle| <= 2e-5 over
every element (which implies the relative bar 1e-4 wherever |oracle| >= 0.2).
For the bf16-projection workload: the fp32 bars against the oracle run with
the same bf16 rounding of X and W, and <= 2e-2 against the fp32 oracle.
Masked positions (t >= sequence_lens[b]), zero-length rows and NaN bit
patterns are compared bit for bit.  The two large workloads run at full size
in the benchmark's launch configuration and are compared on every element of
Y, Y_h and Y_c."""
import dataclasses
import hashlib
import sys

import numpy as np
import pytest
import torch

import oracle
import recurrent_nn_amd as ra
import workloads

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-5, 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ra._lib.load()
    yield


def u32(a):
    return np.ascontiguousarray(a).view(np.uint32)


def to_np(t):
    return None if t is None else t.detach().cpu().numpy()


def run_gpu(c, **extra):
    say(f"  gpu run: {c.name} {extra}")
    Y, Yh, Yc = ra.run_case(c, **extra)
    torch.cuda.synchronize()
    return to_np(Y), to_np(Yh), to_np(Yc)


def check_close(got, ref, what, atol=ATOL, rtol=RTOL, max_abs=None):
    """Elementwise |g - o| <= atol + rtol |o|; with max_abs also max |g - o|
    <= max_abs over every element."""
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    nan_r = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_r), f"{what}: NaN positions differ"
    if nan_r.any():
        assert np.all(u32(got)[nan_r] == 0x7FC00000), f"{what}: NaN not canonical"
    g, r = got[~nan_r].astype(np.float64), ref[~nan_r].astype(np.float64)
    err = np.abs(g - r)
    del g
    bad = err > atol + rtol * np.abs(r)
    mx = float(err.max()) if err.size else 0.0
    say(f"    {what}: n={err.size} max_abs={mx:.3e} "
        f"max_rel(|o|>=0.2)={(err / np.maximum(np.abs(r), 0.2)).max() if err.size else 0:.3e} "
        f"bad={int(bad.sum())}/{err.size}")
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside {atol} + {rtol}|o|"
    if max_abs is not None:
        assert mx <= max_abs, f"{what}: max |gpu - oracle| = {mx:.3e} > {max_abs}"


def y_positions(c, Y, d, b):
    """Y[t, d, b, :] over t for either layout."""
    return Y[:, d, b] if c.layout == 0 else Y[b, :, d]


def check_masks(c, Y, Yh, Yc):
    """Bit-exact: +0.0 at t >= len_b, and zero final states for len_b = 0."""
    if c.sequence_lens is None:
        return
    lens = c.sequence_lens.numpy()
    D = int(c.W.shape[0])
    for d in range(D):
        for b, L in enumerate(lens):
            tail = y_positions(c, Y, d, b)[L:]
            assert np.all(u32(tail) == 0), f"Y not +0.0 past len at d={d} b={b}"
            if L == 0:
                sh = Yh[d, b] if c.layout == 0 else Yh[b, d]
                assert np.all(u32(sh) == 0)
                if Yc is not None:
                    sc = Yc[d, b] if c.layout == 0 else Yc[b, d]
                    assert np.all(u32(sc) == 0)


def compare(c, gpu, ref=None, atol=ATOL, rtol=RTOL, strict=False):
    """Y, Y_h (and Y_c) against the oracle; strict adds max |g - o| <= atol."""
    if ref is None:
        _, *ref = oracle.run(c)
    Y, Yh, Yc = gpu
    mx = atol if strict else None
    check_close(Y, ref[0], "Y", atol, rtol, mx)
    check_close(Yh, ref[1], "Y_h", atol, rtol, mx)
    if c.op == "LSTM":
        check_close(Yc, ref[2], "Y_c", atol, rtol, mx)
    check_masks(c, Y, Yh, Yc)


_ORACLE_CACHE = {}


def oracle_outputs(c, key=None):
    """The oracle's (Y, Y_h, Y_c) for a case, kept for the session under `key`
    (the large workloads are compared by several tests)."""
    if key is None:
        return tuple(oracle.run(c)[1:])
    if key not in _ORACLE_CACHE:
        say(f"  oracle run: {key}")
        _ORACLE_CACHE[key] = tuple(oracle.run(c)[1:])
    return _ORACLE_CACHE[key]


# ---------------------------------------------------------------------------
# The named workloads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["rnn_fwd_s4_b2_i3_h5", "lstm_bidir_s16_b4_i32_h64",
                                  "gru_fwd_s128_b32_i256_h512_lbr0",
                                  "gru_fwd_s128_b32_i256_h512_lbr1"])
def test_small_workloads_match_oracle(name):
    c = workloads.workload(name)
    say(f"case {name}")
    compare(c, run_gpu(c), strict=True)


def test_lstm_bench_workload_every_element():
    name = "lstm_bidir_s512_b64_i1024_h1024"
    c = workloads.workload(name)
    say(f"case {name}: full size on the GPU, every element against the oracle")
    gpu = run_gpu(c)
    compare(c, gpu, oracle_outputs(c, name), strict=True)


def test_gru_bf16_workload_every_element():
    name = "gru_rev_s256_b256_i2048_h2048_bf16"
    c = workloads.workload(name)
    say(f"case {name}: full size on the GPU, every element against the oracle")
    gpu = run_gpu(c)
    # against the oracle with the same bf16 rounding of X and W: the fp32 bars
    compare(c, gpu, oracle_outputs(c, name), strict=True)
    # against the fp32 oracle: the bf16-projection bar
    c32 = dataclasses.replace(c, proj_bf16=False)
    ref32 = oracle_outputs(c32, name + ":fp32")
    check_close(gpu[0], ref32[0], "Y vs fp32 oracle", atol=2e-2, rtol=0.0, max_abs=2e-2)
    check_close(gpu[1], ref32[1], "Y_h vs fp32 oracle", atol=2e-2, rtol=0.0, max_abs=2e-2)


# ---------------------------------------------------------------------------
# Features, ragged shapes and edge cases
# ---------------------------------------------------------------------------

FEATURES = [
    dict(op="RNN", direction="forward", S=9, Bt=70, I=45, H=70, activations=["Relu"]),
    dict(op="RNN", direction="bidirectional", S=6, Bt=5, I=8, H=33, layout=1, with_lens=True,
         activations=["Affine", "LeakyRelu"], alpha=[0.8, 0.1], beta=[0.05]),
    dict(op="GRU", direction="forward", S=8, Bt=20, I=12, H=200, with_lens=True,
         linear_before_reset=0, clip=0.7),
    dict(op="GRU", direction="reverse", S=7, Bt=37, I=24, H=96, with_lens=True,
         linear_before_reset=1, layout=1),
    dict(op="GRU", direction="bidirectional", S=5, Bt=66, I=16, H=40, linear_before_reset=0,
         activations=["HardSigmoid", "Softsign", "Sigmoid", "Elu"], alpha=[0.3, 0.8], beta=[0.45]),
    dict(op="LSTM", direction="forward", S=6, Bt=17, I=20, H=130, with_p=True, clip=0.8,
         with_lens=True),
    dict(op="LSTM", direction="bidirectional", S=5, Bt=9, I=7, H=64, with_p=True, input_forget=1,
         layout=1, with_lens=True),
    dict(op="LSTM", direction="reverse", S=4, Bt=3, I=5, H=11,
         activations=["HardSigmoid", "LeakyRelu", "ScaledTanh"], alpha=[0.3, 0.2, 1.2],
         beta=[0.4, 0.7], with_lens=True),
    dict(op="LSTM", direction="forward", S=3, Bt=4, I=6, H=9,
         activations=["ThresholdedRelu", "Softplus", "Relu"], alpha=[0.1]),
    dict(op="RNN", direction="forward", S=5, Bt=3, I=4, H=6, with_bias=False,
         activations=["Elu"], alpha=[0.5]),
    dict(op="GRU", direction="forward", S=4, Bt=2, I=3, H=7, with_bias=False, with_h0=False,
         linear_before_reset=1, activations=["Sigmoid", "ScaledTanh"], alpha=[1.3], beta=[0.6]),
    dict(op="LSTM", direction="forward", S=24, Bt=32, I=64, H=512, with_lens=True),
    # R streamed with an odd number of k blocks per wave (5 and 7)
    dict(op="RNN", direction="reverse", S=5, Bt=24, I=16, H=300, with_lens=True),
    dict(op="GRU", direction="forward", S=4, Bt=40, I=24, H=420, linear_before_reset=1,
         with_lens=True),
]


# Projection staging: whole k stages (buffer loads), a partial last stage
# (checked loads) and inputs whose K is not a multiple of the 16-byte load
# (checked loads only), for both operand types, with ragged M and N tiles.
# The bf16 cases are held to the fp32 bar against the oracle run with the
# same bf16 rounding of X and W.
STAGING = [
    dict(op="GRU", direction="forward", S=5, Bt=50, I=100, H=70, linear_before_reset=0,
         with_lens=True),                                  # fp32: 3 whole stages + 4
    dict(op="GRU", direction="reverse", S=6, Bt=40, I=72, H=96, linear_before_reset=1,
         with_lens=True, proj_bf16=True),                  # bf16: 1 whole stage + 8
    dict(op="LSTM", direction="bidirectional", S=5, Bt=20, I=30, H=64, with_lens=True,
         proj_bf16=True),                                  # bf16: K % 8 != 0
    dict(op="RNN", direction="forward", S=9, Bt=130, I=136, H=40, layout=1,
         proj_bf16=True),                                  # bf16: 2 whole stages + 8, 3 batch blocks
    dict(op="LSTM", direction="forward", S=4, Bt=8, I=256, H=130, with_p=True,
         proj_bf16=True),                                  # bf16: whole stages only
]


@pytest.mark.parametrize("k", range(len(STAGING)))
def test_projection_staging_cases_match_oracle(k):
    spec = dict(STAGING[k])
    op, direction = spec.pop("op"), spec.pop("direction")
    S, Bt, I, H = spec.pop("S"), spec.pop("Bt"), spec.pop("I"), spec.pop("H")
    lay = spec.pop("layout", 0)
    kw = {key: spec.pop(key) for key in ("with_lens", "with_p") if key in spec}
    c = workloads.random_case(op, direction, S, Bt, I, H, seed=700 + k, layout=lay,
                              with_h0=True, with_c0=(op == "LSTM"),
                              scale=min(0.6, 1.5 / H ** 0.5), **kw, **spec)
    say(f"case {c.name} {STAGING[k]}")
    compare(c, run_gpu(c))


@pytest.mark.parametrize("k", range(len(FEATURES)))
def test_feature_cases_match_oracle(k):
    spec = dict(FEATURES[k])
    op, direction = spec.pop("op"), spec.pop("direction")
    S, Bt, I, H = spec.pop("S"), spec.pop("Bt"), spec.pop("I"), spec.pop("H")
    lay = spec.pop("layout", 0)
    kw = {key: spec.pop(key) for key in ("with_lens", "with_p", "with_bias", "with_h0") if key in spec}
    kw.setdefault("with_h0", True)
    # weights ~ U(+-1.5/sqrt(H)) (at most 0.6) keep the recurrence contractive,
    # as in the named workloads, so that fp32 rounding differences do not grow
    c = workloads.random_case(op, direction, S, Bt, I, H, seed=500 + k, layout=lay,
                              with_c0=(op == "LSTM"), scale=min(0.6, 1.5 / H ** 0.5),
                              **kw, **spec)
    say(f"case {c.name} {FEATURES[k]}")
    compare(c, run_gpu(c))


# The streamed kernel with up to 8 (row, unit) pairs per thread, forced
# through units_per_block: XW of every pair is loaded during the previous
# product, for one phase (GRU linear_before_reset = 0: z and r, then the
# candidate) or both; ragged batch blocks leave threads with fewer pairs.
EIGHT_PAIRS = [
    (dict(op="GRU", direction="bidirectional", S=5, Bt=70, I=16, H=64, with_lens=True,
          linear_before_reset=0), 16),                  # 4 pairs per thread, two phases
    (dict(op="GRU", direction="bidirectional", S=4, Bt=37, I=12, H=96, with_lens=True,
          linear_before_reset=0, clip=0.9), 32),        # 8 pairs per thread, two phases
    (dict(op="LSTM", direction="forward", S=5, Bt=50, I=20, H=72, with_lens=True, with_p=True,
          clip=0.8), 24),                               # 6 pairs per thread, one phase
]


@pytest.mark.parametrize("k", range(len(EIGHT_PAIRS)))
def test_eight_pair_streamed_kernel_matches_oracle(k):
    spec, units = dict(EIGHT_PAIRS[k][0]), EIGHT_PAIRS[k][1]
    op, direction = spec.pop("op"), spec.pop("direction")
    S, Bt, I, H = spec.pop("S"), spec.pop("Bt"), spec.pop("I"), spec.pop("H")
    kw = {key: spec.pop(key) for key in ("with_lens", "with_p") if key in spec}
    c = workloads.random_case(op, direction, S, Bt, I, H, seed=900 + k, with_h0=True,
                              with_c0=(op == "LSTM"), scale=min(0.6, 1.5 / H ** 0.5), **kw, **spec)
    plan = ra.plan_for_case(c, units_per_block=units)
    d = dict(kv.split("=", 1) for kv in plan.describe().split() if "=" in kv)
    pairs = -(-int(d["BT"]) * int(d["U"]) // (64 * int(d["waves"])))
    assert d["resident"] == "0" and pairs > 2, plan.describe()
    say(f"case {c.name} units_per_block={units}: {plan.describe()}")
    compare(c, run_gpu(c, plan=plan))


def test_zero_length_rows_and_masks_bit_exact():
    c = workloads.random_case("LSTM", "bidirectional", 9, 19, 10, 24, seed=7, with_h0=True,
                              with_c0=True, lens=[0, 9, 1, 0, 5, 2, 9, 0, 3, 4, 8, 7, 6, 1, 0, 9, 2,
                                                  5, 3])
    say(f"case {c.name}")
    compare(c, run_gpu(c))


def test_nan_is_canonical_on_gpu():
    c = workloads.random_case("GRU", "bidirectional", 6, 5, 8, 20, seed=3, with_h0=True,
                              lens=[6, 3, 0, 1, 5], linear_before_reset=1)
    X = c.X.numpy().copy()
    X.view(np.uint32)[2, 0, 1] = 0xFFC00123          # a negative NaN with payload
    c.X = torch.from_numpy(X)
    say(f"case {c.name} with an injected NaN")
    compare(c, run_gpu(c))


@pytest.mark.parametrize("op", ["RNN", "GRU", "LSTM"])
def test_zero_size_on_gpu(op):
    c = workloads.random_case(op, "bidirectional", 0, 3, 4, 5, seed=1, with_h0=True,
                              with_c0=(op == "LSTM"))
    say(f"case {c.name}")
    Y, Yh, Yc = run_gpu(c)
    assert Y.size == 0
    assert np.array_equal(u32(Yh), u32(c.initial_h.numpy()))
    if op == "LSTM":
        assert np.array_equal(u32(Yc), u32(c.initial_c.numpy()))
    c = workloads.random_case(op, "forward", 4, 0, 4, 5, seed=1)
    Y, Yh, Yc = run_gpu(c)
    assert Y.size == 0 and Yh.size == 0


# ---------------------------------------------------------------------------
# Paths, grid sizes, determinism and the invariants on the GPU path
# ---------------------------------------------------------------------------

def _digest(out):
    h = hashlib.sha256()
    for a in out:
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("op,attrs", [("LSTM", {}), ("GRU", dict(linear_before_reset=0)),
                                      ("GRU", dict(linear_before_reset=1)), ("RNN", {})])
def test_persistent_and_per_step_paths_agree_bitwise(op, attrs):
    c = workloads.random_case(op, "bidirectional", 11, 40, 24, 96, seed=9, with_lens=True,
                              with_h0=True, with_c0=(op == "LSTM"), with_p=(op == "LSTM"), **attrs)
    say(f"case {c.name}")
    a = run_gpu(c, kernel_path=ra.RNN_PATH_PERSISTENT)
    b = run_gpu(c, kernel_path=ra.RNN_PATH_PER_STEP)
    assert _digest(a) == _digest(b)
    compare(c, a)


def test_results_do_not_depend_on_the_grid():
    c = workloads.random_case("LSTM", "bidirectional", 7, 50, 32, 128, seed=13, with_lens=True,
                              with_h0=True, with_c0=True)
    say(f"case {c.name}")
    digests = set()
    for upb, bt in [(0, 0), (1, 16), (3, 32), (4, 64), (8, 16), (0, 128), (12, 128)]:
        digests.add(_digest(run_gpu(c, units_per_block=upb, batch_tile=bt)))
    assert len(digests) == 1


@pytest.mark.parametrize("op,attrs", [("GRU", dict(linear_before_reset=1)),
                                      ("GRU", dict(linear_before_reset=0)), ("LSTM", {})])
def test_batch_tile_of_128_rows_matches_oracle_and_the_64_row_tile(op, attrs):
    # two batch blocks (128 rows and a ragged 22), lengths, R streamed
    c = workloads.random_case(op, "reverse", 7, 150, 20, 96, seed=61, with_lens=True,
                              with_h0=True, with_c0=(op == "LSTM"), with_p=(op == "LSTM"),
                              scale=1.5 / 96 ** 0.5, **attrs)
    plan = ra.plan_for_case(c, batch_tile=128)
    say(f"case {c.name} {attrs}: {plan.describe()}")
    assert "BT=128" in plan.describe() and "NBB=2" in plan.describe()
    got = run_gpu(c, plan=plan)
    compare(c, got)
    assert _digest(got) == _digest(run_gpu(c, batch_tile=64))


def test_repeated_runs_are_bit_identical():
    c = workloads.workload("gru_fwd_s128_b32_i256_h512_lbr0")
    say(f"case {c.name}")
    plan = ra.plan_for_case(c)
    outs = set()
    for _ in range(3):
        Y, Yh, _ = ra.run_case(c, plan=plan)
        torch.cuda.synchronize()
        outs.add(_digest((to_np(Y), to_np(Yh))))
    assert len(outs) == 1
    plan.check()


def test_invariants_hold_bitwise_on_gpu():
    c = workloads.random_case("GRU", "reverse", 8, 6, 10, 24, seed=21, with_h0=True,
                              lens=[8, 5, 1, 0, 7, 3], linear_before_reset=0)
    say(f"case {c.name}")
    Y, Yh, _ = run_gpu(c)
    # reverse == forward on per-row flipped input
    f = dataclasses.replace(c, direction="forward")
    X = c.X.clone()
    for b, L in enumerate(c.sequence_lens.tolist()):
        X[:L, b] = c.X[:L, b].flip(0)
    f.X = X
    Yf, Yhf, _ = run_gpu(f)
    for b, L in enumerate(c.sequence_lens.tolist()):
        assert np.array_equal(u32(Y[:L, 0, b]), u32(Yf[:L, 0, b][::-1]))
    assert np.array_equal(u32(Yh), u32(Yhf))
    # layout 1 == transposed layout 0
    t = dataclasses.replace(c, layout=1)
    t.X = c.X.transpose(0, 1).contiguous()
    t.initial_h = c.initial_h.transpose(0, 1).contiguous()
    Y1, Yh1, _ = run_gpu(t)
    assert np.array_equal(u32(Y1), u32(np.ascontiguousarray(Y.transpose(2, 0, 1, 3))))
    # state carry: (S1 + S2) == S1 then S2 from Y_h (forward, full length)
    g = workloads.random_case("LSTM", "forward", 9, 6, 10, 24, seed=22, with_h0=True, with_c0=True)
    Yg, Yhg, Ycg = run_gpu(g)
    a = dataclasses.replace(g, seq=4)
    a.X = g.X[:4].contiguous()
    Ya, Yha, Yca = run_gpu(a)
    b = dataclasses.replace(g, seq=5)
    b.X = g.X[4:].contiguous()
    b.initial_h, b.initial_c = torch.from_numpy(Yha), torch.from_numpy(Yca)
    Yb, Yhb, Ycb = run_gpu(b)
    assert np.array_equal(u32(Yg), u32(np.concatenate([Ya, Yb])))
    assert np.array_equal(u32(Ycg), u32(Ycb))


def test_constant_weights_are_packed_once_and_reused():
    c = workloads.random_case("LSTM", "forward", 5, 8, 16, 32, seed=5, with_h0=True)
    say(f"case {c.name}")
    plan = ra.plan_for_case(c, constant_weights=True)
    plan.enable_timing(True)
    a = ra.run_case(c, plan=plan)
    torch.cuda.synchronize()
    b = ra.run_case(c, plan=plan)
    torch.cuda.synchronize()
    assert _digest([to_np(x) for x in a]) == _digest([to_np(x) for x in b])
    t = plan.last_timings()
    assert set(t) == set(ra.STAGES) and all(v >= 0 for v in t.values())
    compare(c, [to_np(x) for x in b])


def test_eight_wave_product_matches_oracle():
    c = workloads.random_case("LSTM", "bidirectional", 9, 40, 48, 512, seed=31, with_lens=True,
                              with_h0=True, with_c0=True, scale=1.5 / 512 ** 0.5)
    say(f"case {c.name} with 8 waves")
    plan = ra.plan_for_case(c, waves_per_block=8)
    assert "waves=8" in plan.describe() and "resident=1" in plan.describe()
    compare(c, run_gpu(c, waves_per_block=8))


@pytest.mark.parametrize("op,attrs", [("LSTM", {}), ("GRU", dict(linear_before_reset=1)),
                                      ("GRU", dict(linear_before_reset=0)), ("RNN", {})])
def test_resident_kernels_without_bias_match_oracle(op, attrs):
    # H = 512 takes the register-resident kernels; B absent is staged as zeros
    c = workloads.random_case(op, "forward", 6, 32, 40, 512, seed=41, with_bias=False,
                              with_lens=True, with_h0=True, with_c0=(op == "LSTM"),
                              scale=1.5 / 512 ** 0.5, **attrs)
    say(f"case {c.name} {attrs}")
    assert "resident=1" in ra.plan_for_case(c).describe()
    compare(c, run_gpu(c))


@pytest.mark.parametrize("halves,inp", [(1, 16), (2, 16), (2, 512)])
def test_a_stalled_barrier_raises_the_device_error_and_the_kernel_exits(halves, inp, monkeypatch):
    # Forced from the host: with RNN_AMD_TEST_WITHHOLD_FLAGS the step loops
    # never store their flags, so every wait between steps runs out its spin
    # limit (1: two polls); the kernel then runs on without waiting and exits
    # normally, and rnn_workspace_check reports the error it raised.  (Input
    # size 512: the two-half kernel with the projection inside.)
    c = workloads.random_case("LSTM", "bidirectional", 8, 64, inp, 1024, seed=3, with_h0=True,
                              scale=1.0 / 32, x_scale=4.0 / inp ** 0.5)
    say(f"case {c.name} with withheld flags, barrier_spin_limit=1, batch_halves={halves}")
    monkeypatch.setenv("RNN_AMD_TEST_WITHHOLD_FLAGS", "1")
    fuse = 2 if inp == 512 else 0
    plan = ra.plan_for_case(c, kernel_path=ra.RNN_PATH_PERSISTENT, barrier_spin_limit=1,
                            batch_halves=halves, fuse_projection=fuse)
    monkeypatch.delenv("RNN_AMD_TEST_WITHHOLD_FLAGS")
    assert "workgroups=256" in plan.describe() and f"halves={halves}" in plan.describe()
    assert ("fused=1" in plan.describe()) == (inp == 512)
    ra.run_case(c, plan=plan)
    torch.cuda.synchronize()
    with pytest.raises(ra.RNNError) as ei:
        plan.check()
    assert ei.value.status == ra.RNN_ERR_DEVICE
    # a plan made without the switch, on the same inputs, is clean and matches the oracle
    plan2 = ra.plan_for_case(c, kernel_path=ra.RNN_PATH_PERSISTENT, batch_halves=halves,
                             fuse_projection=fuse)
    out = ra.run_case(c, plan=plan2)
    torch.cuda.synchronize()
    plan2.check()
    compare(c, [to_np(x) for x in out])


# ---------------------------------------------------------------------------
# Two half-batch groups of waves: bit-identical to one group, and to the oracle
# ---------------------------------------------------------------------------

HALVES = [
    # 2 tiles per half, 2 column tiles, 16 k blocks per wave; peepholes, clip
    dict(op="LSTM", direction="bidirectional", S=7, Bt=64, I=40, H=1024, with_p=True, clip=0.9,
         with_lens=True),
    # ragged second half (18 of 32 rows), padded hidden (500 -> 512), layout 1
    dict(op="GRU", direction="reverse", S=6, Bt=50, I=24, H=500, linear_before_reset=1,
         layout=1, with_lens=True),
    # one tile per half (batch tile 32), second half 4 rows
    dict(op="RNN", direction="forward", S=9, Bt=20, I=16, H=512, with_lens=True),
    # HardSigmoid GRU (its own compiled set), half 1 with 8 rows
    dict(op="GRU", direction="bidirectional", S=5, Bt=40, I=12, H=512, linear_before_reset=1,
         activations=["HardSigmoid", "Tanh"], alpha=[0.25], beta=[0.45]),
    # a set compiled through the run-time switch, input_forget
    dict(op="LSTM", direction="forward", S=5, Bt=33, I=10, H=480, input_forget=1,
         activations=["HardSigmoid", "Softsign", "Tanh"], alpha=[0.3], beta=[0.5]),
]


@pytest.mark.parametrize("k", range(len(HALVES)))
def test_half_batch_halves_match_one_group_bitwise_and_the_oracle(k):
    spec = dict(HALVES[k])
    op, direction = spec.pop("op"), spec.pop("direction")
    S, Bt, I, H = spec.pop("S"), spec.pop("Bt"), spec.pop("I"), spec.pop("H")
    lay = spec.pop("layout", 0)
    kw = {key: spec.pop(key) for key in ("with_lens", "with_p") if key in spec}
    c = workloads.random_case(op, direction, S, Bt, I, H, seed=700 + k, layout=lay,
                              with_h0=True, with_c0=(op == "LSTM"), scale=1.5 / H ** 0.5,
                              **kw, **spec)
    say(f"case {c.name} {HALVES[k]}")
    assert "halves=2" in ra.plan_for_case(c).describe()
    two = run_gpu(c, batch_halves=2)
    one = run_gpu(c, batch_halves=1)
    assert _digest(two) == _digest(one)
    compare(c, two)
    if k == 0:
        per_step = run_gpu(c, batch_halves=2, kernel_path=ra.RNN_PATH_PER_STEP)
        assert _digest(per_step) == _digest(two)


# ---------------------------------------------------------------------------
# The step hand-over over many steps and many workgroups
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("op,attrs", [("LSTM", {}), ("GRU", dict(linear_before_reset=0))])
def test_many_step_handover_matches_oracle(op, attrs):
    # one hidden unit per workgroup: 256 workgroups exchange H at every step
    # (GRU linear_before_reset = 0: twice per step) for 4096 steps; every
    # element is compared, and the first step that differs is named
    c = workloads.random_case(op, "forward", 4096, 16, 16, 256, seed=77, with_h0=True,
                              with_c0=(op == "LSTM"), scale=1.5 / 256 ** 0.5, **attrs)
    plan = ra.plan_for_case(c, units_per_block=1)
    desc = plan.describe()
    say(f"case {c.name} {attrs}: {desc}")
    assert "workgroups=256" in desc and "persist=" in desc
    gpu = run_gpu(c, plan=plan)
    plan.check()
    ref = oracle_outputs(c)
    err = np.abs(gpu[0].astype(np.float64) - ref[0])
    bad = err > ATOL + RTOL * np.abs(ref[0])
    if bad.any():
        t = int(np.argwhere(bad)[0][0])
        raise AssertionError(f"first step differing: {t} (max abs there {err[t].max():.3e})")
    compare(c, gpu, ref, strict=True)


@pytest.mark.parametrize("proj_bf16,exact", [(False, False), (True, False), (False, True),
                                             (True, True)])
def test_projection_row_list_and_whole_tiles_agree_bitwise(proj_bf16, exact, monkeypatch):
    # With sequence_lens the projection computes either the list of rows the
    # step loop reads (built on the device per time chunk) or whole tiles;
    # both give the same bits.  Lengths from 0 to seq, two directions, three
    # time chunks (so the list starts at steps j_base > 0).
    c = workloads.random_case("GRU", "bidirectional", 13, 70, 40, 48, seed=71, with_lens=True,
                              with_h0=True, linear_before_reset=1, proj_bf16=proj_bf16,
                              scale=1.5 / 48 ** 0.5)
    say(f"case {c.name} bf16={proj_bf16} exact={exact}")
    outs = []
    for mode in ("list", "tiles"):
        monkeypatch.setenv("RNN_AMD_TEST_PROJ_ROWS", mode)
        outs.append(run_gpu(c, exact=exact, time_chunk=5))
    monkeypatch.delenv("RNN_AMD_TEST_PROJ_ROWS")
    assert _digest(outs[0]) == _digest(outs[1])
    ref = oracle_outputs(c)
    if exact:
        for what, g, r in zip(("Y", "Y_h"), outs[0], ref):
            assert np.array_equal(u32(g), u32(r)), f"{what}: not bit-exact"
        check_masks(c, *outs[0])
    else:
        compare(c, outs[0], ref)


def test_long_two_half_run_matches_oracle():
    # the two-half kernel with the LSTM benchmark workload's tile shape (64
    # rows in two halves, R resident, 16 k blocks per wave; one column tile)
    # over 2048 steps, i.e. 4096 hand-overs per workgroup; every element is
    # compared, and the first step that differs is named
    c = workloads.random_case("LSTM", "forward", 2048, 64, 64, 1024, seed=83, with_h0=True,
                              with_c0=True, scale=1.0 / 32.0)
    plan = ra.plan_for_case(c)
    desc = plan.describe()
    say(f"case {c.name}: {desc}")
    assert "halves=2" in desc and "MT=4" in desc and "KB=16" in desc
    gpu = run_gpu(c, plan=plan)
    plan.check()
    ref = oracle_outputs(c)
    err = np.abs(gpu[0].astype(np.float64) - ref[0])
    bad = err > ATOL + RTOL * np.abs(ref[0])
    if bad.any():
        t = int(np.argwhere(bad)[0][0])
        raise AssertionError(f"first step differing: {t} (max abs there {err[t].max():.3e})")
    compare(c, gpu, ref, strict=True)


# The two-half kernel's other operators and tiles over hundreds of steps:
# the flag poll inside the product and the next step's XW rows loaded after
# the publish, for GRU (three gates, one column tile), LSTM with lengths and
# a 32-row batch tile, and a reverse RNN; every element is compared
LONG_TWO_HALF = [
    ("GRU", "forward", 512, 64, 256, 1024, {"linear_before_reset": 1}),
    ("LSTM", "bidirectional", 384, 32, 256, 1024, {"with_lens": True}),
    ("RNN", "reverse", 512, 64, 128, 1024, {}),
]


@pytest.mark.parametrize("k", range(len(LONG_TWO_HALF)))
def test_long_two_half_runs_of_each_operator_match_oracle(k):
    op, direction, S, Bt, I, H, kw = LONG_TWO_HALF[k]
    c = workloads.random_case(op, direction, S, Bt, I, H, seed=4242, with_h0=True,
                              with_c0=(op == "LSTM"), scale=1.0 / H ** 0.5, x_scale=0.5, **kw)
    with ra.plan_for_case(c) as plan:
        desc = plan.describe()
    say(f"case {c.name}: {desc}")
    assert "halves=2" in desc and "KB=16" in desc
    compare(c, run_gpu(c), oracle_outputs(c), strict=True)
