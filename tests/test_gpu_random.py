"""Seeded random configurations against the oracle: operator, direction,
layout, shapes (ragged batch and hidden sizes, input sizes that are and are
not whole projection stages), sequence lengths, bias, peepholes, clip,
input_forget, linear_before_reset, activation sets with their alpha/beta
cursors, the bf16 projection, and the run options (exact mode, the
projection inside the step loop where the shape allows it, time chunks, one
launch per step).  Fast mode is held to the fp32 bars (against the oracle
with the same bf16 rounding of X and W where the projection is bf16), exact
mode to bit equality."""
import numpy as np
import pytest

import oracle
import recurrent_nn_amd as ra
import workloads
from tests.test_gpu_parity import check_masks, compare, run_gpu, say, u32

pytestmark = pytest.mark.gpu

ACTS = ["Relu", "Tanh", "Sigmoid", "Affine", "LeakyRelu", "ThresholdedRelu", "ScaledTanh",
        "HardSigmoid", "Elu", "Softsign", "Softplus"]
# activations that stay bounded, for the gates whose outputs feed the state
BOUNDED = ["Tanh", "Sigmoid", "HardSigmoid", "Softsign", "ScaledTanh"]


def _configs(n=100, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        op = ["RNN", "GRU", "LSTM"][k % 3]
        direction = ["forward", "reverse", "bidirectional"][rng.integers(3)]
        # hidden sizes up to 300, or padded to 512 or 1024 (16-column k
        # blocks per wave: 8 or 16, where R stays in registers and the
        # two-half schedule and the fused projection apply)
        big = bool(rng.integers(3) == 0)
        H = (int(rng.choice([rng.integers(449, 513), rng.integers(961, 1025)])) if big
             else int(rng.integers(1, 300)))
        cfg = dict(op=op, direction=direction, S=int(rng.integers(1, 9)),
                   Bt=int(rng.integers(1, 65 if big else 81)), H=H,
                   layout=int(rng.integers(2)), with_lens=bool(rng.integers(2)),
                   with_bias=bool(rng.integers(4) > 0), exact=bool(rng.integers(4) == 0))
        cfg["I"] = int(rng.choice([int(rng.integers(1, 90)), 256, 512] + [256, 512] * big))
        if rng.integers(3) == 0:
            cfg["clip"] = float(rng.uniform(0.3, 2.0))
        if op == "LSTM":
            cfg["with_p"] = bool(rng.integers(2))
            cfg["input_forget"] = int(rng.integers(4) == 0)
        if op == "GRU":
            cfg["linear_before_reset"] = int(rng.integers(2))
        if rng.integers(3) == 0:          # a non-default activation set
            ng = {"RNN": 1, "GRU": 2, "LSTM": 3}[op]
            dirs = 2 if direction == "bidirectional" else 1
            names = [str(rng.choice(BOUNDED if (g < ng - 1 or op == "RNN") else ACTS))
                     for _ in range(dirs) for g in range(ng)]
            cfg["activations"] = names
            cfg["alpha"] = [float(a) for a in rng.uniform(0.1, 1.2, size=3)]
            cfg["beta"] = [float(b) for b in rng.uniform(0.1, 0.9, size=2)]
        cfg["proj_bf16"] = bool(rng.integers(5) == 0)
        cfg["time_chunk"] = int(rng.choice([0, 0, 2, 3]))
        cfg["kernel_path"] = int(rng.choice([0, 0, 0, 2]))
        cfg["fuse"] = bool(rng.integers(4) > 0)
        out.append(cfg)
    return out


CONFIGS = _configs()


@pytest.mark.parametrize("k", range(len(CONFIGS)))
def test_random_configuration_matches_oracle(k):
    spec = dict(CONFIGS[k])
    op, direction = spec.pop("op"), spec.pop("direction")
    S, Bt, I, H = spec.pop("S"), spec.pop("Bt"), spec.pop("I"), spec.pop("H")
    lay = spec.pop("layout")
    exact, chunk, path, fuse = spec.pop("exact"), spec.pop("time_chunk"), spec.pop("kernel_path"), \
        spec.pop("fuse")
    kw = {key: spec.pop(key) for key in ("with_lens", "with_p", "with_bias") if key in spec}
    c = workloads.random_case(op, direction, S, Bt, I, H, seed=3000 + k, layout=lay,
                              with_h0=True, with_c0=(op == "LSTM"),
                              scale=min(0.6, 1.5 / H ** 0.5), x_scale=min(1.0, 4.0 / I ** 0.5),
                              **kw, **spec)
    run = dict(exact=exact, time_chunk=chunk, kernel_path=path)
    if fuse and not exact:
        try:
            ra.plan_for_case(c, fuse_projection=2, **run).close()
            run["fuse_projection"] = 2
        except ra.RNNError:
            pass
    say(f"case {c.name} {CONFIGS[k]} run={run}")
    with ra.plan_for_case(c, **run) as plan:
        say(f"  plan {plan.describe()}")
    gpu = run_gpu(c, **run)
    if exact:
        ref = oracle.run(c)[1:]
        for what, g, r in zip(("Y", "Y_h", "Y_c"), gpu, ref):
            if r is not None:
                assert np.array_equal(u32(g), u32(r)), f"{what}: not bit-exact"
        check_masks(c, *gpu)
    else:
        compare(c, gpu)
