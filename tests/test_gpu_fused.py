"""The input projection computed inside the step loop (fuse_projection = 2):
bit-identical to the separate projection launch (fuse_projection = 1) on
every output, and within the fp32 bars of the oracle.  The cases cover both
places the flag of a half goes out (inside the projection for input sizes
of 512 and more, from the next recurrent product at 256), batch tiles of 64
and 32 (with one column tile two waves hold no projection tile, with two
each wave holds one), sequence
lengths in both directions, layout 1, ragged batch and hidden, the compiled
and run-time activation sets, time chunks and one launch per step."""
import hashlib

import numpy as np
import pytest

import recurrent_nn_amd as ra
import workloads
from tests.test_gpu_parity import ATOL, compare, oracle_outputs, run_gpu, say

pytestmark = pytest.mark.gpu


def _digest(outs):
    h = hashlib.sha256()
    for o in outs:
        if o is not None:
            h.update(np.ascontiguousarray(o).tobytes())
    return h.hexdigest()


FUSED = [
    # the LSTM benchmark workload's tile (64 rows, two column tiles, 16 k
    # blocks per wave); I = 512:
    # the flag goes out inside the projection; peepholes, clip, lengths
    dict(op="LSTM", direction="bidirectional", S=9, Bt=64, I=512, H=1024, with_p=True, clip=0.9,
         with_lens=True),
    # I = 256: the flag from the next recurrent product; ragged batch (50 of
    # 64 rows), padded hidden (500 -> 512), layout 1, reverse
    dict(op="GRU", direction="reverse", S=6, Bt=50, I=256, H=500, linear_before_reset=1,
         layout=1, with_lens=True),
    # batch tile 32 with one column tile: waves 2 and 3 compute no projection
    dict(op="RNN", direction="forward", S=9, Bt=20, I=512, H=512, with_lens=True),
    # HardSigmoid GRU (its own compiled set), I = 768 (three prefetch rounds)
    dict(op="GRU", direction="bidirectional", S=5, Bt=40, I=768, H=512, linear_before_reset=1,
         activations=["HardSigmoid", "Tanh"], alpha=[0.25], beta=[0.45]),
    # a set compiled through the run-time switch, input_forget, I = 1024
    dict(op="LSTM", direction="forward", S=5, Bt=33, I=1024, H=480, input_forget=1,
         activations=["HardSigmoid", "Softsign", "Tanh"], alpha=[0.3], beta=[0.5]),
    # batch tile 32 with two column tiles: each wave one projection tile
    dict(op="LSTM", direction="reverse", S=5, Bt=24, I=512, H=512, with_lens=True,
         plan=dict(units_per_block=8)),
]


def _case(k):
    spec = dict(FUSED[k])
    spec.pop("plan", None)
    op, direction = spec.pop("op"), spec.pop("direction")
    S, Bt, I, H = spec.pop("S"), spec.pop("Bt"), spec.pop("I"), spec.pop("H")
    lay = spec.pop("layout", 0)
    kw = {key: spec.pop(key) for key in ("with_lens", "with_p") if key in spec}
    return workloads.random_case(op, direction, S, Bt, I, H, seed=900 + k, layout=lay,
                                 with_h0=True, with_c0=(op == "LSTM"), scale=1.5 / H ** 0.5,
                                 x_scale=1.0 / I ** 0.5 * 8, **kw, **spec)


@pytest.mark.parametrize("k", range(len(FUSED)))
def test_fused_projection_matches_separate_launch_bitwise_and_the_oracle(k):
    c = _case(k)
    pk = FUSED[k].get("plan", {})
    say(f"case {c.name} {FUSED[k]}")
    desc = ra.plan_for_case(c, fuse_projection=2, **pk).describe()
    say(f"  plan {desc}")
    assert "fused=1" in desc and "halves=2" in desc
    fused = run_gpu(c, fuse_projection=2, **pk)
    sep = run_gpu(c, fuse_projection=1, **pk)
    assert _digest(fused) == _digest(sep)
    compare(c, fused, strict=True)
    if k == 0:
        # one launch per step, and time chunks of 4 steps
        assert _digest(run_gpu(c, fuse_projection=2, kernel_path=ra.RNN_PATH_PER_STEP)) == \
            _digest(fused)
        assert _digest(run_gpu(c, fuse_projection=2, time_chunk=4)) == _digest(fused)


def test_long_fused_run_matches_oracle():
    # the fused kernel with that tile over 1024 steps (2048 hand-overs per
    # workgroup, the flag from inside the projection); every element is
    # compared, and the first step that differs is named
    c = workloads.random_case("LSTM", "forward", 1024, 64, 512, 1024, seed=87, with_h0=True,
                              with_c0=True, scale=1.0 / 32.0, x_scale=0.35)
    plan = ra.plan_for_case(c, fuse_projection=2)
    desc = plan.describe()
    say(f"case {c.name}: {desc}")
    assert "fused=1" in desc and "MT=4" in desc and "KB=16" in desc
    gpu = run_gpu(c, plan=plan)
    plan.check()
    plan.close()
    ref = oracle_outputs(c)
    err = np.abs(gpu[0].astype(np.float64) - ref[0])
    bad = err > ATOL + 1e-4 * np.abs(ref[0])
    if bad.any():
        t = int(np.argwhere(bad)[0][0])
        raise AssertionError(f"first step differing: {t} (max abs there {err[t].max():.3e})")
    compare(c, gpu, ref, strict=True)
