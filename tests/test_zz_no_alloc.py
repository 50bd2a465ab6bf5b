"""The allocation-free entry point rnn_run_noalloc (for callers that cannot
allocate device memory): through the C-ABI, its outputs must equal those of
rnn_run on the same plan and inputs bit for bit (the same kernels run on the
library's own scratch instead of a caller workspace), call after call on the
one shared scratch array, the second call with a smaller input; and they must
meet the oracle's bar.  Sizes beyond the scratch are refused before any
device call."""
import ctypes

import numpy as np
import pytest
import torch

import recurrent_nn_amd as ra
import workloads
from tests.test_gpu_parity import compare, say


def _u32(a):
    return np.ascontiguousarray(a).view(np.uint32)


def _outputs(plan, dev):
    ysh, ssh = plan.output_shapes()
    Y = torch.full(ysh, float("nan"), dtype=torch.float32, device=dev)
    Yh = torch.full(ssh, float("nan"), dtype=torch.float32, device=dev)
    Yc = torch.full(ssh, float("nan"), dtype=torch.float32, device=dev) if plan.op == "LSTM" else None
    return Y, Yh, Yc


def _both(c):
    """(rnn_run outputs, rnn_run_noalloc outputs) of one case, as numpy."""
    dev = torch.device("cuda:0")
    t = {k: (v.to(dev) if v is not None and k != "sequence_lens" else v)
         for k, v in c.tensors().items()}
    with ra.plan_for_case(c) as plan:
        say(f"  {c.name}: {plan.describe()}")
        assert plan.workspace_bytes <= ra.RNN_NOALLOC_SCRATCH_BYTES
        args = (t["X"], t["W"], t["R"], t["B"], t["sequence_lens"], t["initial_h"],
                t["initial_c"], t["P"])
        ref = plan.run(*args, out=_outputs(plan, dev))
        torch.cuda.synchronize()
        plan.check()
        got = plan.run(*args, out=_outputs(plan, dev), noalloc=True)
        torch.cuda.synchronize()
    conv = lambda o: tuple(None if x is None else x.cpu().numpy() for x in o)
    return conv(ref), conv(got)


@pytest.mark.gpu
def test_noalloc_matches_rnn_run_on_two_calls_in_a_row():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ra._lib.load()
    torch.cuda.set_device(0)
    # first the larger input, then a smaller one on the same scratch array,
    # then the larger one again
    names = ["gru_fwd_s128_b32_i256_h512_lbr0", "lstm_bidir_s16_b4_i32_h64",
             "gru_fwd_s128_b32_i256_h512_lbr1"]
    for name in names:
        c = workloads.workload(name)
        say(f"case {name} through rnn_run and rnn_run_noalloc")
        ref, got = _both(c)
        for what, r, g in zip(("Y", "Y_h", "Y_c"), ref, got):
            if r is None:
                assert g is None
                continue
            assert np.array_equal(_u32(r), _u32(g)), f"{name}: {what} differs from rnn_run"
        compare(c, got, strict=True)


def test_noalloc_refuses_plans_beyond_its_scratch_before_any_device_call():
    # a plan whose workspace exceeds the scratch: refused with Unsupported and
    # a message, before any device work (this runs without a GPU)
    c = workloads.workload("lstm_bidir_s512_b64_i1024_h1024", batch_rows=[0])
    c.seq = 4096
    with ra.plan_for_case(c) as plan:
        assert plan.workspace_bytes > ra.RNN_NOALLOC_SCRATCH_BYTES
        st = ra.rnn_run_noalloc(plan.plan, 0, 16, 16, 16)
        assert st == ra.RNN_ERR_UNSUPPORTED
        assert "scratch" in ra.rnn_last_error()
    # more batch rows with sequence_lens than the kernel arguments carry
    c = workloads.random_case("RNN", "forward", 2, ra.RNN_NOALLOC_MAX_LENS_BATCH + 1, 3, 4, seed=1,
                              with_lens=True)
    with ra.plan_for_case(c) as plan:
        lens = np.ones(c.batch, dtype=np.int32)
        st = ra.rnn_run_noalloc(plan.plan, 0, 16, 16, 16, 0, lens)
        assert st == ra.RNN_ERR_UNSUPPORTED
        assert "sequence_lens" in ra.rnn_last_error()
