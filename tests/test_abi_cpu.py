"""The C-ABI without a GPU: the library loads, exports every entry point the
header declares, and raises every plan-time error (and the run-time
sequence_lens error) before touching a device, with the same error class as
the oracle for the same fault."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

import oracle
import recurrent_nn_amd as ra
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "recurrent_nn_amd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rnn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(ra._lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ra._lib.load()
    out = subprocess.run(["nm", "-D", "--defined-only", ra._lib.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if " T " in line)
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_struct_layout_matches_header():
    # sizes of the ABI structs as the C compiler sees them
    src = f'#include "{HEADER}"\n#include <stdio.h>\n#include <stddef.h>\n' \
          'int main(){printf("%zu %zu %zu\\n", sizeof(rnn_attrs), sizeof(rnn_dims), ' \
          'offsetof(rnn_attrs, batch_tile));return 0;}'
    tmp = os.path.join(ROOT, "_build")
    os.makedirs(tmp, exist_ok=True)
    c = os.path.join(tmp, "abi_sizes.c")
    exe = os.path.join(tmp, "abi_sizes")
    open(c, "w").write(src)
    subprocess.run(["gcc", "-o", exe, c], check=True)
    sa, sd, off = map(int, subprocess.run([exe], capture_output=True, text=True).stdout.split())
    assert sa == ctypes.sizeof(ra.rnn_attrs)
    assert sd == ctypes.sizeof(ra.rnn_dims)
    assert off == ra.rnn_attrs.batch_tile.offset


def _plan(op, direction, dims, **kw):
    a, keep = ra.make_attrs(op, direction, **kw)
    st, p = ra.rnn_plan_create(a, ra.rnn_dims(*dims))
    if st == ra.RNN_OK:
        ra.rnn_plan_destroy(p)
    return st


def test_plan_time_errors_match_the_oracle():
    # (description, library status, oracle status) for the same fault
    cases = []
    cases.append((_plan("LSTM", "forward", (4, 3, 4, 5, 2)), "num_directions"))
    cases.append((_plan("LSTM", "sideways", (4, 3, 4, 5, 1)), "direction"))
    cases.append((_plan("LSTM", "forward", (4, 3, 4, 5, 1), hidden_size=6), "hidden_size"))
    cases.append((_plan("LSTM", "forward", (4, 3, 4, 0, 1)), "hidden 0"))
    cases.append((_plan("LSTM", "forward", (4, 3, 4, 5, 1), activations=["Sigmoid", "Tanh"]), "count"))
    cases.append((_plan("LSTM", "forward", (4, 3, 4, 5, 1),
                        activations=["Sigmoid", "Tanh", "Gelu"]), "name"))
    cases.append((_plan("GRU", "forward", (4, 3, 4, 5, 1), input_forget=1), "input_forget"))
    cases.append((_plan("LSTM", "forward", (4, 3, 4, 5, 1), linear_before_reset=1), "lbr"))
    cases.append((_plan("LSTM", "forward", (4, 3, 4, 5, 1), layout=2), "layout"))
    for st, what in cases:
        assert st == ra.RNN_ERR_INVALID_INPUT, what
    # the same faults in the oracle
    c = workloads.random_case("LSTM", "forward", 4, 3, 4, 5, seed=1)
    c.hidden_size_attr = 6
    assert oracle.run(c, raise_on_error=False)[0] == oracle.INVALID_INPUT
    c.hidden_size_attr = 0
    c.activations = ["Sigmoid", "Tanh", "Gelu"]
    assert oracle.run(c, raise_on_error=False)[0] == oracle.INVALID_INPUT


def test_scratch_limit_is_unsupported_at_plan_time():
    # 16 * batch * (seq + 1) = 2^30 - 16 floats: below with constant weights,
    # at the limit once the transposed weights (16 * 7 floats) count.
    dims = (2 ** 26 - 2, 1, 3, 4, 1)
    assert _plan("LSTM", "forward", dims) == ra.RNN_ERR_UNSUPPORTED
    assert _plan("LSTM", "forward", (2 ** 16, 2 ** 10, 3, 4, 1),
                 constant_weights=True) == ra.RNN_ERR_UNSUPPORTED
    # just below the limit a plan is made (nothing is allocated)
    a, keep = ra.make_attrs("LSTM", "forward", constant_weights=True)
    st, p = ra.rnn_plan_create(a, ra.rnn_dims(*dims))
    assert st == ra.RNN_OK
    ra.rnn_plan_destroy(p)
    # the oracle draws the same line
    c = workloads.random_case("LSTM", "forward", 2, 1, 3, 4, seed=2)
    c.seq = dims[0]
    c.sequence_lens = torch.tensor([-1], dtype=torch.int32)
    no = dict(want_y=False, want_yh=False, want_yc=False, raise_on_error=False)
    assert oracle.run(c, **no)[0] == oracle.UNSUPPORTED
    assert oracle.run(c, constant_weights=True, **no)[0] == oracle.INVALID_INPUT


def test_run_time_errors_before_any_device_work():
    p = ra.RNNPlan("GRU", 4, 3, 8, 16)
    fake = 1 << 20          # a 256-aligned address that is never dereferenced
    ws = p.workspace_bytes
    bad = np.array([1, 5, 2], np.int32)      # 5 > seq
    st = ra.rnn_run(p.plan, 0, fake, ws, fake, fake, fake, 0, bad)
    assert st == ra.RNN_ERR_INVALID_INPUT and "sequence_lens" in ra.rnn_last_error()
    st = ra.rnn_run(p.plan, 0, fake, ws, fake, fake, fake, 0, np.array([1, -1, 2], np.int32))
    assert st == ra.RNN_ERR_INVALID_INPUT
    # Y_c / initial_c / P on a GRU plan
    assert ra.rnn_run(p.plan, 0, fake, ws, fake, fake, fake, Y_c=fake) == ra.RNN_ERR_INVALID_INPUT
    assert ra.rnn_run(p.plan, 0, fake, ws, fake, fake, fake, P=fake) == ra.RNN_ERR_INVALID_INPUT
    # missing required inputs, small or misaligned workspace, misaligned X
    assert ra.rnn_run(p.plan, 0, fake, ws, 0, fake, fake) == ra.RNN_ERR_INVALID_INPUT
    assert ra.rnn_run(p.plan, 0, fake, ws - 1, fake, fake, fake) == ra.RNN_ERR_INVALID_INPUT
    assert ra.rnn_run(p.plan, 0, fake + 64, ws, fake, fake, fake) == ra.RNN_ERR_INVALID_INPUT
    assert ra.rnn_run(p.plan, 0, fake, ws, fake + 4, fake, fake) == ra.RNN_ERR_INVALID_INPUT
    assert ra.rnn_run(0, 0, fake, ws, fake, fake, fake) == ra.RNN_ERR_INVALID_INPUT


def test_cell_run_errors_before_any_device_work():
    fake = 1 << 20          # a 256-aligned address that is never dereferenced
    # a plan with more than one step or direction is not a cell plan
    p = ra.RNNPlan("RNN", 2, 3, 8, 16)
    st = ra.rnn_cell_run(p.plan, 0, fake, p.workspace_bytes, fake, 0, 0, fake, fake, 0, 0, fake, 0)
    assert st == ra.RNN_ERR_INVALID_INPUT and "seq_length 1" in ra.rnn_last_error()
    p = ra.RNNPlan("RNN", 1, 3, 8, 16, direction="bidirectional")
    st = ra.rnn_cell_run(p.plan, 0, fake, p.workspace_bytes, fake, 0, 0, fake, fake, 0, 0, fake, 0)
    assert st == ra.RNN_ERR_INVALID_INPUT
    c = ra.RNNCell("GRU", 3, 8, 16, linear_before_reset=1)
    ws = c.workspace_bytes
    # a summed bias cannot carry GRU's reset-after-product candidate bias
    st = ra.rnn_cell_run(c.plan, 0, fake, ws, fake, 0, 0, fake, fake, fake, 0, fake, 0)
    assert st == ra.RNN_ERR_INVALID_INPUT and "linear_before_reset" in ra.rnn_last_error()
    c = ra.RNNCell("LSTM", 3, 8, 16)
    ws = c.workspace_bytes
    # H_out required; rnn_run's checks apply (X, W, R required; workspace size)
    assert ra.rnn_cell_run(c.plan, 0, fake, ws, fake, 0, 0, fake, fake, fake, 0, 0, 0) == \
        ra.RNN_ERR_INVALID_INPUT
    assert ra.rnn_cell_run(c.plan, 0, fake, ws, 0, 0, 0, fake, fake, fake, 0, fake, 0) == \
        ra.RNN_ERR_INVALID_INPUT
    assert ra.rnn_cell_run(c.plan, 0, fake, ws - 1, fake, 0, 0, fake, fake, fake, 0, fake, 0) == \
        ra.RNN_ERR_INVALID_INPUT
    assert ra.rnn_cell_run(c.plan, 0, fake, ws, fake, 0, 0, fake, fake, fake + 2, 0, fake, 0) == \
        ra.RNN_ERR_INVALID_INPUT
    assert ra.rnn_cell_run(0, 0, fake, ws, fake, 0, 0, fake, fake, 0, 0, fake, 0) == \
        ra.RNN_ERR_INVALID_INPUT
    # C / P / C_out are LSTM-only
    r = ra.RNNCell("RNN", 3, 8, 16)
    assert ra.rnn_cell_run(r.plan, 0, fake, r.workspace_bytes, fake, 0, 0, fake, fake, 0, 0, fake,
                           fake) == ra.RNN_ERR_INVALID_INPUT


def test_time_chunks_shrink_the_workspace_and_lift_the_scratch_limit():
    # (the projections held in the workspace: a separate projection launch)
    full = ra.RNNPlan("LSTM", 512, 64, 1024, 1024, direction="bidirectional", fuse_projection=1)
    ch = ra.RNNPlan("LSTM", 512, 64, 1024, 1024, direction="bidirectional", time_chunk=64,
                    fuse_projection=1)
    assert "C=512" in full.describe() and "C=64" in ch.describe()
    assert ch.workspace_bytes < full.workspace_bytes / 4
    # the projection inside the step loop holds no projections at all
    fused = ra.RNNPlan("LSTM", 512, 64, 1024, 1024, direction="bidirectional", fuse_projection=2)
    assert "fused=1" in fused.describe() and "fused=0" in full.describe()
    xw = 2 * 512 * 64 * 4096 * 4
    assert fused.workspace_bytes <= full.workspace_bytes - xw
    # a chunk at least as long as the sequence is the whole sequence
    assert "C=20" in ra.RNNPlan("GRU", 20, 4, 8, 16, time_chunk=50).describe()
    # 2^22 steps x 64 rows x 4 gates x 64 units exceeds 2^30 floats at once,
    # not in chunks of 1024 steps (plan only: nothing is allocated)
    with pytest.raises(ra.RNNError) as ei:
        ra.RNNPlan("LSTM", 1 << 22, 64, 16, 64)
    assert ei.value.status == ra.RNN_ERR_UNSUPPORTED
    p = ra.RNNPlan("LSTM", 1 << 22, 64, 16, 64, time_chunk=1024)
    assert "C=1024" in p.describe()
    with pytest.raises(ra.RNNError):
        ra.RNNPlan("LSTM", 8, 4, 8, 16, time_chunk=-1)


def test_workspace_and_tiling_of_the_named_workloads():
    expect = {
        "lstm_bidir_s512_b64_i1024_h1024": dict(resident="1", workgroups="256", halves="2",
                                                fused="0"),
        "gru_rev_s256_b256_i2048_h2048_bf16": dict(workgroups="256", NBB="2", BT="128", U="16"),
        "gru_fwd_s128_b32_i256_h512_lbr0": dict(phases="2", fused="0"),
    }
    for name, want in expect.items():
        c = workloads.Case(*[None] * 6)
        spec = {"lstm_bidir_s512_b64_i1024_h1024": ("LSTM", "bidirectional", 512, 64, 1024, 1024, {}),
                "gru_rev_s256_b256_i2048_h2048_bf16": ("GRU", "reverse", 256, 256, 2048, 2048,
                                                       dict(linear_before_reset=1, proj_bf16=True)),
                "gru_fwd_s128_b32_i256_h512_lbr0": ("GRU", "forward", 128, 32, 256, 512,
                                                    dict(layout=1))}[name]
        op, d, S, Bt, I, H, kw = spec
        p = ra.RNNPlan(op, S, Bt, I, H, direction=d, **kw)
        desc = dict(kv.split("=") for kv in p.describe().split())
        for k, v in want.items():
            assert desc[k] == v, (name, k, desc[k])
        xw = S * Bt * (2 if d == "bidirectional" else 1) * {"LSTM": 4, "GRU": 3}[op] * H * 4
        if desc["fused"] == "1":      # the projections never leave the step loop
            assert p.workspace_bytes < xw
        else:                         # XW is materialised
            assert p.workspace_bytes >= xw


def test_fused_projection_needs_its_shape():
    # on request where the two-half schedule, an fp32 projection, I in whole
    # 256-input ranges and the W slice in LDS allow it (never automatic);
    # elsewhere the request is an InvalidInput
    assert "fused=0" in ra.RNNPlan("GRU", 6, 50, 256, 500, linear_before_reset=1).describe()
    assert "fused=1" in ra.RNNPlan("GRU", 6, 50, 256, 500, linear_before_reset=1,
                                   fuse_projection=2).describe()
    for kw in (dict(), dict(proj_bf16=True), dict(exact=True), dict(batch_halves=1)):
        I = 40 if not kw else 1024
        p = ra.RNNPlan("LSTM", 3, 64, I, 1024, **kw)
        assert "fused=0" in p.describe(), kw
        with pytest.raises(ra.RNNError) as ei:
            ra.RNNPlan("LSTM", 3, 64, I, 1024, fuse_projection=2, **kw)
        assert ei.value.status == ra.RNN_ERR_INVALID_INPUT
    # the W slice of 32 gate columns over 2048 inputs does not fit in LDS
    with pytest.raises(ra.RNNError):
        ra.RNNPlan("LSTM", 3, 64, 2048, 1024, direction="bidirectional", fuse_projection=2)
    assert "fused=1" in ra.RNNPlan("LSTM", 3, 64, 2048, 1024, fuse_projection=2).describe()
    # off on request; out of range
    assert "fused=0" in ra.RNNPlan("LSTM", 3, 64, 1024, 1024, fuse_projection=1).describe()
    with pytest.raises(ra.RNNError):
        ra.RNNPlan("LSTM", 3, 64, 1024, 1024, fuse_projection=3)


def test_zero_size_plans_need_no_workspace():
    assert ra.RNNPlan("LSTM", 0, 3, 4, 5).workspace_bytes == 0
    assert ra.RNNPlan("GRU", 4, 0, 4, 5).workspace_bytes == 0


def test_units_per_block_override_and_errors():
    p = ra.RNNPlan("LSTM", 8, 20, 16, 40, units_per_block=3)
    assert "U=3" in p.describe()
    with pytest.raises(ra.RNNError):
        ra.RNNPlan("LSTM", 8, 20, 16, 40, units_per_block=0 - 1)
    with pytest.raises(ra.RNNError):
        ra.RNNPlan("LSTM", 8, 20, 16, 40, batch_tile=48)
