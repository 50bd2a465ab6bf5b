"""The benchmark's accounting, on the CPU: the FLOP counts behind the roofline
fractions (nominal and valid work, the fused form charging both products to
its step loop), the counter summaries that turn rocprofv3 files into bytes
per launch (steady dispatches, the copy-kernel scale), and the rule that a
recorded traffic figure is reported only for the sources it was taken on."""
import json
import os

import pytest

import bench
import workloads


def test_flops_count_both_products_per_step_and_the_valid_steps():
    c = workloads.random_case("LSTM", "bidirectional", 6, 5, 7, 9, seed=1, lens=[6, 0, 3, 6, 1])
    fl = bench.flops_per_run(c)
    G, D, H, I = 4, 2, 9, 7
    assert fl["nominal"] == (2.0 * G * H * I * 6 * 5 * D, 2.0 * G * H * H * 6 * 5 * D)
    steps = D * (6 + 0 + 3 + 6 + 1)
    assert fl["valid"] == (2.0 * G * H * I * steps, 2.0 * G * H * H * steps)
    # without lengths the two counts agree
    c2 = workloads.random_case("GRU", "forward", 4, 3, 5, 8, seed=2)
    f2 = bench.flops_per_run(c2)
    assert f2["nominal"] == f2["valid"] == (2.0 * 3 * 8 * 5 * 12, 2.0 * 3 * 8 * 8 * 12)


def _measured(plan, proj_ms, rec_ms):
    return {"plan": plan, "stage_ms": {"pack": 0.01, "projection": proj_ms, "recurrence": rec_ms,
                                       "other": 0.0}}


def test_kernel_figures_separate_and_fused():
    c = workloads.random_case("LSTM", "forward", 8, 4, 16, 32, seed=3)
    fp, fr = bench.flops_per_run(c)["valid"]
    sep = bench.kernel_figures(c, _measured("halves=2 fused=0 exact=0", 2.0, 4.0))
    assert sep["projection"]["flop_valid"] == fp and sep["recurrence"]["flop_valid"] == fr
    assert sep["recurrence"]["frac"] == pytest.approx(fr / 4e-3 / 1e12 / bench.FP32_MFMA_PEAK_TFLOPS)
    assert sep["recurrence"]["us_per_step"] == pytest.approx(4.0 * 1e3 / 8)
    fused = bench.kernel_figures(c, _measured("halves=2 fused=1 exact=0", 0.003, 5.0))
    assert fused["projection"]["fused"] is True and "frac" not in fused["projection"]
    assert fused["recurrence"]["flop_valid"] == fp + fr
    assert fused["recurrence"]["frac"] == pytest.approx((fp + fr) / 5e-3 / 1e12 /
                                                        bench.FP32_MFMA_PEAK_TFLOPS)
    assert not bench.plan_fused(_measured("fused=10", 1, 1))    # whole fields only


def _write_pmc(d, rows, counter="FETCH_SIZE"):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "pmc_counter_collection.csv"), "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for did, name, v in rows:
            f.write(f'{did},"{name}",{counter},{v}\n')


def test_traffic_summary_scales_steady_dispatches_by_the_copy(tmp_path, capsys):
    copy_kib = bench.COPY_BYTES / 1024.0
    # the copy kernel's counters read half its bytes (reads) and all of them (writes)
    _write_pmc(tmp_path / "cf", [(1, "copy", copy_kib / 2), (2, "copy", copy_kib / 2)])
    _write_pmc(tmp_path / "cw", [(1, "copy", copy_kib), (2, "copy", copy_kib)], "WRITE_SIZE")
    rec = "void rnnamd::rec_pipe_kernel<2, 2, 16, 1, 1>(rnnamd::RecArgs)"
    proj = "void rnnamd::proj_gemm_kernel<false>(rnnamd::ProjArgs)"
    # first dispatch cold (larger), then two steady ones
    _write_pmc(tmp_path / "f", [(1, rec, 900.0), (3, rec, 100.0), (5, rec, 300.0),
                                (2, proj, 50.0), (4, proj, 10.0), (6, proj, 30.0)])
    _write_pmc(tmp_path / "w", [(1, rec, 40.0), (3, rec, 20.0), (5, rec, 20.0),
                                (2, proj, 8.0), (4, proj, 8.0), (6, proj, 8.0)], "WRITE_SIZE")
    bench.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
                          str(tmp_path / "cw"), workload="w")
    out = json.loads(capsys.readouterr().out)
    assert out["read_scale"] == pytest.approx(2.0) and out["write_scale"] == pytest.approx(1.0)
    r = out["kernels"]["recurrence"]
    assert r["fetch_kib"] == 200.0 and r["write_kib"] == 20.0
    assert r["first_dispatch_fetch_kib"] == 900.0 and r["dispatches"] == 3
    assert r["traffic_bytes"] == pytest.approx((200.0 * 2 + 20.0) * 1024)
    assert r["source_hash"] == bench.kernel_hash("recurrence", rec)
    assert r["source_hash"] != bench.kernel_hash("recurrence")     # the two-half form's own file
    assert out["kernels"]["projection"]["fetch_kib"] == 20.0


def test_one_counter_file_per_directory(tmp_path):
    _write_pmc(tmp_path / "a", [(1, "k", 1.0)])
    _write_pmc(tmp_path / "a" / "again", [(1, "k", 1.0)])
    with pytest.raises(SystemExit):
        bench._pmc_rows(str(tmp_path / "a"))
    with pytest.raises(SystemExit):
        bench._pmc_rows(str(tmp_path / "empty"))


def test_recorded_traffic_only_for_its_sources(monkeypatch):
    w = "lstm_bidir_s512_b64_i1024_h1024"
    with open(os.path.join(bench.ROOT, "profiles", f"{w}_traffic.json")) as f:
        rec = json.load(f)["kernels"]["recurrence"]
    if rec["source_hash"] == bench.kernel_hash("recurrence", rec["name"]):
        assert bench.measured_traffic(w, "recurrence") == rec["traffic_bytes"]
    assert bench.measured_traffic("no_such_workload", "recurrence") is None
    monkeypatch.setattr(bench, "kernel_hash", lambda stage, name="": "0" * 16)
    assert bench.measured_traffic(w, "recurrence") is None


def test_family_flags_count_for_their_kernels_only(monkeypatch):
    from recurrent_nn_amd import build
    pipe = "void rnnamd::rec_pipe_kernel<2, 2, 16, 1, 1>(rnnamd::RecArgs)"
    four = "void rnnamd::rec_kernel<8, 3, 0, 8, 0, 2, 4>(rnnamd::RecArgs)"
    before = bench.kernel_hash("recurrence", pipe), bench.kernel_hash("recurrence", four)
    flags = dict(build.FAMILY_FLAGS)
    flags[2] = flags.get(2, []) + ["-mllvm", "-some-other-option"]
    monkeypatch.setattr(build, "FAMILY_FLAGS", flags)
    assert bench.kernel_hash("recurrence", pipe) == before[0]
    assert bench.kernel_hash("recurrence", four) != before[1]



def test_source_hash_ignores_comments():
    a = "int f(int x) {\n    return x + 1;   // one more\n}\n"
    b = "/* the successor */\nint f(int x) {\n\n    return x + 1;\n}\n"
    c = "int f(int x) {\n    return x + 2;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
