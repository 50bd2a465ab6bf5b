"""The build's unit list: every instantiation unit gets its family and
activation set, the streamed step-loop families their own device flags, and
every HIP unit the flags the gate arithmetic and the step loops rely on."""
from recurrent_nn_amd import build


def test_instantiation_units_and_their_flags():
    inst = [u for u in build.HIP_UNITS if u[0] == build.INST]
    assert len(inst) == len(build.INST_UNITS) == 25
    for (src, extra, oname), (fam, act) in zip(inst, build.INST_UNITS):
        assert f"-DRNN_FAMILY={fam}" in extra and f"-DRNN_ACT={act}" in extra
        assert oname == f"recurrence_inst_f{fam}_a{act}.o"
        fam_flags = build.FAMILY_FLAGS.get(fam, [])
        assert extra[2:] == fam_flags
        # the accumulators in vector registers only for the streamed families
        assert ("-amdgpu-mfma-vgpr-form" in extra) == (fam in (1, 2))


def test_device_flags():
    f = build.HIP_FLAGS
    assert "-ffp-contract=off" in f                  # no fused multiply-adds in the gates
    assert "-packed-fp32-ops" in f and f[f.index("-packed-fp32-ops") - 1] == "-Xclang"
    assert "-amdgpu-atomic-optimizer-strategy=None" in f
    assert any(x.startswith("--offload-arch=gfx950") for x in f) or build.ARCH != "gfx950"
