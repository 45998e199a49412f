"""Host-side checks of bench.py's profile-derived roofline fields (no GPU needed).

The measured HBM traffic and the issued VALU work in the benchmark line come from the
committed rocprofv3 summary of the solver.  They must be computed from that summary as
documented, and must be null once the solver's source differs from the one the counters
were taken on.
"""
import json

import pytest

import bench


def _profile(tmp_path, sha, **over):
    prof = {
        "kernel_source_sha256_16": sha,
        "workload": "llama70b_stack",
        "weights_per_launch": 1000.0,
        "hbm_bytes_per_weight": 2.5,
        "sq": {
            "hqq_solve_kernel<32>": {"valu_wave_instr_per_launch": 500.0,
                                     "trans_wave_instr_per_launch": 100.0},
            "hqq_solve_kernel<64>": {"valu_wave_instr_per_launch": 600.0,
                                     "trans_wave_instr_per_launch": 120.0},
        },
    }
    prof.update(over)
    path = tmp_path / "pmc.json"
    path.write_text(json.dumps(prof))
    return str(path)


def test_issued_valu_from_a_matching_profile(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_PMC", _profile(tmp_path, bench.kernel_source_hash()))
    n, step_s = 2000.0, 1e-9
    got = bench.issued_valu_from_profile(n, [(2, 32), (4, 64)], step_s)
    # per weight: (500 + 3*100) * 64 / 1000 = 51.2 and (600 + 3*120) * 64 / 1000 = 61.44
    slots = (51.2 + 61.44) * n
    assert got["slots_per_weight"] == pytest.approx((51.2 + 61.44) / 2, abs=0.01)
    assert got["achieved"] == pytest.approx(slots / step_s / 1e12, rel=1e-3)
    assert got["frac"] == pytest.approx(slots / step_s / bench.PEAK_VALU_SLOTS, abs=1e-4)


def test_traffic_from_a_matching_profile(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_PMC", _profile(tmp_path, bench.kernel_source_hash()))
    assert bench.traffic_from_profile(4000.0) == 10000


@pytest.mark.parametrize("over", [{"kernel_source_sha256_16": "0" * 16},
                                  {"workload": "llama7b_stack"},
                                  {"sq": {}}])
def test_profile_fields_are_null_on_another_source_or_workload(tmp_path, monkeypatch, over):
    path = _profile(tmp_path, bench.kernel_source_hash(), **over)
    monkeypatch.setattr(bench, "PROFILE_PMC", path)
    assert bench.issued_valu_from_profile(2000.0, [(2, 32), (4, 64)], 1e-6) is None
    if "sq" not in over:
        assert bench.traffic_from_profile(4000.0) is None


def test_committed_profile_matches_the_solver_source():
    """The committed counters were taken on the solver as it stands, so the benchmark
    reports measured traffic and issued work (retake the profile after a change)."""
    with open(bench.PROFILE_PMC) as f:
        prof = json.load(f)
    assert prof["kernel_source_sha256_16"] == bench.kernel_source_hash()
    assert set(prof["sq"]) == {"hqq_solve_kernel<32>", "hqq_solve_kernel<64>"}


def _variants_profile(tmp_path, sha):
    prof = {"tensor_stop_source_sha256_16": sha, "kernels": {
        "hqq_lockstep_kernel<32, 0, false>": {"dispatches": 14, "total_ms": 1.0,
                                              "valu_wave_instr": 1000.0, "trans_wave_instr": 100.0},
        "hqq_lockstep_kernel<32, 0, true>": {"dispatches": 14, "total_ms": 1.0,
                                             "valu_wave_instr": 500.0, "trans_wave_instr": 50.0},
        "hqq_lockstep_kernel<64, 0, false>": {"dispatches": 14, "total_ms": 1.0,
                                              "valu_wave_instr": 9e9, "trans_wave_instr": 9e9},
        "hqq_tensor_total_kernel": {"dispatches": 28, "total_ms": 0.1,
                                    "valu_wave_instr": 9e9, "trans_wave_instr": 0.0}}}
    path = tmp_path / "variants.json"
    path.write_text(json.dumps(prof))
    return str(path)


def test_tensor_stop_issued_from_a_matching_profile(tmp_path, monkeypatch):
    sha = bench.kernel_source_hash(bench.TENSOR_STOP_SRC)
    monkeypatch.setattr(bench, "PROFILE_VARIANTS", _variants_profile(tmp_path, sha))
    got = bench.tensor_stop_issued_from_profile(32, 7, 1000.0, 1e-6)
    # 14 dispatches over 7 matrices = 2 calls each; only the g = 32 lockstep kernels count:
    # (1000 + 3*100 + 500 + 3*50) * 64 lane-slots over 2 * 1000 weights = 62.4 per weight
    assert got["slots_per_weight"] == pytest.approx(62.4)
    assert got["frac"] == pytest.approx(62.4 * 1000 / 1e-9 / bench.PEAK_VALU_SLOTS, rel=1e-3)


def test_tensor_stop_issued_is_null_on_another_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_VARIANTS", _variants_profile(tmp_path, "0" * 16))
    assert bench.tensor_stop_issued_from_profile(32, 7, 1000.0, 1e-6) is None
    monkeypatch.setattr(bench, "PROFILE_VARIANTS", str(tmp_path / "absent.json"))
    assert bench.tensor_stop_issued_from_profile(32, 7, 1000.0, 1e-6) is None


def test_committed_variants_profile_matches_the_tensor_stop_source():
    with open(bench.PROFILE_VARIANTS) as f:
        prof = json.load(f)
    assert prof["tensor_stop_source_sha256_16"] == bench.kernel_source_hash(bench.TENSOR_STOP_SRC)
