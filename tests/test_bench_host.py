"""Host-side logic of bench.py (no GPU): the HBM-traffic record written from
rocprofv3 counter files and read back for the roofline object, the
algorithmic byte and FLOP figures the bench divides by its timings, and the
refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synthetic import CONFIGS  # noqa: E402

HEADER = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"


def _csv(path, rows):
    with open(path, "w") as f:
        f.write(HEADER)
        for d, name, counter, value in rows:
            f.write(f'{d},"{name}",{counter},{value}\n')
    return str(path)


def test_permute_bytes_of_the_fwd_bwd_workload():
    """R = 65536 routed rows, T = 16384 tokens, H = 7168: rows of 14336 bytes
    in and out, plus the 4- and 8-byte per-row arrays each kernel touches."""
    b = bench.permute_bytes(CONFIGS[4])
    assert b == {"combine": 1174929408, "reverse_combine": 1175453696, "reverse_dispatch": 1174667264}


def test_gemm_rates_use_routed_rows_only():
    """gate/up: 4*H*I FLOPs per routed row; 65536 rows at H=7168, I=2048
    (962072674304 * 4 FLOPs) in 3.7368 ms per step is 1029.84 TFLOP/s; down
    2*H*I per row in 1.8452 ms, 1042.78."""
    p = CONFIGS[4]
    r = bench.gemm_rates({"gateup_gemm": (2, 3.7368, 1.9), "down_gemm": (2, 1.8452, 1.0),
                          "combine": (1, 0.2, 0.2)}, p, 1)
    assert r == {"gateup_gemm": 1029.84, "down_gemm": 1042.78}


def test_traffic_record_round_trip(tmp_path, monkeypatch):
    """Counter values per dispatch, averaged per kernel and scaled by what the
    same counter reads for a 1 GiB copy, come back from the record; a record
    of other kernel sources or another minibatch size yields no traffic."""
    p = CONFIGS[4]
    out = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "traffic_file", lambda q: str(out))
    copy = "__amd_rocclr_copyBuffer(...)"
    gu = "void (anonymous namespace)::gateup_kernel<false>(mok_fwd_args, int, int, int)"
    dh = "(anonymous namespace)::bwd_dh_kernel(mok_bwd_args, int)"
    f = _csv(tmp_path / "f.csv", [(1, gu, "FETCH_SIZE", 1000.0), (2, gu, "FETCH_SIZE", 3000.0),
                                  (3, dh, "FETCH_SIZE", 800.0), (3, dh, "FETCH_SIZE", 200.0)])
    w = _csv(tmp_path / "w.csv", [(1, gu, "WRITE_SIZE", 500.0), (2, gu, "WRITE_SIZE", 700.0),
                                  (3, dh, "WRITE_SIZE", 100.0)])
    cf = _csv(tmp_path / "cf.csv", [(1, copy, "FETCH_SIZE", 524288.0)])       # half the bytes: factor 2
    cw = _csv(tmp_path / "cw.csv", [(1, copy, "WRITE_SIZE", 1048576.0)])      # all of them: factor 1

    class A:
        traffic_record = (f, w, cf, cw)
        config = 4
        minibatch_rows = 0
        ring_slots = 0

    bench.write_traffic_record(A)
    rec = json.loads([ln for ln in open(out) if ln.startswith("{")][-1])
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    assert rec["workload"] == p.name and rec["sources_sha256"] == bench.kernel_sources_sha256()
    k = rec["kernels"]
    # gate/up: fetch (1000 + 3000) / 2 dispatches, write (500 + 700) / 2
    assert k["gateup_gemm"] == {"dispatches": 2, "fetch_kib": 2000.0, "write_kib": 600.0,
                                "bytes_per_launch": (2000 * 2 + 600) * 1024}
    # dh: one dispatch whose counter rows (hardware instances) add up
    assert k["bwd_dh_gemm"]["fetch_kib"] == 1000.0
    assert k["bwd_dh_gemm"]["bytes_per_launch"] == (1000 * 2 + 100) * 1024
    assert "down_gemm" not in k                                            # no counters for it
    mb = rec["minibatch_rows"]
    assert bench.measured_traffic("gateup_gemm", p, mb) == ((2000 * 2 + 600) * 1024, os.path.relpath(out, ROOT))
    assert bench.measured_traffic("down_gemm", p, mb)[0] is None
    assert bench.measured_traffic("gateup_gemm", p, mb + 256)[0] is None
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: "0" * 64)
    assert bench.measured_traffic("gateup_gemm", p, mb) == (None, "kernel sources changed since the counters "
                                                                 "were taken")


def test_traffic_record_needs_the_copy_calibration(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_file", lambda q: str(tmp_path / "traffic.txt"))
    empty = _csv(tmp_path / "e.csv", [])

    class A:
        traffic_record = (empty, empty, empty, empty)
        config = 4
        minibatch_rows = 0
        ring_slots = 0

    with pytest.raises(SystemExit):
        bench.write_traffic_record(A)


def test_committed_traffic_record_is_consistent():
    """The committed record of the headline workload: every kernel's bytes per
    launch are its averaged counters times the stored calibration factors."""
    p = CONFIGS[4]
    rec = json.loads([ln for ln in open(bench.traffic_file(p)) if ln.startswith("{")][-1])
    assert rec["workload"] == p.name
    assert 1.9 < rec["fetch_factor"] < 2.1 and 0.9 < rec["write_factor"] < 1.1
    for name, k in rec["kernels"].items():
        want = (k["fetch_kib"] * rec["fetch_factor"] + k["write_kib"] * rec["write_factor"]) * 1024
        assert abs(k["bytes_per_launch"] - want) <= 2e-5 * want + 1024, name


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr
