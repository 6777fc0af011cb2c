"""bench.py without a GPU: the multi-GPU refusal, the rocprofv3 counter
summaries that turn FETCH_SIZE / WRITE_SIZE into bytes per launch (for the
gate and for the memory read), and the one that turns the hash's SQ
instruction counts into its ALU roofline."""

import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "shards by tokens" in r.stderr


def _counter_csv(path, counter, rows):
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_traffic_summary_calibrates_on_the_copy_probe(tmp_path, monkeypatch):
    import synth
    c = synth.CONFIGS[4]
    copy_bytes = 2 * c.T * c.H
    fwd = "void (anonymous namespace)::gate_fwd_kernel<7, 2, true, 2>(unsigned int, int)"
    bwd = "void (anonymous namespace)::gate_bwd_kernel<7, 2, true, 3, true>(int)"
    cp = "(anonymous namespace)::copy_probe_kernel(unsigned int __vector(4) const*, long)"
    # FETCH_SIZE reads half the bytes and WRITE_SIZE all of them, in KiB; at
    # this shape each gate call is two epoch launches, each with half its bytes
    assert bench.gate_launches(c.T, c.H) == {"gate_fwd_kernel": 2, "gate_bwd_kernel": 2}
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE",
                 [(cp, copy_bytes / 2048)] + [(fwd, 3 * copy_bytes / 4 / 2048)] * 4
                 + [(bwd, copy_bytes / 2048)] * 2)
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE",
                 [(cp, copy_bytes / 1024)] + [(fwd, copy_bytes / 4 / 1024)] * 2
                 + [(bwd, 3 * copy_bytes / 4 / 1024)] * 2)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    rec = bench.traffic_from_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 4)
    assert abs(rec["calibration"]["fetch_scale"] - 2.0) < 1e-12
    assert abs(rec["calibration"]["write_scale"] - 1.0) < 1e-12
    k = rec["kernels"]
    # forward: 3 tensors read, 1 written; backward: 4 read, 3 written
    assert abs(k["gate_fwd_kernel"]["bytes_per_call"] - 2 * copy_bytes) < 1
    assert abs(k["gate_bwd_kernel"]["bytes_per_call"] - 3.5 * copy_bytes) < 1
    saved = json.load(open(tmp_path / f"traffic_{c.name}.json"))
    assert saved["kernel_source_sha256_16"] == bench.kernel_source_hash()
    # the bench line uses it only while the kernel source is unchanged
    assert bench.measured_traffic("gate_bwd_kernel", c.name) == \
        k["gate_bwd_kernel"]["bytes_per_call"]
    saved["kernel_source_sha256_16"] = "0" * 16
    json.dump(saved, open(tmp_path / f"traffic_{c.name}.json", "w"))
    assert bench.measured_traffic("gate_bwd_kernel", c.name) is None


def test_hash_valu_summary_and_alu_roofline(tmp_path, monkeypatch):
    # two dispatches of the 4,194,304-token hash and one small one (ignored)
    fields = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    name = "void (anonymous namespace)::hash_kernel_vec<16, 3>(int const*, long)"
    rows = []
    for disp, grid, valu in ((1, 4194304, 588), (2, 4194304, 590), (3, 32768, 999)):
        waves = grid // 64
        rows += [(disp, grid, "SQ_WAVES", waves), (disp, grid, "SQ_INSTS_VALU", valu * waves),
                 (disp, grid, "SQ_INSTS_SALU", 18 * waves)]
    with open(tmp_path / "sq.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for disp, grid, counter, value in rows:
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Grid_Size": grid,
                        "Counter_Name": counter, "Counter_Value": value})
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    rec = bench.valu_from_counters(str(tmp_path / "sq.csv"))
    assert rec["dispatches"] == 2 and rec["tokens_per_wave"] == 64
    assert rec["valu_insts_per_wave"] == 589 and rec["salu_insts_per_wave"] == 18
    # 1024 SIMDs issue one VALU instruction every 4 cycles at 2.4 GHz
    note = bench.hash_valu_note(30e9)
    want = 1024 * 2.4e9 / 4 * 64 / 589
    assert abs(note["tokens_per_s_at_valu_issue_rate"] - want) < 1
    assert abs(note["frac"] - 30e9 / want) < 1e-12
    saved = json.load(open(tmp_path / "valu_hash_b1024s4096.json"))
    saved["hash_source_sha256_16"] = "0" * 16
    json.dump(saved, open(tmp_path / "valu_hash_b1024s4096.json", "w"))
    assert bench.hash_valu_note(30e9) is None


def test_memory_read_traffic_splits_hash_and_gather(tmp_path, monkeypatch):
    import synth
    c = synth.CONFIGS[4]
    copy_bytes = 2 * c.T * c.H
    gc = synth.GATHER_CONFIGS["t32768_d448"]
    g_algo = gc.T * gc.tables * (4 + 4 * gc.d)
    h_tok = 1024 * 4096
    fields = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    cp = "(anonymous namespace)::copy_probe_kernel(unsigned int __vector(4) const*, long)"
    hk = "void (anonymous namespace)::hash_kernel_vec<16, 3>(int const*, long)"
    gk = "(anonymous namespace)::gather_kernel(int const*, unsigned int __vector(4) const*)"
    for counter, scale in (("FETCH_SIZE", 2.0), ("WRITE_SIZE", 1.0)):
        rows = [(cp, 4194304, copy_bytes / scale / 1024)]
        rows += [(hk, h_tok, (4 * h_tok if counter == "FETCH_SIZE" else 64 * h_tok) / scale / 1024)] * 3
        half = g_algo / 2
        # each gather group follows the small hash of its own indices, and
        # its warm-up makes the group's length vary
        rows += [(hk, 32768, 1.0)]
        rows += [(gk, 8388608, half / scale / 1024)] * 37
        rows += [(hk, 32768, 1.0)]
        rows += [(gk, 8388608, 0.9 * half / scale / 1024)] * 29
        with open(tmp_path / f"{counter}.csv", "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=fields)
            w.writeheader()
            for i, (name, grid, value) in enumerate(rows):
                w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Grid_Size": grid,
                            "Counter_Name": counter, "Counter_Value": value})
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    rec = bench.memory_read_traffic(str(tmp_path / "FETCH_SIZE.csv"),
                                    str(tmp_path / "WRITE_SIZE.csv"))
    assert abs(rec["hash"]["measured_over_algorithmic"] - 1.0) < 1e-12
    assert abs(rec["gather"]["measured_over_algorithmic"] - 1.0) < 1e-12
    assert abs(rec["gather_zipf"]["measured_over_algorithmic"] - 0.9) < 1e-12
    assert bench.memory_read_bytes("gather") == rec["gather"]["bytes_per_launch"]
    saved = json.load(open(tmp_path / bench.MEMORY_READ_TRAFFIC))
    saved["gather_source_sha256_16"] = "0" * 16
    json.dump(saved, open(tmp_path / bench.MEMORY_READ_TRAFFIC, "w"))
    assert bench.memory_read_bytes("gather") is None
    assert bench.memory_read_bytes("hash") == rec["hash"]["bytes_per_launch"]


def test_host_cpu_share_counts_usable_cpus():
    share = bench.host_cpu_share()
    assert 1 <= share["threads"] <= share["affinity_cpus"] <= share["host_cpus"]
    if share["cgroup_cpu_quota"] is not None:
        assert share["threads"] <= max(1, int(share["cgroup_cpu_quota"]))


def test_footprint_summary_attributes_dispatches(tmp_path, monkeypatch):
    H = 7168
    n = bench.FOOTPRINT_COUNTER_LAUNCHES
    fields = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    cp = "(anonymous namespace)::copy_probe_kernel(unsigned int __vector(4) const*, long)"
    bk = "void (anonymous namespace)::gate_bwd_kernel<7, 2, true, 3, true>(long)"
    pk = "void (anonymous namespace)::stream_probe_kernel<4, 3>(long)"
    copy_bytes = 2 * 32768 * H
    for counter, scale in (("FETCH_SIZE", 2.0), ("WRITE_SIZE", 1.0)):
        rows = [(cp, copy_bytes / scale / 1024)]
        for T in bench.FOOTPRINT_COUNTER_TOKENS:
            part = (8 if counter == "FETCH_SIZE" else 6) * T * H
            L = bench.gate_launches(T, H)["gate_bwd_kernel"]    # epoch launches per call
            rows += [(bk, part / L / scale / 1024)] * (n * L)
            rows += [(pk, 1.1 * part / scale / 1024)] * n
        with open(tmp_path / f"{counter}.csv", "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=fields)
            w.writeheader()
            for i, (name, value) in enumerate(rows):
                w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Grid_Size": 1,
                            "Counter_Name": counter, "Counter_Value": value})
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    rec = bench.footprint_from_counters([str(tmp_path / "FETCH_SIZE.csv"),
                                         str(tmp_path / "WRITE_SIZE.csv")])
    for T in bench.FOOTPRINT_COUNTER_TOKENS:
        d = rec["per_tokens"][str(T)]
        assert abs(d["gate_bwd_kernel"]["measured_over_algorithmic"] - 1.0) < 1e-12
        assert abs(d["stream_probe_kernel"]["measured_over_algorithmic"] - 1.1) < 1e-12
