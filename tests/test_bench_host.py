"""Host logic of bench.py: the HBM traffic summary built from rocprofv3 counter
CSVs (no GPU; the CSVs are written here in the profiler's column layout)."""
import csv
import json
import os

import bench

COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
        "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
        "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
        "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write(dirname, counter, rows):
    """rows: (dispatch id, kernel name, value)."""
    os.makedirs(dirname, exist_ok=True)
    with open(os.path.join(dirname, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for did, name, val in rows:
            r = {c: 0 for c in COLS}
            r.update({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": counter,
                      "Counter_Value": val})
            w.writerow(r)


def _kname(short):
    return "void fa::(anonymous namespace)::%s(unsigned short const*, float*)" % short


def test_summarize_counters_scales_by_the_copy_and_maps_kernels(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    mib = 1024
    copy_kib = mib * 1024   # a 1 GiB copy read as 1 GiB: 1 KiB per KiB
    step = []
    did = 0
    for bench_name, names in bench.HEADLINE_KERNELS.items():
        for rep in range(2):   # two dispatches each; the mean is taken
            for i, n in enumerate(names[:1]):
                did += 1
                step.append((did, _kname(n), 100.0 + 10 * rep + i))
    step.append((did + 1, _kname("other_kernel<1>"), 7.0))   # not the headline: ignored
    for counter, scale in (("FETCH_SIZE", 0.5), ("WRITE_SIZE", 1.0)):
        _write(str(tmp_path / ("s_" + counter)), counter, step)
        _write(str(tmp_path / ("c_" + counter)), counter,
               [(1, "__amd_rocclr_copyBuffer", copy_kib * scale),
                (2, "fill kernel", 3.0)])
    bench.summarize_counters(str(tmp_path / "s_FETCH_SIZE"), str(tmp_path / "c_FETCH_SIZE"),
                             str(tmp_path / "s_WRITE_SIZE"), str(tmp_path / "c_WRITE_SIZE"),
                             mib, ["cmd"])
    t = json.loads(out.read_text())
    assert t["copy_counter_per_byte"] == {"FETCH_SIZE": 0.5, "WRITE_SIZE": 1.0}
    assert t["src_digest"] == bench.src_digest(bench.HEADLINE_SOURCES)
    for name in bench.HEADLINE_KERNELS:
        e = t["kernels"][name]
        assert e["FETCH_SIZE_KiB"] == 105.0 and e["WRITE_SIZE_KiB"] == 105.0
        # FETCH reads half a KiB per KiB moved, so 105 KiB counted are 210 KiB moved
        assert e["fetch_bytes"] == 105.0 * 1024 / 0.5
        assert e["write_bytes"] == 105.0 * 1024
        assert e["bytes_per_launch"] == int(105.0 * 1024 * 3)
    # the bench line reads it back while the digest matches the sources
    assert bench.load_traffic("long_causal_prefill") == int(105.0 * 1024 * 3)


def test_bytes_avoided_matches_the_pages_table():
    """512 MiB per head of fp16 scores at N = 16384, four passes over 32 heads."""
    b = bench.bytes_avoided(1, 32, 16384)
    assert b["per_head_MiB"] == 512 and b["total_GiB"] == 64


def test_timing_stats_and_flop_convention():
    s = bench.stats_ms([float(x) for x in range(1, 102)])
    assert s["median"] == 51 and s["p10"] == 11 and s["p90"] == 91 and s["n"] == 101
    assert bench.fwd_flops(1, 32, 16384, 128, True) == 4 * 32 * 16384 ** 2 * 128 / 2
    assert bench.window_pairs(10, 10, 0) == 55 and bench.window_pairs(10, 1, 0) == 10


def test_bench_refuses_more_than_one_gpu(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
