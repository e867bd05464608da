"""Host-side checks of the bench's measurement arithmetic: the scaling of rocprofv3's
FETCH_SIZE / WRITE_SIZE readings by a calibration copy of known size, the grouping of a
call's kernels per launch, and the source-hash guard on stored traffic figures.  Counter
files here are small synthetic CSVs in rocprofv3's column names; nothing touches a GPU or
the committed traffic table."""

import csv
import json

import bench


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for dispatch, kernel, value in rows:
            w.writerow({"Dispatch_Id": dispatch, "Kernel_Name": kernel, "Counter_Name": counter,
                        "Counter_Value": value})


def _bench_line(path, workload, calls, own="page"):
    """A bench line of one workload whose timed calls are {name: (source hash, algorithmic bytes)}."""
    line = {"metric": "m", "config": {"workload": workload, "ownership": own},
            "parts": {"workloads": {workload: {"calls": {c: {"source_hash": h, "algorithmic_bytes": b}
                                                          for c, (h, b) in calls.items()}}}},
            "roofline": {"kernel": next(iter(calls))}}
    with open(path, "w") as f:
        f.write("[bench] some progress line\n" + json.dumps(line) + "\n")


CALIB = "void at::native::vectorized_elementwise_kernel<bitwise_not_kernel_cuda>(int, ...)"


def test_traffic_scaled_by_calibration_copy_and_grouped_per_launch(tmp_path):
    # a 1024 MiB copy reads as 512 MiB of FETCH_SIZE and 1024 MiB of WRITE_SIZE (two rows
    # per dispatch, as per-partition values are), so fetch counts scale by 2 and writes by 1
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    rs = "dcpkv::reshard_kernel(dcpkv::ReshardArgs)"
    other = "dcpkv::reshard_tokens_kernel(dcpkv::TokenReshardArgs)"
    _counter_csv(fetch, "FETCH_SIZE", [(1, CALIB, 262144), (1, CALIB, 262144)] +
                 [(d, rs, v) for d in (2, 3, 4) for v in (600, 400)] + [(5, other, 99999)])
    _counter_csv(write, "WRITE_SIZE", [(1, CALIB, 1048576)] + [(d, rs, 2000) for d in (2, 3, 4)] +
                 [(5, other, 99999)])
    line = tmp_path / "b.json"
    _bench_line(line, "wl", {"reshard_kernel": ("abc", 4_000_000)})
    db = tmp_path / "traffic.json"
    stored = bench.pmc_summarize(str(fetch), str(write), str(line), 1024, path=str(db))
    assert set(stored) == {"wl:reshard_kernel"}
    e = stored["wl:reshard_kernel"]
    assert e["launches"] == 3 and e["algorithmic_bytes_per_launch"] == 4_000_000
    assert e["scale_fetch"] == 2.0 and e["scale_write"] == 1.0
    assert e["fetch_kib_per_launch"] == 1000.0 and e["write_kib_per_launch"] == 2000.0
    assert e["hbm_bytes_per_launch"] == 1000 * 1024 * 2 + 2000 * 1024
    assert bench.load_traffic("wl:reshard_kernel", "abc", path=str(db)) == 4_096_000
    assert bench.load_traffic("wl:reshard_kernel", "changed", path=str(db)) is None
    assert bench.load_traffic("other:reshard_kernel", "abc", path=str(db)) is None


def test_traffic_of_the_decode_call_sums_its_kernels_per_launch(tmp_path):
    # one launch of the call = planner + partial kernel + chunk reduction; launches are counted
    # by the partial kernel; token ownership gets its own key; a call whose kernels are not in
    # the counter files (the reshard here) is left out
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    ks = ["dcpkv::plan_kernel(dcpkv::AttnParams)", "dcpkv::mla_fp8_kernel(dcpkv::AttnParams)",
          "dcpkv::chunk_reduce_kernel(dcpkv::AttnParams)"]
    rows_f, rows_w, d = [(1, CALIB, 524288)], [(1, CALIB, 1048576)], 2
    for _ in range(2):
        for k, fv, wv in zip(ks, (10, 500, 20), (1, 100, 9)):
            rows_f.append((d, k, fv))
            rows_w.append((d, k, wv))
            d += 1
    rows_f.append((d, "dcpkv::lse_merge_kernel(int, long, ...)", 12345))  # not part of the call
    _counter_csv(fetch, "FETCH_SIZE", rows_f)
    _counter_csv(write, "WRITE_SIZE", rows_w)
    line = tmp_path / "b.json"
    _bench_line(line, "mla", {"dcp_decode_partial": ("h1", 10), "reshard_kernel": ("h2", 20)}, own="token")
    db = tmp_path / "traffic.json"
    stored = bench.pmc_summarize(str(fetch), str(write), str(line), 1024, path=str(db))
    e = stored["mla:dcp_decode_partial:token"]
    assert e["launches"] == 2
    assert e["fetch_kib_per_launch"] == 530.0 and e["write_kib_per_launch"] == 110.0
    assert e["hbm_bytes_per_launch"] == 530 * 1024 * 2 + 110 * 1024
    assert set(json.load(open(db))) == {"mla:dcp_decode_partial:token"}


def test_kernel_source_hash_follows_the_sources():
    a = bench.kernel_source_hash(["reshard.hip"])
    assert a == bench.kernel_source_hash(["reshard.hip"]) and len(a) == 16
    assert a != bench.kernel_source_hash(["reshard.hip", "common.h"])


def test_default_run_covers_the_four_full_size_workloads_with_the_long_mix_as_headline():
    a = bench.parse([])
    assert a.workload == "all" and a.gpus == 1
    assert bench.WORKLOADS == ("gqa_bf16_16x4k-32k", "reshard_mla_128k", "mla_fp8_48x100k",
                               "mla_fp8_longmix_verify")
    assert bench.HEADLINE == "mla_fp8_longmix_verify"
    assert 1 <= bench.cpu_workers() <= 16


def test_device_telemetry_never_raises():
    t = bench.device_telemetry()
    assert isinstance(t, dict)
