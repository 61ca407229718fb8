"""Host-side logic of bench.py (no GPU): the algorithmic byte counts the
roofline uses, the single-GPU guard, and the rocprofv3 summaries that the
committed profiles and the bench line's `traffic` come from."""
import csv
import subprocess
import sys

import pytest

import bench

N_LARGE = 32768 * 4096


def test_algorithmic_bytes():
    # per element: compress 2 (bf16 in) + 0.5 (codes) + 1/16 (micro) + 4/256 (block);
    # decompress the payload in and 4 (fp32) out
    ab = bench.algorithmic_bytes(N_LARGE)
    assert ab["compress"] == 346030080 == int(N_LARGE * 2.578125)
    assert ab["decompress"] == 614465536 == int(N_LARGE * 4.578125)


def test_receiver_bytes():
    rb = bench._receiver_bytes()
    n = 4096 * 11008
    payload = 26066944                          # codes + micro + block of one peer
    assert n // 2 + n // 16 + n // 64 == payload
    assert rb["accumulate"] == 388890624 == 8 * payload + 4 * n
    assert rb["requantize"] == 9 * payload      # 8 payloads in, 1 out
    assert rb["requantize_local"] == 7 * payload + 2 * n + payload


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


COUNTER_FIELDS = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _counter_dir(tmp_path, name, counter, rows):
    d = tmp_path / name / "host"
    d.mkdir(parents=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, COUNTER_FIELDS)
        w.writeheader()
        for i, (kernel, grid, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Grid_Size": grid, "Kernel_Name": kernel,
                        "Counter_Name": counter, "Counter_Value": value})
    return str(tmp_path / name)


COPY = "__amd_rocclr_copyBuffer"
COMP = "void (anonymous namespace)::compress_kernel<true>(uint4 const*, long, uint4*, unsigned int*, float*)"
DECOMP = "void (anonymous namespace)::decompress_kernel<true, false>(uint4 const*, uint4 const*, float const*, long, void*)"
G = N_LARGE // 64          # one thread per 64 elements
KIB = bench.COPY_REF_BYTES // 1024


def test_counter_summary_scales_by_the_copy_reference(tmp_path):
    # a counter that reads half of what a copy reads (fetch) and one that reads all of it (write)
    ab = bench.algorithmic_bytes(N_LARGE)
    fetch = _counter_dir(tmp_path, "f", "FETCH_SIZE", [
        (COPY, 131072, KIB / 2), (COPY, 131072, KIB / 2 + 3), (COPY, 131072, KIB / 2 - 3),
        (COPY, 512, 2),                                         # a tiny copy: another grid, ignored
        (COMP, G, 2 * N_LARGE / 1024 / 2), (COMP, G // 4, 1.0),  # a smaller launch: ignored
        (DECOMP, G, (ab["decompress"] - 4 * N_LARGE) / 2048),
    ])
    write = _counter_dir(tmp_path, "w", "WRITE_SIZE", [
        (COPY, 131072, KIB), (COPY, 131072, KIB), (COPY, 131072, KIB),
        (COMP, G, (ab["compress"] - 2 * N_LARGE) / 1024), (DECOMP, G, 4 * N_LARGE / 1024),
    ])
    text = bench.summarize_counters(fetch, write)
    assert "fetch x2.000, write x1.000" in text
    traffic = dict(kv.split("=") for kv in text.splitlines()[-1].split()[1:])
    assert traffic.pop("source") == bench.kernel_source_hash()
    assert int(traffic["compress"]) == ab["compress"]
    assert int(traffic["decompress"]) == ab["decompress"]
    assert "| compress | 32768x4096 |" in text and "| 1.000 |" in text


ACC = "void (anonymous namespace)::accumulate_narrow_kernel<true, false>(Peers, int, long, float*)"
REQ = "void (anonymous namespace)::requantize_narrow_kernel(Peers, int, long, uint4*, unsigned int*, float*)"
REQ_LOCAL = "void (anonymous namespace)::requantize_kernel<true>(Peers, int, long, uint4*, unsigned int*, float*)"


def test_counter_summary_receivers_at_their_layouts_grids(tmp_path):
    # accumulate and the re-quantise without a local slice run one thread per 32
    # elements, the re-quantise with one a thread per 64; launches of other
    # grids are another workload and give no figure
    n, rb = bench.REDUCE_N, bench._receiver_bytes()
    fetch = _counter_dir(tmp_path, "f", "FETCH_SIZE", [
        (COPY, 131072, KIB / 2), (COPY, 131072, KIB / 2), (COPY, 131072, KIB / 2),
        (ACC, n // 32, (rb["accumulate"] - 4 * n) / 2048),
        (REQ, n // 32, 100.0), (REQ_LOCAL, n // 32, 100.0)])
    write = _counter_dir(tmp_path, "w", "WRITE_SIZE", [
        (COPY, 131072, KIB), (COPY, 131072, KIB), (COPY, 131072, KIB),
        (ACC, n // 32, 4 * n / 1024), (REQ, n // 32, 10.0), (REQ_LOCAL, n // 32, 10.0)])
    traffic = dict(kv.split("=") for kv in bench.summarize_counters(fetch, write).splitlines()[-1].split()[1:])
    assert int(traffic["accumulate"]) == rb["accumulate"]
    assert int(traffic["requantize"]) == 2 * 100 * 1024 + 10 * 1024
    assert "requantize_local" not in traffic     # a narrow grid is not its workload


def test_counter_summary_reference_is_the_largest_copies(tmp_path):
    # smaller copies (tensor clones) share the grid-strided copy kernel's grid and
    # are left out; the reference needs its three copies
    fetch = _counter_dir(tmp_path, "f", "FETCH_SIZE", [
        (COPY, 131072, KIB / 2), (COPY, 131072, KIB / 2), (COPY, 131072, KIB / 2),
        (COPY, 131072, KIB / 16), (COPY, 131072, KIB / 200), (COMP, G, 1.0)])
    write = _counter_dir(tmp_path, "w", "WRITE_SIZE", [
        (COPY, 131072, KIB), (COPY, 131072, KIB), (COPY, 131072, KIB),
        (COPY, 131072, KIB / 8), (COMP, G, 1.0)])
    assert "fetch x2.000, write x1.000" in bench.summarize_counters(fetch, write)
    no_ref = _counter_dir(tmp_path, "w2", "WRITE_SIZE", [
        (COPY, 131072, KIB / 8), (COMP, G, 1.0)])
    with pytest.raises(ValueError, match="three reference copies"):
        bench.summarize_counters(fetch, no_ref)


def test_trace_summary(tmp_path, monkeypatch):
    d = tmp_path / "t" / "host"
    d.mkdir(parents=True)
    fields = ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp", "End_Timestamp"]
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fields)
        w.writeheader()
        t = 0
        for grid, us in [(G, 90), (G, 100), (G, 110), (G // 8, 5), (G, 120), (G, 130)]:   # ns timestamps
            w.writerow({"Kernel_Name": DECOMP, "Grid_Size_X": grid, "Grid_Size_Y": 1, "Grid_Size_Z": 1,
                        "Start_Timestamp": t, "End_Timestamp": t + us * 1000})
            t += 10 ** 6
        w.writerow({"Kernel_Name": "some_other_kernel", "Grid_Size_X": 64, "Grid_Size_Y": 1,
                    "Grid_Size_Z": 1, "Start_Timestamp": 0, "End_Timestamp": 5})
    text = bench.summarize_trace(str(tmp_path / "t"))
    rows = [l for l in text.splitlines() if l.startswith("| decompress_kernel")]
    assert rows == ["| decompress_kernel<true, false> | %d | 5 | 110.00 | 110.00 | 90.00 | 130.00 |" % G]
    assert "some_other_kernel" not in text and "per-kernel pass" not in text
    # a 2-step run with a 2-step per-kernel pass: the last two full-size launches
    # are the pass, the two before them the timed region
    monkeypatch.setattr(bench, "KERNEL_PASS", 2)
    text = bench.summarize_trace(str(tmp_path / "t"), timed_steps=2)
    assert "| decompress_kernel<true, false> | per-kernel pass | 2 | 125.00 | 125.00 |" in text
    assert "| decompress_kernel<true, false> | timed region | 2 | 105.00 | 105.00 |" in text


def test_traffic_is_read_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    f = tmp_path / "summary.md"
    f.write_text("text\ntraffic: source=%s compress=11 decompress=22\n" % bench.kernel_source_hash())
    assert bench.measured_traffic(str(f)) == {"compress": 11, "decompress": 22}
    f.write_text("text\ntraffic: source=0123456789abcdef compress=11 decompress=22\n")
    assert bench.measured_traffic(str(f)) is None
    assert bench.measured_traffic(str(tmp_path / "missing.md")) is None


def test_kernel_families():
    """Counter and trace summaries group dispatches by kernel family; the traffic
    twins of the ceilings leg never count as the kernels they mirror."""
    ns = "void (anonymous namespace)::"
    assert bench._short(ns + "decompress_kernel<true, false>(x)") == "decompress"
    assert bench._short(ns + "twin_decompress_kernel(x)") == "twin"
    assert bench._short(ns + "twin_compress_kernel(x)") == "twin"
    assert bench._short(ns + "requantize_narrow_kernel(x)") == "requantize"
    assert bench._short(ns + "requantize_kernel<true>(x)") == "requantize_local"
    assert bench._short(ns + "compress_mx_kernel<true>(x)") == "compress_mx"
    assert bench._short(ns + "accumulate_narrow_kernel<true, false>(x)") == "accumulate"
    assert bench.KERNEL_NAME.search(ns + "accumulate_narrow_kernel<true, false>(x)").group(1) \
        == "accumulate_narrow_kernel<true, false>"
