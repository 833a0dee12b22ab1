"""bench.py without a GPU: its command line (one GPU only, and it says so for more) and the
traffic record it builds from rocprofv3 counter passes."""
import argparse
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    for n in ("2", "8"):
        res = run_bench("--gpus", n)
        assert res.returncode == 2, res
        assert "one GPU" in res.stderr, res.stderr
        assert res.stdout == ""  # no JSON line


def test_help_lists_the_contract_flags():
    res = run_bench("--help")
    assert res.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workload", "--kernel", "--partition"):
        assert flag in res.stdout


def test_block_size_must_be_a_multiple_of_16():
    for bs in ("8", "24"):
        res = run_bench("--block-size", bs)
        assert res.returncode == 2, res
        assert "multiple of 16" in res.stderr, res.stderr
        assert res.stdout == ""



def _counter_csv(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    cols = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(os.path.join(path, "run_counter_collection.csv"), "w") as f:
        f.write(",".join(cols) + "\n")
        for i, (grid, name, value) in enumerate(rows):
            f.write(f'{i},{grid},"{name}",{counter},{value}\n')


def test_record_traffic_scales_by_the_copy_and_averages_the_attention_launches(tmp_path,
                                                                                monkeypatch):
    """--record-traffic reads the two counter passes, takes the scale from the 1 GiB copy
    (FETCH_SIZE reads half of its bytes here, WRITE_SIZE all of them), averages every attention
    dispatch of the decode families it finds (not the merge), and stamps the record with the
    hash of those families' sources."""
    sys.path.insert(0, ROOT)
    import bench

    copy = (131072, "__amd_rocclr_copyBuffer", None)
    sk = "void pagedkv::decode_mfma_sk_kernel<128, 4, 2, 1, 0, 2, false>(pagedkv::DecodeArgs)"
    hw = "void pagedkv::decode_mfma_hw_kernel<128, 4, 2, 2, 0, 2, false>(pagedkv::DecodeArgs)"
    merge = "void pagedkv::decode_reduce_split_kernel<2, 16, 4, false>(pagedkv::DecodeArgs)"
    fetch = [(copy[0], copy[1], 524288.0), (65536, sk, 1000.0), (8192, merge, 77.0),
             (65536, hw, 3000.0)]
    write = [(copy[0], copy[1], 1048576.0), (65536, sk, 10.0), (8192, merge, 5.0),
             (65536, hw, 30.0)]
    _counter_csv(str(tmp_path / "FETCH_SIZE"), "FETCH_SIZE", fetch)
    _counter_csv(str(tmp_path / "WRITE_SIZE"), "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    args = argparse.Namespace(record_traffic=str(tmp_path), kernel="auto", workload="c5")
    bench.record_traffic(args)
    rec = json.loads(out.read_text())["c5"]
    assert rec["kernel"] == "mfma_sk+mfma_hw"
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["launches"] == 2
    assert rec["fetch_bytes_per_launch"] == 2000 * 1024 * 2
    assert rec["write_bytes_per_launch"] == 20 * 1024
    assert rec["bytes_per_launch"] == 2000 * 1024 * 2 + 20 * 1024
    assert rec["kernel_source"] == bench.kernel_source_hash("mfma_sk+mfma_hw")
    assert rec["kernel_source"] != bench.kernel_source_hash("mfma_hw")


def test_event_steps_are_disjoint_spread_and_in_range():
    """The timed steps that carry timing events: disjoint kernel and call sets inside the
    timed steps, spread over them, every step alternating when there are too few."""
    import bench
    for steps, per in ((20, 4), (100, 4), (10, 2), (5, 4), (20, 0), (1, 4), (2, 1)):
        kern, call = bench.event_steps(steps, per)
        assert kern, (steps, per)
        assert not set(kern) & set(call)
        assert all(0 <= i < steps for i in kern + call)
        if steps > 1 and 0 < per and 2 * per < steps:
            assert len(kern) == len(call) == per
            assert kern[0] < steps // per and kern[-1] >= steps - steps // per
        elif steps > 1:
            assert sorted(kern + call) == list(range(steps))


def test_warm_up_counts_steps_and_stops_on_time():
    """Without --warmup the warm-up runs whole groups of five steps until --warmup-seconds
    have passed and records the count; with --warmup it runs exactly that many."""
    import types
    import bench

    class FakeCuda:
        def synchronize(self):
            pass

    torch_stub = types.SimpleNamespace(cuda=FakeCuda())
    calls = []
    args = types.SimpleNamespace(warmup=None, warmup_seconds=0.0)
    n = bench.warm_up(args, torch_stub, lambda: calls.append(1))
    assert n == 5 and args.warmup == 5 and len(calls) == 5  # at least one group of five
    calls.clear()
    args = types.SimpleNamespace(warmup=None, warmup_seconds=0.05)
    n = bench.warm_up(args, torch_stub, lambda: (calls.append(1), __import__("time").sleep(0.002)))
    assert n % 5 == 0 and n >= 15 and args.warmup == n == len(calls)
    calls.clear()
    args = types.SimpleNamespace(warmup=3, warmup_seconds=10.0)
    assert bench.warm_up(args, torch_stub, lambda: calls.append(1)) == 3 and len(calls) == 3
