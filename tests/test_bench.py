"""bench.py's host-side contract, on the CPU: the one-GPU refusal, the HBM
traffic figure that follows the kernel source, the shard replicas that keep
a step's inputs out of the last-level cache, and the CPU-baseline record."""
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (imports no GPU library at module level)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_recorded_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    """The committed counter summary is used only while the kernel source
    hashes to the value it was taken on; any other source gets None."""
    with open(bench.TRAFFIC_FILE) as f:
        text = f.read()
    assert f"kernel_source_sha256_16: {bench.kernel_source_hash()}" in text, \
        "profiles/fused_step_traffic.md was taken on another kernel source"
    got = bench.recorded_traffic("gpt2s-w8")
    assert got is not None and got > 0
    assert bench.recorded_traffic("no-such-workload") is None
    # only for the instance the row was taken on
    row = re.search(r"^\| `([^`]+)` \(gpt2s-w8\) \|", text, re.M)
    assert row is not None
    assert bench.recorded_traffic("gpt2s-w8", row.group(1)) == got
    assert bench.recorded_traffic("gpt2s-w8", "zs::fused_kernel<no such instance>") is None
    other = tmp_path / "zs_kernels.h"
    other.write_text("// a different kernel source\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(other))
    assert bench.recorded_traffic("gpt2s-w8") is None


@pytest.mark.parametrize("step_bytes,want", [(1, 128), (1 << 20, 128), (11_184_832, 96),
                                             (200 << 20, 6), (653308992, 2), (1 << 30, 1),
                                             (18 << 30, 1)])
def test_replicas_cover_a_gigabyte(step_bytes, want):
    """Copies cycled per step: enough that the working set reaches 1 GB
    (past the 256 MB last-level cache), at most 128, at least 1."""
    got = bench.replicas_for(None, step_bytes)
    assert got == want
    assert got == 128 or got * step_bytes >= 1 << 30


def test_pad_elems_rounds_rows_to_256_bytes():
    assert [bench.pad_elems(n) for n in (0, 1, 128, 129, 15554976)] == \
        [0, 128, 128, 256, 15555072]


def test_cpu_baseline_record_on_the_smallest_workload():
    """The oracle timed on a bounded sample: the record's fields, and a
    sample no larger than the workload."""
    r = bench.cpu_baseline("mlp9-w3", target_s=0.3)
    assert r["kind"] == "oracle" and r["unit"] == "params/s"
    assert r["value"] > 0 and r["value_1_thread"] > 0
    assert 1 <= r["cores"] <= 16
    assert r["sample"].startswith("349526 params of the mlp9-w3 rank-0 partition")
    assert r["host_cpus_available"] >= 1


def test_cpu_sample_of_the_7b_state_is_three_windows():
    """The 7B state does not fit host memory: the oracle runs on windows of
    2^26 parameters at the head, the middle and the tail of the shard."""
    from sharded_mixed_precision_zs_amd import synth
    wl = synth.WORKLOADS["7b-full-w1"]
    starts, L = bench.cpu_windows(wl, (6 << 30) // 32)
    assert L == 1 << 26
    assert starts[0] == 0 and starts[-1] == wl.n - L and len(starts) == 3
    assert all(0 <= s and s + L <= wl.n for s in starts)
    small = synth.WORKLOADS["mlp9-w3"]
    assert bench.cpu_windows(small, 1 << 30) == ([0], small.n)


def test_fused_instance_names_match_the_kernel_template():
    from sharded_mixed_precision_zs_amd import synth
    W = synth.WORKLOADS
    assert bench.fused_instance(W["7b-full-w1"]) == \
        "zs::fused_kernel<4, 1, false, false, 0, 0, 0, 5, 64, false>"
    assert bench.fused_instance(W["7p5b-shard-w64"]) == \
        "zs::fused_kernel<4, 2, true, false, 0, 0, 0, 6, 64, false>"
    assert bench.fused_instance(W["1p3b-w4-acc4-fp16"]) == \
        "zs::fused_kernel<4, 2, true, true, 1, 1, 0, 5, 64, false>"
    assert bench.fused_instance(W["gpt2s-w8"]) == \
        "zs::fused_kernel<4, 2, true, false, 0, 0, 0, 6, 64, false>"
    big, small = 40_960_000, 40_959_999  # 20 000 tiles of 2048 and one element short
    assert [bench.fused_shape(w, big) for w in (1, 2, 3, 4, 5, 12, 13, 64)] == \
        [(64, 1, 5, 12), (64, 1, 5, 16), (256, 2, 5, 3), (64, 2, 5, 12), (64, 2, 6, 8),
         (64, 2, 6, 8), (64, 2, 6, 6), (64, 2, 6, 0)]
    assert [bench.fused_shape(w, small) for w in (1, 2, 3, 4, 5, 12, 13, 64)] == \
        [(64, 1, 5, 12), (64, 1, 5, 16), (256, 2, 5, 4), (64, 2, 5, 12), (64, 2, 6, 8),
         (64, 2, 6, 8), (64, 2, 6, 6), (64, 2, 6, 0)]
    assert bench.fused_instance(W["7b-full-w1"], state_layout="grouped") == \
        "zs::fused_kernel<4, 1, false, false, 0, 0, 0, 5, 64, true>"
    assert bench.fused_instance(W["7p5b-shard-w64"], state_layout="grouped") == \
        "zs::fused_kernel<4, 2, true, false, 0, 0, 0, 6, 64, true>"
    assert bench.fused_instance(W["1p3b-w4-acc4-fp16"], state_layout="grouped") == \
        "zs::fused_kernel<4, 2, true, true, 1, 1, 0, 5, 64, true>"
    assert [bench.fused_shape(w, big, "grouped") for w in (1, 3, 4, 5, 12, 13, 64)] == \
        [(64, 1, 5, 12), (64, 1, 5, 16), (64, 2, 5, 12), (64, 2, 6, 8), (64, 2, 6, 8),
         (64, 2, 6, 6), (64, 2, 6, 0)]
    # write windows: W >= 40 and >= 4 GB per launch (the 7.5B shard), uncapped
    assert bench.fused_shape(64, W["7p5b-shard-w64"].n, "grouped") == (64, 2, 6, 0)
    assert bench.write_window_of(64, W["7p5b-shard-w64"].n) == \
        {"period_us": 30.72, "open_fraction": 0.125}
    assert bench.write_window_of(39, 10**9) is None
    assert bench.write_window_of(64, W["7p5b-shard-w64"].n, state_layout="split") is not None
    assert bench.fused_shape(64, W["7p5b-shard-w64"].n) == (64, 2, 6, 0)
    assert bench.write_window_of(64, 4 * 10**9 // 154 - 1) is None
    assert bench.write_window_of(64, 4 * 10**9 // 154 + 1) is not None
    assert bench.fused_bytes_per_param(64, 1) == (140, 14)
    assert bench.fused_bytes_per_param(4, 4) == (24, 14)


def test_variant_sweep_plans_fit_their_workloads(hip_built):
    """Every variant a sweep plan names suits its workload's world size, and
    each plan starts with the production shape at libzeroshard's own cap."""
    from sharded_mixed_precision_zs_amd import synth
    lib = bench._variantlib()
    # the shapes zs_step_fused launches for these workloads, at its own caps
    production = {"7b-full-w1": (49, 2), "gpt2s-w8": (53, 4), "7p5b-shard-w64": (64, 12)}
    for name, plan in bench.VARIANT_SWEEP.items():
        W = synth.WORKLOADS[name].world
        for v, cap, per in plan:
            assert lib.zs_variant_multi(v) == (1 if W > 1 else 0), (name, v)
            assert 0 <= cap <= 32 and 0 <= per <= 8
        assert plan[0] == (*production[name], 0), name
    assert lib.zs_variant_name(49).decode() == "w1: 4-element lane groups, nt stores, nt state loads"
    assert lib.zs_variant_name(64).decode() == \
        "wN: 4-element lane groups, 2 vectors/thread, 64-thread blocks"
    assert lib.zs_variant_name(66).decode() == \
        "wN: 4-element lane groups, 1 vector/thread, 64-thread blocks"
    assert lib.zs_variant_name(70).decode() == \
        "wN: libzeroshard's kernel, 2 vectors/thread, 64-thread blocks"
    assert [lib.zs_variant_tile(v) for v in (49, 64, 66, 70)] == [2048, 512, 256, 512]


def test_shape_sweep_plans_fit_their_shards(hip_built):
    """Every shard of the tile-depth sweep has W > 1, and every alternative
    it times is a multi-worker variant with a cap the launch accepts."""
    lib = bench._variantlib()
    assert len(bench.SHAPE_GRID) == len(set(bench.SHAPE_GRID))
    for W, n in bench.SHAPE_GRID:
        assert W > 1 and n > 0
        for v, cap, per in bench.shape_plan(W):
            assert lib.zs_variant_multi(v) == 1, (W, v)
            assert 0 <= cap <= 32 and per == 0
    assert bench.shape_plan(8)[0] == (50, 3, 0) and bench.shape_plan(12)[0] == (50, 0, 0)
    assert bench.shape_plan(64)[0] == (51, 0, 0)


def test_stream_bounds_combine_the_phases_at_the_step_bytes():
    """The phased bound is the step's bytes over its reads' time alone plus
    its writes' time alone: W = 1 reads 14 and writes 14 B per parameter, the
    7.5B shard reads 140 and writes 14; workloads the probes do not carry
    (other W, accumulated inputs) get none."""
    c = {k: {"gbps": g} for k, g in [
        ("read_only_w1_streams", 7000.0), ("write_only_w1_streams", 5000.0),
        ("step_mix_w1", 6000.0), ("read_only_w64_streams", 7000.0),
        ("write_only_w64_streams", 3500.0), ("step_mix_w64", 6000.0)]}
    roofs = {"7b-full-w1": {"achieved": 5600.0}, "7p5b-shard-w64": {"achieved": 6300.0},
             "gpt2s-w8": {"achieved": 6000.0}, "1p3b-w4-acc4-fp16": {"achieved": 6000.0}}
    b = bench.stream_bounds(c, roofs)
    assert set(b) == {"7b-full-w1", "7p5b-shard-w64"}
    w1 = b["7b-full-w1"]
    assert w1["phased_gbps"] == pytest.approx(28 / (14 / 7000 + 14 / 5000))
    assert w1["fused_pct_of_phased"] == pytest.approx(100 * 5600 / w1["phased_gbps"])
    assert w1["fused_pct_of_no_arithmetic_mix"] == pytest.approx(100 * 5600 / 6000)
    w64 = b["7p5b-shard-w64"]
    assert w64["phased_gbps"] == pytest.approx(154 / (140 / 7000 + 14 / 3500))
    assert bench.stream_bounds({}, roofs) == {}


def test_wave_probe_plans_fit_the_probe():
    """Every shard the wave probe is asked to stream is whole 1024-element
    groups (its grouped state) and whole tiles, with at most 64 gradient
    streams, 1 or 2 vectors per thread and caps the library accepts."""
    plans = [(w, n, vecs, (cap,)) for _, w, _, _, _, vecs, cap, _, n in bench.PROBES]
    plans += list(bench.PROBE_SWEEP)
    for w, n, vecs, caps in plans:
        assert 0 <= w <= 64 and vecs in (1, 2)
        assert n % 1024 == 0 and n % (256 * vecs) == 0
        assert all(0 <= c <= 32 for c in caps)
    assert bench.WINDOW_W64 == (bench.WINDOW_PERIOD_US, bench.WINDOW_OPEN)
