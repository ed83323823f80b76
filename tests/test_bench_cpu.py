"""bench.py on the host: the algorithmic byte counts its roofline uses, the
one-GPU contract, and the HBM-traffic summary built from rocprofv3 counter
files (synthetic files here; no GPU)."""
import csv
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from full_duplex_speech_moshi_amd import synth  # noqa: E402


def test_weight_bytes_per_tick_match_the_shape_arithmetic():
    # 32 layers of 3d^2 + d^2 + 2Fd + dF bf16, the text head, 16 input
    # projections, 6 depformer layers and 16 heads, plus the fp32 norm scales
    # (65 temporal and 13 depformer rows): 13,772,066,816 bytes at 7B.
    assert bench.weight_stream_bytes(synth.FULL) == 13_772_066_816


@pytest.mark.parametrize("n", [0, 1, 250, 3000])
def test_slot_bytes_are_rows_plus_keys(n):
    # 17 temporal + 16 depformer embedding rows, then K and V of every layer
    # for each of the slot's n keys: 172,032 + 524,288 n bytes at 7B.
    assert bench.slot_bytes(synth.FULL, n) == 172_032 + 524_288 * n


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _counter_csv(path, name, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for kern, grid, val in rows:
            w.writerow({"Kernel_Name": kern, "Grid_Size": grid, "Workgroup_Size": 512, "Counter_Name": name,
                        "Counter_Value": val})


def test_traffic_summary_scales_counters_by_the_copy_probe(tmp_path, monkeypatch):
    # a stand-in repository: the summary hashes the kernel sources and writes
    # profiles/traffic_<kernel>_<config>_b<B>.json under ROOT
    src = tmp_path / "full_duplex_speech_moshi_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "kernels.hip").write_bytes(b"// kernels\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    run = tmp_path / "run"
    copy_kib = bench.COPY_PROBE_BYTES / 1024
    (name, wgs), = bench.traffic_parts("gate_up", 1)
    dom = f"void pp::{name}(pp::GemmArgs)"
    grid = wgs * 512
    # FETCH_SIZE reads half the copy probe's bytes (scale 2), WRITE_SIZE all of them
    _counter_csv(str(run / "pmc_fetch" / "c1_counter_collection.csv"), "FETCH_SIZE",
                 [("__amd_rocclr_copyBuffer", 256 * 512, copy_kib / 2), (dom, grid, 1000.0), (dom, grid, 1002.0),
                  (dom, 3 * 512, 5.0), ("void pp::other(pp::GemmArgs)", grid, 7.0)])
    _counter_csv(str(run / "pmc_write" / "c1_counter_collection.csv"), "WRITE_SIZE",
                 [("__amd_rocclr_copyBuffer", 256 * 512, copy_kib), (dom, grid, 4.0), (dom, grid, 4.0)])
    algo = 2_000_000.0
    (run / "traffic_mode.json").write_text(json.dumps({
        "kernel": "gate_up", "config": "C1", "B": 1, "parts": bench.traffic_parts("gate_up", 1),
        "copy_probe_bytes": bench.COPY_PROBE_BYTES, "algorithmic_bytes_per_launch": algo}))
    bench.summarize_traffic(str(run))
    t = json.load(open(tmp_path / "profiles" / "traffic_gate_up_C1_b1.json"))
    assert t["parts"][0]["dispatches"] == 2  # other kernels and other grid sizes are left out
    assert t["fetch_scale"] == pytest.approx(2.0)
    assert t["write_scale"] == pytest.approx(1.0)
    assert t["bytes_per_launch"] == round(1024 * (1001.0 * 2.0 + 4.0))
    assert t["kernel_sources_sha256_16"] == hashlib.sha256(b"// kernels\n").hexdigest()[:16]
    # reported only for the same kernel sources, kernel, workload and launch shape
    assert bench.measured_traffic("gate_up", "C1", 1, algo) == t["bytes_per_launch"]
    assert bench.measured_traffic("gate_up", "C1", 1, 2 * algo) is None
    assert bench.measured_traffic("gate_up", "C4", 32, algo) is None
    assert bench.measured_traffic("attention", "C1", 1, algo) is None
    (src / "device.h").write_bytes(b"// helpers\n")
    assert bench.measured_traffic("gate_up", "C1", 1, algo) is None


def test_traffic_summary_adds_main_loop_and_reduce(tmp_path, monkeypatch):
    # the large-batch gate/up at B = 32: a main loop and an ordered reduce per
    # launch, each averaged over its own dispatches, then added
    src = tmp_path / "full_duplex_speech_moshi_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "kernels.hip").write_bytes(b"// kernels\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    parts = bench.traffic_parts("gate_up", 32)
    assert [p[0] for p in parts] == ["gemm_wide_res_kernel<2, 2, 3>", "gemm_wide_reduce<2, 2>"]
    assert [p[0] for p in bench.traffic_parts("gate_up", 16)] == ["gemm_wide_res_kernel<2, 1, 3>",
                                                                   "gemm_wide_reduce<2, 1>"]
    run = tmp_path / "run"
    copy_kib = bench.COPY_PROBE_BYTES / 1024
    main, red = "void pp::gemm_wide_res_kernel<2, 2, 3>(pp::GemmArgs)", "void pp::gemm_wide_reduce<2, 2>(pp::GemmArgs)"
    _counter_csv(str(run / "pmc_fetch" / "b32_counter_collection.csv"), "FETCH_SIZE",
                 [("__amd_rocclr_copyBuffer", 256 * 512, copy_kib / 2), (main, 472 * 512, 100.0),
                  (main, 472 * 512, 110.0), (red, 704 * 512, 20.0)])
    _counter_csv(str(run / "pmc_write" / "b32_counter_collection.csv"), "WRITE_SIZE",
                 [("__amd_rocclr_copyBuffer", 256 * 512, copy_kib), (main, 472 * 512, 30.0),
                  (red, 704 * 512, 6.0), (red, 704 * 512, 8.0)])
    (run / "traffic_mode.json").write_text(json.dumps({
        "kernel": "gate_up", "config": "sweep", "B": 32, "parts": parts,
        "copy_probe_bytes": bench.COPY_PROBE_BYTES, "algorithmic_bytes_per_launch": 500_000.0}))
    bench.summarize_traffic(str(run))
    t = json.load(open(tmp_path / "profiles" / "traffic_gate_up_sweep_b32.json"))
    assert [p["dispatches"] for p in t["parts"]] == [2, 1]
    assert t["parts"][0]["bytes"] == round(1024 * (105.0 * 2 + 30.0))
    assert t["parts"][1]["bytes"] == round(1024 * (20.0 * 2 + 7.0))
    assert t["bytes_per_launch"] == round(1024 * ((105.0 + 20.0) * 2 + 30.0 + 7.0))
    assert t["traffic_over_algorithmic"] == pytest.approx(t["bytes_per_launch"] / 500_000.0, rel=1e-6)


def test_dominant_kernel_is_the_largest_per_tick():
    # B = 1 from an empty ring: the gate/up GEMM (30 us x 32 layers) beats a
    # 45 us text head launched once and a 6 us decode per layer
    kern = {"gate_up": {"ms": 0.030}, "qkv": {"ms": 0.019}, "down": {"ms": 0.018}, "out_proj": {"ms": 0.0085},
            "attention": {"ms": 0.006}, "text_head": {"ms": 0.045}}
    assert bench.dominant_kernel(kern, 32) == "gate_up"
    # every ring full at B = 32: the decode (255 us per layer) dominates
    kern["attention"]["ms"] = 0.255
    kern["gate_up"]["ms"] = 0.044
    assert bench.dominant_kernel(kern, 32) == "attention"
    # a one-layer model: the text head's single launch can win
    assert bench.dominant_kernel({"gate_up": {"ms": 0.03}, "text_head": {"ms": 0.045}}, 1) == "text_head"
    assert set(bench.KERNEL_LABELS) >= set(kern)


def test_codec_call_bytes_are_the_weights_rows_and_caches():
    # every weight of the manifest once (codebooks excepted: one row per
    # codebook per slot), plus each slot's keys and values over the window
    w = synth.make_codec_weights(synth.CODEC_TINY, seed=0)
    cd = synth.CODEC_TINY
    weights = sum(v.nbytes for k, v in w.items() if not k.startswith(("codebook.", "enc.")))  # the decoder's
    for B, n in ((1, 1), (3, cd.window)):
        rows = B * cd.n_q * cd.d * 2
        cache = B * cd.n_layers * 2 * n * cd.d * 2
        assert bench.codec_call_bytes(cd, B, n) == weights + rows + cache


def test_codec_encode_bytes_are_the_encoder_weights_codebooks_samples_and_caches():
    # every encoder weight and every codebook once, plus each slot's samples
    # and its keys and values over the window
    w = synth.make_codec_weights(synth.CODEC_TINY, seed=0)
    cd = synth.CODEC_TINY
    weights = sum(v.nbytes for k, v in w.items() if k.startswith(("codebook.", "enc.")))
    for B, n in ((1, 1), (3, cd.window)):
        pcm = B * cd.samples * 4
        cache = B * cd.n_layers * 2 * n * cd.d * 2
        assert bench.codec_encode_bytes(cd, B, n) == weights + pcm + cache
