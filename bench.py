"""Benchmark of the lockstep tick on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config C1|C2|C3|C4|sweep] [--cpu-seconds S]

A step is one lockstep tick of the whole hot path (column assembly, embedding
gather-sum, 32 temporal layers against the ring KV, text head, 16-step
depformer, greedy decoding) for every slot.  Default workload: the 7B shape,
B = 1, from an empty ring (250 timed ticks unless --steps says otherwise),
synthetic bf16 weights N(0, 0.02) from seed 0 and uniform user codes from
seed 1; the line also carries a B = 32 elastic sub-record (C4: mixed ring
occupancy, slots joining and leaving), timed by a child run of this script
before this process uses the GPU.  Prints one JSON line on stdout; progress
goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
COPY_PROBE_BYTES = 256 << 20   # a plain device copy of known size, for counter calibration


KERNEL_SOURCES = ("kernels.hip", "kernels.h", "device.h")


def kernel_source_hash() -> str:
    """Hash of the sources the timed kernels are built from."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        path = os.path.join(ROOT, "full_duplex_speech_moshi_amd", "csrc", name)
        if os.path.exists(path):
            h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def traffic_file(kernel: str, config: str, B: int) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{kernel}_{config}_b{B}.json")


def measured_traffic(kernel, config, B, algorithmic_bytes):
    """HBM bytes per launch of a timed kernel from its counter summary
    (rocprofv3 FETCH_SIZE / WRITE_SIZE runs, calibrated on the copy probe),
    or None when there is none for this kernel and workload, the kernels
    changed since the counters were taken, or the launch timed here has
    other algorithmic bytes than the one measured."""
    try:
        t = json.load(open(traffic_file(kernel, config, B)))
    except (OSError, ValueError):
        return None
    if t.get("kernel_sources_sha256_16") != kernel_source_hash():
        return None
    if abs(t.get("algorithmic_bytes_per_launch", 0) - algorithmic_bytes) > 1e-3 * algorithmic_bytes:
        return None
    return t.get("bytes_per_launch")


# The kernels bench.py times one launch of, and what each is.  The GEMMs
# cover all their launches (main loop and reduce on the large-batch path).
KERNEL_LABELS = {
    "gate_up": "temporal gate/up GEMM (EPI_GATED), mean of one launch per layer over all 32 layers",
    "qkv": "temporal QKV GEMM (EPI_QKV), mean of one launch per layer over all 32 layers",
    "down": "temporal down-projection GEMM (EPI_RESID), mean of one launch per layer over all 32 layers",
    "out_proj": "temporal out-projection GEMM (EPI_RESID), mean of one launch per layer over all 32 layers",
    "attention": "attn_kernel<128>: ring decode, mean of one launch per layer over all 32 layers",
    "text_head": "text head GEMM (EPI_LOGITS)",
}


def dominant_kernel(kern: dict, n_layers: int) -> str:
    """The timed kernel with the most time per tick: its time per launch
    times its launches per tick (one per temporal layer, one for the text
    head)."""
    per_tick = {k: v["ms"] * (1 if k == "text_head" else n_layers) for k, v in kern.items()}
    return max(per_tick, key=per_tick.get)


def traffic_parts(kernel: str, B: int):
    """The dispatches that make up one launch of a timed kernel at the 7B
    shape: (kernel-name substring, workgroups or None for any).  The temporal
    gate/up runs as one small-batch launch below B = 14 (704 workgroups, one
    per gate/up row-tile pair) and as main loop plus ordered reduce from
    B = 14 on (one 16-column tile up to B = 16, two above; each wave of the
    main loop takes 3 of the 1408 gate and up weight tiles side by side)."""
    if kernel == "gate_up":
        if B < 14:
            return [["gemm_kernel<2, 1, true, 0>", 704]]
        c = 1 if B <= 16 else 2
        return [[f"gemm_wide_res_kernel<2, {c}, 3>", None], [f"gemm_wide_reduce<2, {c}>", None]]
    if kernel == "attention":
        return [["attn_kernel<128>", None]]
    raise ValueError(f"no counter recipe for {kernel}")


def summarize_traffic(run_dir):
    """Write profiles/traffic_<kernel>_<config>_b<B>.json from two rocprofv3
    counter runs of `bench.py --mode traffic` kept under run_dir: pmc_fetch/
    (FETCH_SIZE) and pmc_write/ (WRITE_SIZE), each with its
    *_counter_collection.csv, and traffic_mode.json (the JSON line that mode
    printed).  The counters are scaled by what they read for the copy probe
    (COPY_PROBE_BYTES read and written).  Each part of the launch (main loop,
    reduce) is averaged over its dispatches, and the parts are added."""
    import csv
    import glob
    meta = json.load(open(os.path.join(run_dir, "traffic_mode.json")))
    parts = meta["parts"]

    def counter(sub, name):
        path = glob.glob(os.path.join(run_dir, sub, "*counter_collection.csv"))[0]
        copy, per = [], [[] for _ in parts]
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != name:
                continue
            v = float(r["Counter_Value"])
            if "copyBuffer" in r["Kernel_Name"]:
                copy.append(v)
                continue
            for i, (sub_name, wgs) in enumerate(parts):
                if sub_name in r["Kernel_Name"] and (wgs is None or
                                                     int(r["Grid_Size"]) == wgs * int(r["Workgroup_Size"])):
                    per[i].append(v)
        if not all(per):
            raise SystemExit(f"{sub}: no dispatches of " + ", ".join(p[0] for p, d in zip(parts, per) if not d))
        return max(copy), [sum(d) / len(d) for d in per], [len(d) for d in per]

    f_copy, f_kern, n = counter("pmc_fetch", "FETCH_SIZE")
    w_copy, w_kern, _ = counter("pmc_write", "WRITE_SIZE")
    kib = meta["copy_probe_bytes"] / 1024
    f_scale, w_scale = kib / f_copy, kib / w_copy
    by = 1024 * (sum(f_kern) * f_scale + sum(w_kern) * w_scale)
    out = {
        "kernel": meta["kernel"], "config": meta["config"], "B": meta["B"],
        "parts": [{"name": p[0], "workgroups": p[1], "dispatches": c, "fetch_kib_raw": f, "write_kib_raw": w,
                   "bytes": round(1024 * (f * f_scale + w * w_scale))}
                  for p, c, f, w in zip(parts, n, f_kern, w_kern)],
        "kernel_sources_sha256_16": kernel_source_hash(),
        "bytes_per_launch": round(by),
        "fetch_scale": f_scale, "write_scale": w_scale,
        "copy_probe_bytes": meta["copy_probe_bytes"],
        "algorithmic_bytes_per_launch": meta["algorithmic_bytes_per_launch"],
        "traffic_over_algorithmic": by / meta["algorithmic_bytes_per_launch"],
    }
    json.dump(out, open(traffic_file(meta["kernel"], meta["config"], meta["B"]), "w"), indent=1)
    print(json.dumps(out))


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def weight_stream_bytes(dm) -> int:
    """bf16 matrices streamed once per tick + fp32 norm scales."""
    d, F, Vt, A = dm.d, dm.ffn, dm.text_card, dm.audio_card
    dd, dF, Q = dm.dep_d, dm.dep_ffn, dm.dep_q
    per_layer = 3 * d * d + d * d + 2 * F * d + d * F
    dep_layer = 3 * dd * dd + dd * dd + 2 * dF * dd + dd * dF
    mats = dm.n_layers * per_layer + Vt * d + Q * dd * d + dm.dep_layers * dep_layer + Q * A * dd
    alphas = (2 * dm.n_layers + 1) * d + (2 * dm.dep_layers + 1) * dd
    return 2 * mats + 4 * alphas


def slot_bytes(dm, n_keys: int) -> int:
    """Embedding rows gathered + KV read and written for one slot at n keys."""
    emb = 17 * dm.d * 2 + dm.dep_q * dm.dep_d * 2
    kv = n_keys * dm.n_layers * 2 * dm.d * 2
    return emb + kv


class Workload:
    """Slots, ring occupancy, forced schedules and per-tick user codes of one
    benchmark configuration.  Ring fills share one seeded N(0,1) bf16 fill
    (seed 3): cost depends only on occupancy, not on the values."""

    def __init__(self, name, dm, W, B, K, WU, synth):
        self.name, self.dm, self.W, self.B = name, dm, W, B
        self.fill_n = [0] * B
        self.sched = [None] * B
        self.events = None
        n = WU + K
        if name in ("C0", "C1"):
            self.codes = [synth.user_codes(1 + 1000 * b, n) for b in range(B)]
        elif name == "C2":
            self.fill_n = [W] * B
            self.codes = [synth.alternating_codes(n) for _ in range(B)]
        elif name == "C3":
            self.fill_n = [int(x) for x in synth.batch_occupancy(B, W)]
            self.sched = [synth.session_open(b, text_card=dm.text_card) for b in range(B)]
            self.codes = [synth.user_codes(1000 + b, n) for b in range(B)]
        elif name == "C4":
            sessions, events = synth.elastic_schedule(B, n, W)
            self.sessions, self.events = sessions, events
            for sess in sessions:
                if sess["start_tick"] == 0:
                    self.fill_n[sess["slot"]] = sess["fill_n"]
            self.codes = [np.zeros((n, 8), np.int32) for _ in range(B)]
            for si, sess in enumerate(sessions):
                end = next((t for t in range(sess["start_tick"] + 1, n) if sess["slot"] in events[t]), n)
                c = synth.user_codes(sess["code_seed"], n)
                self.codes[sess["slot"]][sess["start_tick"]:end] = c[:end - sess["start_tick"]]
        elif name in ("sweep", "sweep_empty"):
            self.fill_n = [W if name == "sweep" else 0] * B
            self.codes = [synth.user_codes(1 + 1000 * b, n) for b in range(B)]
        self.fill = None
        need = max(self.fill_n + [s["fill_n"] for s in getattr(self, "sessions", [])] + [0])
        if need:
            self.fill = synth.ring_fill(dm, 3, need)

    def open_slot(self, eng, b, n_fill, sched):
        eng.slot_reset(b)
        if n_fill:
            eng.ring_fill(b, self.fill[0][:, :n_fill], self.fill[1][:, :n_fill])
        if sched is not None:
            eng.prefill_forced(b, sched)

    def setup(self, eng):
        for b in range(self.B):
            self.open_slot(eng, b, self.fill_n[b], self.sched[b])


def workload_label(config, B, W, K, WU):
    """What was timed, from the actual counts."""
    what = {"C0": f"tiny RQ-Transformer tick, ring window {W}",
            "C1": "7B RQ-Transformer tick, empty ring at the start of the warm-up",
            "C2": f"7B RQ-Transformer tick, ring pre-filled to {W} frames",
            "C3": f"7B RQ-Transformer tick, occupancy U[0,{W}], 92-frame session open",
            "C4": "7B RQ-Transformer tick, elastic batch, mixed occupancy, p=0.01 turnover per slot-tick",
            "sweep": "7B RQ-Transformer tick, all rings full",
            "sweep_empty": "7B RQ-Transformer tick, all rings empty"}[config]
    return f"{what}; B={B}, {WU} warm-up ticks, then {K} timed ticks"


def run_sub_c4(args):
    """The B=32 elastic workload (C4) timed by a child run of this script,
    before this process touches the GPU (one engine per process); returns the
    fields of its JSON line that the sub-record carries, or an error note."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--config", "C4", "--steps", str(args.sub_steps),
           "--warmup", "10", "--cpu-ticks", "0", "--kernel-iters", "5", "--no-sub"]
    log("sub-record: " + " ".join(cmd[1:]))
    r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    if r.returncode != 0 or not lines:
        return {"error": f"C4 child exited with {r.returncode}"}
    c = json.loads(lines[-1])
    keys = ("metric", "value", "unit", "steps", "warmup", "ms_per_step", "p50_tick_ms", "p90_tick_ms", "p99_tick_ms",
            "device_tick_ms", "tick_hbm_roofline_frac_p50", "tick_bytes_p50", "roofline", "kernels_gbs", "config")
    return {k: c[k] for k in keys if k in c}


def codec_call_bytes(cd, B: int, n_keys: int) -> int:
    """Bytes one decode call must move at least: every weight once (bf16
    matrices and conv weights, fp32 norms and biases), each slot's 8 codebook
    rows, and each slot's stored keys and values over n_keys frames."""
    d, F, L, H = cd.d, cd.ffn, cd.n_layers, cd.n_heads
    mats = L * (3 * d * d + d * d + 2 * F * d + d * F)
    c = cd.channels
    conv = c[0] * d * cd.conv_k + c[-1] * cd.conv_k
    bias = c[0] + 1
    for i, s in enumerate(cd.strides):
        ci, co = c[i], c[i + 1]
        conv += co * ci * 2 * s + (co // 2) * co * cd.res_k + co * (co // 2)
        bias += co + co // 2 + co
    norms = (2 * L + 1) * d
    per_slot = cd.n_q * d * 2 + L * 2 * n_keys * d * 2
    return 2 * (mats + conv) + 4 * (norms + bias) + B * per_slot


def codec_encode_bytes(cd, B: int, n_keys: int) -> int:
    """Bytes one encode call must move at least: every encoder weight once,
    every codebook once (each quantiser stage scores its whole codebook),
    each slot's samples, and each slot's stored keys and values over n_keys
    frames."""
    d, F, L = cd.d, cd.ffn, cd.n_layers
    mats = L * (3 * d * d + d * d + 2 * F * d + d * F)
    c, n = cd.channels, len(cd.strides)
    conv = c[-1] * cd.conv_k + d * c[0] * cd.conv_k
    bias = c[-1] + d
    for j in range(n):
        ci, co, st = c[n - j], c[n - 1 - j], cd.strides[n - 1 - j]
        conv += (ci // 2) * ci * cd.res_k + ci * (ci // 2) + co * ci * 2 * st
        bias += ci // 2 + ci + co
    norms = (2 * L + 1) * d
    books = cd.n_q * cd.card * d
    per_slot = cd.samples * 4 + L * 2 * n_keys * d * 2
    return 2 * (mats + conv + books) + 4 * (norms + bias) + B * per_slot


def run_codec(args):
    """The codec decoder on its own: B slots (default 32), the window filled
    by warm-up calls, then timed calls of pp_codec_decode (host clock per
    call, device time of the call's graph from pp_codec_time)."""
    import torch
    from full_duplex_speech_moshi_amd import codec, synth
    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    cd = synth.CODEC
    B = args.batch or 32
    K = args.steps or 200
    WU = max(args.warmup, cd.window)
    w = synth.make_codec_weights(cd, seed=0)
    e = codec.CodecEngine(cd, w, B)
    frames = [synth.agent_frames(60 + b, WU + K) for b in range(B)]
    for t in range(WU):
        e.decode(np.stack([frames[b][t] for b in range(B)]))
    torch.cuda.synchronize()
    ms = np.empty(K)
    for t in range(K):
        c = np.stack([frames[b][WU + t] for b in range(B)])
        t0 = time.perf_counter()
        e.decode(c)
        ms[t] = (time.perf_counter() - t0) * 1e3
    dev_ms = e.time(20)
    # the encoder on the same handle: user audio, the window filled likewise
    pcm = [synth.user_audio(90 + b, WU + K, cd.samples) for b in range(B)]
    for t in range(WU):
        e.encode(np.stack([pcm[b][t] for b in range(B)]))
    torch.cuda.synchronize()
    ems = np.empty(K)
    for t in range(K):
        x = np.stack([pcm[b][WU + t] for b in range(B)])
        t0 = time.perf_counter()
        e.encode(x)
        ems[t] = (time.perf_counter() - t0) * 1e3
    enc_dev_ms = e.time_encode(20)
    e.close()
    by = codec_call_bytes(cd, B, cd.window)
    eby = codec_encode_bytes(cd, B, cd.window)
    return {"metric": "decoded frames/sec (codec, 1920 samples per frame)", "value": B * K / (ms.sum() / 1e3),
            "unit": "frames/s", "steps": K, "warmup": WU, "p50_call_ms": float(np.median(ms)),
            "device_call_ms": dev_ms, "call_bytes": by, "call_hbm_frac": by / (dev_ms * 1e-3) / (PEAK_HBM_GBS * 1e9),
            "encode": {"metric": "encoded frames/sec (1920 samples per frame)", "value": B * K / (ems.sum() / 1e3),
                       "unit": "frames/s", "p50_call_ms": float(np.median(ems)), "device_call_ms": enc_dev_ms,
                       "call_bytes": eby, "call_hbm_frac": eby / (enc_dev_ms * 1e-3) / (PEAK_HBM_GBS * 1e9)},
            "config": {"workload": f"codec decoder and encoder (d {cd.d}, {cd.n_layers} layers each, strides "
                                   f"{list(cd.strides)}), B={B}, window of {cd.window} frames filled by {WU} "
                                   f"warm-up calls, then {K} timed calls, each direction", "B": B}}


def run_sub_codec(args):
    """The codec decoder timed by a child run of this script (B = 32)."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--config", "codec", "--batch", "32", "--steps", "200",
           "--no-sub", "--cpu-ticks", "0"]
    log("sub-record: " + " ".join(cmd[1:]))
    r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    if r.returncode != 0 or not lines:
        return {"error": f"codec child exited with {r.returncode}"}
    return json.loads(lines[-1])


def cpu_baseline(args, dm, W, B, weights, wl, sampling):
    """The oracle as it stands, one slot at a time on the host cores, on a
    bounded sample of the workload: C0-C2 tick slot 0; C3 ticks slots 0 and 1
    in turn, C4 its first four sessions in turn (each with its own ring fill
    and schedule).  The oracle runs slots one after another, so B slots take B
    per-slot ticks: its frames/s does not depend on B, and the B-slot tick time
    it implies is labelled as an extrapolation."""
    from oracle.tick import Oracle
    cores = len(os.sched_getaffinity(0))
    if args.config == "C3":
        picks = [(b, wl.fill_n[b], wl.sched[b], wl.codes[b]) for b in range(min(2, B))]
    elif args.config == "C4":
        picks = []
        for sess in wl.sessions[:4]:
            c = wl.codes[sess["slot"]][sess["start_tick"]:]
            picks.append((sess["slot"], sess["fill_n"], None, c))
    else:
        picks = [(0, wl.fill_n[0], wl.sched[0], wl.codes[0])]
    runs = []
    for slot, n_fill, sched, codes in picks:
        o = Oracle(dm, weights, 1, W)
        if sampling:
            o.set_sampling(sampling["text_temperature"], sampling["audio_temperature"], sampling["top_k"],
                           sampling["top_p"], sampling["repetition_penalty"])
            o.slot_seed(0, 1000 + slot)
        if n_fill:  # the same pre-filled ring and session-open schedule as that slot of the workload
            o.ring_fill(0, wl.fill[0][:, :n_fill], wl.fill[1][:, :n_fill])
        if sched is not None:
            o.prefill_forced(0, sched)
        runs.append([o, codes, 0])
    ts = []
    while len(ts) < args.cpu_ticks and sum(ts) < args.cpu_seconds:
        run = runs[len(ts) % len(runs)]
        o, codes, t = run
        a = time.perf_counter()
        o.step(codes[t % len(codes):t % len(codes) + 1])
        ts.append(time.perf_counter() - a)
        run[2] += 1
        if len(ts) <= 3 or len(ts) % 100 == 0:
            log(f"oracle tick {len(ts) - 1}: {ts[-1]:.3f} s")
    log(f"oracle: {len(ts)} ticks in {sum(ts):.1f} s")
    what = ", ".join(f"slot {s} ({'ring fill of %d frames' % n if n else 'empty ring'}"
                     f"{', session-open schedule' if sc is not None else ''})" for s, n, sc, _ in picks)
    out = {"value": len(ts) / sum(ts), "unit": "frames/s", "cores": cores, "kind": "oracle",
           "sample": f"{len(ts)} slot-ticks of {what}, taken in turn, {sum(ts):.1f} s of host time "
                     f"(numpy fp32, BLAS threads = host cores)",
           "p50_slot_tick_s": float(np.median(ts))}
    if B > 1:
        out["extrapolated_tick_s_for_B"] = {"B": B, "tick_s": B * float(np.median(ts)),
                                            "label": "extrapolation: B x the per-slot-tick p50 (slots run one "
                                                     "after another)"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed ticks (default: the config's own count)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="C1", choices=["C0", "C1", "C2", "C3", "C4", "sweep", "sweep_empty", "codec"])
    ap.add_argument("--batch", type=int, default=None, help="slots (default: the config's own B)")
    ap.add_argument("--cpu-ticks", type=int, default=100000,
                    help="at most this many oracle ticks timed on the host (0: skip the CPU baseline)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle ticks are timed until this much host time has been spent (a bounded sample)")
    ap.add_argument("--kernel-iters", type=int, default=30)
    ap.add_argument("--sampling", action="store_true",
                    help="sample the token choices (text temperature 0.7, audio temperature 0.3, top-p 0.9, "
                         "repetition penalty 1.2) instead of greedy")
    ap.add_argument("--mode", default="bench", choices=["bench", "traffic"],
                    help="traffic: one tick, then --traffic-kernel once per layer outside the graph and the "
                         "copy probe, nothing else (for rocprofv3 --pmc runs)")
    ap.add_argument("--traffic-kernel", default="gate_up", choices=["gate_up", "attention"])
    ap.add_argument("--summarize-traffic", metavar="RUN_DIR", default=None,
                    help="no GPU: write profiles/traffic_<kernel>_<config>_b<B>.json from the counter runs of "
                         "--mode traffic under RUN_DIR")
    ap.add_argument("--no-sub", action="store_true",
                    help="default workload only: skip the B=32 elastic sub-record (C4, timed in a child process)")
    ap.add_argument("--sub-steps", type=int, default=100, help="timed ticks of the C4 sub-record")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: there is no multi-GPU path (sessions shard across GPUs "
              "with no exchange; run one process per GPU)", file=sys.stderr)
        sys.exit(2)

    if args.config == "codec":
        print(json.dumps(run_codec(args)), flush=True)
        return
    sub = None
    if args.config == "C1" and args.batch is None and not args.no_sub and args.mode == "bench":
        sub = {"C4": run_sub_c4(args), "codec": run_sub_codec(args)}

    import torch
    from full_duplex_speech_moshi_amd import pp, synth

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda:0")

    tiny = args.config == "C0"
    dm = synth.TINY if tiny else synth.FULL
    W = synth.TINY_WINDOW if tiny else synth.FULL_WINDOW
    B = args.batch or {"C0": 1, "C1": 1, "C2": 1, "C3": 8, "C4": 32, "sweep": 32, "sweep_empty": 32}[args.config]
    K = args.steps or {"C0": 100, "C1": 250, "C2": 500, "C3": 292, "C4": 300, "sweep": 100,
                       "sweep_empty": 100}[args.config]
    WU = args.warmup

    t0 = time.time()
    weights = synth.make_weights(dm, seed=0)
    log(f"weights generated in {time.time() - t0:.1f} s")
    t0 = time.time()
    dw = pp.upload_weights(dm, weights, dev)
    torch.cuda.synchronize()
    log(f"weights uploaded and packed in {time.time() - t0:.1f} s")
    eng = pp.Engine(dm, weights, B, W, device=dev, device_weights=dw)
    log(f"engine created: B={B} W={W} arena {eng.arena.numel() / 2**30:.2f} GiB")
    sampling = dict(text_temperature=0.7, audio_temperature=0.3, top_k=0, top_p=0.9,
                    repetition_penalty=1.2) if args.sampling else None
    if sampling:
        eng.set_sampling(**sampling)
        for b in range(B):
            eng.slot_seed(b, 1000 + b)
    wl = Workload(args.config, dm, W, B, K, WU, synth)

    t0 = time.time()
    wl.setup(eng)
    log(f"slots opened in {time.time() - t0:.1f} s")
    if args.mode == "traffic":
        eng.step(np.stack([wl.codes[b][0] for b in range(B)]))
        ms, by = eng.time_kernel(args.traffic_kernel, 1)
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        eng.close()
        log(f"traffic mode: {args.traffic_kernel} {ms * 1e3:.1f} us per launch, {by / 1e6:.1f} MB algorithmic; "
            f"copy probe {COPY_PROBE_BYTES} B")
        print(json.dumps({"mode": "traffic", "kernel": args.traffic_kernel, "config": args.config, "B": B,
                          "parts": traffic_parts(args.traffic_kernel, B), "us_per_launch": ms * 1e3,
                          "algorithmic_bytes_per_launch": by, "copy_probe_bytes": COPY_PROBE_BYTES}))
        return
    pos = list(wl.fill_n)
    for t in range(WU):
        eng.step(np.stack([wl.codes[b][t] for b in range(B)]))
    wl.setup(eng)
    log(f"warmup {WU} ticks done; timing {K} ticks")

    tick_ms = np.empty(K)
    n_keys = np.empty((K, B), np.int64)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for t in range(K):
        if wl.events is not None:
            for b in wl.events[WU + t] if WU + t > 0 else []:
                sess = next(x for x in wl.sessions if x["slot"] == b and x["start_tick"] == WU + t)
                wl.open_slot(eng, b, sess["fill_n"], None)
                pos[b] = sess["fill_n"]
        c = np.stack([wl.codes[b][WU + t] for b in range(B)])
        a = time.perf_counter()
        eng.step(c)
        tick_ms[t] = (time.perf_counter() - a) * 1e3
        for b in range(B):
            n_keys[t, b] = min(pos[b] + 1, W)
            pos[b] += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log(f"timed {K} ticks in {wall:.3f} s")

    wbytes = weight_stream_bytes(dm)
    tick_bytes = np.array([wbytes + sum(slot_bytes(dm, int(n)) for n in n_keys[t]) for t in range(K)])
    frac = tick_bytes / (tick_ms * 1e-3) / (PEAK_HBM_GBS * 1e9)
    graph_ms = eng.time_graph(20)
    log(f"device tick (graph replay) {graph_ms:.3f} ms")

    # per-kernel timing, one launch per layer with cold weights
    kern = {}
    for name in ("gate_up", "qkv", "down", "out_proj", "attention", "text_head"):
        ms, by = eng.time_kernel(name, args.kernel_iters)
        kern[name] = dict(ms=ms, bytes=by, gbs=by / (ms * 1e-3) / 1e9)
        log(f"kernel {name}: {ms * 1e3:.1f} us, {by / 1e6:.1f} MB, {kern[name]['gbs']:.0f} GB/s")
    eng.close()

    # copy probe: device-to-device copies of COPY_PROBE_BYTES (each reads and
    # writes that many bytes), the reference for HBM counter calibration and
    # the measured copy bandwidth reported beside the 8 TB/s peak
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_copy = 20
    e0.record()
    for _ in range(n_copy):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    copy_gbs = 2 * COPY_PROBE_BYTES * n_copy / (e0.elapsed_time(e1) * 1e-3) / 1e9
    log(f"device copy: {copy_gbs:.0f} GB/s (read + write of {COPY_PROBE_BYTES >> 20} MiB, {n_copy} copies)")

    dom_name = dominant_kernel(kern, dm.n_layers)
    dom = kern[dom_name]
    tick_total_s = float(np.sum(tick_ms)) / 1e3  # host fills of joining sessions (C4) fall between ticks
    result = {
        "metric": "lockstep frames/sec at 7B shape",
        "value": B * K / tick_total_s,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": WU,
        "ms_per_step": tick_total_s / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload_label(args.config, B, W, K, WU),
                   "B": B, "window": W, "config": args.config, "choice": sampling or "greedy"},
        "p50_tick_ms": float(np.median(tick_ms)),
        "p90_tick_ms": float(np.percentile(tick_ms, 90)),
        "p99_tick_ms": float(np.percentile(tick_ms, 99)),
        "device_tick_ms": graph_ms,
        "tick_hbm_roofline_frac_p50": float(np.median(frac)),
        "tick_bytes_p50": float(np.median(tick_bytes)),
        "roofline": {"bound": "hbm", "kernel": KERNEL_LABELS[dom_name],
                     "achieved": dom["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": dom["gbs"] / PEAK_HBM_GBS,
                     "traffic": measured_traffic(dom_name, args.config, B, dom["bytes"])},
        "device_copy_gbs": copy_gbs,
        "kernels_us": {k: round(v["ms"] * 1e3, 2) for k, v in kern.items()},
        "kernels_gbs": {k: round(v["gbs"], 1) for k, v in kern.items()},
    }

    if args.cpu_ticks > 0:
        result["cpu_baseline"] = cpu_baseline(args, dm, W, B, weights, wl, sampling)
    if sub is not None:
        result["sub"] = sub
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
