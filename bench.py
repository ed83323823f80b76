"""Benchmark of the lockstep tick on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config C1|C2|C3|C4|sweep] [--cpu-ticks N]

A step is one lockstep tick of the whole hot path (column assembly, embedding
gather-sum, 32 temporal layers against the ring KV, text head, 16-step
depformer, greedy decoding) for every slot.  Default workload: the 7B shape,
B = 1, 250 ticks from an empty ring, synthetic bf16 weights N(0, 0.02) from
seed 0 and uniform user codes from seed 1.  Prints one JSON line on stdout;
progress goes to stderr.
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=250)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="C1", choices=["C0", "C1", "C2", "sweep"])
    ap.add_argument("--batch", type=int, default=1, help="slots (sweep / C2 only)")
    ap.add_argument("--cpu-ticks", type=int, default=2, help="oracle ticks timed on the host (0: skip)")
    ap.add_argument("--kernel-iters", type=int, default=30)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (sessions shard across GPUs "
              "with no exchange; run one process per GPU)", file=sys.stderr)
        sys.exit(2)

    import torch
    from full_duplex_speech_moshi_amd import pp, synth

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda:0")

    tiny = args.config == "C0"
    dm = synth.TINY if tiny else synth.FULL
    W = synth.TINY_WINDOW if tiny else synth.FULL_WINDOW
    B = 1 if args.config in ("C0", "C1") else args.batch
    K, WU = args.steps, args.warmup

    t0 = time.time()
    weights = synth.make_weights(dm, seed=0)
    log(f"weights generated in {time.time() - t0:.1f} s")
    t0 = time.time()
    dw = pp.upload_weights(dm, weights, dev)
    torch.cuda.synchronize()
    log(f"weights uploaded in {time.time() - t0:.1f} s")
    eng = pp.Engine(dm, weights, B, W, device=dev, device_weights=dw)
    log(f"engine created: B={B} W={W} arena {eng.arena.numel() / 2**30:.2f} GiB")

    fill_n = [0] * B
    if args.config in ("C2", "sweep") and not tiny:
        fill_n = [W] * B

    def setup():
        for b in range(B):
            eng.slot_reset(b)
            if fill_n[b]:
                kb, vb = synth.ring_fill(dm, 3 + 1000 * b, fill_n[b])
                eng.ring_fill(b, kb, vb)

    codes = [synth.user_codes(1 if b == 0 else 1000 + b, WU + K) if args.config != "C2"
             else synth.alternating_codes(WU + K) for b in range(B)]

    setup()
    for t in range(WU):
        eng.step(np.stack([codes[b][t] for b in range(B)]))
    setup()
    log(f"warmup {WU} ticks done; timing {K} ticks")

    tick_ms = np.empty(K)
    n_keys = np.empty((K, B), np.int64)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for t in range(K):
        c = np.stack([codes[b][WU + t] for b in range(B)])
        a = time.perf_counter()
        eng.step(c)
        tick_ms[t] = (time.perf_counter() - a) * 1e3
        for b in range(B):
            n_keys[t, b] = min(fill_n[b] + t + 1, W)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log(f"timed {K} ticks in {wall:.3f} s")

    wbytes = weight_stream_bytes(dm)
    tick_bytes = np.array([wbytes + sum(slot_bytes(dm, int(n)) for n in n_keys[t]) for t in range(K)])
    frac = tick_bytes / (tick_ms * 1e-3) / (PEAK_HBM_GBS * 1e9)
    graph_ms = eng.time_graph(20)
    log(f"device tick (graph replay) {graph_ms:.3f} ms")

    # dominant kernel: the temporal gate/up projection (largest per-layer weight)
    kern = {}
    for name in ("gate_up", "qkv", "down", "out_proj", "attention", "text_head"):
        ms, by = eng.time_kernel(name, args.kernel_iters)
        kern[name] = dict(ms=ms, bytes=by, gbs=by / (ms * 1e-3) / 1e9)
        log(f"kernel {name}: {ms * 1e3:.1f} us, {by / 1e6:.1f} MB, {kern[name]['gbs']:.0f} GB/s")
    eng.close()

    dom = kern["gate_up"]
    result = {
        "metric": "lockstep frames/sec at 7B shape",
        "value": B * K / wall,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": WU,
        "ms_per_step": wall / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": {"C0": "tiny RQ-Transformer tick, B=1, ring window 32",
                                "C1": "7B RQ-Transformer tick, B=1, empty ring, 250 ticks",
                                "C2": "7B RQ-Transformer tick, ring pre-filled to 3000 frames",
                                "sweep": "7B RQ-Transformer tick, all rings full"}[args.config],
                   "B": B, "window": W, "config": args.config},
        "p50_tick_ms": float(np.median(tick_ms)),
        "p90_tick_ms": float(np.percentile(tick_ms, 90)),
        "p99_tick_ms": float(np.percentile(tick_ms, 99)),
        "device_tick_ms": graph_ms,
        "tick_hbm_roofline_frac_p50": float(np.median(frac)),
        "tick_bytes_p50": float(np.median(tick_bytes)),
        "roofline": {"bound": "hbm", "kernel": "gemm_kernel<EPI_GATED> (temporal gate/up, layer 0)",
                     "achieved": dom["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": dom["gbs"] / PEAK_HBM_GBS, "traffic": None},
        "kernels_us": {k: round(v["ms"] * 1e3, 2) for k, v in kern.items()},
        "kernels_gbs": {k: round(v["gbs"], 1) for k, v in kern.items()},
    }

    if args.cpu_ticks > 0:
        from oracle.tick import Oracle
        cores = len(os.sched_getaffinity(0))
        o = Oracle(dm, weights, 1, W)
        c0 = codes[0]
        ts = []
        for t in range(args.cpu_ticks):
            a = time.perf_counter()
            o.step(c0[t:t + 1])
            ts.append(time.perf_counter() - a)
            log(f"oracle tick {t}: {ts[-1]:.2f} s")
        result["cpu_baseline"] = {"value": len(ts) / sum(ts), "unit": "frames/s", "cores": cores,
                                  "kind": "oracle",
                                  "sample": f"{len(ts)} ticks of one slot from an empty ring "
                                            f"(numpy fp32, BLAS threads = host cores)"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
