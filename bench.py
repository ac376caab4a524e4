"""Benchmark of the streaming RVQ codec decoder on one MI355X.

Workload (default): 128 concurrent streams of the Qwen3-TTS-shaped decoder
(16 codebooks x 2048, latent 1024, x1920 upsampling to 24 kHz, bf16 random
weights), streams at staggered positions (0..500 frames already decoded,
prefilled before timing), every step giving each stream a chunk drawn from
{1, 2, 4, 8, 16} frames.  A step is one decode_chunk call over all 128
streams: the whole hot path (batch assembly, gather-sum, projection, conv
decoder, PCM, state save).  Inputs are seeded synthetic codes.

Prints one JSON line: frames/s (and audio-seconds/s) over the timed steps,
the dominant kernel's roofline fraction from per-kernel HIP-event timing,
and the fp64 CPU oracle's rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_F16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
METRIC = "codec frames/s and audio-sec/s at 128 streams; % of MFMA/HBM roofline"


def layer_model(cfg: dict) -> dict:
    """Algorithmic work per launch class: flops and HBM bytes per unit (the
    unit is what the library's profiler counts: input rows of a conv, frames,
    streams), plus bytes per launch (weights)."""
    import rvq_inputs as RI
    es = 2 if cfg["weight_dtype"] == "bf16" else 4
    ch = RI.channels(cfg)
    rate = [1]
    for s in cfg["strides"]:
        rate.append(rate[-1] * s)
    K, dcb, dl = cfg["K"], cfg["d_cb"], cfg["d_lat"]
    m = {}
    m["rvq_gather"] = dict(fpr=K * dcb, bpr=K * dcb * 2 + K * 4 + dcb * es, wpl=0)
    m["proj"] = dict(fpr=2 * dl * dcb, bpr=es * (dcb + dl), wpl=es * dl * dcb)
    m["in_conv"] = dict(fpr=2 * ch[0] * 7 * dl, bpr=es * (dl + ch[0]), wpl=es * ch[0] * 7 * dl)
    for i, s in enumerate(cfg["strides"]):
        ci, co = ch[i], ch[i + 1]
        m[f"s{i}.convT"] = dict(fpr=2 * s * co * 2 * ci, bpr=es * ci + s * co * (4 + es),
                                wpl=es * s * co * 2 * ci)
        for j in range(2):
            m[f"s{i}.ru{j}.conv7"] = dict(fpr=2 * co * 7 * co, bpr=2 * es * co, wpl=es * 7 * co * co)
            out = (4 + es) * co if j == 0 else es * co
            m[f"s{i}.ru{j}.conv1"] = dict(fpr=2 * co * co, bpr=es * co + 4 * co + out,
                                          wpl=es * co * co)
    m["final_conv"] = dict(fpr=2 * 7 * ch[-1], bpr=es * ch[-1] + 4, wpl=0)
    return m


def flops_per_frame(cfg: dict) -> float:
    lm = layer_model(cfg)
    rate = [1]
    for s in cfg["strides"]:
        rate.append(rate[-1] * s)
    tot = lm["proj"]["fpr"] + lm["in_conv"]["fpr"]
    for i in range(len(cfg["strides"])):
        tot += lm[f"s{i}.convT"]["fpr"] * rate[i]
        for j in range(2):
            tot += (lm[f"s{i}.ru{j}.conv7"]["fpr"] + lm[f"s{i}.ru{j}.conv1"]["fpr"]) * rate[i + 1]
    tot += lm["final_conv"]["fpr"] * rate[-1]
    return float(tot)


def cpu_baseline(cfg: dict, weights: dict, budget_s: float) -> dict:
    """The fp64 oracle on a bounded sample of the same workload: 8 streams
    decoding their per-step chunks (drawn from the same buckets), in
    parallel across streams, for about budget_s seconds of CPU time."""
    import oracle
    import rvq_inputs as RI
    m = oracle.Model(cfg, weights)
    nb = 8
    streams = [m.stream() for _ in range(nb)]
    frames = 0
    t0 = time.perf_counter()
    step = 0
    while True:
        n = RI.c4_chunk_sizes(cfg, step)[:nb]
        codes = np.concatenate([RI.stream_codes(cfg, b, int(n[b]), part=1 + step)
                                for b in range(nb)])
        m.decode_batch(streams, n, codes)
        frames += int(n.sum())
        step += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    fr = RI.get_config("c2")["sample_rate"] / RI.hop(cfg)
    return {"value": frames / dt, "unit": "frames/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{nb} streams x {step} steps of bucketed chunks ({frames} frames, "
                      f"{dt:.1f} s), fp64, parallel across streams",
            "audio_sec_per_s": frames / dt / fr}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--config", default="c4")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build decodes on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); streams would shard across GPUs with no collective, "
              "which is not built.", file=sys.stderr)
        return 2

    import torch

    import rvq_inputs as RI
    import streaming_neural_audio_rvq_amd as snr

    cfg = RI.get_config(args.config)
    w = RI.make_weights(cfg)
    codec = snr.Codec(cfg, RI.weight_bits(w))
    hop = codec.hop
    Bn = cfg["n_streams"]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    # ---- setup (untimed): open streams, prefill staggered offsets ----
    off = RI.c4_offsets(cfg)
    ids = [codec.stream_open() for _ in range(Bn)]
    for b in range(Bn):
        if off[b]:
            codec.stream_prefill(ids[b], RI.stream_codes(cfg, b, int(off[b]), part=0), stream)
    # steps: warmup, timed (codes resident in HBM), profiled, host-codes
    total_steps = args.warmup + 3 * args.steps
    sizes = [RI.c4_chunk_sizes(cfg, j) for j in range(total_steps)]
    packed = [np.concatenate([RI.stream_codes(cfg, b, int(sizes[j][b]), part=1 + j)
                              for b in range(Bn)]) for j in range(total_steps)]
    packed_dev = [torch.from_numpy(p).to(dev) for p in packed]
    pcm = torch.empty(cfg["max_frames_per_call"] * hop, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    for j in range(args.warmup):
        codec.decode_chunk_device(ids, sizes[j], packed_dev[j], pcm, stream)
    torch.cuda.synchronize()

    def timed_run(steps, host_codes: bool):
        fr = int(sum(sizes[j].sum() for j in steps))
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for j in steps:
            if host_codes:
                codec.decode_chunk(ids, sizes[j], packed[j], pcm, stream)
            else:
                codec.decode_chunk_device(ids, sizes[j], packed_dev[j], pcm, stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return fr, max(wall, ev0.elapsed_time(ev1) / 1e3)

    # ---- timed region: K steps, codes already resident in HBM ----
    frames, elapsed = timed_run(range(args.warmup, args.warmup + args.steps), False)
    if codec.device_status() != 0:
        raise RuntimeError("out-of-range codes in the benchmark input")
    fps = frames / elapsed
    frame_rate = cfg["sample_rate"] / hop
    # the same step count with host codes (pinned staging + H2D inside the call)
    h_frames, h_elapsed = timed_run(range(args.warmup + 2 * args.steps,
                                          args.warmup + 3 * args.steps), True)

    # ---- per-kernel HIP-event timing: the same number of steps again ----
    roof = None
    kernels = {}
    lm = layer_model(cfg)
    if not args.no_profile:
        codec.profile_enable(True)
        codec.profile_read()
        p_steps = range(args.warmup + args.steps, args.warmup + 2 * args.steps)
        for j in p_steps:
            codec.decode_chunk_device(ids, sizes[j], packed_dev[j], pcm, stream)
        torch.cuda.synchronize()
        prof = codec.profile_read()
        codec.profile_enable(False)
        for name, r in prof.items():
            if r["launches"] == 0:
                continue
            k = dict(ms_total=r["ms"], launches=r["launches"], avg_us=1e3 * r["ms"] / r["launches"],
                     units=r["units"])
            if name in lm:
                mm = lm[name]
                per_launch_units = r["units"] / r["launches"]
                k["bytes_per_launch"] = per_launch_units * mm["bpr"] + mm["wpl"]
                k["flops_per_launch"] = per_launch_units * mm["fpr"]
            kernels[name] = k
        dom = max((n for n in kernels if "bytes_per_launch" in kernels[n]),
                  key=lambda n: kernels[n]["ms_total"])
        d = kernels[dom]
        sec = d["avg_us"] / 1e6
        ai = d["flops_per_launch"] / d["bytes_per_launch"]
        peak_f = PEAK_F16_TFLOPS if cfg["weight_dtype"] == "bf16" else PEAK_F32_TFLOPS
        ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
        if ai < ridge:
            ach = d["bytes_per_launch"] / sec / 1e9
            roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None}
        else:
            ach = d["flops_per_launch"] / sec / 1e12
            roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak_f,
                    "unit": "TFLOP/s", "frac": round(ach / peak_f, 4), "traffic": None}
        roof["kernel"] = dom
        roof["avg_launch_us"] = round(d["avg_us"], 2)
        roof["alg_bytes_per_launch"] = int(d["bytes_per_launch"])
        roof["alg_flops_per_launch"] = int(d["flops_per_launch"])

    fpf = flops_per_frame(cfg)
    peak_f = PEAK_F16_TFLOPS if cfg["weight_dtype"] == "bf16" else PEAK_F32_TFLOPS
    out = {
        "metric": METRIC,
        "value": round(fps, 1),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if cfg["weight_dtype"] == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {Bn} streams at offsets 0..500, chunks from "
                               "{1,2,4,8,16} per stream per step, 16x2048 codebooks, "
                               "hop 1920 @ 24 kHz, bf16 random weights",
                   "streams": Bn, "frames_timed": frames, "mean_frames_per_step": frames / args.steps},
        "audio_sec_per_s": round(fps / frame_rate, 1),
        "host_codes_frames_per_s": round(h_frames / h_elapsed, 1),
        "mfma_util_alg": round(fps * fpf / (peak_f * 1e12), 4),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, w, args.cpu_baseline_seconds)
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 2)
    if kernels:
        out["kernels"] = {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv)
                              for kk, vv in v.items()} for k, v in
                          sorted(kernels.items(), key=lambda kv: -kv[1]["ms_total"])}
    print(json.dumps(out), flush=True)
    codec.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
