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
import gc
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
    # the input conv reads the latent, or (projection folded into it, decoders
    # without a transformer) [z, 1, 0...] padded to a multiple of the K stage
    # (64 deep for fp16, 16 for fp32)
    gran = 64 if es == 2 else 16
    d_in = dl if cfg["tf_layers"] else (dcb + 1 + gran - 1) // gran * gran
    m["in_conv"] = dict(fpr=2 * ch[0] * 7 * dl, bpr=es * (d_in + ch[0]),
                        wpl=es * ch[0] * 7 * d_in)
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
    # a residual unit in one launch: the k = 7 conv's input, the residual in,
    # its outputs (as the separate 1x1 conv writes them)
    for i in range(len(cfg["strides"])):
        co = ch[i + 1]
        for j in range(2):
            c7, c1 = m[f"s{i}.ru{j}.conv7"], m[f"s{i}.ru{j}.conv1"]
            out = (4 + es) * co if j == 0 else es * co
            m[f"s{i}.ru{j}"] = dict(fpr=c7["fpr"] + c1["fpr"], bpr=es * co + 4 * co + out,
                                    wpl=c7["wpl"] + c1["wpl"])
    # a fused stage counts its output rows: the ConvT's input row is shared by
    # s output rows; only the stage input and output cross HBM (the last
    # stage writes PCM instead of the next stage's operand)
    S = len(cfg["strides"])
    for i, s in enumerate(cfg["strides"]):
        ci, co = ch[i], ch[i + 1]
        t = m[f"s{i}.convT"]
        fpr = t["fpr"] / s + sum(m[f"s{i}.ru{j}.conv7"]["fpr"] + m[f"s{i}.ru{j}.conv1"]["fpr"]
                                 for j in range(2))
        wpl = t["wpl"] + sum(m[f"s{i}.ru{j}.conv7"]["wpl"] + m[f"s{i}.ru{j}.conv1"]["wpl"]
                             for j in range(2))
        if i == S - 1:
            fpr += m["final_conv"]["fpr"]
            bpr = es * ci / s + 4
            # the last fused stage also saves every per-layer halo of the step
            # (read from the layers' buffers, written to the slots): the input
            # conv's, each stage input's, and the residual-unit inputs of the
            # stages without a fused kernel (widths above 64 channels)
            fused = [es == 2 and cfg["act"] == "snake" and ch[k + 1] <= 64 for k in range(S)]
            per_stream = 6 * d_in + sum(ch[:S]) + sum(24 * ch[k + 1] for k in range(S)
                                                       if not fused[k])
            wpl += 2 * es * per_stream * cfg["n_streams"]
        else:
            bpr = es * ci / s + es * co
        m[f"s{i}.fused"] = dict(fpr=fpr, bpr=bpr, wpl=wpl)
    return m


# Vector ALU of the part: 256 CUs x 4 SIMDs, a wave64 instruction every 4
# cycles per SIMD (16 lanes per cycle) at 2.4 GHz, i.e. 39.3 T lane-operations
# per second (the published 157.3 TFLOP/s fp32 counts an FMA as two and packed
# instructions twice); transcendentals (the hardware sine) at a quarter of it.
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
# vector-ALU lane-operation slots of one Snake (multiply, range reduction,
# sine, square, fused multiply-add), measured: 24.8-26 cycles per 64-lane
# wave on one SIMD (bench.py --ceilings: four full-rate instructions and the
# sine at about half rate), i.e. 6.2 slots of 16 lanes per cycle
SNAKE_SLOTS = 6.2


def vector_floor(cfg: dict, cls: str, units: float, flops: float, peak_tflops: float,
                 sec: float) -> dict:
    """The vector-ALU work a fused stage cannot avoid beside its MFMAs: five
    activations per output row and channel (the two residual units' input and
    inner activations, and the stage output's), each a Snake at its measured
    cost (SNAKE_SLOTS lane-operation slots) plus half a conversion
    instruction (two values packed to fp16 per instruction).  The floor is
    that work at the full vector rate; MFMA work at the published peak beside
    it; the two overlapped at best, serial at worst."""
    import rvq_inputs as RI
    ch = RI.channels(cfg)
    i = int(cls[1:cls.index(".")])
    snakes = units * 5 * ch[i + 1]
    slots = snakes * (SNAKE_SLOTS + 0.5) if cfg["act"] == "snake" else snakes * 2.5
    valu_us = slots / VALU_LANE_OPS * 1e6
    mfma_us = flops / (peak_tflops * 1e12) * 1e6
    return {"activations_per_launch": int(snakes), "lane_op_slots_per_launch": int(slots),
            "valu_floor_us": round(valu_us, 1), "mfma_floor_us": round(mfma_us, 1),
            "serial_floor_us": round(valu_us + mfma_us, 1), "measured_us": round(sec * 1e6, 1),
            "frac_of_serial_floor": round((valu_us + mfma_us) / (sec * 1e6), 3)}


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
    if cfg["tf_layers"]:
        # windowed transformer per frame: in/out projections, per layer the
        # QKV, output and MLP projections and the attention products over
        # its window of keys (the full window: the steady state)
        dm = cfg["tf_heads"] * cfg["tf_head_dim"]
        dl = cfg["d_lat"]
        per_layer = 2 * dm * (3 * dm + dm + 2 * cfg["tf_mlp"]) + \
            2 * 2 * cfg["tf_window"] * dm
        tot += 2 * 2 * dl * dm + cfg["tf_layers"] * per_layer
    return float(tot)


WORKLOADS = {
    "c2": "8 streams in lockstep, 8 new frames each per step (F = 64), 16x2048 codebooks, "
          "hop 1920 @ 24 kHz, bf16 random weights",
    "c3": "64 streams in lockstep, 8 new frames each per step (F = 512), 10x1024 codebooks, "
          "4-layer windowed transformer, hop 2048 @ 44.1 kHz, bf16 random weights",
    "c4": "128 streams at offsets 0..500, chunks from {1,2,4,8,16} per stream per step, "
          "16x2048 codebooks, hop 1920 @ 24 kHz, bf16 random weights",
    "c5": "offline: 128 whole utterances of 50..500 frames (valid frames only, no padding), "
          "calls grouping whole utterances up to 16,000 frames, fresh streams; "
          "a step decodes all 128",
}


LEFT_CONTEXT_FRAMES = 16  # stateless re-decode: left frames decoded again with every chunk


def group_calls(n, codes_of, max_frames):
    """Whole streams into calls of at most max_frames frames: lists of
    (stream indices, frames per stream)."""
    out, b0, B = [], 0, len(n)
    while b0 < B:
        b1, tot = b0, 0
        while b1 < B and tot + int(n[b1]) <= max_frames:
            tot += int(n[b1])
            b1 += 1
        out.append(list(range(b0, b1)))
        b0 = b1
    return out


def make_workload(name: str, cfg: dict, codec, total_steps: int, stream,
                  stateless: bool = False) -> dict:
    """Per step, the decode calls (stream ids or None for fresh streams, frames
    per stream, host codes, the same codes in HBM) and the new frames the step
    delivers; streams opened and prefilled here, untimed.  stateless: every
    chunk is decoded again from zero state together with up to 16 earlier
    frames of its stream (fresh streams each call)."""
    import torch
    import rvq_inputs as RI
    dev = torch.device("cuda:0")
    Bn = cfg["n_streams"]

    def call(ids, n, codes):
        n = np.asarray(n, np.int32)
        return (ids, n, codes, torch.from_numpy(codes).to(dev))

    steps = []
    new_frames = []
    if stateless:
        if name not in ("c2", "c4"):
            raise SystemExit("bench.py: the stateless re-decode runs on the c2 and c4 workloads")
        off = RI.c4_offsets(cfg) if name == "c4" else np.zeros(Bn, np.int32)
        hist = [RI.stream_codes(cfg, b, int(off[b]), part=0) for b in range(Bn)]
        for j in range(total_steps):
            n = RI.c4_chunk_sizes(cfg, j) if name == "c4" else np.full(Bn, 8, np.int32)
            new = [RI.stream_codes(cfg, b, int(n[b]), part=1 + j) for b in range(Bn)]
            win = []
            for b in range(Bn):
                left = hist[b][max(0, len(hist[b]) - LEFT_CONTEXT_FRAMES):]
                win.append(np.concatenate([left, new[b]]))
                hist[b] = np.concatenate([hist[b], new[b]])
            wn = np.array([w.shape[0] for w in win], np.int32)
            calls = []
            for grp in group_calls(wn, None, cfg["max_frames_per_call"]):
                calls.append(call(None, wn[grp], np.concatenate([win[b] for b in grp])))
            steps.append(calls)
            new_frames.append(int(n.sum()))
        return {"steps": steps, "new_frames": new_frames, "streams": Bn,
                "desc": f"{name}: {WORKLOADS[name]}; stateless re-decode with "
                        f"{LEFT_CONTEXT_FRAMES} left frames, fresh streams every call"}
    if name == "c4":
        off = RI.c4_offsets(cfg)
        ids = [codec.stream_open() for _ in range(Bn)]
        for b in range(Bn):
            if off[b]:
                codec.stream_prefill(ids[b], RI.stream_codes(cfg, b, int(off[b]), part=0), stream)
        for j in range(total_steps):
            n = RI.c4_chunk_sizes(cfg, j)
            codes = np.concatenate([RI.stream_codes(cfg, b, int(n[b]), part=1 + j)
                                    for b in range(Bn)])
            steps.append([call(ids, n, codes)])
    elif name in ("c2", "c3"):
        ids = [codec.stream_open() for _ in range(Bn)]
        for j in range(total_steps):
            codes = np.concatenate([RI.stream_codes(cfg, b, 8, part=1 + j) for b in range(Bn)])
            steps.append([call(ids, [8] * Bn, codes)])
    elif name == "c5":
        lens = RI.c5_lengths(cfg)
        calls = []
        for grp in group_calls(lens, None, cfg["max_frames_per_call"]):
            codes = np.concatenate([RI.stream_codes(cfg, b, int(lens[b]), part=0) for b in grp])
            calls.append(call(None, lens[grp], codes))
        steps = [calls] * total_steps
    else:
        raise SystemExit(f"bench.py: no workload for config {name!r}")
    return {"steps": steps, "desc": f"{name}: {WORKLOADS[name]}", "streams": Bn}


def blas_reference(torch, cfg: dict, F: int, reps: int = 20) -> dict:
    """The decoder's contractions at F frames per step as plain dense fp16
    GEMMs on the vendor library (torch.mm -> hipBLASLt): no implicit im2col, no
    activation, no residual, no streaming state -- a calibration of what a
    tuned library reaches on these shapes, per launch class of this library
    (a class's GEMMs summed), plus one 8192^3 GEMM."""
    import rvq_inputs as RI
    ch = RI.channels(cfg)
    r = [1]
    for st in cfg["strides"]:
        r.append(r[-1] * st)
    dcb, dl = cfg["d_cb"], cfg["d_lat"]
    d_in = dl if cfg["tf_layers"] else (dcb + 1 + 63) // 64 * 64
    S = len(cfg["strides"])
    shapes = {"in_conv": [(F, ch[0], 7 * d_in)]}
    for i, s in enumerate(cfg["strides"]):
        ci, co = ch[i], ch[i + 1]
        convT = (F * r[i], s * co, 2 * ci)
        conv7 = (F * r[i + 1], co, 7 * co)
        conv1 = (F * r[i + 1], co, co)
        shapes[f"s{i}.convT"] = [convT]
        shapes[f"s{i}.fused"] = [convT, conv7, conv1, conv7, conv1] + (
            [(F * r[S], 1, 7 * co)] if i == S - 1 else [])
        for j in range(2):
            shapes[f"s{i}.ru{j}"] = [conv7, conv1]
            shapes[f"s{i}.ru{j}.conv7"] = [conv7]
            shapes[f"s{i}.ru{j}.conv1"] = [conv1]
    # the classes this library launches for the decoder, in launch order
    classes = {c: shapes[c] for c in launch_sequence(cfg) if c in shapes}
    classes["square 8192"] = [(8192, 8192, 8192)]
    timed = {}
    out = {}
    for cls, gemms in classes.items():
        us = flop = 0.0
        for (M, N, K) in gemms:
            key = (M, N, K)
            if key not in timed:
                a = torch.randn(M, K, dtype=torch.float16, device="cuda:0")
                b = torch.randn(N, K, dtype=torch.float16, device="cuda:0")
                for _ in range(3):
                    torch.mm(a, b.t())
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record()
                for _ in range(reps):
                    torch.mm(a, b.t())
                e1.record()
                torch.cuda.synchronize()
                timed[key] = 1e3 * e0.elapsed_time(e1) / reps
                del a, b
            us += timed[key]
            flop += 2.0 * M * N * K
        out[cls] = {"gemms": [list(g) for g in gemms], "blas_us": round(us, 2),
                    "tflops": round(flop / us / 1e6, 1),
                    "frac": round(flop / us / 1e6 / PEAK_F16_TFLOPS, 4)}
    return out


# (config, timed steps, warm-up steps) of the short runs beside the headline
OTHER_RUNS = (("c2", 32, 4), ("c3", 16, 2), ("c5", 3, 1))


def other_workloads() -> dict:
    """Short runs of the other workloads (child processes of this script, one
    at a time, each under its own time limit): frames/s, audio-s/s and ms per
    step of each, or the reason it has none."""
    import subprocess
    res = {}
    for name, steps, warmup in OTHER_RUNS:
        cmd = [sys.executable, os.path.abspath(__file__), "--config", name, "--steps",
               str(steps), "--warmup", str(warmup), "--no-cpu-baseline", "--no-profile",
               "--no-other-configs"]
        print(f"bench.py: {name} ({steps} steps)", file=sys.stderr, flush=True)
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        except subprocess.TimeoutExpired:
            res[name] = {"error": "time limit"}
            continue
        lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
        if r.returncode != 0 or not lines:
            res[name] = {"error": f"exit {r.returncode}", "stderr": r.stderr[-300:]}
            continue
        rec = json.loads(lines[-1])
        res[name] = {k: rec[k] for k in ("value", "unit", "ms_per_step", "audio_sec_per_s")
                     if k in rec}
        res[name]["workload"] = rec["config"]["workload"]
        res[name]["steps"] = steps
    return res


def write_blas_summary(path: str, out: dict, F: int) -> None:
    """Appends the vendor-GEMM calibration of a run to a text summary: per
    launch class, the library's own average (HIP events in the same run) and
    the plain GEMMs of the same shapes on torch.mm."""
    lines = [f"Run: {out['value']} frames/s, {out['ms_per_step']} ms per step; the plain GEMMs at "
             f"F = {F} frames (the run's mean per step).\n",
             "| class | GEMMs (M, N, K) | vendor GEMM us | TFLOP/s | of 2.5 PFLOP/s | "
             "this library us |", "|---|---|---:|---:|---:|---:|"]
    for cls, v in out["blas_reference"].items():
        g = "; ".join("x".join(str(d) for d in gm) for gm in v["gemms"])
        lib = f"{v['library_us']:.1f}" if "library_us" in v else "-"
        lines.append(f"| {cls} | {g} | {v['blas_us']:.1f} | {v['tflops']:.0f} | {v['frac']:.3f} | "
                     f"{lib} |")
    with open(path, "a") as fh:
        fh.write("\n".join(lines) + "\n")


def cpu_baseline(name: str, cfg: dict, weights: dict, budget_s: float) -> dict:
    """The fp64 oracle on a bounded sample of the same workload, for about
    budget_s seconds, parallel across streams: 8 streams decoding per-step
    chunks drawn like the workload's (streamed workloads), or whole
    utterances one after another (offline workload)."""
    import oracle
    import rvq_inputs as RI
    m = oracle.Model(cfg, weights)
    frames = 0
    t0 = time.perf_counter()
    step = 0
    if name == "c5":
        lens = RI.c5_lengths(cfg)
        while True:
            b = step % len(lens)
            m.stream().decode(RI.stream_codes(cfg, b, int(lens[b]), part=0))
            frames += int(lens[b])
            step += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        sample = f"{step} whole utterances ({frames} frames)"
    else:
        nb = 8
        streams = [m.stream() for _ in range(nb)]
        while True:
            n = (RI.c4_chunk_sizes(cfg, step)[:nb] if name == "c4"
                 else np.full(nb, 8, np.int32))
            codes = np.concatenate([RI.stream_codes(cfg, b, int(n[b]), part=1 + step)
                                    for b in range(nb)])
            m.decode_batch(streams, n, codes)
            frames += int(n.sum())
            step += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        sample = f"{nb} streams x {step} steps of the workload's chunks ({frames} frames)"
    dt = time.perf_counter() - t0
    fr = cfg["sample_rate"] / RI.hop(cfg)
    cpu = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                cpu = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": frames / dt, "unit": "frames/s", "cores": oracle.num_threads(),
            "cpu_model": cpu, "host_cpus": os.cpu_count(), "kind": "oracle",
            "sample": f"{sample}, {dt:.1f} s, fp64, parallel across streams and channels",
            "audio_sec_per_s": frames / dt / fr}


def graph_latency(torch, codec, cfg, stream, reps: int = 50) -> dict:
    """Latency of one-stream steps (1 and 8 new frames), each waited for:
    eager decode_chunk against decode_chunk_graph; medians in microseconds."""
    import rvq_inputs as RI
    out = {}
    for n in (1, 8):
        pcm = torch.empty(n * codec.hop, dtype=torch.float32, device="cuda:0")
        res = {}
        for mode in ("eager", "graph"):
            sid = codec.stream_open()
            fn = codec.decode_chunk_graph if mode == "graph" else codec.decode_chunk
            ts = []
            for r in range(reps + 5):
                codes = RI.stream_codes(cfg, 0, n, part=1000 + r)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                fn([sid], [n], codes, pcm, stream)
                torch.cuda.synchronize()
                if r >= 5:
                    ts.append(time.perf_counter() - t0)
            codec.stream_close(sid)
            res[mode] = round(1e6 * float(np.median(ts)), 1)
        out[f"{n}_frame_step_us"] = res
    return out


def cu_masked_stream(torch, lo: int, hi: int):
    """A stream (default priority) whose kernels run on CUs [lo, hi) only."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    words = (n_cu + 31) // 32
    mask = (ctypes.c_uint32 * words)()
    for cu in range(lo, hi):
        mask[cu // 32] |= 1 << (cu % 32)
    handle = ctypes.c_void_p()
    rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(handle), ctypes.c_uint32(words), mask)
    if rc != 0:
        raise RuntimeError(f"hipExtStreamCreateWithCUMask failed ({rc})")
    return torch.cuda.ExternalStream(handle.value)


def cotenant_run(args, torch, timed_run, timed_frames, dec_stream, steps, solo_fps) -> dict:
    """The same decode steps beside a synthetic stage-0 stand-in: back-to-back
    bf16 8192^3 GEMMs on a second stream, enqueued to outlast the decode.
    Decode frames/s alone and beside the load, and the slowdown."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    a = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda:0")
    b = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda:0")
    if args.cotenant == "masked":
        k = max(1, min(n_cu - 1, int(round(n_cu * args.cu_fraction))))
        dec = cu_masked_stream(torch, 0, k)
        load = cu_masked_stream(torch, k, n_cu)
        alone = timed_run(steps, False, dec)
        solo = alone[0] / alone[1]
    else:
        k = n_cu
        dec = torch.cuda.Stream()
        load = torch.cuda.Stream()
        alone = timed_run(steps, False, dec)
        solo = alone[0] / alone[1]
    # time one GEMM on the load stream, then enqueue enough for 6x the decode time
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(load):
        torch.matmul(a, b)
        e0.record(load)
        torch.matmul(a, b)
        e1.record(load)
    torch.cuda.synchronize()
    gemm_ms = e0.elapsed_time(e1)
    # decode time alone, from the frames of these steps at the solo rate
    decode_ms = 1e3 * timed_frames(steps) / max(1.0, solo)
    n_gemm = 0
    started = torch.cuda.Event()
    with torch.cuda.stream(load):
        le0 = torch.cuda.Event(enable_timing=True)
        le0.record(load)
        while n_gemm * gemm_ms < 6 * decode_ms + 2 * gemm_ms:
            torch.matmul(a, b)
            n_gemm += 1
            if n_gemm == 2:
                started.record(load)
    le1 = torch.cuda.Event(enable_timing=True)
    le1.record(load)
    # the decode starts once the load runs (two GEMMs done), so that the two
    # overlap whatever order the queues are served in
    dec.wait_event(started)
    fr, el = timed_run(steps, False, dec, alone=False)
    torch.cuda.synchronize()
    load_tflops = n_gemm * 2 * 8192 ** 3 / (le0.elapsed_time(le1) / 1e3) / 1e12
    co = fr / el
    return {"mode": args.cotenant, "decode_cus": k, "load": "bf16 GEMM 8192^3 back to back",
            "gemm_ms_alone": round(gemm_ms, 3), "gemms": n_gemm,
            "load_tflops": round(load_tflops, 1),
            "decode_frames_per_s_alone": round(solo, 1),
            "decode_frames_per_s_beside_load": round(co, 1),
            "decode_slowdown": round(solo / co - 1.0, 4)}


def step_indices(warmup: int, steps: int, profiled: bool) -> list:
    """Chunk-schedule indices of the decode steps a run dispatches, in order:
    warmup, timed (codes in HBM), profiled (unless skipped), host codes."""
    idx = list(range(warmup + steps))
    if profiled:
        idx += list(range(warmup + steps, warmup + 2 * steps))
    return idx + list(range(warmup + 2 * steps, warmup + 3 * steps))


def kernel_class(name: str, cfg: dict) -> str:
    """Library launch class of a dispatched kernel name, as the library's own
    profiler names it, where the name alone decides it."""
    import re
    import rvq_inputs as RI
    mm = re.search(r"stage_kernel<(\d+), (\d+), (\d+), (true|false)", name)
    if mm:
        C, S = int(mm.group(1)), int(mm.group(2))
        ch = RI.channels(cfg)
        for i, st in enumerate(cfg["strides"]):
            if ch[i + 1] == C and st == S:
                return f"s{i}.fused"
    for key, cls in (("halo_save", "halo_save"), ("rvq_gather", "rvq_gather"),
                     ("final_conv", "final_conv")):
        if key in name:
            return cls
    return ""


def launch_sequence(cfg: dict) -> list:
    """Launch classes of one decode call of a decoder without a transformer,
    in the order the library enqueues them (split-K reductions and runtime
    copies aside): the gather, the input conv (the projection folded in), then
    per stage either its fused kernel or the ConvT and the residual units (one
    launch each at 128 channels, two below)."""
    import rvq_inputs as RI
    if cfg["tf_layers"]:
        raise SystemExit("launch_sequence: decoders without a transformer only")
    ch = RI.channels(cfg)
    es = 2 if cfg["weight_dtype"] == "bf16" else 4
    seq = ["rvq_gather", "in_conv"]
    for i in range(len(cfg["strides"])):
        if es == 2 and cfg["act"] == "snake" and ch[i + 1] <= 64:
            seq.append(f"s{i}.fused")
            continue
        seq.append(f"s{i}.convT")
        for j in range(2):
            if es == 2 and ch[i + 1] == 128:
                seq.append(f"s{i}.ru{j}")
            else:
                seq += [f"s{i}.ru{j}.conv7", f"s{i}.ru{j}.conv1"]
    return seq


def label_dispatches(rows: list, cfg: dict) -> list:
    """(class, row) for the library's dispatches of whole decode calls: each
    call opens with its gather launch; a split-K reduction is counted with the
    launch it completes; runtime copies are left out."""
    seq = launch_sequence(cfg)
    out, pos = [], None
    for r in sorted(rows, key=lambda r: int(r["Dispatch_Id"])):
        name = r["Kernel_Name"]
        if "snrvq" not in name:
            continue
        if "rvq_gather" in name:
            pos = 0
        elif pos is None:
            continue
        elif "splitk_reduce" in name:
            out.append((out[-1][0], r))
            continue
        else:
            pos += 1
        if pos >= len(seq):
            raise SystemExit("label_dispatches: more launches in a call than the sequence")
        want = kernel_class(name, cfg)
        if want and want != seq[pos]:
            raise SystemExit(f"label_dispatches: launch {pos} is {want}, expected {seq[pos]}")
        out.append((seq[pos], r))
    return out


def calls_per_step(name: str, cfg: dict) -> int:
    """Decode calls one step of the workload makes: the offline workload
    groups its utterances into several calls, the streaming ones make one."""
    if name != "c5":
        return 1
    import rvq_inputs as RI
    return len(group_calls(RI.c5_lengths(cfg), None, cfg["max_frames_per_call"]))


def _steady(rows: list, n_steps: int) -> list:
    """Dispatches of the decode steps: the last n_steps decode calls, each
    opened by its gather launch (the first kernel of every call), and
    everything after them."""
    starts = sorted(int(r["Dispatch_Id"]) for r in rows if "rvq_gather" in r["Kernel_Name"])
    if len(starts) < n_steps:
        raise SystemExit("trace holds fewer decode calls than the run's steps")
    first = starts[len(starts) - n_steps]
    return [r for r in rows if int(r["Dispatch_Id"]) >= first]


def counter_table(path: str, args, cfg: dict, out: list, res: dict) -> None:
    """Per launch class, the counters of one rocprofv3 --pmc run over the
    decode steps, summed over each class's dispatches and divided by the
    steps; the classes' kernel time beside them."""
    import csv
    fn = [f for f in os.listdir(path) if f.endswith("counter_collection.csv")][0]
    disp = {}
    for r in csv.DictReader(open(os.path.join(path, fn))):
        d = disp.setdefault(int(r["Dispatch_Id"]), {
            "Kernel_Name": r["Kernel_Name"], "Dispatch_Id": r["Dispatch_Id"],
            "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), "c": {}})
        d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    idx = step_indices(args.pmc_warmup, args.pmc_steps, False)
    names = sorted({k for d in disp.values() for k in d["c"]})
    agg = {}
    for cls, d in label_dispatches(_steady(list(disp.values()), len(idx)), cfg):
        a = agg.setdefault(cls, {"ns": 0, **{k: 0.0 for k in names}})
        a["ns"] += d["ns"]
        for k, v in d["c"].items():
            a[k] += v
    n = len(idx)
    out.append(f"## Counters per launch class ({', '.join(names)}), per step\n")
    out.append("| class | us | " + " | ".join(names) + " |")
    out.append("|---|---:|" + "---:|" * len(names))
    tab = res.setdefault("counters", {})
    for cls in launch_sequence(cfg):
        if cls not in agg:
            continue
        a = agg[cls]
        out.append(f"| {cls} | {a['ns'] / n / 1e3:.1f} | " +
                   " | ".join(f"{a[k] / n:.4g}" for k in names) + " |")
        t = tab.setdefault(cls, {"us": round(a["ns"] / n / 1e3, 2)})
        t.update({k: a[k] / n for k in names})
    out.append("")


def derived_table(args, cfg: dict, out: list, res: dict) -> None:
    """Ratios per launch class from the counter tables, where their counters
    were collected: matrix pipes busy (of the SIMD cycles at the nominal
    2.4 GHz over the class's time), LDS / other-VALU / SALU instructions per
    MFMA, the share of wave time spent waiting (SQ_WAIT_ANY over
    SQ_WAVE_CYCLES), and the share of busy matrix-pipe cycles in which a
    VALU instruction issued beside it."""
    tab = res.get("counters", {})
    need = ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_LDS", "SQ_INSTS_VALU",
            "SQ_INSTS_SALU", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES")
    rows = [(c, v) for c, v in tab.items() if all(k in v for k in need)]
    if not rows:
        return
    n_simd = 4 * args.n_cu
    out.append("## Derived per launch class\n")
    out.append("| class | us | MFMA busy at 2.4 GHz | LDS instr / MFMA | other VALU / MFMA | "
               "SALU / MFMA | waiting share of wave time | VALU beside busy MFMA |")
    out.append("|---|---:|---:|---:|---:|---:|---:|---:|")
    der = res.setdefault("derived", {})
    for c, v in rows:
        m = max(v["SQ_INSTS_MFMA"], 1.0)
        busy = v["SQ_VALU_MFMA_BUSY_CYCLES"] / (n_simd * v["us"] * 2400.0)
        d = {"mfma_busy": busy, "lds_per_mfma": v["SQ_INSTS_LDS"] / m,
             "valu_per_mfma": (v["SQ_INSTS_VALU"] - v["SQ_INSTS_MFMA"]) / m,
             "salu_per_mfma": v["SQ_INSTS_SALU"] / m,
             "wait_share": v["SQ_WAIT_ANY"] / max(v["SQ_WAVE_CYCLES"], 1.0),
             "coexec_share": v["SQ_VALU_MFMA_COEXEC_CYCLES"] /
             max(v["SQ_VALU_MFMA_BUSY_CYCLES"], 1.0)}
        if v["SQ_INSTS_MFMA"] == 0:
            out.append(f"| {c} | {v['us']:.1f} | 0 | - | - | - | {d['wait_share']:.2f} | - |")
        else:
            out.append(f"| {c} | {v['us']:.1f} | {busy:.3f} | {d['lds_per_mfma']:.2f} | "
                       f"{d['valu_per_mfma']:.2f} | {d['salu_per_mfma']:.2f} | "
                       f"{d['wait_share']:.2f} | {d['coexec_share']:.3f} |")
        der[c] = {k: round(x, 4) for k, x in d.items()}
    out.append("")


def mfma_summary(args, cfg: dict, out: list, res: dict) -> None:
    """Matrix-core use over the decode steps of a counter run with
    SQ_INSTS_MFMA and SQ_VALU_MFMA_BUSY_CYCLES: MFMA instructions (every one a
    16x16x32 fp16 product, 16,384 FLOP) and the matrix pipes' busy cycles
    summed over all SIMDs, against the SIMDs' cycles at the nominal 2.4 GHz
    over the dispatches' own durations."""
    import csv
    import rvq_inputs as RI
    path = args.pmc_mfma
    fn = [f for f in os.listdir(path) if f.endswith("counter_collection.csv")][0]
    disp = {}
    for r in csv.DictReader(open(os.path.join(path, fn))):
        d = disp.setdefault(int(r["Dispatch_Id"]), {
            "name": r["Kernel_Name"], "Kernel_Name": r["Kernel_Name"],
            "Dispatch_Id": r["Dispatch_Id"],
            "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    idx = step_indices(args.pmc_warmup, args.pmc_steps, False)
    frames = sum(int(RI.c4_chunk_sizes(cfg, j).sum()) for j in idx)
    st = _steady(list(disp.values()), len(idx))
    n_simd = 4 * args.n_cu
    agg = {}
    for d in st:
        a = agg.setdefault(d["name"], {"n": 0, "ns": 0, "mfma": 0.0, "busy": 0.0})
        a["n"] += 1
        a["ns"] += d["ns"]
        a["mfma"] += d.get("SQ_INSTS_MFMA", 0.0)
        a["busy"] += d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
    tot = {k: sum(a[k] for a in agg.values()) for k in ("ns", "mfma", "busy")}
    nominal = 2.4e9  # cycles per second the published peak assumes
    flops = 16384.0 * tot["mfma"]
    alg = frames * flops_per_frame(cfg)
    steps = len(idx)
    out.append("## Matrix-core use over the decode steps\n")
    busy = tot["busy"] / (n_simd * tot["ns"] * 1e-9 * nominal)
    out.append(f"{steps} decode steps, {frames / steps:.0f} frames per step. Executed MFMA work "
               f"{flops / steps / 1e9:.1f} GFLOP per step against {alg / steps / 1e9:.1f} GFLOP "
               f"algorithmic (the fused stages recompute their tile halos); "
               f"{tot['busy'] / max(tot['mfma'], 1):.1f} busy cycles per MFMA. Over the kernel "
               f"time the matrix pipes of all {n_simd} SIMDs were busy {busy:.3f} of their "
               f"cycles at the nominal 2.4 GHz; executed work ran at "
               f"{flops / (tot['ns'] * 1e-9) / 1e12:.0f} TFLOP/s, algorithmic work at "
               f"{alg / (tot['ns'] * 1e-9) / 1e12:.0f} TFLOP/s "
               f"({alg / (tot['ns'] * 1e-9) / (PEAK_F16_TFLOPS * 1e12):.3f} of the published "
               f"{PEAK_F16_TFLOPS / 1000:.1f} PFLOP/s).\n")
    out.append("| kernel | calls | avg us | MFMA busy at 2.4 GHz | executed TFLOP/s |")
    out.append("|---|---:|---:|---:|---:|")
    res["mfma"] = {"busy_fraction_nominal": round(busy, 4),
                   "executed_tflops": round(flops / (tot["ns"] * 1e-9) / 1e12, 1),
                   "algorithmic_tflops": round(alg / (tot["ns"] * 1e-9) / 1e12, 1),
                   "executed_gflop_per_step": round(flops / steps / 1e9, 2),
                   "algorithmic_gflop_per_step": round(alg / steps / 1e9, 2)}
    for k, a in sorted(agg.items(), key=lambda kv: -kv[1]["ns"])[:args.top]:
        if a["mfma"] == 0:
            continue
        short = k if len(k) < 90 else k[:87] + "..."
        b = a["busy"] / (n_simd * a["ns"] * 1e-9 * nominal)
        out.append(f"| `{short}` | {a['n']} | {a['ns'] / a['n'] / 1e3:.1f} | {b:.3f} | "
                   f"{16384.0 * a['mfma'] / (a['ns'] * 1e-9) / 1e12:.0f} |")
    out.append("")


def cotenant_trace_summary(path: str) -> list:
    """Decode kernels of a --cotenant run's kernel trace, inside and outside
    the window in which the GEMM load ran (from the third GEMM, after the two
    timed alone, to the last one's end): calls and average duration per
    kernel, and the decode kernels' total time per decode step."""
    import csv
    fn = [f for f in os.listdir(path) if f.endswith("kernel_trace.csv")][0]
    rows = list(csv.DictReader(open(os.path.join(path, fn))))
    gemm = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows
                  if r["Kernel_Name"].startswith("Cijk_"))
    if len(gemm) < 3:
        raise SystemExit("cotenant trace: fewer than three GEMM dispatches")
    w0, w1 = gemm[2][0], max(e for _, e in gemm[2:])
    agg = {}
    steps = {"alone": 0, "beside": 0}
    for r in rows:
        name = r["Kernel_Name"]
        if "snrvq" not in name:
            continue
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        where = "beside" if t0 >= w0 and t1 <= w1 else "alone"
        if "rvq_gather" in name:
            steps[where] += 1
        a = agg.setdefault(name, {"alone": [0, 0], "beside": [0, 0]})
        a[where][0] += 1
        a[where][1] += t1 - t0
    out = [f"Load window: {(w1 - w0) / 1e6:.2f} ms, {len(gemm) - 2} GEMMs. Decode steps: "
           f"{steps['alone']} outside the window (warm-up, the timed solo pass, prefill "
           f"included), {steps['beside']} inside it.\n",
           "| kernel | calls alone | avg us alone | calls beside load | avg us beside load |",
           "|---|---:|---:|---:|---:|"]
    tot = {"alone": 0, "beside": 0}
    for name, a in sorted(agg.items(), key=lambda kv: -kv[1]["beside"][1])[:12]:
        short = name if len(name) < 80 else name[:77] + "..."
        cells = []
        for k in ("alone", "beside"):
            n, t = a[k]
            tot[k] += t
            cells += [str(n), f"{t / n / 1e3:.1f}" if n else "-"]
        out.append(f"| `{short}` | " + " | ".join(cells) + " |")
    out.append("")
    return out


def rocprof_summary(args) -> int:
    """Text summary of a rocprofv3 kernel trace of this benchmark, and of two
    counter runs (FETCH_SIZE, WRITE_SIZE) scaled by the same counters of a
    plain negation kernel of known size."""
    import csv
    import hashlib
    import rvq_inputs as RI
    cfg = RI.get_config(args.config)
    lm = layer_model(cfg)
    rate = [1]
    for st in cfg["strides"]:
        rate.append(rate[-1] * st)
    out = []
    res = {"config": args.config}
    if args.kt:
        rows = list(csv.DictReader(open(os.path.join(args.kt, "kt_kernel_trace.csv"))))
        idx = step_indices(args.kt_warmup, args.kt_steps, True)
        cps = calls_per_step(args.config, cfg)
        st = _steady(rows, len(idx) * cps)
        agg = {}
        for r in st:
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            a = agg.setdefault(r["Kernel_Name"], [0, 0.0])
            a[0] += 1
            a[1] += d
        tot = sum(v[1] for v in agg.values())
        out.append(f"## Kernel time over the {len(idx)} decode steps "
                   f"({len(st)} dispatches; setup and prefill excluded)\n")
        out.append("| kernel | class | calls | avg us | total ms | % |")
        out.append("|---|---|---:|---:|---:|---:|")
        res["kernels"] = {}
        for k, (n, t) in sorted(agg.items(), key=lambda kv: -kv[1][1])[:args.top]:
            cls = kernel_class(k, cfg)
            short = k if len(k) < 90 else k[:87] + "..."
            out.append(f"| `{short}` | {cls} | {n} | {t / n:.1f} | {t / 1e3:.3f} | "
                       f"{100 * t / tot:.1f} |")
            if cls:
                res["kernels"][cls] = {"calls": n, "avg_us": round(t / n, 2)}
        out.append(f"\nSum over the steps: {tot / 1e3:.3f} ms, {tot / len(idx):.1f} us per step.\n")
        logs = [os.path.join(args.kt, "..", f) for f in ("kt_bench.log",)]
        if args.kt_json or os.path.exists(logs[0]):
            lines = open(args.kt_json or logs[0]).read().splitlines()
            rec = json.loads([ln for ln in lines if ln.startswith("{")][-1])
            ks = rec.get("kernels", {})
            out.append("The same run's own HIP-event timing (its profiled pass of "
                       f"{args.kt_steps} steps), for the classes named above:\n")
            out.append("| class | rocprofv3 avg us | HIP events avg us |")
            out.append("|---|---:|---:|")
            for cls, v in res["kernels"].items():
                if cls in ks:
                    out.append(f"| {cls} | {v['avg_us']:.1f} | {ks[cls]['avg_us']:.1f} |")
            res["bench_value"] = rec.get("value")
            out.append(f"\nThat run's throughput under the tracer: {rec.get('value')} frames/s.\n")
            if ks:
                tot_k = sum(v["ms_total"] for v in ks.values())
                out.append("Every launch class of the library over that profiled pass "
                           "(HIP events around each launch):\n")
                out.append("| class | launches | avg us | total ms | % |")
                out.append("|---|---:|---:|---:|---:|")
                for cls, v in sorted(ks.items(), key=lambda kv: -kv[1]["ms_total"]):
                    out.append(f"| {cls} | {v['launches']} | {v['avg_us']:.1f} | "
                               f"{v['ms_total']:.3f} | {100 * v['ms_total'] / tot_k:.1f} |")
                tf = sum(v["ms_total"] for c, v in ks.items() if c.startswith("tf."))
                if tf:
                    res["transformer_share"] = round(tf / tot_k, 4)
                    out.append(f"\nThe transformer's launches (tf.*) take {100 * tf / tot_k:.1f}% "
                               "of the library's kernel time.\n")
                else:
                    out.append("")
        stats = os.path.join(args.kt, "kt_kernel_stats.csv")
        if os.path.exists(stats):
            srows = list(csv.DictReader(open(stats)))[:8]
            out.append("`--stats` over the whole process (setup and prefill included):\n")
            out.append("| kernel | calls | avg us | % |")
            out.append("|---|---:|---:|---:|")
            for r in srows:
                k = r["Name"] if len(r["Name"]) < 90 else r["Name"][:87] + "..."
                out.append(f"| `{k}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                           f"{r['Percentage']} |")
            out.append("")
    if args.pmc_fetch and args.pmc_write:
        if args.config != "c4":
            raise SystemExit("counter summaries are built for the 128-stream workload only")
        idx = step_indices(args.pmc_warmup, args.pmc_steps, False)
        frames = [int(RI.c4_chunk_sizes(cfg, j).sum()) for j in idx]
        res["copy_mib"] = args.copy_mib
        per_cls = {}
        whole = {}  # every dispatch of the decode steps
        for tag, path in (("FETCH_SIZE", args.pmc_fetch), ("WRITE_SIZE", args.pmc_write)):
            fn = [f for f in os.listdir(path) if f.endswith("counter_collection.csv")][0]
            rows = [r for r in csv.DictReader(open(os.path.join(path, fn)))
                    if r["Counter_Name"] == tag]
            neg = [r for r in rows if "neg_kernel" in r["Kernel_Name"]]
            if len(neg) != 1:
                raise SystemExit(f"{tag}: expected one negation dispatch, found {len(neg)}")
            factor = args.copy_mib * 1024.0 / float(neg[0]["Counter_Value"])
            res[f"{tag}_factor"] = round(factor, 4)
            st = _steady(rows, len(idx))
            seen = {}
            for r in st:
                step_bytes = float(r["Counter_Value"]) * 1024.0 * factor
                whole[tag] = whole.get(tag, 0.0) + step_bytes
                if tag == "FETCH_SIZE":
                    whole["kernel_ns"] = whole.get("kernel_ns", 0.0) + (
                        int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                cls = kernel_class(r["Kernel_Name"], cfg)
                if not cls.endswith(".fused"):
                    continue
                j = seen.get(cls, 0)
                seen[cls] = j + 1
                i = int(cls[1:cls.index(".")])
                units = frames[j] * rate[i + 1]
                c = per_cls.setdefault(cls, {"units": 0, "FETCH_SIZE": 0.0, "WRITE_SIZE": 0.0,
                                             "raw": {}})
                if tag == "FETCH_SIZE":
                    c["units"] += units
                c[tag] += float(r["Counter_Value"]) * 1024.0 * factor
                c["raw"].setdefault(tag, []).append(float(r["Counter_Value"]))
        out.append("## HBM traffic of the fused stage kernels\n")
        out.append(f"Calibration: for one negation kernel that reads and writes {args.copy_mib} "
                   f"MiB, FETCH_SIZE times {res['FETCH_SIZE_factor']} and WRITE_SIZE times "
                   f"{res['WRITE_SIZE_factor']} give the known size; the counters below are "
                   "scaled by these factors.\n")
        out.append("| class | dispatches | output rows | fetch B/row | write B/row | "
                   "total B/row | algorithmic B/row |")
        out.append("|---|---:|---:|---:|---:|---:|---:|")
        res["traffic"] = {}
        for cls, c in sorted(per_cls.items()):
            f, w = c["FETCH_SIZE"] / c["units"], c["WRITE_SIZE"] / c["units"]
            n = len(c["raw"]["FETCH_SIZE"])
            alg = lm[cls]["bpr"] + lm[cls]["wpl"] * n / c["units"]
            out.append(f"| {cls} | {n} | {c['units']} | {f:.1f} | {w:.1f} | {f + w:.1f} | "
                       f"{alg:.1f} |")
            res["traffic"][cls] = {"bytes_per_unit": round(f + w, 3)}
        # every launch class, by launch order within each call
        by_cls = {}
        for tag, path in (("FETCH_SIZE", args.pmc_fetch), ("WRITE_SIZE", args.pmc_write)):
            fn = [f for f in os.listdir(path) if f.endswith("counter_collection.csv")][0]
            rows = [r for r in csv.DictReader(open(os.path.join(path, fn)))
                    if r["Counter_Name"] == tag]
            factor = res[f"{tag}_factor"]
            for cls, r in label_dispatches(_steady(rows, len(idx)), cfg):
                c = by_cls.setdefault(cls, {"FETCH_SIZE": 0.0, "WRITE_SIZE": 0.0, "ns": 0})
                c[tag] += float(r["Counter_Value"]) * 1024.0 * factor
                if tag == "FETCH_SIZE":
                    c["ns"] += int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        nsteps = len(idx)
        mean_f = sum(frames) / nsteps
        out.append(f"\nEvery launch class, per step ({mean_f:.0f} frames), against the bytes "
                   "it must move (its operands, outputs and weights once):\n")
        out.append("| class | fetch MB | write MB | total MB | algorithmic MB | ratio | "
                   "GB/s over its own time |")
        out.append("|---|---:|---:|---:|---:|---:|---:|")
        res["traffic_by_class"] = {}
        for cls in launch_sequence(cfg):
            if cls not in by_cls:
                continue
            c = by_cls[cls]
            f, w = c["FETCH_SIZE"] / nsteps, c["WRITE_SIZE"] / nsteps
            # the unit rows of a class: frames, a ConvT's input rows, else the
            # stage's output rows
            i = 0 if cls in ("rvq_gather", "in_conv") else int(cls[1:cls.index(".")]) + (
                0 if cls.endswith(".convT") else 1)
            alg = mean_f * rate[i] * lm[cls]["bpr"] + lm[cls]["wpl"] if cls in lm else None
            t = c["ns"] * 1e-9 / nsteps
            out.append(f"| {cls} | {f / 1e6:.1f} | {w / 1e6:.1f} | {(f + w) / 1e6:.1f} | "
                       + (f"{alg / 1e6:.1f} | {(f + w) / alg:.2f} | " if alg else "| | ")
                       + f"{(f + w) / t / 1e9:.0f} |")
            res["traffic_by_class"][cls] = {"bytes_per_step": round(f + w),
                                            "algorithmic_bytes_per_step":
                                                round(alg) if alg else None}
        step_b = (whole["FETCH_SIZE"] + whole["WRITE_SIZE"]) / nsteps
        step_s = whole["kernel_ns"] * 1e-9 / nsteps
        out.append(f"\nWhole decode step (every dispatch of the {nsteps} counted steps, "
                   f"{sum(frames) / nsteps:.0f} frames per step): "
                   f"{whole['FETCH_SIZE'] / nsteps / 1e6:.1f} MB fetched + "
                   f"{whole['WRITE_SIZE'] / nsteps / 1e6:.1f} MB written = "
                   f"{step_b / 1e6:.1f} MB per step ({step_b / (sum(frames) / nsteps) / 1e3:.1f} kB "
                   f"per frame); over the counter run's own kernel time ({step_s * 1e6:.0f} us per "
                   f"step) that is {step_b / step_s / 1e9:.0f} GB/s, "
                   f"{step_b / step_s / 8e12:.3f} of the 8 TB/s HBM peak.\n")
        res["step_hbm"] = {"bytes_per_step": round(step_b), "kernel_us_per_step":
                           round(step_s * 1e6, 1), "GB_per_s": round(step_b / step_s / 1e9, 1),
                           "frames_per_step": sum(frames) / nsteps}
        res["library_source_sha256"] = source_digest()
        res["stage_source_sha256"] = stage_digest()
        out.append("\nThe traffic holds for the code whose SHA-256 is recorded below (the stage "
                   "kernel's: kernels_stage.hip then internal.h; the whole library's), comments "
                   "and whitespace aside; bench.py reports it only while the code matches.\n")
    if args.pmc_mfma:
        mfma_summary(args, cfg, out, res)
    for path in args.pmc_any or []:
        counter_table(path, args, cfg, out, res)
    if args.pmc_any:
        derived_table(args, cfg, out, res)
    if args.blas_json:
        lines = open(args.blas_json).read().splitlines()
        rec = json.loads([ln for ln in lines if ln.startswith("{")][-1])
        out.append("## Vendor GEMMs on the decoder's shapes\n")
        tmp = args.rocprof_summary + ".blas.tmp" if args.rocprof_summary != "-" else None
        F = int(round(rec["config"]["mean_frames_per_step"]))
        if tmp:
            write_blas_summary(tmp, rec, F)
            out.append(open(tmp).read())
            os.remove(tmp)
        res["blas_reference"] = {k: {kk: v[kk] for kk in ("blas_us", "tflops", "frac", "library_us")
                                     if kk in v} for k, v in rec["blas_reference"].items()}
    if args.cotenant_trace:
        out.append("## Decode kernels alone and beside the GEMM load\n")
        out += cotenant_trace_summary(args.cotenant_trace)
    out.append("```json\n" + json.dumps(res, indent=1) + "\n```")
    text = "\n".join(out) + "\n"
    if args.rocprof_summary == "-":
        print(text)
    else:
        with open(args.rocprof_summary, "a") as fh:
            fh.write(text)
    return 0


def stored_traffic(cls: str, units_per_launch: float):
    """HBM bytes per launch of a fused stage class from the committed counter
    summary, or None when absent or taken from other kernel source."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "stage_fused__qwen_128_streams__hbm_counters.md")
    if not os.path.exists(path):
        return None
    mm = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not mm:
        return None
    rec = json.loads(mm.group(1))
    t = rec.get("traffic", {}).get(cls)
    if rec.get("stage_source_sha256") != stage_digest() or not t:
        return None
    return t["bytes_per_unit"] * units_per_launch


def code_text(path: str) -> bytes:
    """A C/C++/HIP source without its comments and with runs of whitespace
    collapsed: what a digest of the code should see (string and character
    literals are kept as they are)."""
    src = open(path, encoding="utf-8").read()
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            while i < n and src[i] != "\n":
                i += 1
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split()).encode()


def stage_digest() -> str:
    """SHA-256 over the fused stage kernel's code (kernels_stage.hip, then
    internal.h; comments and whitespace do not count)."""
    import hashlib
    src = os.path.join(ROOT, "streaming_neural_audio_rvq_amd", "csrc")
    h = hashlib.sha256()
    for fn in ("kernels_stage.hip", "internal.h"):
        h.update(code_text(os.path.join(src, fn)))
    return h.hexdigest()


def source_digest() -> str:
    """SHA-256 over every library source file's code (name order; comments
    and whitespace do not count)."""
    import hashlib
    src = os.path.join(ROOT, "streaming_neural_audio_rvq_amd", "csrc")
    h = hashlib.sha256()
    for fn in sorted(os.listdir(src)):
        h.update(code_text(os.path.join(src, fn)))
    return h.hexdigest()


def stored_ceilings() -> dict:
    """The JSON record of the committed ceilings summary (bench.py
    --ceilings), or {} when absent."""
    import re
    path = os.path.join(ROOT, "profiles", "part_ceilings__mi355x.md")
    if not os.path.exists(path):
        return {}
    mm = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    return json.loads(mm.group(1)) if mm else {}


def measured_mfma_peak():
    """The highest v_mfma_f32_16x16x32_f16 rate of the committed ceilings
    summary, TFLOP/s, or None when absent."""
    rates = [r["tflops"] for r in stored_ceilings().get("mfma", [])
             if r.get("shape") == "16x16x32 f16"]
    return max(rates) if rates else None


def measured_hbm_peak():
    """The highest HBM streaming rate (reads + writes) of the committed
    ceilings summary, GB/s, or None when absent."""
    rates = [r["gbps"] for r in stored_ceilings().get("hbm", [])]
    return max(rates) if rates else None


def stored_step_hbm():
    """HBM bytes per decoded frame of the whole decode step (every kernel),
    from the committed counter summary of the 128-stream workload, or None
    when absent or taken from other library source."""
    import re
    path = os.path.join(ROOT, "profiles", "stage_fused__qwen_128_streams__hbm_counters.md")
    if not os.path.exists(path):
        return None
    mm = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not mm:
        return None
    rec = json.loads(mm.group(1))
    st = rec.get("step_hbm", {})
    if rec.get("library_source_sha256") != source_digest() or not st.get("frames_per_step"):
        return None
    return st["bytes_per_step"] / st["frames_per_step"]


def ceilings(summary: str | None) -> int:
    """The part's own rates (libsnrvq_probes.so): MFMA throughput with no
    memory traffic, conflict-free LDS reads, Snake throughput on the vector
    ALU, and MFMA with Snake work in the same waves -- in separate blocks and
    interleaved -- against the sum of their times alone; each with the shader
    clock its waves saw.  One JSON line; with `summary`, a markdown table
    appended to that file."""
    import ctypes as C
    lib_path = os.path.join(ROOT, "streaming_neural_audio_rvq_amd", "libsnrvq_probes.so")
    if not os.path.exists(lib_path):
        raise SystemExit(f"{lib_path} is missing: build it first "
                         "(python -c 'import __graft_entry__ as g; g.build()')")

    class Res(C.Structure):
        _fields_ = [("us", C.c_double), ("rate", C.c_double), ("clock_ghz", C.c_double)]

    L = C.CDLL(lib_path)
    n_cu = L.probe_cu_count()
    reps = 5

    def call(fn, *a):
        r = Res()
        rc = fn(*[C.c_int(v) for v in a], C.c_int(reps), C.byref(r))
        if rc:
            raise SystemExit(f"probe {fn.__name__}{a} failed: {rc}")
        return {"us": round(r.us, 2), "rate": r.rate, "clock_ghz": round(r.clock_ghz, 3)}

    out = {"n_cu": n_cu, "mfma": [], "lds": [], "overlap": []}
    for kind, name in ((0, "16x16x32 f16"), (1, "32x32x16 f16")):
        for wps in (1, 2, 3):
            r = call(L.probe_mfma, kind, wps, 20000)
            r.update(shape=name, waves_per_simd=wps, tflops=round(r.pop("rate"), 1))
            # cycles per MFMA on one SIMD at the clock the waves saw (multiply-adds
            # per MFMA: 8192 for 16x16x32, 16384 for 32x32x16)
            macs = 8192 if kind == 0 else 16384
            r["cycles_per_mfma"] = round(2 * macs * n_cu * 4 * r["clock_ghz"] * 1e9
                                         / (r["tflops"] * 1e12), 2)
            out["mfma"].append(r)
            print(json.dumps(r), flush=True)
    for wps in (1, 2, 4):
        r = call(L.probe_lds, wps, 20000)
        r.update(waves_per_simd=wps, tbps=round(r.pop("rate"), 2))
        r["bytes_per_clk_cu"] = round(r["tbps"] * 1e12 / (n_cu * r["clock_ghz"] * 1e9), 1)
        out["lds"].append(r)
        print(json.dumps(r), flush=True)
    out["hbm"] = []
    for bpc in (1, 2, 4, 16):
        r = Res()
        rc = L.probe_hbm(C.c_int(2048), C.c_int(bpc), C.c_int(reps), C.byref(r))
        if rc:
            raise SystemExit(f"probe_hbm failed: {rc}")
        rec = {"mib_per_buffer": 2048, "blocks_per_cu": bpc, "us": round(r.us, 1),
               "gbps": round(r.rate, 1), "frac_of_8tbps": round(r.rate / PEAK_HBM_GBS, 3)}
        out["hbm"].append(rec)
        print(json.dumps(rec), flush=True)
    out["gload"] = []
    for wps in (1, 2, 4):
        r = call(L.probe_gload, wps, 4000)
        r.update(waves_per_simd=wps, tbps=round(r.pop("rate"), 2))
        r["bytes_per_clk_cu"] = round(r["tbps"] * 1e12 / (n_cu * r["clock_ghz"] * 1e9), 1)
        out["gload"].append(r)
        print(json.dumps(r), flush=True)
    for wps in (2, 3):
        t = {}
        for mode, name in ((0, "snake"), (1, "mfma"), (2, "blocked"), (3, "interleaved")):
            r = call(L.probe_overlap, mode, wps, 4000)
            t[name] = r
        alone = t["snake"]["us"] + t["mfma"]["us"]
        rec = {"waves_per_simd": wps, "us_snake": t["snake"]["us"], "us_mfma": t["mfma"]["us"],
               "us_blocked": t["blocked"]["us"], "us_interleaved": t["interleaved"]["us"],
               "blocked_of_sum": round(t["blocked"]["us"] / alone, 3),
               "interleaved_of_sum": round(t["interleaved"]["us"] / alone, 3),
               "snakes_per_s": t["snake"]["rate"],
               # vector-ALU cycles of one wave's Snake (64 lanes) on its SIMD
               "cycles_per_wave_snake": round(t["snake"]["clock_ghz"] * 1e9 * n_cu * 4 * 64
                                              / t["snake"]["rate"], 2),
               "clock_ghz": t["snake"]["clock_ghz"]}
        out["overlap"].append(rec)
        print(json.dumps(rec), flush=True)
    print(json.dumps(out), flush=True)
    if summary:
        lines = ["", "## Ceilings of the part (`bench.py --ceilings`)", "",
                 f"{n_cu} compute units. Each probe: one untimed launch, then {reps} timed "
                 "launches (HIP events) of CUs x waves-per-SIMD work-groups of 256 threads; "
                 "the clock is the waves' cycle counter against the 100 MHz counter.", "",
                 "| MFMA | waves/SIMD | us | TFLOP/s | of 2.5 PFLOP/s | clock GHz | cycles per MFMA |",
                 "|---|---:|---:|---:|---:|---:|---:|"]
        for r in out["mfma"]:
            lines.append(f"| {r['shape']} | {r['waves_per_simd']} | {r['us']} | {r['tflops']} | "
                         f"{r['tflops'] / 2500:.3f} | {r['clock_ghz']} | {r['cycles_per_mfma']} |")
        lines += ["", "| LDS reads | waves/SIMD | us | TB/s | bytes per clock per CU | clock GHz |",
                  "|---|---:|---:|---:|---:|---:|"]
        for r in out["lds"]:
            lines.append(f"| ds_read_b128, conflict-free | {r['waves_per_simd']} | {r['us']} | "
                         f"{r['tbps']} | {r['bytes_per_clk_cu']} | {r['clock_ghz']} |")
        lines += ["", "| HBM streaming y = x + 1 (2 x 2 GiB) | work-groups per CU | us | GB/s (read + write) | "
                  "of 8 TB/s |", "|---|---:|---:|---:|---:|"]
        for r in out["hbm"]:
            lines.append(f"| float4 loads and stores | {r['blocks_per_cu']} | {r['us']} | {r['gbps']} | "
                         f"{r['frac_of_8tbps']} |")
        lines += ["", "| global -> LDS direct loads (L2-resident) | waves/SIMD | us | TB/s | "
                  "bytes per clock per CU | clock GHz |", "|---|---:|---:|---:|---:|---:|"]
        for r in out["gload"]:
            lines.append(f"| global_load_lds 16 B/lane, 8 KiB per wave in flight | "
                         f"{r['waves_per_simd']} | {r['us']} | {r['tbps']} | "
                         f"{r['bytes_per_clk_cu']} | {r['clock_ghz']} |")
        lines += ["", "MFMA and Snake work in the same waves (16 MFMAs 16x16x32 f16 and 32 Snakes "
                  "per iteration): time in separate blocks and interleaved (one MFMA, two Snakes), "
                  "against the sum of the two alone.", "",
                  "| waves/SIMD | Snakes alone us | MFMAs alone us | blocked us | interleaved us | "
                  "blocked / sum | interleaved / sum | Snakes/s | cycles per wave Snake | clock GHz |",
                  "|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
        for r in out["overlap"]:
            lines.append(f"| {r['waves_per_simd']} | {r['us_snake']} | {r['us_mfma']} | "
                         f"{r['us_blocked']} | {r['us_interleaved']} | {r['blocked_of_sum']} | "
                         f"{r['interleaved_of_sum']} | {r['snakes_per_s']:.3g} | "
                         f"{r['cycles_per_wave_snake']} | {r['clock_ghz']} |")
        lines += ["", "```json", json.dumps(out), "```", ""]
        with open(summary, "a") as fh:
            fh.write("\n".join(lines))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--config", default="c4")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true")
    ap.add_argument("--cotenant", choices=["shared", "masked"],
                    help="also time the steps beside a synthetic bf16 GEMM load on another "
                         "stream (default priority): sharing all CUs, or with the decode "
                         "stream and the load stream on disjoint CU masks")
    ap.add_argument("--cu-fraction", type=float, default=0.5,
                    help="share of the CUs in the decode stream's mask (--cotenant masked)")
    ap.add_argument("--graph", action="store_true",
                    help="run every step through decode_chunk_graph (host codes, one graph "
                         "launch per step, captured once per frame bucket)")
    ap.add_argument("--blas-reference", action="store_true",
                    help="also time the decoder's contractions as plain dense fp16 GEMMs on the "
                         "vendor library (torch.mm) at the workload's mean frames per step")
    ap.add_argument("--blas-summary", help="with --blas-reference: append its table to this file")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the short runs of the other workloads (c2, c3, c5) that the "
                         "default 128-stream run reports beside its own line")
    ap.add_argument("--stateless", action="store_true",
                    help="comparison: decode every chunk again from zero state with up to 16 "
                         "left frames (the pages' stateless variant) instead of carrying state")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run one plain streaming kernel (negation) that reads and "
                         "writes this many MiB: the known-size reference for HBM counters")
    ap.add_argument("--rocprof-summary", metavar="OUT",
                    help="summarise rocprofv3 output of earlier runs of this benchmark "
                         "into OUT (appended; '-' prints) instead of running")
    ap.add_argument("--kt", help="rocprofv3 --kernel-trace output directory")
    ap.add_argument("--kt-steps", type=int, default=16)
    ap.add_argument("--kt-json", help="the traced run's output (default: kt_bench.log "
                                      "beside the trace directory)")
    ap.add_argument("--kt-warmup", type=int, default=2)
    ap.add_argument("--pmc-fetch", help="rocprofv3 --pmc FETCH_SIZE output directory")
    ap.add_argument("--pmc-write", help="rocprofv3 --pmc WRITE_SIZE output directory")
    ap.add_argument("--blas-json", help="with --rocprof-summary: the output of a --blas-reference run, "
                         "tabulated")
    ap.add_argument("--pmc-any", action="append",
                    help="rocprofv3 --pmc output directory of any counters: a per-class table "
                         "over the decode steps (repeatable)")
    ap.add_argument("--pmc-mfma", help="rocprofv3 --pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES "
                    "output directory")
    ap.add_argument("--cotenant-trace", help="rocprofv3 --kernel-trace output directory of a "
                    "--cotenant run (summarised with --rocprof-summary)")
    ap.add_argument("--n-cu", type=int, default=256, help="compute units (counter summaries)")
    ap.add_argument("--pmc-steps", type=int, default=2)
    ap.add_argument("--pmc-warmup", type=int, default=1)
    ap.add_argument("--top", type=int, default=30)
    ap.add_argument("--ceilings", action="store_true",
                    help="instead of decoding: the part's own MFMA, LDS and vector-ALU rates "
                         "(libsnrvq_probes.so)")
    ap.add_argument("--ceilings-summary", help="with --ceilings: append the tables to this file")
    args = ap.parse_args()
    if args.rocprof_summary:
        return rocprof_summary(args)
    if args.ceilings:
        return ceilings(args.ceilings_summary)
    if args.graph:
        args.no_profile = True  # graph steps record no per-kernel events
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build decodes on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); streams would shard across GPUs with no collective, "
              "which is not built.", file=sys.stderr)
        return 2

    # the other workloads, each a short run of this script in a child process
    # (before this process touches the GPU), reported beside the headline line
    others = None
    if (args.config == "c4" and not args.no_other_configs and not
            (args.graph or args.stateless or args.cotenant or args.blas_reference or
             args.copy_mib)):
        others = other_workloads()

    import torch

    import rvq_inputs as RI
    import streaming_neural_audio_rvq_amd as snr

    if args.copy_mib:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    cfg = RI.get_config(args.config)
    if args.graph:  # one spare slot for the single-stream latency probe
        cfg["max_streams"] += 1
    w = RI.make_weights(cfg)
    codec = snr.Codec(cfg, RI.weight_bits(w))
    hop = codec.hop
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    # steps: warmup, timed (codes resident in HBM), profiled, host-codes
    total_steps = args.warmup + 3 * args.steps
    wl = make_workload(args.config, cfg, codec, total_steps, stream, args.stateless)
    pcm = torch.empty(cfg["max_frames_per_call"] * hop, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def run_step(j, host_codes=False, st=None):
        st = stream if st is None else st
        for ids, n, codes, codes_dev in wl["steps"][j]:
            fresh = ids is None
            if fresh:
                ids = [codec.stream_open() for _ in range(len(n))]
            if args.graph and not fresh:
                codec.decode_chunk_graph(ids, n, codes, pcm, st)
            elif host_codes:
                codec.decode_chunk(ids, n, codes, pcm, st)
            else:
                codec.decode_chunk_device(ids, n, codes_dev, pcm, st)
            if fresh:
                for i in ids:
                    codec.stream_close(i)

    def step_frames(j):
        if "new_frames" in wl:
            return wl["new_frames"][j]
        return int(sum(int(np.sum(n)) for _, n, _, _ in wl["steps"][j]))

    for j in range(args.warmup):
        run_step(j)
    torch.cuda.synchronize()

    clocks = []  # (wall, GPU events) seconds of every timed run

    def timed_run(steps, host_codes: bool, st=None, alone=True):
        """Frames and seconds of the steps on stream st.  alone=False: other
        work runs on the device, so only this stream's events time it.  The
        garbage collector is paused while the steps are enqueued (as timeit
        does), so a collection cannot stall the host and idle the device."""
        st = stream if st is None else st
        fr = sum(step_frames(j) for j in steps)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        if alone:
            torch.cuda.synchronize()
        gc_was = gc.isenabled()
        gc.collect()
        gc.disable()
        t0 = time.perf_counter()
        ev0.record(st)
        for j in steps:
            run_step(j, host_codes, st)
        ev1.record(st)
        if gc_was:
            gc.enable()
        if not alone:
            ev1.synchronize()
            return fr, ev0.elapsed_time(ev1) / 1e3
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        clocks.append((wall, ev0.elapsed_time(ev1) / 1e3))
        return fr, max(wall, ev0.elapsed_time(ev1) / 1e3)

    graph_info = None
    if args.graph:
        # one untimed pass over the timed steps' chunk schedule captures the
        # graph of every frame bucket they use; the timed pass then replays
        for j in range(args.warmup, args.warmup + args.steps):
            run_step(j)
        torch.cuda.synchronize()
        i0 = codec.get_info()
        graph_info = {"captures_before_timing": i0.graph_captures}
    # ---- timed region: K steps, codes already resident in HBM ----
    frames, elapsed = timed_run(range(args.warmup, args.warmup + args.steps), False)
    timed_clocks = clocks[-1]
    if args.graph:
        i1 = codec.get_info()
        graph_info["captures_in_timed_steps"] = i1.graph_captures - i0.graph_captures
        graph_info["replays_in_timed_steps"] = i1.graph_replays - i0.graph_replays
        fr = [step_frames(j) for j in range(args.warmup, args.warmup + args.steps)]
        graph_info["frame_buckets"] = sorted({(f + 31) // 32 * 32 if f > 32 else
                                              1 << (f - 1).bit_length() for f in fr})
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
            run_step(j)
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
        if dom.endswith(".fused"):
            roof["traffic"] = stored_traffic(dom, d["units"] / d["launches"])
            if roof["traffic"] is not None:
                roof["traffic"] = int(roof["traffic"])
        roof["kernel"] = dom
        roof["avg_launch_us"] = round(d["avg_us"], 2)
        roof["alg_bytes_per_launch"] = int(d["bytes_per_launch"])
        roof["alg_flops_per_launch"] = int(d["flops_per_launch"])
        if dom.endswith(".fused"):
            roof["vector_alu"] = vector_floor(cfg, dom, d["units"] / d["launches"],
                                              d["flops_per_launch"], peak_f, sec)
        mp = measured_mfma_peak()
        if roof["bound"] == "mfma" and mp and cfg["weight_dtype"] == "bf16":
            # context beside the published peak: what the part's matrix cores
            # delivered to the kernels' MFMA shape with no memory traffic
            roof["measured_peak"] = {"value": mp, "unit": "TFLOP/s",
                                     "frac": round(roof["achieved"] / mp, 4),
                                     "source": "profiles/part_ceilings__mi355x.md"}

    glat = None
    if args.graph:
        glat = graph_latency(torch, codec, cfg, stream)

    cot = None
    if args.cotenant:
        cot = cotenant_run(args, torch, timed_run, lambda st: sum(step_frames(j) for j in st),
                           stream,
                           range(args.warmup, args.warmup + args.steps), fps)

    fpf = flops_per_frame(cfg)
    peak_f = PEAK_F16_TFLOPS if cfg["weight_dtype"] == "bf16" else PEAK_F32_TFLOPS
    out = {
        "metric": (METRIC if args.config == "c4" and not (args.stateless or args.graph)
                   else f"codec frames/s ({args.config}{', stateless' if args.stateless else ''}"
                        f"{', graph replay' if args.graph else ''})"),
        "value": round(fps, 1),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 4),
        "ms_per_step_wall": round(1e3 * timed_clocks[0] / args.steps, 4),
        "ms_per_step_gpu_events": round(1e3 * timed_clocks[1] / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if cfg["weight_dtype"] == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl["desc"], "streams": wl["streams"], "frames_timed": frames,
                   "mean_frames_per_step": frames / args.steps,
                   "decoded_frames_per_new_frame": round(
                       sum(int(np.sum(n)) for j in range(args.warmup, args.warmup + args.steps)
                           for _, n, _, _ in wl["steps"][j]) / frames, 3)},
        "audio_sec_per_s": round(fps / frame_rate, 1),
        "host_codes_frames_per_s": round(h_frames / h_elapsed, 1),
        "mfma_util_alg": round(fps * fpf / (peak_f * 1e12), 4),
        "roofline": roof,
    }
    bpf = stored_step_hbm() if args.config == "c4" and not (args.stateless or args.graph) else None
    out["step_hbm"] = None if bpf is None else {
        "bytes_per_frame": round(bpf), "achieved": round(bpf * fps / 1e9, 1),
        "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(bpf * fps / 1e9 / PEAK_HBM_GBS, 4),
        "source": "FETCH_SIZE + WRITE_SIZE of every dispatch of the step (committed counter "
                  "summary) x this run's frames/s"}
    hp = measured_hbm_peak()
    if out["step_hbm"] and hp:
        out["step_hbm"]["measured_peak"] = {
            "value": hp, "unit": "GB/s", "frac": round(out["step_hbm"]["achieved"] / hp, 4),
            "source": "profiles/part_ceilings__mi355x.md"}
    if others:
        out["other_workloads"] = others
    if cot:
        out["cotenant"] = cot
    if glat:
        out["graph_latency"] = glat
    if graph_info:
        out["graphs"] = graph_info
    if args.blas_reference:
        out["blas_reference"] = blas_reference(torch, cfg, int(round(frames / args.steps)))
        for k, v in out["blas_reference"].items():
            if k in kernels:
                v["library_us"] = round(kernels[k]["avg_us"], 2)
        if args.blas_summary:
            write_blas_summary(args.blas_summary, out, int(round(frames / args.steps)))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.config, cfg, w, args.cpu_baseline_seconds)
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
