"""GPU parity on the workloads as configured, through every decode entry point.

The 128-stream workload runs through decode_chunk_device (codes resident in
HBM, the launch sequence the benchmark times), through decode_chunk_graph
(graphs keyed by frame bucket, replayed) and twice over (bitwise
repeatability); the Qwen-shaped decoder runs 8 streams x 200 frames with the
chunk ramp, with zero biases (so the peak amplitude is the signal itself, not
a DC offset), with the optional output tanh, with a prefill longer than one
call, layer by layer against the oracle's taps, and beside a GEMM load on
another stream.

Bar: per stream, max|gpu - oracle| <= 2e-3 max|oracle| (bf16 weights); where
the biases put a DC offset under the signal, the error relative to the AC
peak max|oracle - mean| is bounded too (``AC_BOUND``).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import rvq_inputs as RI
import streaming_neural_audio_rvq_amd as snr
from _util import analytic_left_context, host_weights, rel_err, tol_for

pytestmark = pytest.mark.gpu

# Error relative to the AC peak (max|oracle - mean(oracle)|) on the standard
# N(0, 0.02) weights, whose biases give the PCM a DC offset of about 9x its
# AC peak.  The fp16 operands' rounding (2^-11 relative per stored operand)
# reaches the output through ~23 layers: measured up to 2.7e-3 of the AC
# peak on these workloads (err/peak <= 2.6e-4 there), so this bound leaves
# 1.5x of margin.  The zero-bias test below holds the unscaled 2e-3 bar where
# peak and signal coincide.
AC_BOUND = 4e-3


def say(*a):
    print(*a, flush=True)


def open_codec(cfg, w):
    return snr.Codec(cfg, host_weights(cfg, w))


def check(tag, got, ref, tol, ac_bound=AC_BOUND):
    e, ac = rel_err(got, ref)
    say(f"{tag}: err/peak {e:.3e} AC-rel {ac:.3e}")
    assert e <= tol, f"{tag}: err/peak {e:.3e} > {tol}"
    assert ac <= ac_bound, f"{tag}: AC-relative error {ac:.3e} > {ac_bound}"
    return e, ac


# --------------------------------------------------------------------------
# The 128-stream workload: staggered offsets, bucketed chunks
# --------------------------------------------------------------------------
C4_STEPS = 8


@pytest.fixture(scope="module")
def c4():
    """Weights, the step schedule, the sampled streams and their oracle PCM
    for every step (each sampled stream decoded by the oracle from zero state
    L frames before its first checked step: exact, by the left-context pin)."""
    cfg = RI.get_config("c4")
    w = RI.make_weights(cfg)
    Bn = cfg["n_streams"]
    off = RI.c4_offsets(cfg)
    pre = [RI.stream_codes(cfg, b, int(off[b]), part=0) for b in range(Bn)]
    n = [RI.c4_chunk_sizes(cfg, j) for j in range(C4_STEPS)]
    step_codes = [[RI.stream_codes(cfg, b, int(n[j][b]), part=1 + j) for b in range(Bn)]
                  for j in range(C4_STEPS)]
    # min and max offsets, a stream of each chunk size at some step, seeded rest
    sample = {int(np.argmin(off)), int(np.argmax(off))}
    for v in cfg["buckets"]:
        for j in range(C4_STEPS):
            hits = np.flatnonzero(n[j] == v)
            if hits.size:
                sample.add(int(hits[0]))
                break
    for b in np.random.default_rng(3).permutation(Bn):
        if len(sample) >= 8:
            break
        sample.add(int(b))
    sample = sorted(sample)
    H = RI.hop(cfg)
    L = analytic_left_context(cfg) + 1
    m = oracle.Model(cfg, w)
    streams, codes, w0s = [], [], []
    for b in sample:
        w0 = max(0, int(off[b]) - L)
        hist = np.concatenate([pre[b][w0:]] + [step_codes[j][b] for j in range(C4_STEPS)])
        streams.append(m.stream(w0))
        codes.append(hist)
        w0s.append(w0)
    pcm = m.decode_batch(streams, [c.shape[0] for c in codes], np.concatenate(codes))
    ref, at = {}, 0
    for b, c, w0 in zip(sample, codes, w0s):
        full = pcm[at * H:(at + c.shape[0]) * H]
        at += c.shape[0]
        pos = int(off[b]) - w0
        for j in range(C4_STEPS):
            k = int(n[j][b])
            ref[(j, b)] = full[pos * H:(pos + k) * H]
            pos += k
    say(f"c4 fixture: sampled streams {sample}, offsets {[int(off[b]) for b in sample]}")
    return dict(cfg=cfg, w=w, off=off, pre=pre, n=n, codes=step_codes, sample=sample, ref=ref)


def c4_open_streams(codec, d):
    ids = [codec.stream_open() for _ in range(d["cfg"]["n_streams"])]
    for b, i in enumerate(ids):
        if d["off"][b]:
            codec.stream_prefill(i, d["pre"][b])
    return ids


def c4_run(codec, d, ids, mode):
    """The 8 steps through one entry point; per step the PCM on the host."""
    outs = []
    for j in range(C4_STEPS):
        n = d["n"][j]
        packed = np.concatenate(d["codes"][j])
        pcm = torch.empty(int(n.sum()) * codec.hop, dtype=torch.float32, device="cuda")
        if mode == "device":
            codec.decode_chunk_device(ids, n, torch.from_numpy(packed).cuda(), pcm)
        elif mode == "graph":
            codec.decode_chunk_graph(ids, n, packed, pcm)
        else:
            codec.decode_chunk(ids, n, packed, pcm)
        outs.append(pcm.cpu().numpy())
    return outs


def c4_check(d, outs, tag, H):
    tol = tol_for(d["cfg"])
    sizes = set()
    for j, host in enumerate(outs):
        cu = np.concatenate([[0], np.cumsum(d["n"][j])])
        for b in d["sample"]:
            got = host[cu[b] * H:cu[b + 1] * H]
            check(f"{tag} step {j} stream {b} n {d['n'][j][b]}", got, d["ref"][(j, b)], tol)
            sizes.add(int(d["n"][j][b]))
    assert sizes == set(d["cfg"]["buckets"])


def test_c4_device_codes_vs_oracle_and_bitwise_repeat(c4):
    """The benchmark's timed path: 128 streams, codes in HBM, 8 steps of
    mixed chunks {1, 2, 4, 8, 16}; sampled streams against the oracle at
    every step, every chunk size covered.  Then all streams are closed,
    reopened (other state slots), prefilled again and the same 8 steps
    decoded again: every sample of every stream bit for bit the same."""
    codec = open_codec(c4["cfg"], c4["w"])
    ids = c4_open_streams(codec, c4)
    first = c4_run(codec, c4, ids, "device")
    assert codec.device_status() == 0
    c4_check(c4, first, "c4 device", codec.hop)
    for i in ids:
        codec.stream_close(i)
    ids = c4_open_streams(codec, c4)
    again = c4_run(codec, c4, ids, "device")
    for j, (x, y) in enumerate(zip(first, again)):
        assert np.array_equal(x, y), f"step {j}: repeated run differs"
    say("c4 device: repeated run bitwise identical over", C4_STEPS, "steps x 128 streams")
    codec.close()


def test_c4_graph_buckets_replay_vs_oracle(c4):
    """decode_chunk_graph on the same 8 steps: each step runs as the graph of
    its frame bucket (the mixed per-stream chunks ride in the metadata).
    First pass: captures, each bucket once; the sampled streams against the
    oracle.  Second pass over reopened streams: every step replays a
    captured graph, bit for bit the same PCM as the first pass, and within
    the bound of the eager path's PCM."""
    codec = open_codec(c4["cfg"], c4["w"])
    ids = c4_open_streams(codec, c4)
    first = c4_run(codec, c4, ids, "graph")
    info = codec.get_info()
    F = [int(n.sum()) for n in c4["n"]]
    # graph keys: (streams incl. the pad stream, bucket frames)
    buckets = {(128 + (f % 32 != 0), (f + 31) // 32 * 32) for f in F}
    say(f"c4 graph: frames per step {F}, graphs {sorted(buckets)}, "
        f"captures {info.graph_captures}, replays {info.graph_replays}")
    assert info.graph_captures == len(buckets)
    assert info.graph_replays == C4_STEPS - len(buckets)
    c4_check(c4, first, "c4 graph", codec.hop)
    for i in ids:
        codec.stream_close(i)
    ids = c4_open_streams(codec, c4)
    again = c4_run(codec, c4, ids, "graph")
    info2 = codec.get_info()
    assert info2.graph_captures == info.graph_captures
    assert info2.graph_replays == info.graph_replays + C4_STEPS
    for j, (x, y) in enumerate(zip(first, again)):
        assert np.array_equal(x, y), f"step {j}: replay differs from the first pass"
    for i in ids:
        codec.stream_close(i)
    ids = c4_open_streams(codec, c4)
    eager = c4_run(codec, c4, ids, "host")
    tol = tol_for(c4["cfg"])
    H = codec.hop
    for j in range(C4_STEPS):
        cu = np.concatenate([[0], np.cumsum(c4["n"][j])])
        worst = max(rel_err(first[j][cu[b] * H:cu[b + 1] * H],
                            eager[j][cu[b] * H:cu[b + 1] * H].astype(np.float64))[0]
                    for b in range(len(ids)))
        say(f"c4 graph vs eager step {j}: worst err/peak {worst:.3e}, "
            f"bitwise {np.array_equal(first[j], eager[j])}")
        assert worst <= tol
    codec.close()


# --------------------------------------------------------------------------
# The Qwen-shaped decoder as configured: 8 streams x 200 frames, chunk ramp
# --------------------------------------------------------------------------
def lockstep(codec, ids, codes, plan):
    H = codec.hop
    B = len(ids)
    outs = [[] for _ in range(B)]
    at = 0
    for n in plan:
        packed = np.concatenate([codes[b][at:at + n] for b in range(B)])
        pcm = torch.empty(B * n * H, dtype=torch.float32, device="cuda")
        codec.decode_chunk(ids, [n] * B, packed, pcm)
        host = pcm.cpu().numpy()
        for b in range(B):
            outs[b].append(host[b * n * H:(b + 1) * n * H])
        at += n
    return [np.concatenate(o) for o in outs]


def test_c2_as_configured_8x200_ramp_vs_oracle():
    cfg = RI.get_config("c2")
    w = RI.make_weights(cfg)
    B, T = cfg["n_streams"], cfg["n_frames"]
    plan = RI.C2_CHUNKS
    assert sum(plan) == T
    say(f"case c2 as configured: {B} streams x {T} frames, plan {plan}")
    codes = [RI.stream_codes(cfg, b, T) for b in range(B)]
    codec = open_codec(cfg, w)
    ids = [codec.stream_open() for _ in range(B)]
    got = lockstep(codec, ids, codes, plan)
    m = oracle.Model(cfg, w)
    ref = m.decode_batch([m.stream() for _ in range(B)], [T] * B, np.concatenate(codes))
    H = codec.hop
    for b in range(B):
        check(f"c2 8x200 stream {b}", got[b], ref[b * T * H:(b + 1) * T * H], tol_for(cfg))
    codec.close()


def test_c2_zero_bias_peak_is_signal():
    """With every bias zero the PCM has no DC offset, so max|oracle| is the
    signal's own peak and the 2e-3 bar is as strict as it reads."""
    cfg = RI.get_config("c2", zero_bias=True)
    w = RI.make_weights(cfg)
    assert all(not np.any(v) for k, v in w.items() if k.endswith(".bias"))
    B, plan = 4, [1, 2, 4, 8, 8, 8, 5]
    T = sum(plan)
    codes = [RI.stream_codes(cfg, b, T, part=4) for b in range(B)]
    codec = open_codec(cfg, w)
    ids = [codec.stream_open() for _ in range(B)]
    got = lockstep(codec, ids, codes, plan)
    m = oracle.Model(cfg, w)
    ref = m.decode_batch([m.stream() for _ in range(B)], [T] * B, np.concatenate(codes))
    H = codec.hop
    for b in range(B):
        r = ref[b * T * H:(b + 1) * T * H]
        say(f"zero-bias stream {b}: mean {r.mean():.2e}, peak {np.abs(r).max():.2e}")
        assert abs(r.mean()) < 0.1 * np.abs(r).max()
        e, ac = rel_err(got[b], r)
        say(f"zero-bias stream {b}: err/peak {e:.3e} (AC-rel {ac:.3e})")
        assert e <= 2e-3 and ac <= 2e-3
    codec.close()


@pytest.mark.parametrize("per_layer", [False, True])
def test_final_tanh_vs_oracle(per_layer):
    """The optional output tanh on both output paths: the fused last stage
    and the per-layer final conv kernel."""
    cfg = RI.get_config("c2", final_tanh=True, per_layer=per_layer)
    w = RI.make_weights(cfg)
    B, plan = 2, [1, 2, 4, 8, 3]
    T = sum(plan)
    codes = [RI.stream_codes(cfg, b, T, part=6) for b in range(B)]
    codec = open_codec(cfg, w)
    ids = [codec.stream_open() for _ in range(B)]
    got = lockstep(codec, ids, codes, plan)
    m = oracle.Model(cfg, w)
    raw = oracle.Model(dict(cfg, final_tanh=False), w)
    for b in range(B):
        ref = m.decode_full(codes[b])
        assert not np.array_equal(ref, raw.decode_full(codes[b]))
        check(f"final tanh per_layer={per_layer} stream {b}", got[b], ref, tol_for(cfg))
    codec.close()


def test_prefill_longer_than_one_call():
    """stream_prefill of more frames than max_frames_per_call is split into
    several decodes; the state it leaves continues exactly (the next chunks
    against the oracle's decode of prefix + chunks)."""
    cfg = RI.get_config("c2", max_streams=4, max_frames_per_call=64)
    w = RI.make_weights(cfg)
    pre, plan = 150, [1, 8, 16]
    codes = RI.stream_codes(cfg, 9, pre + sum(plan), part=2)
    codec = open_codec(cfg, w)
    sid = codec.stream_open()
    codec.stream_prefill(sid, codes[:pre])
    H = codec.hop
    outs, at = [], pre
    for n in plan:
        pcm = torch.empty(n * H, dtype=torch.float32, device="cuda")
        codec.decode_chunk([sid], [n], codes[at:at + n], pcm)
        outs.append(pcm.cpu().numpy())
        at += n
    L = analytic_left_context(cfg) + 1
    w0 = pre - L
    ref = oracle.Model(cfg, w).stream(w0).decode(codes[w0:])[L * H:]
    check(f"prefill {pre} frames in calls of <= 64, then {plan}", np.concatenate(outs), ref,
          tol_for(cfg))
    codec.close()


# --------------------------------------------------------------------------
# Layer by layer: the captured conv operands against the oracle's taps
# --------------------------------------------------------------------------
def test_layer_captures_vs_oracle_taps():
    """Every conv operand of the decoder (per-layer codec: every layer
    stored) against the oracle's tap at the same point, three ragged streams
    in one call; the fused codec refuses the operands its stage kernels keep
    on chip and returns the same values for the rest."""
    cfg = RI.get_config("c2", per_layer=True)
    w = RI.make_weights(cfg)
    n = [3, 5, 2]
    codes = [RI.stream_codes(cfg, b, n[b], part=8) for b in range(3)]
    m = oracle.Model(cfg, w)
    S = len(cfg["strides"])
    layer = open_codec(cfg, w)
    fused = open_codec(dict(cfg, per_layer=False), w)
    caps = {}
    for tag, codec in (("layer", layer), ("fused", fused)):
        ids = [codec.stream_open() for _ in range(3)]
        pcm = torch.empty(sum(n) * codec.hop, dtype=torch.float32, device="cuda")
        codec.decode_chunk(ids, n, np.concatenate(codes), pcm)
        for tap in range(3 * S + 1):
            rows, C = oracle.tap_shape(cfg, tap, sum(n))
            dst = torch.empty(rows * C, dtype=torch.float32, device="cuda")
            try:
                codec.debug_capture(snr.CAPTURE_LAYER0 + tap, dst)
            except snr.CodecError as e:
                assert tag == "fused" and e.code == snr.CODEC_EINVAL
                continue
            caps[(tag, tap)] = dst.cpu().numpy().reshape(rows, C)
    for tap in range(3 * S + 1):
        ref = np.concatenate([m.stream().decode_tap(codes[b], tap)[1] for b in range(3)])
        got = caps[("layer", tap)]
        e = float(np.max(np.abs(got - ref))) / float(np.max(np.abs(ref)))
        say(f"tap {tap} {ref.shape}: err/peak {e:.3e}")
        assert e <= 2e-3
        if ("fused", tap) in caps:
            assert np.array_equal(caps[("fused", tap)], got)
    # the stage kernels keep stages 3 and 4's residual-unit inputs on chip
    assert ("fused", 3 * 3 + 1) not in caps and ("fused", 3 * S) not in caps
    layer.close()
    fused.close()


# --------------------------------------------------------------------------
# Co-tenancy: the decode beside a GEMM load on another stream
# --------------------------------------------------------------------------
def cu_masked_stream(lo, hi):
    hip = ctypes.CDLL("libamdhip64.so")
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    words = (n_cu + 31) // 32
    mask = (ctypes.c_uint32 * words)()
    for cu in range(lo, hi):
        mask[cu // 32] |= 1 << (cu % 32)
    h = ctypes.c_void_p()
    assert hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), ctypes.c_uint32(words), mask) == 0
    return hip, h


@pytest.mark.parametrize("mode", ["shared", "masked"])
def test_decode_beside_gemm_load(mode):
    """The pages' deployment runs the codec beside stage 0 on one GPU.  Here
    the decode runs on one stream while bf16 GEMMs run back to back on
    another (every stream at default priority; "masked": disjoint CU sets).
    The PCM equals the decode alone bit for bit and the oracle within the
    bound: sharing the GPU changes timing only."""
    cfg = RI.get_config("c2")
    w = RI.make_weights(cfg)
    B, plan = 8, [1, 2, 4, 8, 8]
    T = sum(plan)
    codes = [RI.stream_codes(cfg, b, T, part=10) for b in range(B)]
    codec = open_codec(cfg, w)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    handles = []
    if mode == "masked":
        hip, h1 = cu_masked_stream(0, n_cu // 2)
        _, h2 = cu_masked_stream(n_cu // 2, n_cu)
        handles = [h1, h2]
        dec = torch.cuda.ExternalStream(h1.value)
        load = torch.cuda.ExternalStream(h2.value)
    else:
        dec, load = torch.cuda.Stream(), torch.cuda.Stream()
    a = torch.randn(4096, 4096, dtype=torch.bfloat16, device="cuda")
    bm = torch.randn(4096, 4096, dtype=torch.bfloat16, device="cuda")

    def run(with_load):
        ids = [codec.stream_open() for _ in range(B)]
        torch.cuda.synchronize()
        if with_load:  # enough GEMMs to outlast the decode
            with torch.cuda.stream(load):
                for _ in range(400):
                    torch.matmul(a, bm)
        outs = [[] for _ in range(B)]
        at = 0
        # everything on the decode stream: a copy on the null stream would
        # wait for the load (CU-masked streams are blocking streams)
        with torch.cuda.stream(dec):
            for n in plan:
                packed = np.concatenate([cd[at:at + n] for cd in codes])
                pcm = torch.empty(B * n * codec.hop, dtype=torch.float32, device="cuda")
                codec.decode_chunk(ids, [n] * B, packed, pcm, stream=dec)
                host = pcm.cpu().numpy()
                for b in range(B):
                    outs[b].append(host[b * n * codec.hop:(b + 1) * n * codec.hop])
                at += n
        busy = not load.query()
        torch.cuda.synchronize()
        for i in ids:
            codec.stream_close(i)
        return [np.concatenate(o) for o in outs], busy

    solo, _ = run(False)
    beside, busy = run(True)
    say(f"co-tenant {mode}: load still running when the decode ended: {busy}")
    assert busy, "the load ended before the decode: no overlap"
    m = oracle.Model(cfg, w)
    for b in range(B):
        assert np.array_equal(solo[b], beside[b]), f"stream {b}: differs beside the load"
    for b in (0, B - 1):
        check(f"co-tenant {mode} stream {b}", beside[b], m.decode_full(codes[b]), tol_for(cfg))
    codec.close()
    for h in handles:
        hip.hipStreamDestroy(h)
