"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle.

Bar: per stream, max|gpu - oracle| <= tol * max|oracle| with tol = 1e-5 for
fp32 weights and 2e-3 for bf16 weights; codebook indexing bit-exact; the
GPU's streamed and whole-utterance decodes within the same bound; repeated
runs bitwise identical.
"""
import numpy as np
import pytest
import torch

import oracle
import rvq_inputs as RI
import streaming_neural_audio_rvq_amd as snr
from _util import analytic_left_context, host_weights, rel_err, tol_for

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def open_codec(cfg, w=None):
    w = RI.make_weights(cfg) if w is None else w
    return snr.Codec(cfg, host_weights(cfg, w))


def run_lockstep(codec, ids, codes, plan):
    """All streams decode chunk sizes plan[0], plan[1], ... in lockstep.
    codes[b] is [T, K]; returns per-stream concatenated PCM (numpy f32)."""
    hop = codec.hop
    B = len(ids)
    outs = [[] for _ in range(B)]
    at = 0
    for n in plan:
        packed = np.concatenate([codes[b][at:at + n] for b in range(B)])
        pcm = torch.empty(B * n * hop, dtype=torch.float32, device="cuda")
        codec.decode_chunk(ids, [n] * B, packed, pcm)
        host = pcm.cpu().numpy()
        for b in range(B):
            outs[b].append(host[b * n * hop:(b + 1) * n * hop])
        at += n
    return [np.concatenate(o) for o in outs]


def decode_full_gpu(codec, codes_list):
    """Whole-utterance decode of every stream in one call (fresh streams)."""
    ids = [codec.stream_open() for _ in codes_list]
    n = [c.shape[0] for c in codes_list]
    pcm = torch.empty(sum(n) * codec.hop, dtype=torch.float32, device="cuda")
    codec.decode_chunk(ids, n, np.concatenate(codes_list), pcm)
    host = pcm.cpu().numpy()
    out, at = [], 0
    for k in n:
        out.append(host[at * codec.hop:(at + k) * codec.hop])
        at += k
    for i in ids:
        codec.stream_close(i)
    return out


# --------------------------------------------------------------------------
def test_c1_fp32_streamed_and_full_vs_oracle():
    cfg = RI.get_config("c1")
    say("case c1 fp32: 1 stream x 50 frames, chunks", RI.C1_CHUNKS)
    w = RI.make_weights(cfg)
    codes = RI.stream_codes(cfg, 0, cfg["n_frames"])
    ref = oracle.Model(cfg, w).decode_full(codes)
    c = open_codec(cfg, w)
    sid = c.stream_open()
    streamed = run_lockstep(c, [sid], [codes], RI.C1_CHUNKS)[0]
    full = decode_full_gpu(c, [codes])[0]
    e_s, ac_s = rel_err(streamed, ref)
    e_f, _ = rel_err(full, ref)
    e_sf, _ = rel_err(streamed, full.astype(np.float64))
    say(f"c1 err/peak streamed {e_s:.3e} (AC-rel {ac_s:.3e}) full {e_f:.3e} streamed-vs-full {e_sf:.3e}")
    assert e_s <= 1e-5 and e_f <= 1e-5 and e_sf <= 1e-5


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_index_probe_gather_bit_exact(name):
    """Codebook indexing, bit for bit: integer probe tables (sums exact in
    fp16 and fp32) gathered for three ragged streams; the captured RVQ sum
    equals the oracle's.  The Fish-shaped decoder (projection not folded)
    also hands out the projected latent, with an identity projection equal
    to the oracle's bit for bit too; the others fold the projection into the
    input conv and refuse that capture."""
    cfg = RI.get_config(name, max_streams=8, max_frames_per_call=64) if name == "c3" \
        else RI.get_config(name)
    say("case index probe", name)
    w = RI.index_probe_weights(cfg)
    m = oracle.Model(cfg, w)
    n = [5, 8, 11]
    codes = np.concatenate([RI.stream_codes(cfg, b, n[b]) for b in range(3)])
    z_ref = m.rvq_sum(codes)
    assert np.array_equal(z_ref, np.round(z_ref))  # integer sums, exact everywhere
    c = open_codec(cfg, w)
    ids = [c.stream_open() for _ in n]
    pcm = torch.empty(sum(n) * c.hop, dtype=torch.float32, device="cuda")
    c.decode_chunk(ids, n, codes, pcm)
    cap = torch.empty(sum(n) * cfg["d_cb"], dtype=torch.float32, device="cuda")
    c.debug_capture(snr.CAPTURE_RVQ_SUM, cap)
    got = cap.cpu().numpy().reshape(sum(n), cfg["d_cb"]).astype(np.float64)
    assert np.array_equal(got, z_ref)
    lat = torch.empty(sum(n) * cfg["d_lat"], dtype=torch.float32, device="cuda")
    if cfg["tf_layers"]:
        _, u_ref, _ = m.stream().decode(codes, capture=True)  # rows are independent per frame
        c.debug_capture(snr.CAPTURE_LATENT, lat)
        got = lat.cpu().numpy().reshape(sum(n), cfg["d_lat"]).astype(np.float64)
        assert np.array_equal(got, u_ref)
    else:
        with pytest.raises(snr.CodecError):
            c.debug_capture(snr.CAPTURE_LATENT, lat)


def test_c2_streamed_ramp_vs_oracle_and_full():
    cfg = RI.get_config("c2")
    plan = [1, 2, 4, 8, 8, 8]
    B = 3
    say("case c2 bf16:", B, "streams, lockstep chunks", plan)
    w = RI.make_weights(cfg)
    T = sum(plan)
    codes = [RI.stream_codes(cfg, b, T) for b in range(B)]
    m = oracle.Model(cfg, w)
    refs = [m.decode_full(cd) for cd in codes]
    c = open_codec(cfg, w)
    ids = [c.stream_open() for _ in range(B)]
    streamed = run_lockstep(c, ids, codes, plan)
    full = decode_full_gpu(c, codes)
    tol = tol_for(cfg)
    for b in range(B):
        e, ac = rel_err(streamed[b], refs[b])
        ef, _ = rel_err(full[b], refs[b])
        esf, _ = rel_err(streamed[b], full[b].astype(np.float64))
        say(f"stream {b}: err/peak {e:.3e} (AC-rel {ac:.3e}) full {ef:.3e} "
            f"streamed-vs-full {esf:.3e} bitwise={np.array_equal(streamed[b], full[b])}")
        assert e <= tol and ef <= tol and esf <= tol


def test_single_frame_utterance_decodes():
    # a one-frame request whose final chunk is that one frame must decode
    cfg = RI.get_config("c2")
    say("case single-frame utterance")
    w = RI.make_weights(cfg)
    codes = RI.stream_codes(cfg, 7, 1)
    ref = oracle.Model(cfg, w).decode_full(codes)
    c = open_codec(cfg, w)
    got = decode_full_gpu(c, [codes])[0]
    torch.cuda.synchronize()
    assert got.shape == ref.shape
    assert rel_err(got, ref)[0] <= tol_for(cfg)


def test_ragged_mixed_batch_and_prefill():
    # streams at different positions with different chunk sizes in one call,
    # after a prefill; compared with the oracle's whole-utterance decode.
    cfg = RI.get_config("c2")
    say("case ragged batch + prefill")
    w = RI.make_weights(cfg)
    m = oracle.Model(cfg, w)
    c = open_codec(cfg, w)
    pre = [0, 5, 13, 2]
    steps = [[3, 1, 16, 2], [1, 7, 1, 9]]
    tot = [pre[b] + sum(s[b] for s in steps) for b in range(4)]
    codes = [RI.stream_codes(cfg, b, tot[b], part=9) for b in range(4)]
    ids = [c.stream_open() for _ in range(4)]
    for b in range(4):
        if pre[b]:
            c.stream_prefill(ids[b], codes[b][:pre[b]])
    at = list(pre)
    outs = [[] for _ in range(4)]
    for st in steps:
        packed = np.concatenate([codes[b][at[b]:at[b] + st[b]] for b in range(4)])
        pcm = torch.empty(sum(st) * c.hop, dtype=torch.float32, device="cuda")
        c.decode_chunk(ids, st, packed, pcm)
        host = pcm.cpu().numpy()
        o = 0
        for b in range(4):
            outs[b].append(host[o * c.hop:(o + st[b]) * c.hop])
            o += st[b]
            at[b] += st[b]
    H = c.hop
    for b in range(4):
        ref = m.decode_full(codes[b])[pre[b] * H:]
        got = np.concatenate(outs[b])
        e, ac = rel_err(got, ref)
        say(f"stream {b} pre={pre[b]}: err/peak {e:.3e} AC-rel {ac:.3e}")
        assert e <= tol_for(cfg)


def test_repeat_runs_bitwise_identical():
    cfg = RI.get_config("c2")
    say("case determinism")
    w = RI.make_weights(cfg)
    codes = [RI.stream_codes(cfg, b, 12) for b in range(5)]
    c = open_codec(cfg, w)
    a = decode_full_gpu(c, codes)
    b = decode_full_gpu(c, codes)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_three_buffer_tiles_bitwise_equal_double_buffered():
    """The three-stage-buffer half tiles change how K stages are staged, not
    the order of the sums: with K never split, steps whose frame-rate layers
    take them (96 streams x 8 frames: there a 128 x 64 tile reaches 1.5
    work-groups per CU and a 128 x 128 tile does not) decode bit for bit as
    with double-buffered tiles only; the second step continues from the
    first's state.  Stream 0 is also checked against the oracle."""
    cfg = RI.get_config("c2", max_streams=96, max_frames_per_call=1024, no_split_k=True)
    w = RI.make_weights(cfg)
    B, plan = 96, [8, 8]
    codes = [RI.stream_codes(cfg, b, sum(plan)) for b in range(B)]
    outs = []
    for variant in (cfg, dict(cfg, two_stage_buffers=True)):
        say(f"case three-buffer tiles: two_stage_buffers={variant.get('two_stage_buffers', False)}")
        codec = open_codec(variant, w)
        ids = [codec.stream_open() for _ in range(B)]
        outs.append(run_lockstep(codec, ids, codes, plan))
        codec.close()
    for x, y in zip(*outs):
        assert np.isfinite(x).all()
        assert np.array_equal(x, y)
    ref = oracle.Model(cfg, w).decode_full(codes[0])
    e, ac = rel_err(outs[0][0], ref)
    say(f"stream 0: err/peak {e:.3e} AC-rel {ac:.3e}")
    assert e <= tol_for(cfg)


def test_tall_tiles_bitwise_equal_128_row_tiles():
    """The 160-row tiles change which rows a work-group holds, not the order
    of any sum: 112 streams x 8 frames (896 frames, where the 128-row tiles of
    the stage-1 convs, the stage-2 ConvT and the stage-2 residual units would
    overflow whole rounds of two work-groups per CU by a few) decode bit for
    bit as with 128-row tiles only, over two steps; stream 0 is also checked
    against the oracle."""
    cfg = RI.get_config("c2", max_streams=112, max_frames_per_call=1024, no_split_k=True)
    B, plan = 112, [8, 8]
    F = B * plan[0]
    assert snr.conv_plan(F * 40, 256, 256, 7, flags=snr.FLAG_NO_SPLIT_K)[0] == "h160x128k64"
    assert snr.conv_plan(F * 8, 5 * 256, 512, 2, flags=snr.FLAG_NO_SPLIT_K)[0] == "h160x128k64"
    w = RI.make_weights(cfg)
    codes = [RI.stream_codes(cfg, b, sum(plan)) for b in range(B)]
    outs = []
    for variant in (cfg, dict(cfg, no_tall_tiles=True)):
        say(f"case tall tiles: no_tall_tiles={variant.get('no_tall_tiles', False)}")
        codec = open_codec(variant, w)
        ids = [codec.stream_open() for _ in range(B)]
        outs.append(run_lockstep(codec, ids, codes, plan))
        codec.close()
    for x, y in zip(*outs):
        assert np.isfinite(x).all()
        assert np.array_equal(x, y)
    ref = oracle.Model(cfg, w).decode_full(codes[0])
    e, ac = rel_err(outs[0][0], ref)
    say(f"stream 0: err/peak {e:.3e} AC-rel {ac:.3e}")
    assert e <= tol_for(cfg)


def test_c4_full_scale_sampled_parity():
    """The headline workload: 128 streams at staggered offsets (prefilled),
    steps of mixed chunk sizes {1,2,4,8,16}; sampled streams' chunks are
    checked against the oracle, which decodes each from its left-context
    window (exact, since an output frame depends on at most L earlier frames)."""
    cfg = RI.get_config("c4")
    steps = 3
    say("case c4: 128 streams, offsets 0..500, steps", steps)
    w = RI.make_weights(cfg)
    c = open_codec(cfg, w)
    Bn = cfg["n_streams"]
    off = RI.c4_offsets(cfg)
    ids = [c.stream_open() for _ in range(Bn)]
    hist = [RI.stream_codes(cfg, b, int(off[b]), part=0) for b in range(Bn)]
    for b in range(Bn):
        if off[b]:
            c.stream_prefill(ids[b], hist[b])
    # sampled streams: the smallest and largest offsets, one stream per chunk
    # bucket of the last step, the rest seeded; every step of each is checked
    n_last = RI.c4_chunk_sizes(cfg, steps - 1)
    sample = {int(np.argmin(off)), int(np.argmax(off))}
    sample |= {int(np.flatnonzero(n_last == v)[0]) for v in cfg["buckets"]}
    for b in np.random.default_rng(3).permutation(Bn):
        if len(sample) >= 8:
            break
        sample.add(int(b))
    sample = sorted(sample)
    outs = []
    for j in range(steps):
        n = RI.c4_chunk_sizes(cfg, j)
        step_codes = [RI.stream_codes(cfg, b, int(n[b]), part=1 + j) for b in range(Bn)]
        pcm = torch.empty(int(n.sum()) * c.hop, dtype=torch.float32, device="cuda")
        c.decode_chunk(ids, n, np.concatenate(step_codes), pcm)
        starts = [hist[b].shape[0] for b in range(Bn)]
        for b in range(Bn):
            hist[b] = np.concatenate([hist[b], step_codes[b]])
        outs.append((n, starts, pcm.cpu().numpy()))
    H = c.hop
    L = analytic_left_context(cfg) + 1
    m = oracle.Model(cfg, w)
    buckets = set()
    for j, (n, starts, host) in enumerate(outs):
        cu = np.concatenate([[0], np.cumsum(n)])
        for b in sample:
            start = starts[b]
            w0 = max(0, start - L)
            ref = m.stream(w0).decode(hist[b][w0:start + int(n[b])])[(start - w0) * H:]
            got = host[cu[b] * H:cu[b + 1] * H]
            e, ac = rel_err(got, ref)
            say(f"c4 step {j} stream {b} offset {off[b]} pos {start} n {n[b]}: "
                f"err/peak {e:.3e} AC-rel {ac:.3e}")
            assert e <= tol_for(cfg)
            buckets.add(int(n[b]))
    assert buckets == set(cfg["buckets"])


# --------------------------------------------------------------------------
# Windowed causal transformer (Fish-DAC-shaped decoder)
# --------------------------------------------------------------------------
def test_c3_transformer_streamed_vs_oracle():
    """Two streams, 8-frame chunks past the 32-frame window (ring wraps),
    plus a third stream joining late in 1-frame and ramp chunks."""
    cfg = RI.get_config("c3", max_streams=8, max_frames_per_call=64)
    say("case c3: transformer + conv decoder, chunks of 8 past the window")
    w = RI.make_weights(cfg)
    m = oracle.Model(cfg, w)
    c = open_codec(cfg, w)
    plan = [8] * 5 + [3]
    T = sum(plan)
    codes = [RI.stream_codes(cfg, b, T) for b in range(2)]
    ids = [c.stream_open() for _ in range(2)]
    got = run_lockstep(c, ids, codes, plan)
    # decoder input after the transformer for the last step, both streams
    cap = torch.empty(2 * plan[-1] * cfg["d_lat"], dtype=torch.float32, device="cuda")
    c.debug_capture(snr.CAPTURE_DEC_INPUT, cap)
    cap = cap.cpu().numpy().reshape(2, plan[-1], cfg["d_lat"])
    for b in range(2):
        pcm_ref, _, x_ref = m.stream().decode(codes[b], capture=True)
        e, ac = rel_err(got[b], pcm_ref)
        ex, _ = rel_err(cap[b], x_ref[-plan[-1]:])
        say(f"c3 stream {b}: err/peak {e:.3e} (AC-rel {ac:.3e}); transformer output err/peak {ex:.3e}")
        assert e <= tol_for(cfg)
        assert ex <= tol_for(cfg)
    # a late stream with ramp chunks, decoded in the same calls as stream 0
    c2 = open_codec(cfg, w)
    late_codes = RI.stream_codes(cfg, 5, 15)
    a, bb = c2.stream_open(), c2.stream_open()
    outs = []
    at = 0
    for n in [1, 2, 4, 8]:
        pcm = torch.empty((n + 8) * c2.hop, dtype=torch.float32, device="cuda")
        c2.decode_chunk([a, bb], [n, 8], np.concatenate([late_codes[at:at + n], codes[0][:8]]), pcm)
        outs.append(pcm.cpu().numpy()[: n * c2.hop])
        at += n
    e, _ = rel_err(np.concatenate(outs), m.decode_full(late_codes))
    say(f"c3 late ramp stream: err/peak {e:.3e}")
    assert e <= tol_for(cfg)


def test_c3_full_scale_sampled_parity():
    """64 streams x 300 frames in 8-frame chunks (F = 512 per step); sampled
    chunks are checked against the oracle decoding the left-context window
    (135 frames for this decoder) at the true absolute positions."""
    cfg = RI.get_config("c3")
    say("case c3 full scale: 64 streams x 300 frames, 8-frame chunks")
    w = RI.make_weights(cfg)
    c = open_codec(cfg, w)
    Bn, T = cfg["n_streams"], cfg["n_frames"]
    codes = [RI.stream_codes(cfg, b, T) for b in range(Bn)]
    ids = [c.stream_open() for _ in range(Bn)]
    H = c.hop
    keep = {}
    at = 0
    for k, n in enumerate(RI.C3_CHUNKS):
        pcm = torch.empty(Bn * n * H, dtype=torch.float32, device="cuda")
        c.decode_chunk(ids, [n] * Bn, np.concatenate([cd[at:at + n] for cd in codes]), pcm)
        if k in (2, 30):
            keep[k] = (at, n, pcm.cpu().numpy())
        at += n
    m = oracle.Model(cfg, w)
    L = analytic_left_context(cfg) + 1
    for k, b in ((2, 17), (30, 3), (30, 62)):
        start, n, host = keep[k]
        w0 = max(0, start - L)
        ref = m.stream(w0).decode(codes[b][w0:start + n])[(start - w0) * H:]
        got = host[b * n * H:(b + 1) * n * H]
        e, ac = rel_err(got, ref)
        say(f"c3 chunk {k} stream {b} pos {start}: err/peak {e:.3e} AC-rel {ac:.3e}")
        assert e <= tol_for(cfg)


def test_c3_query_blocks_short_window_and_graph():
    """The attention's query blocks (up to 16 frames of one stream per
    work-group): two streams with ragged chunks of up to 40 frames in one call
    (three blocks of one stream), a 5-frame window whose ring wraps every 4
    frames, and the same decode through decode_chunk_graph (blocks listed up to
    the frame bucket's bound, the spare ones empty).  Against the oracle: each
    stream's PCM, and the transformer's output of the last call."""
    cfg = RI.get_config("c3", max_streams=4, max_frames_per_call=96, tf_window=5)
    w = RI.make_weights(cfg)
    m = oracle.Model(cfg, w)
    plans = [[40, 3, 1, 20], [1, 17, 5, 16]]  # per stream, decoded in the same calls
    codes = [RI.stream_codes(cfg, b, sum(plans[b]), part=13) for b in range(2)]
    refs = [m.stream().decode(codes[b], capture=True) for b in range(2)]
    say("case c3 query blocks: window 5, chunks", plans)
    for use_graph in (False, True):
        c = open_codec(cfg, w)
        ids = [c.stream_open() for _ in range(2)]
        outs, at = [[], []], [0, 0]
        for k in range(len(plans[0])):
            n = [plans[0][k], plans[1][k]]
            packed = np.concatenate([codes[b][at[b]:at[b] + n[b]] for b in range(2)])
            pcm = torch.empty(sum(n) * c.hop, dtype=torch.float32, device="cuda")
            if use_graph:
                c.decode_chunk_graph(ids, n, packed, pcm)
            else:
                c.decode_chunk(ids, n, packed, pcm)
            host = pcm.cpu().numpy()
            outs[0].append(host[:n[0] * c.hop])
            outs[1].append(host[n[0] * c.hop:sum(n) * c.hop])
            at = [at[b] + n[b] for b in range(2)]
        if not use_graph:
            cap = torch.empty(sum(n) * cfg["d_lat"], dtype=torch.float32, device="cuda")
            c.debug_capture(snr.CAPTURE_DEC_INPUT, cap)
            cap = cap.cpu().numpy().reshape(sum(n), cfg["d_lat"])
        for b in range(2):
            pcm_ref, _, x_ref = refs[b]
            e, ac = rel_err(np.concatenate(outs[b]), pcm_ref)
            say(f"c3 query blocks {'graph' if use_graph else 'eager'} stream {b}: "
                f"err/peak {e:.3e} (AC-rel {ac:.3e})")
            assert e <= tol_for(cfg)
            if not use_graph:
                rows = cap[:n[0]] if b == 0 else cap[n[0]:]
                ex, _ = rel_err(rows, x_ref[-n[b]:])
                say(f"  transformer output of the last call: err/peak {ex:.3e}")
                assert ex <= tol_for(cfg)
        c.close()


# --------------------------------------------------------------------------
# Fused per-stage kernels vs the per-layer launch sequence: same arithmetic
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["c2", "c3"])
def test_fused_stages_bitwise_equal_per_layer(name):
    cfg = RI.get_config(name, max_streams=8, max_frames_per_call=128)
    say("case fused vs per-layer", name)
    w = RI.make_weights(cfg)
    fused = open_codec(cfg, w)
    layer = open_codec(dict(cfg, per_layer=True), w)
    steps = [[1, 3, 16, 2, 1], [8, 1, 1, 5, 2], [2, 16, 4, 1, 7]]
    codes = [RI.stream_codes(cfg, b, sum(s[b] for s in steps), part=3) for b in range(5)]
    outs, states = {}, {}
    for tag, c in (("fused", fused), ("layer", layer)):
        ids = [c.stream_open() for _ in range(5)]
        at = [0] * 5
        res = []
        for st in steps:
            packed = np.concatenate([codes[b][at[b]:at[b] + st[b]] for b in range(5)])
            pcm = torch.empty(sum(st) * c.hop, dtype=torch.float32, device="cuda")
            c.decode_chunk(ids, st, packed, pcm)
            res.append(pcm.cpu().numpy())
            for b in range(5):
                at[b] += st[b]
        outs[tag] = np.concatenate(res)
        states[tag] = [c.read_state(i) for i in ids]
    # the saved left contexts too: the fused stages write their own and the
    # last one saves the per-layer ones; the per-layer path saves all in one launch
    for a, b in zip(states["fused"], states["layer"]):
        assert np.array_equal(a, b)
    d = np.abs(outs["fused"] - outs["layer"])
    say(f"{name}: max |fused - per-layer| = {d.max():.3e}")
    if d.max() > 0:
        hop = fused.hop
        bad = np.nonzero(d)[0]
        say(f"  {len(bad)} of {d.size} samples differ; first at sample {bad[0]} "
            f"(frame {bad[0] // hop}, offset {bad[0] % hop}); last {bad[-1]}")
        off = np.bincount(bad % hop, minlength=hop)
        say(f"  per-offset counts (first 64): {off[:64].tolist()}")
    assert np.array_equal(outs["fused"], outs["layer"])


# --------------------------------------------------------------------------
# Offline ceiling: whole-utterance decode of 128 ragged utterances
# --------------------------------------------------------------------------
def ramp_plan(T, ramp=(1, 2, 4), steady=8):
    """Chunk sizes ramp[0], ramp[1], ..., then `steady`, the last chunk the
    remainder (the streamed workload's schedule for an utterance of T frames)."""
    plan, at = [], 0
    for n in list(ramp) + [steady] * T:
        if at >= T:
            break
        plan.append(min(n, T - at))
        at += plan[-1]
    return plan


def test_c5_offline_whole_vs_streamed_vs_oracle():
    """128 utterances of 50..500 frames. (1) Whole-utterance decode, calls
    grouping whole utterances up to the per-call frame limit (valid frames
    only: the ragged batch needs no padding). (2) The same codes streamed
    with the ramp 1, 2, 4, 8, ... in lockstep, streams dropping out as they
    end. (1) and (2) agree within the bf16 bound; (3) sampled windows of both
    agree with the oracle; (4) a padded decode (pad code 0 up to 500 frames)
    gives the same valid samples as the ragged one."""
    cfg = RI.get_config("c5")
    w = RI.make_weights(cfg)
    c = open_codec(cfg, w)
    H = c.hop
    Bn = cfg["n_streams"]
    lens = RI.c5_lengths(cfg)
    codes = [RI.stream_codes(cfg, b, int(lens[b]), part=0) for b in range(Bn)]
    say(f"case c5: {Bn} utterances, {int(lens.sum())} frames, lengths {lens.min()}..{lens.max()}")

    # (1) whole-utterance decode, grouped by the per-call limit
    maxF = cfg["max_frames_per_call"]
    full = [None] * Bn
    b0 = 0
    while b0 < Bn:
        b1, tot = b0, 0
        while b1 < Bn and tot + lens[b1] <= maxF:
            tot += int(lens[b1])
            b1 += 1
        outs = decode_full_gpu(c, codes[b0:b1])
        for i, o in enumerate(outs):
            full[b0 + i] = o
        b0 = b1

    # (2) streamed in lockstep with per-stream ramps
    plans = [ramp_plan(int(t)) for t in lens]
    ids = [c.stream_open() for _ in range(Bn)]
    got = [[] for _ in range(Bn)]
    at = [0] * Bn
    for j in range(max(len(p) for p in plans)):
        act = [b for b in range(Bn) if j < len(plans[b])]
        n = [plans[b][j] for b in act]
        packed = np.concatenate([codes[b][at[b]:at[b] + k] for b, k in zip(act, n)])
        pcm = torch.empty(sum(n) * H, dtype=torch.float32, device="cuda")
        c.decode_chunk([ids[b] for b in act], n, packed, pcm)
        host = pcm.cpu().numpy()
        o = 0
        for b, k in zip(act, n):
            got[b].append(host[o * H:(o + k) * H])
            o += k
            at[b] += k
    for i in ids:
        c.stream_close(i)
    worst = 0.0
    for b in range(Bn):
        s = np.concatenate(got[b])
        assert s.shape == full[b].shape
        e, _ = rel_err(s, full[b])
        worst = max(worst, e)
        assert e <= tol_for(cfg), f"stream {b}: streamed vs full err/peak {e:.3e}"
    say(f"c5 streamed vs full: worst err/peak {worst:.3e}")

    # (3) sampled windows against the oracle
    m = oracle.Model(cfg, w)
    L = analytic_left_context(cfg) + 1
    sample = sorted({int(np.argmin(lens)), int(np.argmax(lens))} |
                    {int(b) for b in np.random.default_rng(5).choice(Bn, 2, replace=False)})
    for b in sample:
        T = int(lens[b])
        for start in sorted({0, T // 2, T - 8}):
            w0 = max(0, start - L)
            ref = m.stream(w0).decode(codes[b][w0:start + 8])[(start - w0) * H:]
            for tag, src in (("full", full[b]), ("streamed", np.concatenate(got[b]))):
                e, ac = rel_err(src[start * H:(start + 8) * H], ref)
                say(f"c5 stream {b} len {T} frames {start}..{start + 8} {tag}: "
                    f"err/peak {e:.3e} AC-rel {ac:.3e}")
                assert e <= tol_for(cfg)

    # (4) padded decode: 32 streams padded with code 0 to the longest length
    grp = list(range(32))
    Tmax = cfg["max_len"]
    pad = [np.concatenate([codes[b], np.zeros((Tmax - lens[b], cfg["K"]), np.int32)])
           for b in grp]
    outs = decode_full_gpu(c, pad)
    same = 0
    for b, o in zip(grp, outs):
        v = o[:int(lens[b]) * H]
        e, _ = rel_err(v, full[b])
        assert e <= tol_for(cfg), f"stream {b}: padded vs ragged err/peak {e:.3e}"
        same += int(np.array_equal(v, full[b]))
    say(f"c5 padded vs ragged: {same} of {len(grp)} streams bitwise equal")
    c.close()


# --------------------------------------------------------------------------
# Stateless window re-decode (comparison variant)
# --------------------------------------------------------------------------
def test_stateless_window_redecode_matches_stateful_c2():
    """The pages' stateless variant decodes each chunk again from zero state
    together with up to 16 earlier frames and keeps the new frames' samples.
    For the Qwen-shaped decoder (left context 11 frames <= 16) that equals the
    stateful decode in exact arithmetic: here within the bf16 bound, against
    both the GPU's stateful decode and the oracle.  The window lengths are the
    ones the chunk policy predicts."""
    from oracle import policy
    cfg = RI.get_config("c2")
    w = RI.make_weights(cfg)
    c = open_codec(cfg, w)
    H = c.hop
    B, T = 4, 60
    plan = policy.chunk_plan(T)
    codes = [RI.stream_codes(cfg, b, T, part=0) for b in range(B)]
    say("case stateless c2: plan", plan)
    ids = [c.stream_open() for _ in range(B)]
    stateful = run_lockstep(c, ids, codes, plan)
    for i in ids:
        c.stream_close(i)
    got = [[] for _ in range(B)]
    wins, at = set(), 0
    for n in plan:
        w0 = max(0, at - 16)
        wins.add(at + n - w0)
        outs = decode_full_gpu(c, [cb[w0:at + n] for cb in codes])
        for b in range(B):
            got[b].append(outs[b][(at - w0) * H:])
        at += n
    assert wins <= set(policy.window_frame_counts(16)), sorted(wins)
    m = oracle.Model(cfg, w)
    for b in range(B):
        g = np.concatenate(got[b])
        e, _ = rel_err(g, stateful[b])
        assert e <= tol_for(cfg), f"stream {b}: stateless vs stateful err/peak {e:.3e}"
    ref = m.stream().decode(codes[0])
    e, ac = rel_err(np.concatenate(got[0]), ref)
    say(f"stateless stream 0 vs oracle: err/peak {e:.3e} AC-rel {ac:.3e}; windows {sorted(wins)}")
    assert e <= tol_for(cfg)
    c.close()


# --------------------------------------------------------------------------
# Graph replay (one launch per step for a repeated chunk shape)
# --------------------------------------------------------------------------
def test_graph_replay_vs_eager_and_oracle():
    """decode_chunk_graph runs each step as the graph of its frame bucket
    (next power of two up to 32 frames), the spare frames on a pad stream.
    Replays are interleaved with eager decode_chunk steps of the same codes
    and with host synchronisations; bucket shapes change and come back.  A
    step whose frame count is a bucket size runs the eager launch sequence
    exactly: bit for bit the eager PCM.  A padded step may split K
    differently: within the bound of the eager PCM.  Every graph stream
    against the oracle's whole-utterance decode."""
    cfg = RI.get_config("c2")
    w = RI.make_weights(cfg)
    c = open_codec(cfg, w)
    H = c.hop
    B = 4
    plan = [1, 2, 4, 8, 8, 8, 8, 3, 8, 8, 2, 8, 8, 5, 3]
    T = sum(plan)
    codes = [RI.stream_codes(cfg, b, T, part=7) for b in range(B)]
    ids_g = [c.stream_open() for _ in range(B)]
    ids_e = [c.stream_open() for _ in range(B)]
    pcm_g = torch.empty(max(plan) * B * H, dtype=torch.float32, device="cuda")
    at = 0
    say("case graph replay: plan", plan)
    graph_out = [[] for _ in range(B)]
    for k, n in enumerate(plan):
        packed = np.concatenate([cb[at:at + n] for cb in codes])
        c.decode_chunk_graph(ids_g, [n] * B, packed, pcm_g)
        torch.cuda.synchronize()
        got = pcm_g[:n * B * H].cpu().numpy()
        pcm_e = torch.empty(n * B * H, dtype=torch.float32, device="cuda")
        c.decode_chunk(ids_e, [n] * B, packed, pcm_e)
        ref = pcm_e.cpu().numpy()
        F = n * B
        exact = F & (F - 1) == 0  # a bucket size: no pad stream
        if exact:
            assert np.array_equal(got, ref), f"step {k} (n={n}): graph differs from eager"
        for b in range(B):
            e, _ = rel_err(got[b * n * H:(b + 1) * n * H], ref[b * n * H:(b + 1) * n * H].astype(np.float64))
            assert e <= tol_for(cfg), f"step {k} stream {b}: graph vs eager {e:.3e}"
            graph_out[b].append(got[b * n * H:(b + 1) * n * H])
        at += n
    info = c.get_info()
    say(f"graphs captured {info.graph_captures}, replays {info.graph_replays}")
    keys = set()
    for n in plan:  # (streams incl. the pad stream, bucket frames)
        F = n * B
        Fb = 1 << (F - 1).bit_length() if F <= 32 else (F + 31) // 32 * 32
        keys.add((B + (Fb > F), Fb))
    assert info.graph_captures == len(keys) and info.graph_replays == len(plan) - len(keys)
    m = oracle.Model(cfg, w)
    for b in range(B):
        e, ac = rel_err(np.concatenate(graph_out[b]), m.decode_full(codes[b]))
        say(f"graph stream {b} vs oracle: err/peak {e:.3e} AC-rel {ac:.3e}")
        assert e <= tol_for(cfg)
    c.close()


# --------------------------------------------------------------------------
# ELU decoder (per-layer path everywhere, residual-unit GEMM included)
# --------------------------------------------------------------------------
def test_elu_decoder_vs_oracle():
    """The Qwen-shaped decoder with ELU instead of Snake (the selectable
    activation): no fused stage applies, so every conv runs on the per-layer
    kernels; 8 streams x 16 frames put enough rows into stage 2 for its
    residual units to run as single launches.  Against the oracle."""
    cfg = RI.get_config("c2", act="elu")
    w = RI.make_weights(cfg)
    c = open_codec(cfg, w)
    B = 8
    plan = [3, 16, 5]
    codes = [RI.stream_codes(cfg, b, sum(plan), part=11) for b in range(B)]
    say("case ELU decoder: plan", plan)
    ids = [c.stream_open() for _ in range(B)]
    got = run_lockstep(c, ids, codes, plan)
    m = oracle.Model(cfg, w)
    for b in (0, 5):
        ref = m.stream().decode(codes[b])
        e, ac = rel_err(got[b], ref)
        say(f"ELU stream {b}: err/peak {e:.3e} AC-rel {ac:.3e}")
        assert e <= tol_for(cfg)
    c.close()


# --------------------------------------------------------------------------
# Fused stages: the per-stream tile table in LDS (steps of up to 512 streams)
# and the search in global memory beyond it give the same PCM.  K is not
# split (a split depends on the step's rows and changes the summation order),
# so a stream's arithmetic does not depend on the other streams of its step.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("B", [512, 520])
def test_fused_stage_stream_table_lds_and_global_agree(B):
    # 512: the full LDS table against halves of it; 520: the global search
    cfg = RI.get_config("c2", max_streams=B, max_frames_per_call=2 * B, no_split_k=True)
    say("case stream table", B, "streams")
    w = RI.make_weights(cfg)
    codec = open_codec(cfg, w)
    n = [1 + (b % 2) for b in range(B)]
    codes = [RI.stream_codes(cfg, b, n[b], part=5) for b in range(B)]
    whole = decode_full_gpu(codec, codes)          # one call of all B streams
    halves = decode_full_gpu(codec, codes[:B // 2]) + decode_full_gpu(codec, codes[B // 2:])
    for b in range(B):
        assert np.array_equal(whole[b], halves[b]), b
    codec.close()
