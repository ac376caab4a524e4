"""Pins of the fp64 oracle against things other than itself.

Each layer is checked against a library routine (torch fp64 on the CPU,
numpy), a closed form, an invariant or brute force; the whole decoder is
checked against an independent torch composition on the tiny configuration,
the streaming invariant (streamed == whole-utterance, bitwise) and the
analytic receptive field.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import rvq_inputs as RI
from _util import analytic_first_frame, analytic_left_context

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def t64(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


# --------------------------------------------------------------------------
# Convolutions
# --------------------------------------------------------------------------
@pytest.mark.parametrize("k,d,Ci,Co,T", [(7, 1, 5, 4, 13), (7, 3, 3, 6, 40), (1, 1, 8, 8, 9),
                                          (2, 1, 4, 3, 5)])
def test_causal_conv_matches_torch_conv1d(k, d, Ci, Co, T):
    H = (k - 1) * d
    x = rng.normal(size=(Ci, H + T))
    W = rng.normal(size=(Co, Ci, k))
    b = rng.normal(size=Co)
    y = oracle.causal_conv(x, W, b, d)
    ref = F.conv1d(t64(x)[None], t64(W), t64(b), dilation=d)[0].numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_causal_conv_brute_force_zero_context():
    # y[o][t] = b[o] + sum_j sum_c W[o][c][j] x[c][t - (k-1-j) d], x = 0 before t = 0
    k, d, Ci, Co, T = 7, 3, 2, 3, 25
    x = rng.normal(size=(Ci, T))
    W = rng.normal(size=(Co, Ci, k))
    b = rng.normal(size=Co)
    xe = np.concatenate([np.zeros((Ci, (k - 1) * d)), x], axis=1)
    y = oracle.causal_conv(xe, W, b, d)
    for o in range(Co):
        for t in range(T):
            acc = b[o]
            for j in range(k):
                tt = t - (k - 1 - j) * d
                if tt >= 0:
                    acc += sum(W[o, c, j] * x[c, tt] for c in range(Ci))
            assert abs(acc - y[o, t]) < 1e-12


@pytest.mark.parametrize("s,Ci,Co,T", [(4, 3, 5, 6), (5, 2, 2, 1), (2, 4, 3, 9), (8, 3, 2, 3)])
def test_conv_transpose_matches_torch(s, Ci, Co, T):
    W = rng.normal(size=(Ci, Co, 2 * s))
    b = rng.normal(size=Co)
    x = rng.normal(size=(Ci, T))
    prev = rng.normal(size=(Ci, 1))
    # zero left context: torch output cropped to the first T s samples
    y0 = oracle.conv_transpose(np.concatenate([np.zeros((Ci, 1)), x], 1), W, b, s)
    ref0 = F.conv_transpose1d(t64(x)[None], t64(W), t64(b), stride=s)[0].numpy()[:, : T * s]
    np.testing.assert_allclose(y0, ref0, rtol=1e-12, atol=1e-12)
    # nonzero left context = the previous input sample: shift by one input
    y1 = oracle.conv_transpose(np.concatenate([prev, x], 1), W, b, s)
    ref1 = F.conv_transpose1d(t64(np.concatenate([prev, x], 1))[None], t64(W), t64(b),
                              stride=s)[0].numpy()[:, s: s + T * s]
    np.testing.assert_allclose(y1, ref1, rtol=1e-12, atol=1e-12)


def test_conv_transpose_scatter_definition():
    # out[o][i s + j] += x[c][i] W[c][o][j] for every input i and tap j
    s, Ci, Co, T = 3, 2, 2, 4
    W = rng.normal(size=(Ci, Co, 2 * s))
    b = rng.normal(size=Co)
    x = rng.normal(size=(Ci, T))
    full = np.zeros((Co, (T + 1) * s + s))
    for c in range(Ci):
        for i in range(T):
            for j in range(2 * s):
                full[:, i * s + j] += x[c, i] * W[c, :, j]
    full += b[:, None]
    y = oracle.conv_transpose(np.concatenate([np.zeros((Ci, 1)), x], 1), W, b, s)
    np.testing.assert_allclose(y, full[:, : T * s], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Elementwise maps
# --------------------------------------------------------------------------
def test_snake_special_values():
    alpha = np.array([0.5, 1.0, 1.5])
    # Snake(0) = 0
    assert np.all(oracle.snake(np.zeros((3, 4)), alpha) == 0.0)
    # at alpha x = pi/2 the sine is 1: Snake(x) = x + 1/alpha
    x = (np.pi / 2 / alpha)[:, None] * np.ones((3, 2))
    np.testing.assert_allclose(oracle.snake(x, alpha), x + (1 / alpha)[:, None], rtol=1e-14)
    # period pi/alpha of the added term: Snake(x + pi/alpha) - Snake(x) = pi/alpha
    x = rng.normal(size=(3, 7))
    sh = (np.pi / alpha)[:, None]
    np.testing.assert_allclose(oracle.snake(x + sh, alpha) - oracle.snake(x, alpha),
                               np.broadcast_to(sh, x.shape), rtol=1e-9, atol=1e-12)
    # small x: Snake(x) = x + alpha x^2 - alpha^3 x^4 / 3 + O(x^6)
    x = np.full((3, 1), 1e-3)
    np.testing.assert_allclose(oracle.snake(x, alpha)[:, 0],
                               1e-3 + alpha * 1e-6 - alpha ** 3 * 1e-12 / 3, rtol=1e-14)


def test_elu_gelu_layernorm_match_torch():
    x = rng.normal(size=257) * 3
    np.testing.assert_allclose(oracle.elu(x), F.elu(t64(x)).numpy(), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(oracle.gelu(x), F.gelu(t64(x)).numpy(), rtol=1e-13, atol=1e-15)
    g, b = rng.normal(size=257), rng.normal(size=257)
    ref = F.layer_norm(t64(x)[None], (257,), t64(g), t64(b), eps=1e-5)[0].numpy()
    np.testing.assert_allclose(oracle.layer_norm(x, g, b), ref, rtol=1e-12, atol=1e-13)


def test_linear_matches_numpy():
    W, b, x = rng.normal(size=(9, 13)), rng.normal(size=9), rng.normal(size=13)
    np.testing.assert_allclose(oracle.linear(W, b, x), W @ x + b, rtol=1e-13)


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------
def test_rope_complex_rotation_and_relative_position():
    H, hd = 3, 8
    x = rng.normal(size=H * hd)
    for pos in (0, 1, 17, 500):
        y = oracle.rope(x, H, hd, pos)
        for h in range(H):
            v = x[h * hd:(h + 1) * hd]
            z = v[: hd // 2] + 1j * v[hd // 2:]
            theta = pos * 10000.0 ** (-np.arange(hd // 2) * 2.0 / hd)
            zr = z * np.exp(1j * theta)
            np.testing.assert_allclose(y[h * hd: h * hd + hd // 2], zr.real, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(y[h * hd + hd // 2:(h + 1) * hd], zr.imag, rtol=1e-12,
                                       atol=1e-12)
    # the rotated dot product depends only on the position difference
    q, k = rng.normal(size=hd), rng.normal(size=hd)
    a = oracle.rope(q, 1, hd, 40) @ oracle.rope(k, 1, hd, 33)
    b = oracle.rope(q, 1, hd, 107) @ oracle.rope(k, 1, hd, 100)
    assert abs(a - b) < 1e-10


def test_window_attention_matches_sdpa_with_band_mask():
    H, hd, W, T = 2, 8, 4, 11
    q = rng.normal(size=(T, H * hd))
    k = rng.normal(size=(T, H * hd))
    v = rng.normal(size=(T, H * hd))
    out = np.stack([oracle.window_attention(q[t], k[max(0, t - W + 1): t + 1],
                                            v[max(0, t - W + 1): t + 1], H, hd) for t in range(T)])
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    mask = torch.from_numpy((j <= i) & (j > i - W))
    qt = t64(q).view(T, H, hd).transpose(0, 1)
    kt = t64(k).view(T, H, hd).transpose(0, 1)
    vt = t64(v).view(T, H, hd).transpose(0, 1)
    ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask).transpose(0, 1).reshape(T, -1)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# RVQ gather-and-sum
# --------------------------------------------------------------------------
def test_rvq_sum_index_probe_exact():
    cfg = RI.get_config("c2")
    w = RI.index_probe_weights(cfg)
    m = oracle.Model(cfg, w)
    codes = RI.stream_codes(cfg, 0, 37)
    z = m.rvq_sum(codes)
    # closed form of the probe tables, summed exactly in integers
    d = np.arange(cfg["d_cb"])
    ref = np.zeros((37, cfg["d_cb"]), np.int64)
    for k in range(cfg["K"]):
        ref += ((7 * codes[:, k:k + 1].astype(np.int64) + 3 * d + 11 * k) % 251) - 125
    assert np.array_equal(z, ref.astype(np.float64))
    # and the numpy gather of the random tables
    w2 = RI.make_weights(cfg)
    m2 = oracle.Model(cfg, w2)
    z2 = m2.rvq_sum(codes)
    ref2 = sum(w2[f"rvq.codebook.{k}"].astype(np.float64)[codes[:, k]] for k in range(cfg["K"]))
    np.testing.assert_allclose(z2, ref2, rtol=1e-13, atol=1e-15)


def test_rvq_rejects_out_of_range_code():
    facts = json.load(open(os.path.join(GOLD, "frame_facts.json")))["qwen3_tts"]
    cfg = RI.get_config("c1")
    m = oracle.Model(cfg, RI.make_weights(cfg))
    codes = RI.stream_codes(cfg, 0, 3)
    codes[1, 2] = facts["eos_code"]  # EOS 2150 lies outside any codebook of this size
    with pytest.raises(ValueError):
        m.stream().decode(codes)


# --------------------------------------------------------------------------
# Whole decoder on the tiny configuration: independent torch composition
# --------------------------------------------------------------------------
def torch_decode_full(cfg, w, codes, taps=None):
    """Whole-utterance decode of the network, composed from torch fp64 library
    ops (conv1d / conv_transpose1d with explicit causal padding).  ``taps``,
    a dict, receives every conv operand [rows, C] keyed like the oracle's
    decode_tap (3 i: stage i's transposed-conv input; 3 i + 1 + j: its
    residual unit j's input; 3 S: the final conv's input)."""
    taps = {} if taps is None else taps
    T = codes.shape[0]
    W = {k: t64(v) for k, v in w.items()}
    z = sum(W[f"rvq.codebook.{k}"][torch.from_numpy(codes[:, k].astype(np.int64))]
            for k in range(cfg["K"]))
    u = z @ W["rvq.proj.weight"].T + W["rvq.proj.bias"]            # [T, d_lat]
    x = u.T[None]                                                    # [1, C, T]

    def act(x, a):
        if cfg["act"] == "elu":
            return F.elu(x)
        a = a[None, :, None]
        return x + torch.sin(a * x) ** 2 / a

    def cconv(x, wt, bt, d):
        k = wt.shape[-1]
        return F.conv1d(F.pad(x, ((k - 1) * d, 0)), wt, bt, dilation=d)

    x = cconv(x, W["dec.in_conv.weight"], W["dec.in_conv.bias"], 1)
    for i, s in enumerate(cfg["strides"]):
        p = f"dec.stage.{i}."
        n = x.shape[-1]
        a = act(x, W[p + "snake.alpha"])
        taps[3 * i] = a[0].T.numpy()
        x = F.conv_transpose1d(a, W[p + "convT.weight"], W[p + "convT.bias"], stride=s)[..., : n * s]
        for j, d in enumerate((1, 3)):
            q = p + f"ru.{j}."
            a = act(x, W[q + "snake1.alpha"])
            taps[3 * i + 1 + j] = a[0].T.numpy()
            h = cconv(a, W[q + "conv7.weight"], W[q + "conv7.bias"], d)
            h = F.conv1d(act(h, W[q + "snake2.alpha"]), W[q + "conv1.weight"], W[q + "conv1.bias"])
            x = x + h
    a = act(x, W["dec.out.snake.alpha"])
    taps[3 * len(cfg["strides"])] = a[0].T.numpy()
    y = cconv(a, W["dec.out.conv.weight"], W["dec.out.conv.bias"], 1)
    return y[0, 0].numpy()


@pytest.mark.parametrize("act", ["snake", "elu"])
def test_whole_decoder_c1_matches_torch_composition(act):
    cfg = RI.get_config("c1", act=act)
    w = RI.make_weights(cfg)
    codes = RI.stream_codes(cfg, 0, cfg["n_frames"])
    m = oracle.Model(cfg, w)
    pcm = m.decode_full(codes)
    ref = torch_decode_full(cfg, w, codes)
    assert pcm.shape == (cfg["n_frames"] * RI.hop(cfg),)
    np.testing.assert_allclose(pcm, ref, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("act", ["snake", "elu"])
def test_decoder_taps_match_torch_composition(act):
    """Every conv operand the oracle can hand out (its layer taps) equals the
    torch composition's at the same point, and taking a tap leaves the PCM
    bit for bit unchanged; a streamed decode's taps concatenate to the whole
    decode's."""
    cfg = RI.get_config("c1", act=act)
    w = RI.make_weights(cfg)
    T = 20
    codes = RI.stream_codes(cfg, 2, T)
    m = oracle.Model(cfg, w)
    ref_taps = {}
    ref = torch_decode_full(cfg, w, codes, ref_taps)
    full = m.decode_full(codes)
    S = len(cfg["strides"])
    assert sorted(ref_taps) == list(range(3 * S + 1))
    for tap, want in ref_taps.items():
        pcm, got = m.stream().decode_tap(codes, tap)
        assert got.shape == want.shape == oracle.tap_shape(cfg, tap, T)
        assert np.array_equal(pcm, full)
        np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)
        s = m.stream()
        parts = [s.decode_tap(codes[a:b], tap)[1] for a, b in ((0, 3), (3, 4), (4, T))]
        assert np.array_equal(np.concatenate(parts), got)
    np.testing.assert_allclose(full, ref, rtol=1e-10, atol=1e-12)


def test_final_tanh_is_tanh_of_raw_output():
    """The optional output tanh (off in every workload) maps each raw PCM
    sample through tanh and nothing else: against numpy's tanh of the raw
    decode, including a decode whose raw samples reach |x| > 1 (scaled output
    conv) so that the saturation is exercised."""
    for scale in (1.0, 1000.0):
        cfg = RI.get_config("c1")
        w = dict(RI.make_weights(cfg))
        w["dec.out.conv.weight"] = w["dec.out.conv.weight"] * np.float32(scale)
        codes = RI.stream_codes(cfg, 4, 12)
        raw = oracle.Model(cfg, w).decode_full(codes)
        sq = oracle.Model(dict(cfg, final_tanh=True), w).decode_full(codes)
        if scale > 1:
            assert np.max(np.abs(raw)) > 1.5
        np.testing.assert_allclose(sq, np.tanh(raw), rtol=4e-16, atol=1e-300)
        assert not np.array_equal(sq, raw)


# --------------------------------------------------------------------------
# Streaming invariant: streamed == whole-utterance, bit for bit
# --------------------------------------------------------------------------
def small(cfg_name, **kw):
    """Narrow variant of a configuration: same strides, kernels, dilations,
    window and head count structure, fewer channels (fast on the CPU)."""
    cfg = RI.get_config(cfg_name, **kw)
    cfg.update(d_cb=16, d_lat=64, E=64)
    if cfg["tf_layers"]:
        cfg.update(tf_heads=2, tf_head_dim=8, tf_mlp=32)
    return cfg


def stream_in_chunks(m, codes, chunks):
    s = m.stream()
    out, at = [], 0
    for n in chunks:
        out.append(s.decode(codes[at: at + n]))
        at += n
    assert at == codes.shape[0]
    return np.concatenate(out)


@pytest.mark.parametrize("name,chunks", [
    ("c1", RI.C1_CHUNKS),
    ("c1", [1] * 50),
    ("c1", [50]),
    ("c2", RI.C2_CHUNKS[:6] + [3]),
    ("c3", [1, 2, 4, 8, 8, 8, 8, 1]),
])
def test_streamed_equals_full_bitwise(name, chunks):
    cfg = RI.get_config("c1") if name == "c1" else small(name)
    w = RI.make_weights(cfg)
    T = sum(chunks)
    codes = RI.stream_codes(cfg, 0, T)
    m = oracle.Model(cfg, w)
    full = m.decode_full(codes)
    streamed = stream_in_chunks(m, codes, chunks)
    assert np.array_equal(full, streamed)


def test_streamed_equals_full_bitwise_c2_full_width_short():
    cfg = RI.get_config("c2")
    w = RI.make_weights(cfg)
    codes = RI.stream_codes(cfg, 3, 4)
    m = oracle.Model(cfg, w)
    assert np.array_equal(m.decode_full(codes), stream_in_chunks(m, codes, [1, 2, 1]))


def test_decode_batch_equals_per_stream():
    cfg = RI.get_config("c1")
    m = oracle.Model(cfg, RI.make_weights(cfg))
    n = np.array([3, 1, 5], np.int32)
    codes = [RI.stream_codes(cfg, b, int(n[b])) for b in range(3)]
    streams = [m.stream() for _ in range(3)]
    pcm = m.decode_batch(streams, n, np.concatenate(codes))
    ref = np.concatenate([m.decode_full(c) for c in codes])
    assert np.array_equal(pcm, ref)


# --------------------------------------------------------------------------
# Receptive field: perturbation vs the analytic left context
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name,expect", [("c1", 16), ("c2", 11), ("c3", 135)])
def test_left_context_frames(name, expect):
    assert analytic_left_context(RI.get_config(name)) == expect


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_receptive_field_perturbation(name):
    cfg = RI.get_config("c1") if name == "c1" else small(name)
    if name == "c3":
        cfg.update(tf_window=4)     # same structure, shorter window keeps the test fast
    H = RI.hop(cfg)
    L = analytic_left_context(cfg)
    f = L + 3
    T = f + L + 4
    # A dependency that runs through ~20 layers of N(0, 0.02) weights is far
    # below fp64 resolution, so the perturbation is one huge codebook row:
    # every sample that depends on frame f at all then changes.
    w = dict(RI.make_weights(cfg))
    cb = w["rvq.codebook.0"].astype(np.float64).copy()
    cb[-1, :] = 1e60
    w["rvq.codebook.0"] = cb
    m = oracle.Model(cfg, w)
    codes = RI.stream_codes(cfg, 0, T)
    codes[:, 0] %= cfg["E"] - 1
    base = m.decode_full(codes)
    pert = codes.copy()
    pert[f, 0] = cfg["E"] - 1
    y = m.decode_full(pert)
    assert np.all(np.isfinite(y))
    changed = np.nonzero(base != y)[0]
    firsts = np.array([analytic_first_frame(cfg, n) for n in range(T * H)])
    last = int(np.nonzero(firsts <= f)[0].max())
    assert changed.min() == f * H
    assert np.array_equal(base[: f * H], y[: f * H])
    assert np.array_equal(base[last + 1:], y[last + 1:])
    if not cfg["tf_layers"]:
        assert changed.max() == last
    else:
        # LayerNorm rescales the perturbation to O(1) inside the transformer,
        # so its far edge is checked at the transformer output (frame level);
        # the conv decoder's edge is checked by the configurations without one.
        _, _, x0 = m.stream().decode(codes, capture=True)
        _, _, x1 = m.stream().decode(pert, capture=True)
        rows = np.nonzero(np.any(x0 != x1, axis=1))[0]
        reach = cfg["tf_layers"] * (cfg["tf_window"] - 1)
        assert rows.min() == f and rows.max() == f + reach
        assert len(rows) == reach + 1


def test_window_decode_from_left_context_is_exact():
    # decoding from L frames before a chunk with a zero state reproduces the
    # full decode of that chunk bit for bit (used for sampled parity at scale)
    cfg = small("c2")
    L = analytic_left_context(cfg)
    H = RI.hop(cfg)
    m = oracle.Model(cfg, RI.make_weights(cfg))
    codes = RI.stream_codes(cfg, 0, 40)
    full = m.decode_full(codes)
    start, n = 25, 6
    win = m.stream(start - L).decode(codes[start - L: start + n])
    assert np.array_equal(win[L * H:], full[start * H:(start + n) * H])


def test_window_decode_exact_with_attention():
    cfg = small("c3")
    cfg.update(tf_window=4)
    L = 11 + cfg["tf_layers"] * 3
    H = RI.hop(cfg)
    m = oracle.Model(cfg, RI.make_weights(cfg))
    codes = RI.stream_codes(cfg, 0, L + 12)
    full = m.decode_full(codes)
    start, n = L + 5, 4
    win = m.stream(start - L).decode(codes[start - L: start + n])
    assert np.array_equal(win[L * H:], full[start * H:(start + n) * H])


# --------------------------------------------------------------------------
# Frame rates and hops fixed by the pages
# --------------------------------------------------------------------------
def test_hops_and_frame_rates():
    facts = json.load(open(os.path.join(GOLD, "frame_facts.json")))
    c2, c3 = RI.get_config("c2"), RI.get_config("c3")
    q = facts["qwen3_tts"]
    assert (c2["K"], c2["E"]) == (q["codebooks"], q["codebook_size"])
    assert RI.hop(c2) * 1000 / c2["sample_rate"] == q["frame_ms"]
    assert c2["sample_rate"] / RI.hop(c2) == q["frame_rate_hz"]
    f = facts["fish_drama3"]
    assert c3["K"] == f["codebooks"] and c3["sample_rate"] == f["sample_rate"]
    assert round(c3["sample_rate"] / RI.hop(c3), 1) == f["frames_per_audio_second"]
    assert q["eos_code"] >= c2["E"]


# --------------------------------------------------------------------------
# Windowed transformer: independent torch composition
# --------------------------------------------------------------------------
def torch_transformer(cfg, w, u, pos0=0):
    """Pre-norm windowed causal transformer from torch fp64 library ops:
    layer_norm, linear, RoPE as a complex rotation, SDPA with a band mask,
    erf GELU."""
    W = {k: t64(v) for k, v in w.items()}
    T = u.shape[0]
    H, hd, win = cfg["tf_heads"], cfg["tf_head_dim"], cfg["tf_window"]
    dm = H * hd
    h = F.linear(t64(u), W["tf.in_proj.weight"], W["tf.in_proj.bias"])
    pos = torch.arange(pos0, pos0 + T, dtype=torch.float64)
    inv = 10000.0 ** (-torch.arange(hd // 2, dtype=torch.float64) * 2.0 / hd)
    rot = torch.polar(torch.ones(T, hd // 2, dtype=torch.float64), pos[:, None] * inv[None])

    def rope(x):  # [T, H, hd]
        z = torch.complex(x[..., : hd // 2], x[..., hd // 2:]) * rot[:, None, :]
        return torch.cat([z.real, z.imag], -1)

    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    mask = (j <= i) & (j > i - win)
    for l in range(cfg["tf_layers"]):
        p = f"tf.layer.{l}."
        a = F.layer_norm(h, (dm,), W[p + "ln1.weight"], W[p + "ln1.bias"], eps=1e-5)
        qkv = F.linear(a, W[p + "attn.qkv.weight"], W[p + "attn.qkv.bias"])
        q, k, v = (qkv[:, n * dm:(n + 1) * dm].reshape(T, H, hd) for n in range(3))
        q, k = rope(q), rope(k)
        att = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1),
                                             v.transpose(0, 1), attn_mask=mask)
        h = h + F.linear(att.transpose(0, 1).reshape(T, dm), W[p + "attn.out.weight"],
                         W[p + "attn.out.bias"])
        a = F.layer_norm(h, (dm,), W[p + "ln2.weight"], W[p + "ln2.bias"], eps=1e-5)
        f = F.gelu(F.linear(a, W[p + "mlp.fc1.weight"], W[p + "mlp.fc1.bias"]))
        h = h + F.linear(f, W[p + "mlp.fc2.weight"], W[p + "mlp.fc2.bias"])
    h = F.layer_norm(h, (dm,), W["tf.ln_f.weight"], W["tf.ln_f.bias"], eps=1e-5)
    return F.linear(h, W["tf.out_proj.weight"], W["tf.out_proj.bias"]).numpy()


def test_transformer_matches_torch_composition():
    cfg = small("c3")
    cfg.update(tf_window=5)
    w = RI.make_weights(cfg)
    m = oracle.Model(cfg, w)
    codes = RI.stream_codes(cfg, 0, 23)
    _, u, x = m.stream().decode(codes, capture=True)
    ref = torch_transformer(cfg, w, u)
    np.testing.assert_allclose(x, ref, rtol=1e-10, atol=1e-12)
    # the projected latent itself is the gathered sum through the projection
    z = m.rvq_sum(codes)
    np.testing.assert_allclose(u, z @ w["rvq.proj.weight"].astype(np.float64).T
                               + w["rvq.proj.bias"], rtol=1e-12, atol=1e-14)


def test_transformer_positions_continue_across_chunks():
    # RoPE positions are absolute: a stream opened at position p0 matches the
    # torch composition evaluated at positions p0, p0 + 1, ...
    cfg = small("c3")
    w = RI.make_weights(cfg)
    m = oracle.Model(cfg, w)
    codes = RI.stream_codes(cfg, 0, 9)
    _, u, x = m.stream(pos0=321).decode(codes, capture=True)
    np.testing.assert_allclose(x, torch_transformer(cfg, w, u, pos0=321), rtol=1e-10, atol=1e-12)
