"""Seeded synthetic inputs for the streaming RVQ codec decoder.

This module is shared by the fp64 oracle's tests and by the GPU path's tests
and benchmark.  It holds *no* arithmetic of the decoder itself: only the
decoder shapes (five workload configurations), the canonical parameter list
and its random initialisation, bf16 rounding of those parameters, and the
seeded code / offset / chunk-size draws.

Workloads (the shapes of the pages' two codecs):
  c1  tiny fp32 decoder, 4 codebooks x 256, 16 samples per frame
  c2  Qwen3-TTS-shaped: 16 codebooks x 2048 entries, 12.5 Hz frames
      upsampled x1920 to 24 kHz (AI-infra handbook, "Qwen3-TTS" case:
      model description and the vocoder section)
  c3  Fish-DAC-shaped: 10 codebooks x 1024 entries, hop 2048 at 44.1 kHz,
      with a windowed causal transformer before the upsampler (AREX article
      on vLLM-Omni / Fish Audio Drama 3, "two stages share one card")
  c4  the c2 decoder at 128 concurrent streams at staggered positions
  c5  the c2 decoder decoding 128 whole utterances of 50..500 frames

Seeds: weights 0, codes 1, schedule (offsets, chunk sizes, lengths) 2, all
through numpy's PCG64 ``default_rng``.  Per-stream and per-step draws use a
SeedSequence key ``[seed, stream, step]`` so that a draw never depends on
how many other streams or steps are requested.
"""
from __future__ import annotations

import copy
from collections import OrderedDict

import numpy as np

SEED_W = 0
SEED_C = 1
SEED_S = 2

# ---------------------------------------------------------------------------
# Decoder shapes
# ---------------------------------------------------------------------------
_BASE_C2 = dict(
    K=16, E=2048, d_cb=512, d_lat=1024,
    strides=[8, 5, 4, 3, 4], sample_rate=24000,
    act="snake", final_tanh=False,
    tf_layers=0, tf_heads=0, tf_head_dim=0, tf_window=0, tf_mlp=0,
    weight_dtype="bf16",
)

CONFIGS: dict[str, dict] = {
    "c1": dict(
        K=4, E=256, d_cb=32, d_lat=64,
        strides=[4, 4], sample_rate=16000,
        act="snake", final_tanh=False,
        tf_layers=0, tf_heads=0, tf_head_dim=0, tf_window=0, tf_mlp=0,
        weight_dtype="fp32",
        max_streams=8, max_frames_per_call=256,
        n_streams=1, n_frames=50,
    ),
    "c2": dict(_BASE_C2, max_streams=16, max_frames_per_call=512,
               n_streams=8, n_frames=200),
    "c3": dict(
        K=10, E=1024, d_cb=512, d_lat=1024,
        strides=[8, 8, 4, 4, 2], sample_rate=44100,
        act="snake", final_tanh=False,
        tf_layers=4, tf_heads=8, tf_head_dim=64, tf_window=32, tf_mlp=2048,
        weight_dtype="bf16",
        max_streams=64, max_frames_per_call=512,
        n_streams=64, n_frames=300,
    ),
    "c4": dict(_BASE_C2, max_streams=128, max_frames_per_call=2048,
               n_streams=128, max_offset=500, buckets=[1, 2, 4, 8, 16]),
    "c5": dict(_BASE_C2, max_streams=128, max_frames_per_call=16000,
               n_streams=128, min_len=50, max_len=500),
}


def get_config(name: str, **overrides) -> dict:
    cfg = copy.deepcopy(CONFIGS[name])
    cfg["name"] = name
    cfg.update(overrides)
    return cfg


def hop(cfg: dict) -> int:
    h = 1
    for s in cfg["strides"]:
        h *= s
    return h


def channels(cfg: dict) -> list[int]:
    """Channel width entering each upsample stage, then its output: C0..CS."""
    c = [cfg["d_lat"]]
    for _ in cfg["strides"]:
        c.append(c[-1] // 2)
    return c


# ---------------------------------------------------------------------------
# Canonical parameter list and random initialisation
# ---------------------------------------------------------------------------
def param_specs(cfg: dict) -> list[tuple[str, tuple, str]]:
    """(name, shape, init kind) in canonical drawing order.

    init kind: "w" weight/bias ~ N(0, 0.02); "alpha" Snake alpha ~ U[0.5, 1.5];
    "gamma" LayerNorm scale 1 + N(0, 0.02).  Conv weights use PyTorch layouts:
    Conv1d [C_out, C_in, k], ConvTranspose1d [C_in, C_out, k].
    """
    K, E, dcb, dl = cfg["K"], cfg["E"], cfg["d_cb"], cfg["d_lat"]
    out: list[tuple[str, tuple, str]] = []
    for k in range(K):
        out.append((f"rvq.codebook.{k}", (E, dcb), "w"))
    out.append(("rvq.proj.weight", (dl, dcb), "w"))
    out.append(("rvq.proj.bias", (dl,), "w"))
    L = cfg["tf_layers"]
    if L:
        dm = cfg["tf_heads"] * cfg["tf_head_dim"]
        mlp = cfg["tf_mlp"]
        out.append(("tf.in_proj.weight", (dm, dl), "w"))
        out.append(("tf.in_proj.bias", (dm,), "w"))
        for l in range(L):
            p = f"tf.layer.{l}."
            out += [
                (p + "ln1.weight", (dm,), "gamma"), (p + "ln1.bias", (dm,), "w"),
                (p + "attn.qkv.weight", (3 * dm, dm), "w"), (p + "attn.qkv.bias", (3 * dm,), "w"),
                (p + "attn.out.weight", (dm, dm), "w"), (p + "attn.out.bias", (dm,), "w"),
                (p + "ln2.weight", (dm,), "gamma"), (p + "ln2.bias", (dm,), "w"),
                (p + "mlp.fc1.weight", (mlp, dm), "w"), (p + "mlp.fc1.bias", (mlp,), "w"),
                (p + "mlp.fc2.weight", (dm, mlp), "w"), (p + "mlp.fc2.bias", (dm,), "w"),
            ]
        out.append(("tf.ln_f.weight", (dm,), "gamma"))
        out.append(("tf.ln_f.bias", (dm,), "w"))
        out.append(("tf.out_proj.weight", (dl, dm), "w"))
        out.append(("tf.out_proj.bias", (dl,), "w"))
    ch = channels(cfg)
    out.append(("dec.in_conv.weight", (ch[0], dl, 7), "w"))
    out.append(("dec.in_conv.bias", (ch[0],), "w"))
    for i, s in enumerate(cfg["strides"]):
        ci, co = ch[i], ch[i + 1]
        p = f"dec.stage.{i}."
        out.append((p + "snake.alpha", (ci,), "alpha"))
        out.append((p + "convT.weight", (ci, co, 2 * s), "w"))
        out.append((p + "convT.bias", (co,), "w"))
        for j in range(2):
            q = p + f"ru.{j}."
            out += [
                (q + "snake1.alpha", (co,), "alpha"),
                (q + "conv7.weight", (co, co, 7), "w"), (q + "conv7.bias", (co,), "w"),
                (q + "snake2.alpha", (co,), "alpha"),
                (q + "conv1.weight", (co, co, 1), "w"), (q + "conv1.bias", (co,), "w"),
            ]
    out.append(("dec.out.snake.alpha", (ch[-1],), "alpha"))
    out.append(("dec.out.conv.weight", (1, ch[-1], 7), "w"))
    out.append(("dec.out.conv.bias", (1,), "w"))
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


_WEIGHT_CACHE: dict = {}


def make_weights(cfg: dict, seed: int = SEED_W) -> "OrderedDict[str, np.ndarray]":
    """Random-init parameters as float32 arrays holding their exact values.

    For bf16 configurations every value is rounded to bf16 (the stored value);
    ``weight_bits`` gives the matching uint16 patterns.  With
    ``cfg["zero_bias"]`` every bias (names ending in ``.bias``) is zero
    instead; all other parameters keep the values they have without it.
    """
    zero_bias = bool(cfg.get("zero_bias", False))
    key = (cfg["K"], cfg["E"], cfg["d_cb"], cfg["d_lat"], tuple(cfg["strides"]),
           cfg["tf_layers"], cfg["tf_heads"], cfg["tf_head_dim"], cfg["tf_mlp"],
           cfg["weight_dtype"], seed, zero_bias)
    if key in _WEIGHT_CACHE:
        return _WEIGHT_CACHE[key]
    rng = np.random.default_rng(seed)
    out: "OrderedDict[str, np.ndarray]" = OrderedDict()
    for name, shape, kind in param_specs(cfg):
        if kind == "alpha":
            v = rng.uniform(0.5, 1.5, size=shape).astype(np.float32)
        elif kind == "gamma":
            v = (1.0 + rng.normal(0.0, 0.02, size=shape)).astype(np.float32)
        else:
            v = rng.normal(0.0, 0.02, size=shape).astype(np.float32)
        if cfg["weight_dtype"] == "bf16":
            v = bf16_to_f32(bf16_bits(v)).reshape(shape)
        if zero_bias and name.endswith(".bias"):
            v = np.zeros(shape, np.float32)
        out[name] = v
    _WEIGHT_CACHE[key] = out
    return out


def weight_bits(weights: "OrderedDict[str, np.ndarray]") -> "OrderedDict[str, np.ndarray]":
    """uint16 bf16 patterns of already bf16-valued float32 arrays (exact)."""
    return OrderedDict((k, bf16_bits(v)) for k, v in weights.items())


def index_probe_weights(cfg: dict) -> "OrderedDict[str, np.ndarray]":
    """Integer codebooks and an identity projection for bit-exact gather checks.

    C_k[r, d] = ((7 r + 3 d + 11 k) mod 251) - 125: integers in [-125, 125].
    A sum of up to 16 such rows stays below 2048 in magnitude, so it is exact
    in fp16, bf16 storage of the entries is exact, and fp32 sums are exact.
    The projection is [I; 0] with zero bias, so the latent equals the sum.
    All decoder parameters after the projection keep their random values.
    """
    w = OrderedDict((k, v.copy()) for k, v in make_weights(cfg).items())
    E, dcb, dl = cfg["E"], cfg["d_cb"], cfg["d_lat"]
    r = np.arange(E)[:, None]
    d = np.arange(dcb)[None, :]
    for k in range(cfg["K"]):
        w[f"rvq.codebook.{k}"] = (((7 * r + 3 * d + 11 * k) % 251) - 125).astype(np.float32)
    p = np.zeros((dl, dcb), np.float32)
    p[np.arange(min(dl, dcb)), np.arange(min(dl, dcb))] = 1.0
    w["rvq.proj.weight"] = p
    w["rvq.proj.bias"] = np.zeros((dl,), np.float32)
    return w


# ---------------------------------------------------------------------------
# Codes, offsets, chunk sizes
# ---------------------------------------------------------------------------
def stream_codes(cfg: dict, stream: int, n: int, part: int = 0,
                 seed: int = SEED_C) -> np.ndarray:
    """Uniform codes [n, K] (int32) for one stream; ``part`` selects an
    independent block (0: the utterance / prefix, 1+j: step j)."""
    rng = np.random.default_rng([seed, stream, part])
    return rng.integers(0, cfg["E"], size=(n, cfg["K"])).astype(np.int32)


def c4_offsets(cfg: dict, seed: int = SEED_S) -> np.ndarray:
    """Staggered start positions: frames already decoded per stream (0..500)."""
    rng = np.random.default_rng([seed, 0])
    return rng.integers(0, cfg["max_offset"] + 1, size=cfg["n_streams"]).astype(np.int32)


def c4_chunk_sizes(cfg: dict, step: int, seed: int = SEED_S) -> np.ndarray:
    """New frames per stream in one batched step, drawn from the buckets."""
    rng = np.random.default_rng([seed, 1 + step])
    return rng.choice(np.asarray(cfg["buckets"]), size=cfg["n_streams"]).astype(np.int32)


def c5_lengths(cfg: dict, seed: int = SEED_S) -> np.ndarray:
    rng = np.random.default_rng([seed, 0])
    return rng.integers(cfg["min_len"], cfg["max_len"] + 1, size=cfg["n_streams"]).astype(np.int32)


# Chunk schedules of the streamed workloads: ramp 1, 2, 4 frames, then a
# steady 8, and a final chunk with whatever remains.
C1_CHUNKS = [1, 2, 4] + [8] * 5 + [3]
C2_CHUNKS = [1, 2, 4] + [8] * 24 + [1]
C3_CHUNKS = [8] * 37 + [4]
