"""fp64 CPU oracle of the streaming RVQ codec decoder (ctypes front end).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the GPU library (``streaming_neural_audio_rvq_amd``) and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, fixed reduction order);
this file only marshals numpy arrays.  ``policy.py`` holds the host-side chunk
ramp policy of the streaming vocoder, written from the pages' description.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

MAX_STAGES = 8
ACT = {"snake": 0, "elu": 1}


def build(verbose: bool = False) -> str:
    """Compile oracle.c with gcc (fp64, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O3", "-fno-fast-math", "-ffp-contract=off", "-march=x86-64-v3",
           "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", _SO + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


class _Cfg(C.Structure):
    _fields_ = [("K", C.c_int), ("E", C.c_int), ("d_cb", C.c_int), ("d_lat", C.c_int),
                ("n_stages", C.c_int), ("strides", C.c_int * MAX_STAGES),
                ("act", C.c_int), ("final_tanh", C.c_int),
                ("tf_layers", C.c_int), ("tf_heads", C.c_int), ("tf_head_dim", C.c_int),
                ("tf_window", C.c_int), ("tf_mlp", C.c_int)]


_lib = None
_D = C.POINTER(C.c_double)
_I32 = C.POINTER(C.c_int32)


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        build()
    L = C.CDLL(_SO)
    L.orc_model_new.restype = C.c_void_p
    L.orc_model_new.argtypes = [C.POINTER(_Cfg)]
    L.orc_model_set.restype = C.c_int
    L.orc_model_set.argtypes = [C.c_void_p, C.c_char_p, _D, C.c_long]
    L.orc_model_missing.argtypes = [C.c_void_p]
    L.orc_model_param_name.restype = C.c_char_p
    L.orc_model_param_name.argtypes = [C.c_void_p, C.c_int]
    L.orc_model_n_params.argtypes = [C.c_void_p]
    L.orc_model_hop.argtypes = [C.c_void_p]
    L.orc_model_free.argtypes = [C.c_void_p]
    L.orc_stream_new.restype = C.c_void_p
    L.orc_stream_new.argtypes = [C.c_void_p, C.c_long]
    L.orc_stream_free.argtypes = [C.c_void_p]
    L.orc_stream_pos.restype = C.c_long
    L.orc_stream_pos.argtypes = [C.c_void_p]
    L.orc_stream_decode.argtypes = [C.c_void_p, _I32, C.c_int, _D, _D, _D]
    L.orc_stream_decode_tap.argtypes = [C.c_void_p, _I32, C.c_int, _D, C.c_int, _D]
    L.orc_decode_batch.argtypes = [C.POINTER(C.c_void_p), C.c_int, _I32, _I32, _D]
    L.orc_snake.argtypes = [_D, _D, C.c_int, C.c_long, _D]
    L.orc_elu.argtypes = [_D, C.c_long, _D]
    L.orc_gelu.argtypes = [_D, C.c_long, _D]
    L.orc_layer_norm.argtypes = [_D, _D, _D, C.c_int, C.c_double, _D]
    L.orc_linear.argtypes = [_D, _D, _D, C.c_int, C.c_int, _D]
    L.orc_causal_conv.argtypes = [_D, C.c_int, C.c_long, _D, _D, C.c_int, C.c_int, C.c_int, _D]
    L.orc_conv_transpose.argtypes = [_D, C.c_int, C.c_long, _D, _D, C.c_int, C.c_int, _D]
    L.orc_rope.argtypes = [_D, C.c_int, C.c_int, C.c_long]
    L.orc_window_attention.argtypes = [_D, _D, _D, C.c_int, C.c_int, C.c_int, _D]
    L.orc_rvq_sum.argtypes = [C.c_void_p, _I32, C.c_int, _D]
    L.orc_num_threads.restype = C.c_int
    _lib = L
    return L


def _d(a: np.ndarray):
    return a.ctypes.data_as(_D)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Layer-level entry points (used by the pins)
# ---------------------------------------------------------------------------
def snake(x, alpha):
    x = _f64(x)
    C_, T = x.shape
    y = np.empty_like(x)
    lib().orc_snake(_d(x), _d(_f64(alpha)), C_, T, _d(y))
    return y


def elu(x):
    x = _f64(x)
    y = np.empty_like(x)
    lib().orc_elu(_d(x), x.size, _d(y))
    return y


def gelu(x):
    x = _f64(x)
    y = np.empty_like(x)
    lib().orc_gelu(_d(x), x.size, _d(y))
    return y


def layer_norm(x, g, b, eps=1e-5):
    x = _f64(x)
    y = np.empty_like(x)
    lib().orc_layer_norm(_d(x), _d(_f64(g)), _d(_f64(b)), x.size, eps, _d(y))
    return y


def linear(W, b, x):
    W = _f64(W)
    x = _f64(x)
    O, I = W.shape
    y = np.empty(O)
    bb = _f64(b) if b is not None else None
    lib().orc_linear(_d(W), _d(bb) if bb is not None else None, _d(x), O, I, _d(y))
    return y


def causal_conv(x_ext, W, b, d):
    """x_ext [Ci][(k-1) d + T] (left context first) -> [Co][T]."""
    x_ext = _f64(x_ext)
    W = _f64(W)
    Co, Ci, k = W.shape
    T = x_ext.shape[1] - (k - 1) * d
    y = np.empty((Co, T))
    bb = _f64(b) if b is not None else None
    lib().orc_causal_conv(_d(x_ext), Ci, T, _d(W), _d(bb) if bb is not None else None,
                          Co, k, d, _d(y))
    return y


def conv_transpose(x_ext, W, b, s):
    """x_ext [Ci][1 + T] (column 0 = previous input) -> [Co][T s]."""
    x_ext = _f64(x_ext)
    W = _f64(W)
    Ci, Co, k = W.shape
    assert k == 2 * s
    T = x_ext.shape[1] - 1
    y = np.empty((Co, T * s))
    bb = _f64(b) if b is not None else None
    lib().orc_conv_transpose(_d(x_ext), Ci, T, _d(W), _d(bb) if bb is not None else None,
                             Co, s, _d(y))
    return y


def rope(x, H, hd, pos):
    x = _f64(x).copy()
    lib().orc_rope(_d(x), H, hd, pos)
    return x


def window_attention(q, keys, vals, H, hd):
    q = _f64(q)
    keys = _f64(keys)
    vals = _f64(vals)
    out = np.empty(H * hd)
    lib().orc_window_attention(_d(q), _d(keys), _d(vals), keys.shape[0], H, hd, _d(out))
    return out


# ---------------------------------------------------------------------------
# Whole decoder
# ---------------------------------------------------------------------------
class Model:
    """The decoder of one configuration with fp64 copies of its parameters."""

    def __init__(self, cfg: dict, weights: dict):
        c = _Cfg()
        c.K, c.E, c.d_cb, c.d_lat = cfg["K"], cfg["E"], cfg["d_cb"], cfg["d_lat"]
        c.n_stages = len(cfg["strides"])
        for i, s in enumerate(cfg["strides"]):
            c.strides[i] = s
        c.act = ACT[cfg["act"]]
        c.final_tanh = int(bool(cfg["final_tanh"]))
        c.tf_layers, c.tf_heads, c.tf_head_dim = cfg["tf_layers"], cfg["tf_heads"], cfg["tf_head_dim"]
        c.tf_window, c.tf_mlp = cfg["tf_window"], cfg["tf_mlp"]
        L = lib()
        self._h = L.orc_model_new(C.byref(c))
        if not self._h:
            raise ValueError("oracle: bad configuration")
        self.cfg = cfg
        for name, v in weights.items():
            a = _f64(v).ravel()
            rc = L.orc_model_set(self._h, name.encode(), _d(a), a.size)
            if rc:
                raise ValueError(f"oracle: parameter {name}: status {rc}")
        miss = L.orc_model_missing(self._h)
        if miss >= 0:
            raise ValueError(f"oracle: parameter {L.orc_model_param_name(self._h, miss).decode()} not set")
        self.hop = L.orc_model_hop(self._h)

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.orc_model_free(self._h)
            self._h = None

    def stream(self, pos0: int = 0) -> "Stream":
        return Stream(self, pos0)

    def decode_full(self, codes: np.ndarray, pos0: int = 0) -> np.ndarray:
        """Whole-utterance decode from an all-zero left context."""
        return self.stream(pos0).decode(codes)

    def rvq_sum(self, codes: np.ndarray) -> np.ndarray:
        codes = np.ascontiguousarray(codes, dtype=np.int32)
        z = np.empty((codes.shape[0], self.cfg["d_cb"]))
        rc = lib().orc_rvq_sum(self._h, codes.ctypes.data_as(_I32), codes.shape[0], _d(z))
        if rc:
            raise ValueError("oracle: code out of range")
        return z

    def decode_batch(self, streams, n, codes) -> np.ndarray:
        """One chunk for each stream, decoded in parallel across streams."""
        n = np.ascontiguousarray(n, dtype=np.int32)
        codes = np.ascontiguousarray(codes, dtype=np.int32)
        pcm = np.empty(int(n.sum()) * self.hop)
        arr = (C.c_void_p * len(streams))(*[s._h for s in streams])
        rc = lib().orc_decode_batch(arr, len(streams), n.ctypes.data_as(_I32),
                                    codes.ctypes.data_as(_I32), _d(pcm))
        if rc:
            raise ValueError(f"oracle: decode status {rc}")
        return pcm


class Stream:
    """One stream's decoder state (left contexts, KV windows, position)."""

    def __init__(self, model: Model, pos0: int = 0):
        self.model = model
        self._h = lib().orc_stream_new(model._h, pos0)

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.orc_stream_free(self._h)
            self._h = None

    @property
    def pos(self) -> int:
        return lib().orc_stream_pos(self._h)

    def decode(self, codes: np.ndarray, capture: bool = False):
        codes = np.ascontiguousarray(codes, dtype=np.int32)
        n = codes.shape[0]
        pcm = np.empty(n * self.model.hop)
        dl = self.model.cfg["d_lat"]
        cu = np.empty((n, dl)) if capture else None
        cx = np.empty((n, dl)) if capture else None
        rc = lib().orc_stream_decode(self._h, codes.ctypes.data_as(_I32), n, _d(pcm),
                                     _d(cu) if capture else None, _d(cx) if capture else None)
        if rc == -1:
            raise ValueError("oracle: code out of range")
        if rc:
            raise ValueError(f"oracle: decode status {rc}")
        return (pcm, cu, cx) if capture else pcm

    def decode_tap(self, codes: np.ndarray, tap: int):
        """Decode like ``decode`` and also return one conv operand of the
        decoder, [rows][C] time-major: tap 3 i is stage i's transposed-conv
        input, 3 i + 1 + j the input of its residual unit j, 3 S the final
        conv's input (S = number of stages)."""
        codes = np.ascontiguousarray(codes, dtype=np.int32)
        n = codes.shape[0]
        pcm = np.empty(n * self.model.hop)
        out = np.empty(tap_shape(self.model.cfg, tap, n))
        rc = lib().orc_stream_decode_tap(self._h, codes.ctypes.data_as(_I32), n, _d(pcm), tap,
                                         _d(out))
        if rc:
            raise ValueError(f"oracle: decode status {rc}")
        return pcm, out


def tap_shape(cfg: dict, tap: int, n: int) -> tuple[int, int]:
    """(rows, channels) of decoder tap ``tap`` for n frames (see decode_tap)."""
    S = len(cfg["strides"])
    ch = [cfg["d_lat"]]
    rate = [1]
    for s in cfg["strides"]:
        ch.append(ch[-1] // 2)
        rate.append(rate[-1] * s)
    if tap == 3 * S:
        return n * rate[S], ch[S]
    i, k = divmod(tap, 3)
    return (n * rate[i], ch[i]) if k == 0 else (n * rate[i + 1], ch[i + 1])


def weights_f64(weights: dict) -> dict:
    return {k: np.asarray(v, dtype=np.float64) for k, v in weights.items()}


def num_threads() -> int:
    return lib().orc_num_threads()
