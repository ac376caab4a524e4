"""Python binding of the MI355X streaming RVQ codec decoder (``libsnrvq.so``).

Argument marshalling only: every step of a decode runs in the library's HIP
kernels.  PyTorch supplies device memory (``pcm`` tensors) and HIP streams.
The names follow the C ABI in ``include/snrvq.h``.  The library must have
been built (``_build.build()``, or ``__graft_entry__.build()``); loading fails
loudly otherwise -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import operator
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# SNRVQ_LIBRARY names another build of the same library (the host-sanitized
# libsnrvq_hostsan.so); by default the in-tree libsnrvq.so
LIB_PATH = os.environ.get("SNRVQ_LIBRARY") or os.path.join(HERE, "libsnrvq.so")

CODEC_OK, CODEC_EINVAL, CODEC_ESTREAM, CODEC_EDUP, CODEC_ERANGE = 0, 1, 2, 3, 4
CODEC_ENOSLOT, CODEC_ETOOBIG, CODEC_ENOMEM, CODEC_EHIP = 5, 6, 7, 8
DTYPE_F32, DTYPE_BF16, DTYPE_F16 = 0, 1, 2
ACT = {"snake": 0, "elu": 1}
CAPTURE_LATENT, CAPTURE_DEC_INPUT, CAPTURE_RVQ_SUM, CAPTURE_LAYER0 = 0, 1, 2, 3
FLAG_PER_LAYER = 1
FLAG_NO_SPLIT_K = 2
FLAG_TWO_STAGE_BUFFERS = 4
FLAG_NO_TALL_TILES = 8
MAX_STAGES = 8

ERROR_NAMES = {1: "EINVAL", 2: "ESTREAM", 3: "EDUP", 4: "ERANGE", 5: "ENOSLOT", 6: "ETOOBIG",
               7: "ENOMEM", 8: "EHIP"}


class CodecError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


class codec_tensor(C.Structure):
    _fields_ = [("name", C.c_char_p), ("dtype", C.c_int32), ("ndim", C.c_int32),
                ("shape", C.c_int64 * 4), ("host_data", C.c_void_p)]


class codec_cfg(C.Structure):
    _fields_ = [("K", C.c_int32), ("E", C.c_int32), ("d_cb", C.c_int32), ("d_lat", C.c_int32),
                ("n_stages", C.c_int32), ("strides", C.c_int32 * MAX_STAGES),
                ("sample_rate", C.c_int32), ("act", C.c_int32), ("final_tanh", C.c_int32),
                ("tf_layers", C.c_int32), ("tf_heads", C.c_int32), ("tf_head_dim", C.c_int32),
                ("tf_window", C.c_int32), ("tf_mlp", C.c_int32), ("weight_dtype", C.c_int32),
                ("max_streams", C.c_int32), ("max_frames_per_call", C.c_int32),
                ("flags", C.c_int32)]


class codec_info_t(C.Structure):
    _fields_ = [("hop", C.c_int32), ("sample_rate", C.c_int32), ("K", C.c_int32),
                ("E", C.c_int32), ("left_context_frames", C.c_int32),
                ("max_streams", C.c_int32), ("max_frames_per_call", C.c_int32),
                ("open_streams", C.c_int32), ("compute_dtype", C.c_int32),
                ("state_bytes_per_stream", C.c_int64), ("weight_bytes", C.c_int64),
                ("workspace_bytes", C.c_int64), ("graph_captures", C.c_int64),
                ("graph_replays", C.c_int64)]


_I32P = C.POINTER(C.c_int32)
_lib = None

EXPORTS = ["codec_open", "codec_close", "codec_info", "codec_last_error", "stream_open",
           "stream_close", "stream_prefill", "decode_chunk", "decode_chunk_device",
           "decode_chunk_graph", "decode_chunk_device_noalloc",
           "codec_device_status", "codec_debug_capture", "codec_debug_read_state",
           "codec_profile_enable", "codec_profile_read", "codec_chunk_plan",
           "codec_initial_chunk_size", "codec_debug_conv_plan"]


def lib():
    """Load the built library (raises if it was never built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    L = C.CDLL(LIB_PATH)
    L.codec_open.argtypes = [C.POINTER(codec_tensor), C.c_int32, C.POINTER(codec_cfg),
                             C.POINTER(C.c_void_p)]
    L.codec_close.argtypes = [C.c_void_p]
    L.codec_info.argtypes = [C.c_void_p, C.POINTER(codec_info_t)]
    L.codec_last_error.restype = C.c_char_p
    L.codec_last_error.argtypes = [C.c_void_p]
    L.stream_open.argtypes = [C.c_void_p, _I32P]
    L.stream_close.argtypes = [C.c_void_p, C.c_int32]
    L.stream_prefill.argtypes = [C.c_void_p, C.c_int32, _I32P, C.c_int32, C.c_void_p]
    L.decode_chunk.argtypes = [C.c_void_p, C.c_int32, _I32P, _I32P, _I32P, C.c_void_p,
                               C.c_int64, C.c_void_p]
    L.decode_chunk_device.argtypes = [C.c_void_p, C.c_int32, _I32P, _I32P, C.c_void_p,
                                      C.c_void_p, C.c_int64, C.c_void_p]
    L.decode_chunk_graph.argtypes = [C.c_void_p, C.c_int32, _I32P, _I32P, _I32P, C.c_void_p,
                                     C.c_int64, C.c_void_p]
    L.decode_chunk_device_noalloc.argtypes = [C.c_void_p, C.c_int32, _I32P, _I32P, C.c_void_p,
                                              C.c_void_p, C.c_int64, C.c_void_p]
    L.codec_device_status.argtypes = [C.c_void_p, C.POINTER(C.c_int64)]
    L.codec_debug_capture.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_int64, C.c_void_p]
    L.codec_debug_read_state.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_int64,
                                         C.POINTER(C.c_int64)]
    L.codec_profile_enable.argtypes = [C.c_void_p, C.c_int32]
    L.codec_profile_read.argtypes = [C.c_void_p, C.c_int32, C.POINTER(C.c_char_p),
                                     C.POINTER(C.c_double), C.POINTER(C.c_int64),
                                     C.POINTER(C.c_int64), _I32P]
    L.codec_chunk_plan.argtypes = [C.c_int32, _I32P, C.c_int32, C.c_int32, C.c_int32, _I32P,
                                   C.c_int32, _I32P]
    L.codec_initial_chunk_size.argtypes = [C.c_int64, C.c_int32, C.c_int32, C.c_int32,
                                                     _I32P]
    L.codec_debug_conv_plan.argtypes = [C.c_int32] * 7 + [C.POINTER(C.c_char_p), _I32P]
    _lib = L
    return L


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_I32P)


def _stream_handle(stream) -> C.c_void_p:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    if hasattr(stream, "cuda_stream"):
        return C.c_void_p(stream.cuda_stream)
    return C.c_void_p(int(stream))


def _check(rc: int, handle=None):
    if rc != CODEC_OK:
        msg = lib().codec_last_error(handle).decode()
        raise CodecError(rc, msg)


def make_cfg(cfg: dict) -> codec_cfg:
    c = codec_cfg()
    c.K, c.E, c.d_cb, c.d_lat = cfg["K"], cfg["E"], cfg["d_cb"], cfg["d_lat"]
    c.n_stages = len(cfg["strides"])
    for i, s in enumerate(cfg["strides"]):
        c.strides[i] = s
    c.sample_rate = cfg.get("sample_rate", 0)
    c.act = ACT[cfg.get("act", "snake")]
    c.final_tanh = int(bool(cfg.get("final_tanh", False)))
    c.tf_layers = cfg.get("tf_layers", 0)
    c.tf_heads = cfg.get("tf_heads", 0)
    c.tf_head_dim = cfg.get("tf_head_dim", 0)
    c.tf_window = cfg.get("tf_window", 0)
    c.tf_mlp = cfg.get("tf_mlp", 0)
    c.weight_dtype = DTYPE_BF16 if cfg["weight_dtype"] == "bf16" else DTYPE_F32
    c.max_streams = cfg["max_streams"]
    c.max_frames_per_call = cfg["max_frames_per_call"]
    c.flags = (FLAG_PER_LAYER if cfg.get("per_layer", False) else 0) | \
        (FLAG_NO_SPLIT_K if cfg.get("no_split_k", False) else 0) | \
        (FLAG_TWO_STAGE_BUFFERS if cfg.get("two_stage_buffers", False) else 0) | \
        (FLAG_NO_TALL_TILES if cfg.get("no_tall_tiles", False) else 0) | \
        sum(1 << (8 + i) for i in cfg.get("per_layer_stages", ()))
    return c


def make_tensors(weights: dict, weight_dtype: str):
    """codec_tensor array over the given host arrays.  bf16 weights are passed
    as their uint16 bit patterns; the arrays are kept alive by the caller."""
    keep = []
    arr = (codec_tensor * len(weights))()
    for i, (name, v) in enumerate(weights.items()):
        v = np.ascontiguousarray(v)
        if weight_dtype == "bf16":
            if v.dtype != np.uint16:
                raise TypeError(f"{name}: bf16 weights must be uint16 bit patterns")
            dt = DTYPE_BF16
        else:
            v = np.ascontiguousarray(v, dtype=np.float32)
            dt = DTYPE_F32
        nb = name.encode()
        keep += [v, nb]
        arr[i].name = nb
        arr[i].dtype = dt
        arr[i].ndim = v.ndim
        for d in range(v.ndim):
            arr[i].shape[d] = v.shape[d]
        arr[i].host_data = v.ctypes.data
    return arr, keep


class Codec:
    """An open codec: weights, state slots and workspace on the current device."""

    def __init__(self, cfg: dict, weights: dict):
        L = lib()
        self.cfg = dict(cfg)
        c = make_cfg(cfg)
        arr, keep = make_tensors(weights, cfg["weight_dtype"])
        h = C.c_void_p()
        rc = L.codec_open(arr, len(weights), C.byref(c), C.byref(h))
        del keep
        _check(rc, None)
        self._h = h
        self.info = self.get_info()
        self.hop = self.info.hop

    def close(self):
        if getattr(self, "_h", None):
            _check(lib().codec_close(self._h), None)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def get_info(self) -> codec_info_t:
        o = codec_info_t()
        _check(lib().codec_info(self._h, C.byref(o)), self._h)
        return o

    def last_error(self) -> str:
        return lib().codec_last_error(self._h).decode()

    def stream_open(self) -> int:
        sid = C.c_int32()
        _check(lib().stream_open(self._h, C.byref(sid)), self._h)
        return sid.value

    def stream_close(self, sid: int):
        _check(lib().stream_close(self._h, int(sid)), self._h)

    def stream_prefill(self, sid: int, codes, stream=None):
        codes = _i32(codes)
        n = codes.shape[0] if codes.ndim == 2 else 0
        _check(lib().stream_prefill(self._h, int(sid), _ptr(codes), n, _stream_handle(stream)),
               self._h)

    def decode_chunk(self, stream_ids, n_frames, codes, pcm, stream=None):
        """codes: host int32 [sum n, K] packed stream after stream (or dense
        [B, n, K]); pcm: a float32 CUDA tensor with >= sum(n) * hop elements."""
        ids = _i32(stream_ids)
        n = _i32(n_frames)
        codes = _i32(codes)
        _check(lib().decode_chunk(self._h, len(ids), _ptr(ids), _ptr(n), _ptr(codes),
                                  C.c_void_p(pcm.data_ptr()), pcm.numel(),
                                  _stream_handle(stream)), self._h)

    def decode_chunk_graph(self, stream_ids, n_frames, codes, pcm, stream=None):
        """decode_chunk replayed from the graph of its (B, frame bucket); same
        arguments, results within the parity bound."""
        ids = _i32(stream_ids)
        n = _i32(n_frames)
        codes = _i32(codes)
        _check(lib().decode_chunk_graph(self._h, len(ids), _ptr(ids), _ptr(n), _ptr(codes),
                                        C.c_void_p(pcm.data_ptr()), pcm.numel(),
                                        _stream_handle(stream)), self._h)

    def decode_chunk_device(self, stream_ids, n_frames, codes_dev, pcm, stream=None):
        """codes_dev: an int32 CUDA tensor [sum n, K] already on the device."""
        ids = _i32(stream_ids)
        n = _i32(n_frames)
        _check(lib().decode_chunk_device(self._h, len(ids), _ptr(ids), _ptr(n),
                                         C.c_void_p(codes_dev.data_ptr()),
                                         C.c_void_p(pcm.data_ptr()), pcm.numel(),
                                         _stream_handle(stream)), self._h)

    def decode_chunk_device_noalloc(self, stream_ids, n_frames, codes_dev, pcm, stream=None):
        """decode_chunk_device with its scratch in the library's static device
        array (allocates nothing)."""
        ids = _i32(stream_ids)
        n = _i32(n_frames)
        _check(lib().decode_chunk_device_noalloc(self._h, len(ids), _ptr(ids), _ptr(n),
                                                 C.c_void_p(codes_dev.data_ptr()),
                                                 C.c_void_p(pcm.data_ptr()), pcm.numel(),
                                                 _stream_handle(stream)), self._h)

    def device_status(self) -> int:
        """Number of out-of-range device-resident codes since the last call
        (raises CodecError ERANGE when nonzero)."""
        bad = C.c_int64()
        _check(lib().codec_device_status(self._h, C.byref(bad)), self._h)
        return bad.value

    def debug_capture(self, what: int, dst, stream=None):
        _check(lib().codec_debug_capture(self._h, what, C.c_void_p(dst.data_ptr()), dst.numel(),
                                         _stream_handle(stream)), self._h)

    def read_state(self, sid: int) -> np.ndarray:
        """The stream's state slot (conv left contexts) as raw bytes."""
        n = C.c_int64()
        _check(lib().codec_debug_read_state(self._h, int(sid), None, 0, C.byref(n)), self._h)
        buf = np.empty(n.value, np.uint8)
        _check(lib().codec_debug_read_state(self._h, int(sid), buf.ctypes.data, buf.size,
                                            C.byref(n)), self._h)
        return buf

    def profile_enable(self, on: bool = True):
        _check(lib().codec_profile_enable(self._h, int(on)), self._h)

    def profile_read(self) -> dict:
        cap = 256
        names = (C.c_char_p * cap)()
        ms = (C.c_double * cap)()
        launches = (C.c_int64 * cap)()
        units = (C.c_int64 * cap)()
        n = C.c_int32()
        _check(lib().codec_profile_read(self._h, cap, names, ms, launches, units, C.byref(n)),
               self._h)
        return {names[i].decode(): dict(ms=ms[i], launches=launches[i], units=units[i])
                for i in range(min(n.value, cap))}


def chunk_plan(total: int, ramp=(1, 2, 4), steady: int = 8, initial: int = 0) -> list[int]:
    """The library's chunk ramp policy (host only)."""
    r = _i32(list(ramp))
    cap = max(16, total + 1)
    out = np.zeros(cap, np.int32)
    n = C.c_int32()
    rc = lib().codec_chunk_plan(int(total), _ptr(r), len(r), int(steady), int(initial), _ptr(out),
                                cap, C.byref(n))
    _check(rc, None)
    return out[: n.value].tolist()


def initial_chunk_size(requested, steady: int, fallback: int = 0) -> int:
    """First-chunk size of a request in frames (``None``: the fallback), capped
    at the steady chunk size; the library validates it.  A request that is
    not an integer raises TypeError here (marshalling); the library's
    rejections (steady below 1, a negative size) raise ValueError."""
    if requested is None:
        has, v = 0, 0
    else:
        if isinstance(requested, bool):
            raise TypeError("a chunk size is a frame count, not a flag")
        try:
            v = operator.index(requested)
        except TypeError:
            raise TypeError(f"chunk size {requested!r} is not an integer frame count") from None
        has = 1
    out = C.c_int32()
    rc = lib().codec_initial_chunk_size(int(v), has, int(steady), int(fallback), C.byref(out))
    if rc != CODEC_OK:
        raise ValueError(lib().codec_last_error(None).decode())
    return out.value


def conv_plan(M: int, N: int, Cin: int, taps: int, fp16: bool = True, n_cu: int = 256,
              flags: int = 0) -> tuple[str, int]:
    """The conv GEMM planner's (tile name, K splits) for one launch shape
    (host logic; for tests and inspection)."""
    name = C.c_char_p()
    splits = C.c_int32()
    rc = lib().codec_debug_conv_plan(int(M), int(N), int(Cin), int(taps), int(bool(fp16)),
                                     int(n_cu), int(flags), C.byref(name), C.byref(splits))
    if rc != CODEC_OK:
        raise ValueError(lib().codec_last_error(None).decode())
    return name.value.decode(), splits.value
