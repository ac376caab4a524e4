"""CPU-only checks of the HIP library's host side: it loads, exports every
function its header declares, and its host-only policy and argument checks
behave as specified.  No kernel runs here."""
import ctypes as C
import json
import os
import re

import numpy as np
import pytest

import rvq_inputs as RI
import streaming_neural_audio_rvq_amd as snr
from oracle import policy

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "chunk_plan_qwen3_tts.json")))


def header_functions():
    text = open(os.path.join(ROOT, "include", "snrvq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    L = snr.lib()
    declared = header_functions()
    assert len(declared) >= 13
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(snr.EXPORTS) == declared


def test_probe_library_exports_its_header():
    """The micro-benchmark library (include/snrvq_probes.h) exports every
    function its header declares; without a GPU it counts no CUs and refuses
    to run."""
    text = open(os.path.join(ROOT, "include", "snrvq_probes.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"^\s*int\s+(\w+)\s*\(", text, flags=re.M)))
    assert names == ["probe_cu_count", "probe_gload", "probe_hbm", "probe_lds", "probe_mfma",
                     "probe_overlap"]
    L = C.CDLL(os.path.join(ROOT, "streaming_neural_audio_rvq_amd", "libsnrvq_probes.so"))
    for name in names:
        assert hasattr(L, name), name
    if L.probe_cu_count() == 0:  # no device here
        res = (C.c_double * 3)()
        assert L.probe_mfma(0, 1, 10, 1, res) == 1


def test_chunk_plan_printed_example():
    plan = snr.chunk_plan(sum(GOLD["new_frames_per_decode"]), GOLD["ramp"], GOLD["steady"])
    assert plan == GOLD["new_frames_per_decode"]
    assert policy.decode_points(plan)[:6] == GOLD["decode_points_first_six"]


def test_chunk_plan_matches_oracle_policy():
    rng = np.random.default_rng(5)
    for _ in range(300):
        total = int(rng.integers(0, 120))
        ramp = tuple(int(v) for v in rng.integers(1, 12, size=int(rng.integers(0, 5))))
        steady = int(rng.integers(1, 17))
        initial = int(rng.integers(0, 20)) if rng.random() < 0.3 else 0
        if not ramp and initial == 0:
            ramp = (steady,)
        assert snr.chunk_plan(total, ramp, steady, initial) == \
            policy.chunk_plan(total, ramp, steady, initial), (total, ramp, steady, initial)


def test_initial_chunk_size_matches_oracle_policy():
    cases = [(None, 8, 0), (None, 8, 3), (5, 8, 0), (40, 8, 0), (0, 8, 0), (8, 8, 1),
             (np.int32(7), 4, 0), (3, 1, 0)]
    for req, steady, fb in cases:
        assert snr.initial_chunk_size(req, steady, fb) == \
            policy.initial_chunk_size(req, steady, fb), (req, steady, fb)
    for req, steady, fb in [(3, 0, 0), (-1, 8, 0), (None, 8, -1)]:
        with pytest.raises(ValueError):
            snr.initial_chunk_size(req, steady, fb)
    for bad in ("5", 2.5, True):
        with pytest.raises(TypeError):
            snr.initial_chunk_size(bad, 8)


def _bits(cfg, w):
    return RI.weight_bits(w) if cfg["weight_dtype"] == "bf16" else w


def open_err(cfg, weights):
    with pytest.raises(snr.CodecError) as ei:
        snr.Codec(cfg, weights)
    return ei.value


def test_open_rejects_bad_config_before_touching_a_device():
    cfg = RI.get_config("c1")
    w = RI.make_weights(cfg)
    e = open_err(dict(cfg, K=0), w)
    assert e.code == snr.CODEC_EINVAL and "K=0" in str(e)
    e = open_err(dict(cfg, strides=[]), w)
    assert e.code == snr.CODEC_EINVAL
    e = open_err(dict(cfg, max_frames_per_call=0), w)
    assert e.code == snr.CODEC_EINVAL
    e = open_err(dict(cfg, d_lat=48), RI.make_weights(dict(cfg, d_lat=48)))
    assert e.code == snr.CODEC_EINVAL and "multiple" in str(e)


def test_open_rejects_bad_weight_manifest():
    cfg = RI.get_config("c1")
    w = dict(RI.make_weights(cfg))
    missing = {k: v for k, v in w.items() if k != "dec.out.conv.bias"}
    e = open_err(cfg, missing)
    assert e.code == snr.CODEC_EINVAL and "dec.out.conv.bias" in str(e) and "missing" in str(e)
    bad = dict(w)
    bad["dec.stage.0.convT.weight"] = np.zeros((3, 3, 3), np.float32)
    e = open_err(cfg, bad)
    assert e.code == snr.CODEC_EINVAL and "shape" in str(e)
    extra = dict(w)
    extra["dec.bogus"] = np.zeros(3, np.float32)
    e = open_err(cfg, extra)
    assert e.code == snr.CODEC_EINVAL and "dec.bogus" in str(e)
    # fp32 tensors for a configuration whose weights are bf16: dtype mismatch
    import ctypes as C
    cfg2 = RI.get_config("c2")
    w2 = RI.make_weights(cfg2)
    arr, keep = snr.make_tensors(w2, "fp32")
    h = C.c_void_p()
    rc = snr.lib().codec_open(arr, len(w2), C.byref(snr.make_cfg(cfg2)), C.byref(h))
    assert rc == snr.CODEC_EINVAL and not h.value
    assert b"dtype" in snr.lib().codec_last_error(None)
    with pytest.raises(TypeError):
        snr.make_tensors(w2, "bf16")  # the binding wants bit patterns for bf16


def test_open_without_gpu_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    cfg = RI.get_config("c1")
    e = open_err(cfg, RI.make_weights(cfg))
    assert e.code == snr.CODEC_EHIP


def test_conv_planner_choices_on_the_128_stream_shapes():
    """The planner's tile and K-split choices for the 128-stream decoder's
    layers at 794 frames on 256 CUs (host logic only)."""
    F = 794
    # frame-rate layers: a 128 x 128 tile would leave CUs idle, a three-buffer
    # half tile reaches 1.5 work-groups per CU unsplit
    assert snr.conv_plan(F * 8, 512, 512, 7) == ("h128x64k64b3", 1)    # stage-0 k7 conv
    assert snr.conv_plan(F, 8 * 512, 1024, 2) == ("h128x64k64b3", 1)   # stage-0 transposed conv
    assert snr.conv_plan(F * 8, 512, 512, 1) == ("h128x64k64b3", 1)    # stage-0 1x1 conv
    # layers that fill the GPU with 128 x 128 tiles
    assert snr.conv_plan(F * 40, 256, 256, 7) == ("h128x128k64", 1)    # stage-1 k7 conv
    assert snr.conv_plan(F * 8, 5 * 256, 512, 2) == ("h128x128k64", 1)  # stage-1 transposed conv
    assert snr.conv_plan(F * 40, 4 * 128, 256, 2) == ("h128x128k64", 1)  # stage-2 transposed conv
    # few rows, long K: the input conv splits K; the short-K projection does not
    tile, sp = snr.conv_plan(F, 1024, 1024, 7)
    assert sp > 1 and (1024 * 7 // 64) // sp >= 8
    assert snr.conv_plan(F, 1024, 512, 1)[1] == 1


def test_conv_planner_small_steps_take_64x64_tiles():
    """Layers of steps of a few frames (little work per CU) take the 64 x 64
    tile, K split up to 1.5 work-groups per CU with at least 8 K stages per
    split, and K of at most 16 stages unsplit (timed on the Qwen-shaped decoder's
    first layers at 1, 8 and 64 frames per step)."""
    for F in (1, 8):
        assert snr.conv_plan(F, 1024, 1024, 7) == ("h64x64k64", 14)      # input conv
        assert snr.conv_plan(F, 8 * 512, 1024, 2) == ("h64x64k64", 4)    # stage-0 transposed conv
        assert snr.conv_plan(F * 8, 512, 512, 7) == ("h64x64k64", 7)     # stage-0 k7 conv
        assert snr.conv_plan(F * 8, 512, 512, 1) == ("h64x64k64", 1)     # stage-0 1x1 conv
        assert snr.conv_plan(F * 8, 5 * 256, 512, 2) == ("h64x64k64", 1)  # 16 K stages: unsplit
    assert snr.conv_plan(64, 1024, 1024, 7) == ("h64x64k64", 14)
    assert snr.conv_plan(64 * 8, 512, 512, 7) == ("h64x64k64", 6)        # 64 tiles x 6 = 384
    assert snr.conv_plan(64 * 40, 256, 256, 7) == ("h64x64k64", 3)       # 160 tiles x 3 = 480
    # 512 frames: 128 x 128 unsplit from 1.25 work-groups per CU, half tiles from one
    assert snr.conv_plan(512 * 40, 256, 256, 7) == ("h128x128k64", 1)  # 320 tiles
    assert snr.conv_plan(512, 8 * 512, 1024, 2) == ("h128x64k64b3", 1)  # 256 tiles
    assert snr.conv_plan(512 * 8, 512, 512, 7) == ("h128x64k64b3", 1)
    # 160-row tiles where 128 x 128 tiles would overflow whole rounds of two
    # work-groups per CU by a few (the 128-stream steps above ~819 frames)
    assert snr.conv_plan(800 * 40, 256, 256, 7) == ("h128x128k64", 1)    # 500 tiles
    assert snr.conv_plan(848 * 40, 256, 256, 7) == ("h160x128k64", 1)    # 530 -> 424
    assert snr.conv_plan(848 * 8, 5 * 256, 512, 2) == ("h160x128k64", 1)  # 530 -> 430
    assert snr.conv_plan(848 * 40, 256, 256, 7, flags=snr.FLAG_NO_TALL_TILES) == \
        ("h128x128k64", 1)
    # no split where the flags forbid it; the 794-frame input conv keeps the large tiles
    assert snr.conv_plan(8, 1024, 1024, 7, flags=snr.FLAG_NO_SPLIT_K) == ("h64x64k64", 1)
    assert snr.conv_plan(794, 1024, 1024, 7)[0] != "h64x64k64"


def test_conv_planner_flags_and_invariants():
    F = 794
    NO_SPLIT, TWO_BUF = snr.FLAG_NO_SPLIT_K, snr.FLAG_TWO_STAGE_BUFFERS
    assert snr.conv_plan(F, 1024, 1024, 7, flags=NO_SPLIT)[1] == 1
    assert not snr.conv_plan(F * 8, 512, 512, 7, flags=TWO_BUF)[0].endswith("b3")
    rng = np.random.default_rng(11)
    for _ in range(400):
        M = int(rng.integers(1, 400_000))
        N = int(rng.choice([32, 64, 128, 192, 256, 512, 1024, 1280, 1536, 2048, 4096]))
        Cin = int(rng.choice([32, 64, 128, 256, 512, 1024]))
        taps = int(rng.choice([1, 2, 7]))
        flags = int(rng.choice([0, NO_SPLIT, TWO_BUF, NO_SPLIT | TWO_BUF, snr.FLAG_NO_TALL_TILES]))
        tile, sp = snr.conv_plan(M, N, Cin, taps, flags=flags)
        bm, bn, bk = (int(v) for v in re.match(r"h(\d+)x(\d+)(?:k(\d+))?", tile).groups("32"))
        assert N % bn == 0 and Cin % bk == 0, (M, N, Cin, taps, tile)
        assert sp >= 1 and (sp == 1 or (Cin * taps // bk) // sp >= 8), (M, N, Cin, taps, sp)
        assert sp * M * N <= 16 << 20 or sp == 1
        if flags & NO_SPLIT:
            assert sp == 1
        if flags & TWO_BUF:
            assert not tile.endswith("b3")
        if flags & snr.FLAG_NO_TALL_TILES:
            assert not tile.startswith("h160")
        if tile.startswith("h160"):  # only in place of an unsplit 128 x 128 tile
            assert sp == 1 and N % 128 == 0
    with pytest.raises(ValueError):
        snr.conv_plan(0, 64, 64, 1)

