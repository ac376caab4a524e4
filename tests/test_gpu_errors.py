"""GPU-side error paths of the C ABI: each failing call returns its code, with
a message naming the offending value, and changes no state."""
import numpy as np
import pytest
import torch

import rvq_inputs as RI
import streaming_neural_audio_rvq_amd as snr
from _util import host_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def small_codec():
    cfg = RI.get_config("c1", max_streams=3, max_frames_per_call=20)
    return cfg, snr.Codec(cfg, host_weights(cfg, RI.make_weights(cfg)))


def decode(c, ids, n, codes):
    pcm = torch.empty(max(1, sum(n)) * c.hop, dtype=torch.float32, device="cuda")
    c.decode_chunk(ids, n, codes, pcm)
    return pcm.cpu().numpy()


def err_of(fn):
    with pytest.raises(snr.CodecError) as ei:
        fn()
    return ei.value


def test_error_codes_and_no_state_change(small_codec):
    cfg, c = small_codec
    print("case error paths", flush=True)
    a = c.stream_open()
    b = c.stream_open()
    codes = RI.stream_codes(cfg, 0, 6)
    pcm = torch.empty(6 * c.hop, dtype=torch.float32, device="cuda")

    # EOS-sized code (2150) is outside the codebook
    bad = codes[:3].copy()
    bad[1, 2] = 2150
    e = err_of(lambda: c.decode_chunk([a], [3], bad, pcm))
    assert e.code == snr.CODEC_ERANGE and "2150" in str(e)
    # duplicate stream in one call
    e = err_of(lambda: c.decode_chunk([a, a], [1, 1], codes[:2], pcm))
    assert e.code == snr.CODEC_EDUP
    # unknown stream
    e = err_of(lambda: c.decode_chunk([999], [1], codes[:1], pcm))
    assert e.code == snr.CODEC_ESTREAM
    # non-positive chunk
    e = err_of(lambda: c.decode_chunk([a, b], [2, 0], codes[:2], pcm))
    assert e.code == snr.CODEC_EINVAL
    # too many frames in one call
    big = RI.stream_codes(cfg, 1, 21)
    big_pcm = torch.empty(21 * c.hop, dtype=torch.float32, device="cuda")
    e = err_of(lambda: c.decode_chunk([a], [21], big, big_pcm))
    assert e.code == snr.CODEC_ETOOBIG
    # PCM buffer too small
    e = err_of(lambda: c.decode_chunk([a], [6], codes, pcm[: 6 * c.hop - 1]))
    assert e.code == snr.CODEC_EINVAL

    # none of the failed calls touched a's state: a decodes like b, a fresh twin
    x = decode(c, [a], [6], codes)
    y = decode(c, [b], [6], codes)
    assert np.array_equal(x, y)
    c.stream_close(a)
    c.stream_close(b)


def test_slots_exhaust_and_close_then_reopen(small_codec):
    cfg, c = small_codec
    print("case slots", flush=True)
    ids = [c.stream_open() for _ in range(3)]
    e = err_of(c.stream_open)
    assert e.code == snr.CODEC_ENOSLOT
    codes = RI.stream_codes(cfg, 2, 9)
    # close mid-utterance, reopen: the new stream starts from zero state
    decode(c, [ids[0]], [4], codes[:4])
    c.stream_close(ids[0])
    e = err_of(lambda: c.decode_chunk([ids[0]], [1], codes[:1],
                                      torch.empty(c.hop, device="cuda")))
    assert e.code == snr.CODEC_ESTREAM
    new = c.stream_open()
    assert new not in ids
    x = decode(c, [new], [9], codes)
    y = decode(c, [ids[1]], [9], codes)
    assert np.array_equal(x, y)
    for i in (new, ids[1], ids[2]):
        c.stream_close(i)


def test_device_resident_codes_match_host_codes_and_count_bad_codes(small_codec):
    cfg, c = small_codec
    print("case device-resident codes", flush=True)
    a = c.stream_open()
    b = c.stream_open()
    codes = RI.stream_codes(cfg, 4, 7)
    x = decode(c, [a], [7], codes)
    pcm = torch.empty(7 * c.hop, dtype=torch.float32, device="cuda")
    c.decode_chunk_device([b], [7], torch.from_numpy(codes).cuda(), pcm)
    assert np.array_equal(x, pcm.cpu().numpy())
    assert c.device_status() == 0
    bad = codes.copy()
    bad[2, 1] = 2150
    bad[5, 0] = -3
    c.decode_chunk_device([b], [7], torch.from_numpy(bad).cuda(), pcm)
    e = err_of(c.device_status)
    assert e.code == snr.CODEC_ERANGE and "2 out-of-range" in str(e)
    assert c.device_status() == 0  # the count resets
    c.stream_close(a)
    c.stream_close(b)
