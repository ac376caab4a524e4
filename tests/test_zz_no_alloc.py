"""decode_chunk_device_noalloc: the step's scratch in the library's static
device array instead of the codec's buffers; checked against
decode_chunk_device on the same codes, two calls in a row (the second
smaller), and against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import rvq_inputs as RI
import streaming_neural_audio_rvq_amd as snr
from _util import host_weights, rel_err, tol_for

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_noalloc_matches_decode_chunk_device(name):
    """c2: the Qwen-shaped decoder; c3: the Fish-shaped decoder, whose
    transformer's per-step tables (attention query blocks) also live in the
    static array's metadata region."""
    if name == "c2":
        cfg = RI.get_config("c2", max_streams=16, max_frames_per_call=256)
        calls = [[8, 3, 16, 1, 8, 4], [2, 1, 4]]  # the second call smaller, same streams
    else:
        cfg = RI.get_config("c3", max_streams=8, max_frames_per_call=64)
        calls = [[8, 3, 20, 1], [2, 1, 4]]
    w = RI.make_weights(cfg)
    codec = snr.Codec(cfg, host_weights(cfg, w))
    H = codec.hop
    B = len(calls[0])
    total = [sum(c[b] for c in calls if b < len(c)) for b in range(B)]
    codes = [RI.stream_codes(cfg, b, total[b], part=12) for b in range(B)]
    ids_ref = [codec.stream_open() for _ in range(B)]
    ids_new = [codec.stream_open() for _ in range(B)]
    got = {"ref": [[] for _ in range(B)], "new": [[] for _ in range(B)]}
    at = [0] * B
    for k, n in enumerate(calls):
        Bk = len(n)
        packed = np.concatenate([codes[b][at[b]:at[b] + n[b]] for b in range(Bk)])
        dev = torch.from_numpy(packed).cuda()
        for tag, ids, fn in (("ref", ids_ref, codec.decode_chunk_device),
                             ("new", ids_new, codec.decode_chunk_device_noalloc)):
            pcm = torch.empty(int(sum(n)) * H, dtype=torch.float32, device="cuda")
            fn(ids[:Bk], n, dev, pcm)
            host = pcm.cpu().numpy()
            o = 0
            for b in range(Bk):
                got[tag][b].append(host[o * H:(o + n[b]) * H])
                o += n[b]
        for b in range(Bk):
            x, y = got["new"][b][-1], got["ref"][b][-1]
            e, _ = rel_err(x, y.astype(np.float64))
            print(f"call {k} stream {b} n {n[b]}: noalloc vs device err/peak {e:.3e} "
                  f"bitwise {np.array_equal(x, y)}", flush=True)
            assert e <= tol_for(cfg)
            at[b] += n[b]
    assert codec.device_status() == 0
    m = oracle.Model(cfg, w)
    for b in range(B):
        e, ac = rel_err(np.concatenate(got["new"][b]), m.decode_full(codes[b]))
        print(f"stream {b}: noalloc vs oracle err/peak {e:.3e} AC-rel {ac:.3e}", flush=True)
        assert e <= tol_for(cfg)
    codec.close()
