"""CPU checks of the benchmark's algorithmic work model: the FLOPs per frame
that every utilisation figure divides by, against the per-layer sums derived
from the decoder's definition (causal convs, polyphase transposed convs,
residual units, projections, windowed attention)."""
import importlib.util
import os

import pytest

import rvq_inputs as RI

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def direct_flops_per_frame(cfg: dict) -> float:
    """FLOPs of one frame written out layer by layer from the network's
    definition (2 per multiply-add), independently of the benchmark's model."""
    ch = RI.channels(cfg)
    K, dcb, dl = cfg["K"], cfg["d_cb"], cfg["d_lat"]
    f = 2 * dcb * dl                      # codebook-space sum -> latent projection
    f += 2 * 7 * dl * ch[0]               # input conv, kernel 7
    r = 1
    for i, s in enumerate(cfg["strides"]):
        ci, co = ch[i], ch[i + 1]
        f += r * s * co * 2 * ci * 2      # transposed conv, kernel 2s: 2 taps per output
        r *= s
        f += 2 * r * (2 * 7 * co * co + 2 * co * co)  # two residual units (k7 + 1x1)
    f += 2 * r * 7 * ch[-1]               # final conv to one channel
    if cfg["tf_layers"]:
        dm = cfg["tf_heads"] * cfg["tf_head_dim"]
        f += 2 * 2 * dl * dm              # in / out projections
        for _ in range(cfg["tf_layers"]):
            f += 2 * dm * 3 * dm + 2 * dm * dm + 2 * 2 * dm * cfg["tf_mlp"]
            f += 2 * 2 * cfg["tf_window"] * dm  # scores and weighted values, full window
    return float(f)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_flops_per_frame_matches_the_layer_sum(name):
    cfg = RI.get_config(name)
    assert _bench().flops_per_frame(cfg) == pytest.approx(direct_flops_per_frame(cfg), rel=1e-12)


def test_flops_per_frame_values():
    b = _bench()
    # Qwen-shaped decoder: 467.48 MFLOP per frame; Fish-shaped: 715.26 (27.53 of them
    # in the windowed transformer); the tiny fp32 decoder: 0.39
    assert b.flops_per_frame(RI.get_config("c2")) / 1e6 == pytest.approx(467.476, abs=1e-3)
    assert b.flops_per_frame(RI.get_config("c3")) / 1e6 == pytest.approx(715.26, abs=0.01)
    assert b.flops_per_frame(RI.get_config("c1")) / 1e6 == pytest.approx(0.3927, abs=1e-4)


def test_code_digest_ignores_comments_not_code(tmp_path):
    """The provenance digest that ties stored counter summaries to the
    library's code: comments and whitespace do not change it, code and string
    literals do."""
    b = _bench()
    a = tmp_path / "a.hip"
    a.write_text('int f() { return 1; } // one\n/* block\n comment */ const char *s = "a//b";\n')
    c = tmp_path / "c.hip"
    c.write_text('int f()  {\n  return 1;   }\nconst char *s = "a//b"; // other words\n')
    d = tmp_path / "d.hip"
    d.write_text('int f() { return 2; }\nconst char *s = "a//b";\n')
    e = tmp_path / "e.hip"
    e.write_text('int f() { return 1; }\nconst char *s = "a/b";\n')
    assert b.code_text(str(a)) == b.code_text(str(c))
    assert b.code_text(str(a)) != b.code_text(str(d))
    assert b.code_text(str(a)) != b.code_text(str(e))
    assert b"//" in b.code_text(str(a))  # inside the string literal
    assert b"one" not in b.code_text(str(a)) and b"block" not in b.code_text(str(a))


def test_measured_mfma_peak_is_read_from_the_committed_ceilings():
    """The bench line's measured-peak context comes from the committed
    ceilings summary: the best 16x16x32 f16 MFMA rate, below the published
    2.5 PFLOP/s."""
    b = _bench()
    mp = b.measured_mfma_peak()
    assert mp is not None and 1000.0 < mp <= 2516.6
    hp = b.measured_hbm_peak()
    assert hp is not None and 1000.0 < hp <= 8000.0
