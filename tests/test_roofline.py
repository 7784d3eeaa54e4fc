"""The bandwidth model against the Helix summary's TP roofline numbers."""

import json
import os

import pytest

from long_context_decode_split_amd import configs, roofline


def test_page_roofline(golden_dir):
    with open(os.path.join(golden_dir, "kv_read_roofline.json")) as f:
        g = json.load(f)
    rd = g["readings"]
    for tp, us in g["us_by_tp"].items():
        got = roofline.page_kv_read_us(g["batch"], rd["tokens"], g["kv_heads"], int(tp), rd["head_dim"],
                                       rd["bytes_per_element"], rd["hbm_bytes_per_s"])
        assert got == pytest.approx(us, rel=1e-12), (tp, got, us)


def test_workload_bytes():
    w = configs.LLAMA405B_SHARE
    assert roofline.kv_bytes(w, [w.ctx] * w.B) == 8 * 2**20 * 512
    m = configs.DEEPSEEK_MLA
    assert roofline.kv_bytes(m, [m.ctx] * m.B) == 8 * 2**20 * 1152
    f = configs.FP8_GQA
    assert roofline.kv_bytes(f, [f.ctx] * f.B) == 32 * 2**20 * (256 + 0.5)
    x = configs.MXFP4_RAGGED
    assert roofline.kv_bytes_per_token(x.Dk, x.Dv, False, "mxfp4") == 136
    assert roofline.attn_flops(w, [w.ctx] * w.B) == 8 * 2**20 * 16 * 2 * 256
