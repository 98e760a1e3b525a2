"""bench.py's algorithmic byte counts (the numerators of its roofline
fractions) against totals worked out by hand from the cache layout: K and V
rows of 512 bytes (bf16, head_dim 128), q in bf16, fp32 outputs and lse, int32
ids. The selections used choose chunks that lie wholly outside the tail."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
import gsa_inputs as gi  # noqa: E402


def _first_chunks(units, k):
    return np.tile(np.arange(k), (units, 1))


def test_decode_bytes_gqa_32k():
    cfg = gi.CONFIGS["gqa_32k"]                 # 256 units, 2048 gists, C 16, k 16, T 64
    sel = _first_chunks(256, 16)
    # 256 x (2048 gists + 64 tail) rows + q | 256 x 16 x 16 raw rows + out, lse, ids
    want_all = 256 * 2112 * 512 + 32 * 32 * 128 * 2 + 256 * 256 * 512 + 32 * 32 * 129 * 4 + 256 * 16 * 4
    assert want_all == 311_185_408
    assert sum(bench.decode_bytes(cfg, sel)) == want_all
    # the rules: gist K rows only; "selected" adds the chosen gists' V rows
    assert sum(bench.decode_bytes(cfg, sel, "none")) == want_all - 256 * 2048 * 256 == 176_967_680
    assert sum(bench.decode_bytes(cfg, sel, "selected")) == 176_967_680 + 256 * 16 * 256 == 178_016_256


def test_hier_bytes_hier_1m():
    cfg = gi.CONFIGS["hier_1m"]                 # 32 units, 4096 level-2 gists, G 16, k2 8, k1 16, T 64
    sel1 = _first_chunks(32, 16)
    q = 4 * 32 * 128 * 2
    out = 4 * 32 * 129 * 4 + 32 * (16 + 8) * 4
    nb = bench.hier_bytes(cfg, sel1)
    assert nb["l2"] == 32 * (4096 + 64) * 512 + q
    assert nb["cand"] == 32 * 128 * 512          # 8 chosen groups x 16 children, no ungrouped gists
    assert nb["unfold"] == 32 * 256 * 512 + out
    assert sum(nb.values()) == 74_550_784
    none = bench.hier_bytes(cfg, sel1, "none")
    assert none["l2"] == 32 * 4096 * 256 + q and none["cand"] == 32 * 128 * 256
    assert none["unfold"] == 32 * (256 + 64) * 512 + out
    assert sum(none.values()) == 39_947_776
    assert sum(bench.hier_bytes(cfg, sel1, "selected").values()) == 39_947_776 + 32 * 16 * 256


def test_prefill_flops_prefill_64k():
    cfg = gi.CONFIGS["prefill_64k"]             # queries 61440..65535, C 16, k 16, window 64, Hq 32, D 128
    # eligible gists floor(t / 16): each of 3840..4095 for 16 queries; 16 chosen chunks of 16
    # rows and a 64-row window for every query; 4 D flops per (query head, row)
    gists = 16 * sum(range(3840, 4096))
    rows = gists + 4096 * 16 * 16 + 4096 * 64
    total, gist_qk = bench.prefill_flops(cfg)
    assert total == rows * 32 * 128 * 4 == 287_729_254_400
    assert gist_qk == gists * 32 * 128 * 2


def test_counter_traffic_only_for_the_source_it_was_taken_on():
    """The committed counter bytes are reported only while the kernel source
    they were measured on is the one built; they equal the scaled counters
    (FETCH_SIZE x 2, WRITE_SIZE x 1, KiB -> bytes)."""
    import json
    t = json.load(open(bench.TRAFFIC_FILE))
    for key, e in t.items():
        if key.startswith("_"):
            continue
        scaled = (e["fetch_kib"] * e["fetch_scale"] + e["write_kib"] * e["write_scale"]) * 1024
        assert abs(e["bytes_per_launch"] - scaled) <= 1024, key
        assert bench.measured_traffic(key, e["source_sha"]) == e["bytes_per_launch"]
        assert bench.measured_traffic(key, "0" * 16) is None
