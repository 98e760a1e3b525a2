"""GPU parity of gsa_decode in its one-workgroup-per-unit launch (bf16,
head_dim 128, topk <= 64): one workgroup per (batch, kv-head) unit with 256
or more units and at most 4096 gists, otherwise several workgroups per unit
(with topk > 0 they hand their partial states and group scores to a second
launch that selects, unfolds and merges; with topk = 0 the unit's last
workgroup merges).
Checked against the fp64 oracle: bit-exact selections, outputs and lse within
the stated tolerance (tests/gpu_util.py).
"""
import dataclasses

import numpy as np
import pytest
import torch

import gsa_inputs as gi
from conftest import to_np
from gpu_util import say
from test_parity_decode import run_decode, sample_units

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_gsa_amd
    decode_gsa_amd.lib()          # raises if the library is missing: no fallback
    return decode_gsa_amd


def cfg_of(name, **kw):
    return dataclasses.replace(gi.CONFIGS[name], **kw)


# (config, units compared: None = every unit, else that many sampled)
CASES = [
    (cfg_of("gqa_32k", n_raw=4096), None),                                  # 256 units, g = 4
    (cfg_of("gqa_32k", n_q_heads=8, n_raw=3000, n_gist=187, tail=40), None),    # g = 1, ragged
    (cfg_of("gqa_32k", n_q_heads=16, n_raw=2048, tail=5), 64),             # g = 2
    (cfg_of("gqa_32k", n_q_heads=64, n_raw=2048), 64),                     # g = 8
    (cfg_of("gqa_32k", batch=40, n_raw=1500, tail=12), 64),                # 320 units, shortest tail
    (cfg_of("gqa_32k", n_raw=4096, topk=40), 64),                          # k > 16: top-4 threshold
    (cfg_of("c8_131k", batch=32, n_raw=8192), 48),                         # C = 8, k = 64
    (cfg_of("c32_131k", batch=32, n_raw=8192), 48),                        # C = 32
    (cfg_of("gqa_32k", n_raw=2048, topk=0, plant="none"), 64),             # gists + tail only
    (cfg_of("gqa_32k", n_raw=1024, topk=64, plant="none"), 64),            # every chunk selected
    (cfg_of("gqa_32k", n_raw=12, n_gist=0, topk=0, tail=12, plant="none"), 64),   # no gists
    (cfg_of("gqa_32k", n_raw=65536, tail=300), 12),                        # 4096 gists: the LDS limit
    (cfg_of("gqa_32k", n_raw=65552, tail=64), 12),                         # 4097 gists: two workgroups per unit
    # several workgroups per unit
    (cfg_of("c8_131k", n_raw=32768), None),                                # 64 units x 4, C = 8, k = 64
    (cfg_of("c32_131k", n_raw=65536), 32),                                 # 64 units x 4, C = 32
    (cfg_of("gqa_32k", batch=1, n_kv_heads=1, n_q_heads=4, n_raw=8192, tail=70), None),   # 1 unit x 40
    (cfg_of("gqa_32k", batch=3, n_kv_heads=2, n_q_heads=16, n_raw=9000, n_gist=562, tail=40), None),  # ragged
    (cfg_of("gqa_32k", batch=2, n_raw=4096, topk=0, plant="none"), None),  # gists + tail only
    (cfg_of("gqa_32k", batch=1, n_raw=16384 * 16, tail=64), 8),            # 16384 gists: the selection limit
    (cfg_of("gqa_32k", batch=1, n_kv_heads=1, n_q_heads=4, n_raw=65536, topk=64, tail=64), None),  # 1 unit x 65, k = 64
]


@pytest.mark.parametrize("case", range(len(CASES)), ids=[f"unit{i}" for i in range(len(CASES))])
def test_decode_unit_path(gsa, case):
    cfg, n = CASES[case]
    say(f"decode unit-path {cfg} units={'all' if n is None else n}")
    inp = gi.make_decode(cfg, 3000 + case, device="cuda")
    units = None if n is None else sample_units(cfg, n=n, seed=case)
    err = run_decode(gsa, inp, cfg, units=units)
    say(f"  max err / rms = {err:.2e}")


def test_decode_unit_ties_fall_back_to_radix(gsa):
    """q = 0: all 2048 group scores are +-0, more ties at the threshold than the
    candidate buffer holds, so the radix select decides: chunks 0..k-1, with
    the tail starting inside chunk k-1."""
    C, M, k = 16, 128, 16
    T = M * C - ((k - 1) * C + 8)
    cfg = cfg_of("gqa_32k", n_raw=M * C, topk=k, tail=T, plant="none")
    say(f"decode unit-path ties {cfg}")
    inp = gi.make_decode(cfg, 3100, device="cuda")
    inp.q.zero_()
    inp.k_cache.neg_()
    out, lse, sel = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=C, topk=k, tail=T)
    torch.cuda.synchronize()
    assert (to_np(sel) == np.arange(k)[None, None, :]).all()
    run_decode(gsa, inp, cfg, units=sample_units(cfg, n=32, seed=1))


@pytest.mark.parametrize("batch", [32, 2], ids=["one-wg", "split"])
def test_decode_unit_ties_radix_any_split(gsa, batch):
    """All scores equal: the radix select over the scores in the workspace
    decides, with one workgroup per unit and with several."""
    C, M, k = 16, 256, 16
    T = 64
    cfg = cfg_of("gqa_32k", batch=batch, n_raw=M * C, topk=k, tail=T, plant="none")
    say(f"decode unit-path ties {cfg}")
    inp = gi.make_decode(cfg, 3104 + batch, device="cuda")
    inp.q.zero_()
    out, lse, sel = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=C, topk=k, tail=T)
    torch.cuda.synchronize()
    assert (to_np(sel) == np.arange(k)[None, None, :]).all()
    run_decode(gsa, inp, cfg, units=sample_units(cfg, n=16, seed=4))


def test_decode_unit_selects_chunk_inside_tail(gsa):
    """A planted chunk whose raw rows all lie in the tail is attended once."""
    cfg = cfg_of("gqa_32k", n_raw=2048, topk=4, tail=40, plant="none")
    say(f"decode unit-path chunk in tail {cfg}")
    inp = gi.make_decode(cfg, 3101, device="cuda")
    C = cfg.chunk
    g = cfg.n_q_heads // cfg.n_kv_heads
    last = cfg.M - 1
    qbar = inp.q.float().view(cfg.batch, cfg.n_kv_heads, g, -1).mean(2)
    inp.k_cache[:, :, last * (C + 1) + C] = (qbar / qbar.norm(dim=-1, keepdim=True) * 40).to(
        inp.k_cache.dtype)
    out, lse, sel = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=C, topk=4, tail=40)
    torch.cuda.synchronize()
    assert (to_np(sel)[..., -1] == last).all()
    run_decode(gsa, inp, cfg, units=sample_units(cfg, n=32, seed=2))


def test_decode_unit_repeatable(gsa):
    cfg = cfg_of("gqa_32k", n_raw=4096)
    inp = gi.make_decode(cfg, 3102, device="cuda")
    a = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=16, topk=16, tail=64)
    b = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=16, topk=16, tail=64)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


def test_decode_unit_ties_inside_candidates(gsa):
    """Equal group scores at the k-th place, few enough for the candidate
    buffer: 10 gists share the best score and 10 the second best; with k = 16
    all of the first group and the 6 smallest ids of the second are chosen."""
    cfg = cfg_of("gqa_32k", n_raw=4096, topk=16, plant="none")
    say(f"decode unit-path partial ties {cfg}")
    inp = gi.make_decode(cfg, 3103, device="cuda")
    C = cfg.chunk
    g = cfg.n_q_heads // cfg.n_kv_heads
    qbar = inp.q.float().view(cfg.batch, cfg.n_kv_heads, g, -1).mean(2)
    unit_dir = qbar / qbar.norm(dim=-1, keepdim=True)
    first = [7 + 19 * i for i in range(10)]
    second = [4 + 23 * i for i in range(10)]      # disjoint from the first group
    for ids, mag in ((first, 40.0), (second, 30.0)):
        for m in ids:
            inp.k_cache[:, :, m * (C + 1) + C] = (unit_dir * mag).to(inp.k_cache.dtype)
    out, lse, sel = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=C, topk=16, tail=cfg.tail)
    torch.cuda.synchronize()
    want = np.array(sorted(first + sorted(second)[:6]))
    assert (to_np(sel) == want[None, None, :]).all()
    run_decode(gsa, inp, cfg, units=sample_units(cfg, n=24, seed=3))


@pytest.mark.parametrize("n_raw", [16 * 4096, 16 * 16384])
def test_decode_unit_ties_across_splits(gsa, n_raw):
    """Several workgroups per unit, each handing on its own top-k: 10 gists
    share the best score and 12 the second best, spread over every split, and
    8 more of the second score sit together in the last split. With k = 16 the
    first group and the 6 smallest ids of the second are chosen, so the
    candidates of different splits must break the tie by id."""
    cfg = cfg_of("gqa_32k", batch=1, n_kv_heads=2, n_q_heads=8, n_raw=n_raw, topk=16, plant="none")
    say(f"decode unit-path ties across splits {cfg}")
    inp = gi.make_decode(cfg, 3110, device="cuda")
    C, M = cfg.chunk, cfg.M
    g = cfg.n_q_heads // cfg.n_kv_heads
    qbar = inp.q.float().view(cfg.batch, cfg.n_kv_heads, g, -1).mean(2)
    unit_dir = qbar / qbar.norm(dim=-1, keepdim=True)
    first = [(M // 10) * i + 3 for i in range(10)]
    second = [(M // 12) * i + 5 for i in range(12)] + [M - 20 + i for i in range(8)]
    for ids, mag in ((first, 40.0), (second, 30.0)):
        for m in ids:
            inp.k_cache[:, :, m * (C + 1) + C] = (unit_dir * mag).to(inp.k_cache.dtype)
    out, lse, sel = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=C, topk=16, tail=cfg.tail)
    torch.cuda.synchronize()
    assert gsa.gsa_profile_marks() == 3        # stream launch + select-unfold-merge launch
    want = np.array(sorted(first + sorted(second)[:6]))
    assert (to_np(sel) == want[None, None, :]).all()
    run_decode(gsa, inp, cfg)
