"""GPU parity of gsa_decode / gsa_decode_hier against the fp64 oracle.

Selected chunk indices must match bit for bit; outputs within the stated
tolerance (tests/gpu_util.py). Small cases compare every unit; the full-size
workloads run in the launch configuration the benchmark times and compare
sampled units.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gsa_inputs as gi
import oracle
from conftest import to_np
from gpu_util import check_lse, check_out, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_gsa_amd
    decode_gsa_amd.lib()          # raises if the library is missing: no fallback
    return decode_gsa_amd


def run_decode(gsa, inp, cfg, units=None, gist_set="all"):
    """Run the GPU path once, then compare the listed units (default: all) with
    the oracle, copying only those units' cache slabs to the host."""
    out, lse, sel = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=cfg.chunk,
                                   topk=cfg.topk, tail=cfg.tail, n_gist=cfg.M, gist_set=gist_set)
    torch.cuda.synchronize()
    g = cfg.n_q_heads // cfg.n_kv_heads
    us = [(b, j) for b in range(cfg.batch) for j in range(cfg.n_kv_heads)] if units is None else units
    got, ref, got_l, ref_l = [], [], [], []
    for b, j in us:
        r = oracle.decode_unit(to_np(inp.q[b, j * g:(j + 1) * g]), to_np(inp.k_cache[b, j]),
                               to_np(inp.v_cache[b, j]), n_raw=cfg.n_raw, n_gist=cfg.M,
                               chunk=cfg.chunk, topk=cfg.topk, tail=cfg.tail, gist_set=gist_set)
        if cfg.topk > 0:
            np.testing.assert_array_equal(to_np(sel[b, j]), r["sel"], err_msg=f"unit {(b, j)}")
        got.append(to_np(out[b, j * g:(j + 1) * g]))
        ref.append(r["out"])
        got_l.append(to_np(lse[b, j * g:(j + 1) * g]))
        ref_l.append(r["lse"])
    err = check_out(np.stack(got), np.stack(ref), cfg.dtype, cfg.name)
    check_lse(np.stack(got_l), np.stack(ref_l), cfg.dtype, cfg.name)
    return err


def small(name, **kw):
    return dataclasses.replace(gi.CONFIGS[name], **kw)


# ---------------------------------------------------------------- small ---

CASES = [
    ("tiny_f32", {}),                                           # the parity config itself
    ("gqa_32k", dict(batch=2, n_raw=4096)),                     # 16x, several splits
    ("gqa_32k", dict(batch=3, n_kv_heads=2, n_q_heads=16, n_raw=2009, n_gist=125, tail=16)),
    ("c8_131k", dict(batch=1, n_raw=8192)),                     # C=8, k=64
    ("c32_131k", dict(batch=1, n_raw=8192)),                    # C=32
    ("gqa_32k", dict(batch=2, n_q_heads=8, n_raw=3000, n_gist=187, tail=40)),   # g=1, ragged
    ("gqa_32k", dict(batch=1, n_q_heads=16, n_raw=2048)),       # g=2
    ("gqa_32k", dict(batch=1, n_q_heads=64, n_raw=2048)),       # g=8
    ("gqa_32k", dict(batch=2, head_dim=64, n_raw=4096)),        # bf16, D=64
    ("gqa_32k", dict(batch=1, dtype="f32", n_raw=4096)),        # fp32, D=128
    ("tiny_f32", dict(chunk=7, n_raw=700, topk=5, tail=9, plant="none")),
    ("gqa_32k", dict(batch=1, chunk=1, n_raw=600, topk=30, tail=3, plant="none")),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(CASES)])
def test_decode_small(gsa, name, kw):
    cfg = small(name, **kw)
    say(f"decode small {cfg}")
    inp = gi.make_decode(cfg, 2000, device="cuda")
    err = run_decode(gsa, inp, cfg)
    say(f"  max err / rms = {err:.2e}")


def test_decode_k_zero_and_k_all(gsa):
    for k in (0, 128):
        cfg = small("gqa_32k", batch=2, n_raw=2048, topk=k, plant="none")
        say(f"decode k={k}")
        inp = gi.make_decode(cfg, 2001, device="cuda")
        run_decode(gsa, inp, cfg)


def test_decode_q_zero_ties_and_tail_overlap(gsa):
    """q = 0: every score is +-0, so chunks 0..k-1 win; the tail overlaps chunk k-1."""
    C, M, k = 16, 64, 8
    T = M * C - ((k - 1) * C + 8)             # tail starts mid-way through chunk k-1
    cfg = small("gqa_32k", batch=2, n_raw=M * C, topk=k, tail=T, plant="none")
    inp = gi.make_decode(cfg, 2002, device="cuda")
    inp.q.zero_()
    inp.k_cache.neg_()                         # mixes -0 and +0 products
    out, lse, sel = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=C, topk=k, tail=T)
    torch.cuda.synchronize()
    assert (to_np(sel) == np.arange(k)[None, None, :]).all()
    run_decode(gsa, inp, cfg)


def test_decode_selects_chunk_inside_tail(gsa):
    """A planted chunk that lies inside the tail: its rows must be attended once."""
    cfg = small("gqa_32k", batch=1, n_raw=2048, topk=4, tail=40, plant="none")
    inp = gi.make_decode(cfg, 2003, device="cuda")
    C = cfg.chunk
    g = cfg.n_q_heads // cfg.n_kv_heads
    last = cfg.M - 1                           # its raw rows are all in the tail
    for j in range(cfg.n_kv_heads):
        qbar = inp.q[0, j * g:(j + 1) * g].float().mean(0)
        inp.k_cache[0, j, last * (C + 1) + C] = (qbar / qbar.norm() * 40).to(inp.k_cache.dtype)
    out, lse, sel = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=C, topk=4, tail=40)
    torch.cuda.synchronize()
    assert (to_np(sel)[..., -1] == last).all()
    run_decode(gsa, inp, cfg)


@pytest.mark.parametrize("kw", [
    # more gists than one workgroup per unit keeps (split path, one unit per
    # kv-head): the unit's last workgroup selects among 20000 scores
    dict(batch=1, n_kv_heads=2, n_q_heads=8, n_raw=16 * 20000 + 7, topk=16, tail=64),
    # fp32, D = 64: 5000 scores, several rounds of loads per thread
    dict(batch=1, n_kv_heads=2, n_q_heads=4, head_dim=64, dtype="f32", n_raw=8 * 5000, chunk=8, topk=8, tail=8),
    # just above and at the single-round bound (4096 scores)
    dict(batch=2, n_kv_heads=1, n_q_heads=2, dtype="f32", head_dim=64, n_raw=16 * 4097, topk=12, tail=16),
    dict(batch=2, n_kv_heads=1, n_q_heads=2, dtype="f32", head_dim=64, n_raw=16 * 4096, topk=12, tail=16),
])
def test_decode_split_path_many_gists(gsa, kw):
    cfg = small("gqa_32k", **kw)
    say(f"split path {kw}")
    inp = gi.make_decode(cfg, 2100, device="cuda")
    err = run_decode(gsa, inp, cfg)
    say(f"  max err / rms = {err:.2e}, {gsa.gsa_profile_marks() - 1} launches")


def test_decode_no_gists(gsa):
    cfg = small("gqa_32k", batch=2, n_raw=12, n_gist=0, topk=0, tail=12, plant="none")
    inp = gi.make_decode(cfg, 2004, device="cuda")
    run_decode(gsa, inp, cfg)


def test_decode_repeatable_and_stream(gsa):
    cfg = small("gqa_32k", batch=2, n_raw=4096)
    inp = gi.make_decode(cfg, 2005, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        a = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=16, topk=16, tail=64, stream=s)
        b = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=16, topk=16, tail=64, stream=s)
    s.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[2], b[2]) and torch.equal(a[1], b[1])


def test_decode_on_a_stream_that_is_not_current(gsa):
    """stream=s while another stream is current and no workspace is given: the
    binding allocates the outputs and the zero-filled workspace on s, so the
    fill is ordered before the launch (the several-workgroups-per-unit launch
    uses the workspace's arrival counters). Checked against the oracle, then
    again after the allocator has had the chance to reuse the freed memory."""
    cfg = small("c32_131k", batch=2, n_kv_heads=2, n_q_heads=8, n_raw=65536)
    inp = gi.make_decode(cfg, 2011, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = cfg.n_q_heads // cfg.n_kv_heads
    for rep in range(2):
        out, lse, sel = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=cfg.chunk,
                                       topk=cfg.topk, tail=cfg.tail, stream=s)
        junk = torch.full((1 << 22,), 7, dtype=torch.uint8, device="cuda")   # current stream
        s.synchronize()
        del junk
        for b in range(cfg.batch):
            for j in range(cfg.n_kv_heads):
                r = oracle.decode_unit(to_np(inp.q[b, j * g:(j + 1) * g]), to_np(inp.k_cache[b, j]),
                                       to_np(inp.v_cache[b, j]), n_raw=cfg.n_raw, n_gist=cfg.M,
                                       chunk=cfg.chunk, topk=cfg.topk, tail=cfg.tail)
                np.testing.assert_array_equal(to_np(sel[b, j]), r["sel"])
                check_out(to_np(out[b, j * g:(j + 1) * g]), r["out"], cfg.dtype, f"rep {rep}")
                check_lse(to_np(lse[b, j * g:(j + 1) * g]), r["lse"], cfg.dtype, f"rep {rep}")


# ----------------------------------------------------------- full sizes ---

def sample_units(cfg, n=6, seed=0):
    rng = np.random.default_rng(seed)
    allu = [(b, j) for b in range(cfg.batch) for j in range(cfg.n_kv_heads)]
    pick = {allu[0], allu[-1]}
    while len(pick) < min(n, len(allu)):
        pick.add(allu[int(rng.integers(len(allu)))])
    return sorted(pick)


@pytest.mark.parametrize("name", ["gqa_32k", "c8_131k", "c32_131k"])
def test_decode_full_size_sampled(gsa, name):
    cfg = gi.CONFIGS[name]
    say(f"decode full {name}")
    inp = gi.make_decode(cfg, 1000 + {"gqa_32k": 2, "c8_131k": 3, "c32_131k": 4}[name],
                         device="cuda")
    # every unit's selection must be the planted (margin >= 0.5) set
    out, lse, sel = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=cfg.chunk,
                                   topk=cfg.topk, tail=cfg.tail)
    torch.cuda.synchronize()
    assert torch.equal(sel.long(), inp.planted)
    err = run_decode(gsa, inp, cfg, units=sample_units(cfg))
    say(f"  sampled max err / rms = {err:.2e}")


@pytest.mark.parametrize("name,dtype,topk", [("gqa_32k", "f32", 64), ("c8_131k", "bf16", 80)])
def test_decode_full_size_split_path_sampled(gsa, name, dtype, topk):
    """The split path (fp32; bf16 with k > 64) at a full workload size: every
    unit's selection against the oracle's on sampled units, their outputs
    element by element."""
    cfg = dataclasses.replace(gi.CONFIGS[name], dtype=dtype, topk=topk, plant="none")
    say(f"decode full split path {name} {dtype} k={topk}")
    inp = gi.make_decode(cfg, 1100, device="cuda")
    err = run_decode(gsa, inp, cfg, units=sample_units(cfg, n=4, seed=7))
    say(f"  sampled max err / rms = {err:.2e}")


# ------------------------------------------------------------ two-level ---

def run_hier(gsa, inp, cfg, units=None, gist_set="all"):
    b = cfg.base
    out, lse, s2, s1 = gsa.gsa_decode_hier(inp.q, inp.k_cache, inp.v_cache, inp.k_l2, inp.v_l2,
                                           chunk=b.chunk, fanout=cfg.fanout, topk1=b.topk,
                                           topk2=cfg.topk2, tail=b.tail, n_gist=b.M, gist_set=gist_set)
    torch.cuda.synchronize()
    g = b.n_q_heads // b.n_kv_heads
    us = ([(x, j) for x in range(b.batch) for j in range(b.n_kv_heads)] if units is None
          else units)
    errs = []
    for (x, j) in us:
        r = oracle.decode_hier_unit(to_np(inp.q[x, j * g:(j + 1) * g]), to_np(inp.k_cache[x, j]),
                                    to_np(inp.v_cache[x, j]), to_np(inp.k_l2[x, j]),
                                    to_np(inp.v_l2[x, j]), n_raw=b.n_raw, n_gist=b.M,
                                    chunk=b.chunk, fanout=cfg.fanout, topk1=b.topk,
                                    topk2=cfg.topk2, tail=b.tail, gist_set=gist_set)
        if cfg.topk2 > 0:
            np.testing.assert_array_equal(to_np(s2[x, j]), r["sel2"])
        if b.topk > 0:
            np.testing.assert_array_equal(to_np(s1[x, j]), r["sel1"])
        errs.append((to_np(out[x, j * g:(j + 1) * g]), r["out"], to_np(lse[x, j * g:(j + 1) * g]),
                     r["lse"]))
    got = np.stack([e[0] for e in errs])
    ref = np.stack([e[1] for e in errs])
    err = check_out(got, ref, b.dtype, b.name)
    check_lse(np.stack([e[2] for e in errs]), np.stack([e[3] for e in errs]), b.dtype, b.name)
    return err


HIER_CASES = [
    dict(batch=2, n_raw=16 * 16 * 64, fanout=16, topk2=8),            # 64 groups
    dict(batch=1, n_raw=16 * (16 * 20 + 5) + 9, n_gist=16 * 20 + 5, fanout=16, topk2=3,
         topk=10, plant="none"),                                        # orphans + partial chunk
    dict(batch=1, n_raw=16 * 16 * 8, fanout=16, topk2=8, topk=128, plant="none"),  # all chosen
    dict(batch=1, n_raw=16 * 16 * 8, fanout=16, topk2=0, topk=0, plant="none"),
    dict(batch=4, n_raw=16 * 8 * 40 + 16 * 5, fanout=8, topk2=6, topk=12),   # 5 orphans, k1 <= 64
    dict(batch=2, n_raw=16 * 16 * 16, fanout=16, topk2=16, topk=64, plant="none"),  # every group chosen
    dict(batch=1, n_raw=16 * 4 * 300, fanout=4, topk2=40, topk=20, plant="none"),   # k2 > 16
    # split path with many level-2 gists: the level-2 workgroups' top-k2
    # candidates feed the level-2 selection (fp32, and bf16 with k1 > 64)
    dict(batch=1, n_kv_heads=2, n_q_heads=8, dtype="f32", head_dim=64, n_raw=16 * 16 * 2000, fanout=16,
         topk2=8, topk=16),
    dict(batch=1, n_kv_heads=2, n_q_heads=8, n_raw=16 * 16 * 2000, fanout=16, topk2=8, topk=80),
]


@pytest.mark.parametrize("kw", HIER_CASES)
def test_hier_small(gsa, kw):
    kw = dict(kw)
    fanout, topk2 = kw.pop("fanout"), kw.pop("topk2")
    base = dataclasses.replace(gi.CONFIGS["hier_1m"].base, **kw)
    cfg = gi.HierConfig(base, fanout, topk2)
    say(f"hier small {kw} G={fanout} k2={topk2}")
    inp = gi.make_hier(cfg, 3000, device="cuda")
    err = run_hier(gsa, inp, cfg)
    say(f"  max err / rms = {err:.2e}")


# the selection rules on the split path (fp32, head_dim 64, k1 > 64): the
# level-2 and candidate passes only route, the set's own pass attends
HIER_SPLIT_SET_CASES = [
    dict(batch=1, n_kv_heads=2, n_q_heads=8, dtype="f32", head_dim=64, n_raw=16 * (16 * 20 + 5) + 9,
         n_gist=16 * 20 + 5, fanout=16, topk2=3, topk=10, plant="none"),          # orphans + partial chunk
    dict(batch=2, n_kv_heads=2, n_q_heads=4, head_dim=64, n_raw=16 * 8 * 40 + 16 * 5, fanout=8, topk2=6,
         topk=12),                                                               # bf16, D = 64
    dict(batch=1, n_kv_heads=2, n_q_heads=8, n_raw=16 * 16 * 2000, fanout=16, topk2=8, topk=80),   # k1 > 64
    dict(batch=1, n_kv_heads=2, n_q_heads=8, dtype="f32", head_dim=64, n_raw=16 * 16 * 2000, fanout=16,
         topk2=8, topk=16),                                                      # level-2 candidates
    dict(batch=1, n_kv_heads=2, n_q_heads=8, dtype="f32", head_dim=64, n_raw=16 * 16 * 8 + 7, fanout=16,
         topk2=2, topk=0, plant="none"),                                         # k1 = 0: the tail only
]


@pytest.mark.parametrize("gist_set", ["selected", "none"])
@pytest.mark.parametrize("kw", HIER_SPLIT_SET_CASES)
def test_hier_split_selection_rules(gsa, kw, gist_set):
    kw = dict(kw)
    fanout, topk2 = kw.pop("fanout"), kw.pop("topk2")
    base = dataclasses.replace(gi.CONFIGS["hier_1m"].base, **kw)
    cfg = gi.HierConfig(base, fanout, topk2)
    say(f"hier split {gist_set} {kw} G={fanout} k2={topk2}")
    inp = gi.make_hier(cfg, 3100, device="cuda")
    err = run_hier(gsa, inp, cfg, gist_set=gist_set)
    say(f"  max err / rms = {err:.2e}")


def test_hier_full_size_sampled(gsa):
    cfg = gi.CONFIGS["hier_1m"]
    say("hier full 1M")
    inp = gi.make_hier(cfg, 1004, device="cuda")
    b = cfg.base
    out, lse, s2, s1 = gsa.gsa_decode_hier(inp.q, inp.k_cache, inp.v_cache, inp.k_l2, inp.v_l2,
                                           chunk=b.chunk, fanout=cfg.fanout, topk1=b.topk,
                                           topk2=cfg.topk2, tail=b.tail)
    torch.cuda.synchronize()
    assert torch.equal(s2.long(), inp.planted2) and torch.equal(s1.long(), inp.planted1)
    err = run_hier(gsa, inp, cfg, units=[(0, 0), (1, 3), (3, 7)])
    say(f"  sampled max err / rms = {err:.2e}")


def test_workspace_reused_across_calls_and_shapes(gsa):
    """One zeroed workspace serves many calls of different shapes and both entry
    points: the control words must return to zero after every call."""
    import decode_gsa_amd as g
    ws = g.new_workspace(64 << 20)
    cfgs = [small("gqa_32k", batch=2, n_raw=4096), small("c8_131k", batch=1, n_raw=4096),
            small("gqa_32k", batch=1, n_q_heads=8, n_raw=1000, n_gist=62, tail=16)]
    inps = [gi.make_decode(c, 2100 + i, device="cuda") for i, c in enumerate(cfgs)]
    hcfg = gi.HierConfig(dataclasses.replace(gi.CONFIGS["hier_1m"].base, batch=1,
                                             n_raw=16 * 16 * 32), 16, 8)
    hinp = gi.make_hier(hcfg, 2200, device="cuda")
    ref = [gsa.gsa_decode(x.q, x.k_cache, x.v_cache, chunk=c.chunk, topk=c.topk, tail=c.tail,
                          n_gist=c.M) for c, x in zip(cfgs, inps)]
    b = hcfg.base
    href = gsa.gsa_decode_hier(hinp.q, hinp.k_cache, hinp.v_cache, hinp.k_l2, hinp.v_l2,
                               chunk=b.chunk, fanout=16, topk1=b.topk, topk2=8, tail=b.tail)
    for rep in range(3):
        for c, x, r in zip(cfgs, inps, ref):
            o = gsa.gsa_decode(x.q, x.k_cache, x.v_cache, chunk=c.chunk, topk=c.topk,
                               tail=c.tail, n_gist=c.M, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(o[0], r[0]) and torch.equal(o[2], r[2])
        o = gsa.gsa_decode_hier(hinp.q, hinp.k_cache, hinp.v_cache, hinp.k_l2, hinp.v_l2,
                                chunk=b.chunk, fanout=16, topk1=b.topk, topk2=8, tail=b.tail,
                                workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o[0], href[0]) and torch.equal(o[3], href[3])
        assert ctrl_words_zero(ws, c.batch * c.n_kv_heads)
    assert ctrl_words_zero(ws, b.batch * b.n_kv_heads)


def ctrl_words_zero(ws, units):
    # one 256-byte block of control words per (batch, kv-head) unit
    return int(ws[:256 * units].count_nonzero()) == 0


@pytest.mark.parametrize("batch,n_raw", [(2, 4096), (8, 4096), (1, 2048)])
def test_decode_bit_identical_over_repeats(gsa, batch, n_raw):
    """Many calls with fresh and with reused workspaces give bit-identical
    results, and the first one matches the oracle (cross-workgroup hand-offs
    inside the launch must never read stale data)."""
    import decode_gsa_amd as g
    cfg = small("gqa_32k", batch=batch, n_raw=n_raw)
    inp = gi.make_decode(cfg, 2300 + batch, device="cuda")
    run_decode(gsa, inp, cfg)
    first = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=16, topk=16, tail=64)
    ws = g.new_workspace(g.decode_workspace_size(g.decode_params(
        batch, 32, 8, 128, n_raw, n_raw // 16, 16, 16, 64)))
    bad = 0
    for rep in range(40):
        o = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=16, topk=16, tail=64,
                           workspace=ws if rep % 2 else None)
        torch.cuda.synchronize()
        same = (torch.equal(o[0], first[0]) and torch.equal(o[1], first[1])
                and torch.equal(o[2], first[2]))
        bad += 0 if same else 1
    assert bad == 0, f"{bad} of 40 repeats differ"
