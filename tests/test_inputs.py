"""Checks of the seeded input generator (CPU): determinism, bf16 rounding, and
that the planted margins make the oracle's top-k unambiguous."""
import dataclasses

import numpy as np
import pytest
import torch

import gsa_inputs as gi
import oracle
from conftest import to_np


def small_decode(name="gqa_32k", **kw):
    base = dict(batch=2, n_raw=4096)
    base.update(kw)
    return dataclasses.replace(gi.CONFIGS[name], **base)


def test_deterministic_per_seed():
    cfg = small_decode()
    a, b = gi.make_decode(cfg, 7), gi.make_decode(cfg, 7)
    assert a.seed == b.seed
    assert torch.equal(a.q, b.q) and torch.equal(a.k_cache, b.k_cache)
    assert torch.equal(a.v_cache, b.v_cache)
    c = gi.make_decode(cfg, 7 + 100)
    assert not torch.equal(a.k_cache, c.k_cache)


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even mantissa (1.0);
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6 -> 1 + 2^-6
    x = torch.tensor([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20])
    y = gi._store(x, "bf16").float()
    assert y.tolist() == [1.0, 1 + 2 ** -6, -1.0, 1 + 2 ** -7]


def test_tiny_f32_config_shapes_and_margin():
    cfg = gi.CONFIGS["tiny_f32"]
    inp = gi.make_decode(cfg, 1001)
    assert tuple(inp.k_cache.shape) == (1, 1, 4352, 64)
    assert inp.k_cache.dtype == torch.float32
    assert inp.min_gap >= cfg.margin


@pytest.mark.parametrize("name,kw", [("gqa_32k", {}), ("c8_131k", {"n_raw": 8192}),
                                     ("c32_131k", {"n_raw": 8192}),
                                     ("tiny_f32", {"batch": 1})])
def test_planted_chunks_are_the_oracle_topk(name, kw):
    cfg = small_decode(name, **kw)
    inp = gi.make_decode(cfg, 1000)
    out, lse, sel = oracle.decode(to_np(inp.q), to_np(inp.k_cache), to_np(inp.v_cache),
                                  chunk=cfg.chunk, topk=cfg.topk, tail=cfg.tail)
    np.testing.assert_array_equal(sel, to_np(inp.planted))
    # realized gap measured with the oracle's own scores
    g = cfg.n_q_heads // cfg.n_kv_heads
    for b in range(cfg.batch):
        for j in range(cfg.n_kv_heads):
            r = oracle.decode_unit(to_np(inp.q[b, j * g:(j + 1) * g]), to_np(inp.k_cache[b, j]),
                                   to_np(inp.v_cache[b, j]), n_raw=cfg.n_raw, n_gist=cfg.M,
                                   chunk=cfg.chunk, topk=cfg.topk, tail=cfg.tail)
            S = r["scores"]
            pl = to_np(inp.planted[b, j])
            rest = np.setdiff1d(np.arange(cfg.M), pl)
            assert S[pl].min() - S[rest].max() >= cfg.margin - 1e-9
            # planted chunks never touch the tail
            assert (pl.max() + 1) * cfg.chunk <= cfg.n_raw - cfg.tail


def test_hier_planted_levels_match_oracle():
    base = dataclasses.replace(gi.CONFIGS["hier_1m"].base, batch=1, n_raw=16 * 16 * 48)
    cfg = gi.HierConfig(base, fanout=16, topk2=8)
    inp = gi.make_hier(cfg, 1004)
    out, lse, sel2, sel1 = oracle.decode_hier(
        to_np(inp.q), to_np(inp.k_cache), to_np(inp.v_cache), to_np(inp.k_l2), to_np(inp.v_l2),
        chunk=base.chunk, fanout=16, topk1=base.topk, topk2=8, tail=base.tail)
    np.testing.assert_array_equal(sel2, to_np(inp.planted2))
    np.testing.assert_array_equal(sel1, to_np(inp.planted1))
    assert min(inp.min_gap2, inp.min_gap1) >= base.margin


def test_prefill_planted_blocks_match_oracle_on_sampled_queries():
    cfg = dataclasses.replace(gi.CONFIGS["prefill_64k"], n_raw=8192, n_q=256)
    inp = gi.make_prefill(cfg, 1005)
    assert inp.min_gap >= cfg.margin
    qs = [(i, j) for i in (0, 1, 63, 64, 130, 255) for j in (0, 5, 7)]
    out, sel = oracle.prefill(to_np(inp.q), to_np(inp.k_cache), to_np(inp.v_cache),
                              chunk=cfg.chunk, topk=cfg.topk, window=cfg.window,
                              q_start=cfg.q_start, queries=qs)
    for i, j in qs:
        np.testing.assert_array_equal(sel[j, i], to_np(inp.planted[i // cfg.q_block, j]))


# ------------------------------------- variable lengths, levels, streams ---

@pytest.mark.parametrize("n_min,n_max,chunk", [(16, 4000, 16), (300, 8192, 16), (80, 3000, 8), (1, 40, 4)])
def test_varlen_lengths_keep_the_layout(n_min, n_max, chunk):
    """Every generated (n, m) pair is a valid interleaved cache: gists only of
    complete chunks, at most one full chunk waiting for its gist; both kinds
    of sequence end (ragged tail, full chunk without its gist) occur."""
    n, m = gi.varlen_lengths(64, n_min, n_max, chunk, 11)
    assert len(n) == len(m) == 64
    for a, b in zip(n, m):
        assert n_min <= a <= n_max
        assert b * chunk <= a <= b * chunk + chunk
    assert n == gi.varlen_lengths(64, n_min, n_max, chunk, 11)[0]      # seeded


def test_level_sizes_and_make_levels_shapes():
    assert gi.level_sizes(1010, 3, 4) == [1010, 336, 112, 37]
    q, k, v, ku, vu = gi.make_levels(2, 8, 2, 64, 16 * 100 + 5, 100, 16, 4, 3, 5, values="int")
    assert q.shape == (2, 8, 64) and k.shape == (2, 2, 1705, 64)
    assert [t.shape[2] for t in ku] == [25, 6] and [t.shape[2] for t in vu] == [25, 6]
    assert set(torch.unique(k.float()).tolist()) <= {-2.0, -1.0, 0.0, 1.0, 2.0}
    q2 = gi.make_levels(2, 8, 2, 64, 16 * 100 + 5, 100, 16, 4, 3, 5, values="int")[0]
    assert torch.equal(q, q2)                                           # seeded


def test_token_stream_and_gist_shapes():
    s = gi.make_token_stream(3, 8, 2, 64, 50, 8, 2)
    assert s.raw_k.shape == (50, 3, 2, 64) and s.gist_k.shape == (6, 3, 2, 64)
    assert s.gist_q.shape == (6, 3, 8, 64) and s.q.shape == (3, 8, 64)
    q, k, v = gi.make_gist(8, 2, 128, 16 * 10, 10, 10, 3)
    assert q.shape == (8, 10, 128) and k.shape == (2, 170, 128) and k.dtype == torch.bfloat16
