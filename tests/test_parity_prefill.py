"""GPU parity of gsa_prefill_blocksparse against the fp64 oracle.

Selections must match bit for bit; outputs within the stated tolerance
(tests/gpu_util.py). Small cases compare every (query, kv-head); the
full-size workload runs in the launch configuration the benchmark times,
checks every selection against the planted chunks and compares sampled
queries with the oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gsa_inputs as gi
import oracle
from conftest import to_np
from gpu_util import check_out, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_gsa_amd
    decode_gsa_amd.lib()          # raises if the library is missing: no fallback
    return decode_gsa_amd


def run_prefill(gsa, inp, cfg, queries=None):
    out, sel = gsa.gsa_prefill_blocksparse(inp.q, inp.k_cache, inp.v_cache, chunk=cfg.chunk,
                                           topk=cfg.topk, window=cfg.window, q_start=cfg.q_start,
                                           n_gist=cfg.M)
    torch.cuda.synchronize()
    g = cfg.n_q_heads // cfg.n_kv_heads
    todo = ([(i, j) for j in range(cfg.n_kv_heads) for i in range(cfg.n_q)] if queries is None
            else queries)
    K = [to_np(inp.k_cache[j]) for j in range(cfg.n_kv_heads)]
    V = [to_np(inp.v_cache[j]) for j in range(cfg.n_kv_heads)]
    qn = to_np(inp.q)
    on = to_np(out)
    sn = to_np(sel) if cfg.topk > 0 else None
    got, ref = [], []
    for i, j in todo:
        r = oracle.prefill_query(qn[j * g:(j + 1) * g, i], K[j], V[j], t=cfg.q_start + i,
                                 n_raw=cfg.n_raw, n_gist=cfg.M, chunk=cfg.chunk, topk=cfg.topk,
                                 window=cfg.window)
        if cfg.topk > 0:
            np.testing.assert_array_equal(sn[j, i], r["sel"], err_msg=f"query {i} kv-head {j}")
        got.append(on[j * g:(j + 1) * g, i])
        ref.append(r["out"])
    return check_out(np.stack(got), np.stack(ref), cfg.dtype, cfg.name), out, sel


def small(**kw):
    return dataclasses.replace(gi.CONFIGS["prefill_64k"], **kw)


CASES = [
    # planted selections, several query blocks and a ragged last block
    dict(n_raw=4096, n_q=200, n_kv_heads=2, n_q_heads=8, topk=8),
    dict(n_raw=4096, n_q=130, n_kv_heads=2, n_q_heads=2, topk=8),            # g = 1
    dict(n_raw=4096, n_q=64, n_kv_heads=1, n_q_heads=2, topk=16),            # g = 2
    dict(n_raw=4096, n_q=200, n_kv_heads=2, n_q_heads=16, topk=8),           # g = 8
    dict(n_raw=4096, n_q=96, n_kv_heads=2, n_q_heads=8, topk=0),             # gists + window only
    dict(n_raw=3000, n_gist=187, n_q=70, n_kv_heads=1, n_q_heads=4, topk=8, chunk=16),  # partial chunk
    dict(n_raw=4096, n_q=128, n_kv_heads=1, n_q_heads=4, topk=32, chunk=8, window=40),  # k = 32, C = 8
    dict(n_raw=4096, n_q=64, n_kv_heads=1, n_q_heads=4, topk=16, chunk=32, window=100),
    # small integers: exact scores, ties decided by index; every position is a
    # query (t < C has no gist, |eligible| < k pads with -1, windows and
    # selected chunks overlap)
    dict(n_raw=520, n_q=520, n_kv_heads=2, n_q_heads=8, topk=8, chunk=16, window=20, values="int"),
    dict(n_raw=300, n_gist=37, n_q=300, n_kv_heads=1, n_q_heads=4, topk=5, chunk=8, window=3,
         values="int"),
    dict(n_raw=256, n_q=256, n_kv_heads=1, n_q_heads=2, topk=32, chunk=4, window=1, values="int"),
    dict(n_raw=520, n_q=520, n_kv_heads=1, n_q_heads=8, topk=8, chunk=16, window=20, values="int"),  # g = 8
    # k above 32: candidate lists of 32 entries, a union of up to 64 k chunks
    dict(n_raw=4096, n_q=160, n_kv_heads=2, n_q_heads=8, topk=48, chunk=8, window=40),
    dict(n_raw=600, n_q=600, n_kv_heads=1, n_q_heads=4, topk=64, chunk=4, window=10, values="int"),
]


@pytest.mark.parametrize("kw", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_prefill_small(gsa, kw):
    cfg = small(**kw)
    say(f"prefill small {cfg}")
    inp = gi.make_prefill(cfg, 300 + len(kw), device="cuda")
    err, _, sel = run_prefill(gsa, inp, cfg)
    if inp.planted is not None and cfg.topk > 0:
        blk = torch.arange(cfg.n_q, device=sel.device) // cfg.q_block
        assert torch.equal(sel.permute(1, 0, 2).long(), inp.planted[blk])
    say(f"  max err / rms = {err:.2e}")


def test_prefill_repeatable(gsa):
    cfg = small(n_raw=4096, n_q=128, n_kv_heads=2, n_q_heads=8, topk=8)
    say(f"prefill repeatable {cfg}")
    inp = gi.make_prefill(cfg, 7, device="cuda")
    args = dict(chunk=cfg.chunk, topk=cfg.topk, window=cfg.window, q_start=cfg.q_start, n_gist=cfg.M)
    o1, s1 = gsa.gsa_prefill_blocksparse(inp.q, inp.k_cache, inp.v_cache, **args)
    o2, s2 = gsa.gsa_prefill_blocksparse(inp.q, inp.k_cache, inp.v_cache, **args)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert torch.equal(o1, o2)


def test_prefill_full_size_sampled(gsa):
    """The 64K-token, 4096-query workload in the benchmark's launch shape:
    every selection equals the planted set; sampled outputs match the oracle."""
    cfg = gi.CONFIGS["prefill_64k"]
    say(f"prefill full {cfg}")
    inp = gi.make_prefill(cfg, 2000 + 5, device="cuda")
    rng = np.random.default_rng(11)
    qs = [(int(i), int(j)) for i, j in zip(rng.integers(0, cfg.n_q, 48),
                                           rng.integers(0, cfg.n_kv_heads, 48))]
    qs += [(0, 0), (cfg.n_q - 1, cfg.n_kv_heads - 1), (63, 3), (64, 4)]
    err, _, sel = run_prefill(gsa, inp, cfg, queries=qs)
    blk = torch.arange(cfg.n_q, device=sel.device) // cfg.q_block
    assert torch.equal(sel.permute(1, 0, 2).long(), inp.planted[blk])
    say(f"  max err / rms = {err:.2e}")


def test_prefill_beyond_65536_gists(gsa):
    """70000 gists (a 1.12M-token context): chunk ids above 2^16 in the
    selection, its index tie rule and the attention's chunk union. Integer
    values make scores exact, so ties at the k-th place are decided by id."""
    cfg = small(n_raw=16 * 70000, n_q=128, n_kv_heads=1, n_q_heads=4, topk=16, chunk=16, window=64,
                values="int")
    say(f"prefill beyond 65536 gists {cfg}")
    inp = gi.make_prefill(cfg, 6100, device="cuda")
    qs = [(i, 0) for i in range(0, cfg.n_q, 5)] + [(cfg.n_q - 1, 0)]
    err, _, sel = run_prefill(gsa, inp, cfg, queries=qs)
    assert int(sel.max()) >= 65536          # ids past 16 bits were chosen
    say(f"  max err / rms = {err:.2e}")


@pytest.mark.parametrize("topk", [16, 32, 64])
def test_prefill_all_scores_tied(gsa, topk):
    """q = 0: every group score is 0, so a query keeps the topk smallest
    eligible gist indices. More tied candidates than the candidate lists can
    hold after a bisection prune, so the exact radix selection (ties by
    index) decides."""
    cfg = small(n_raw=4096, n_q=192, n_kv_heads=2, n_q_heads=8, topk=topk, chunk=8, window=24)
    say(f"prefill all scores tied {cfg}")
    inp = gi.make_prefill(cfg, 4100 + topk, device="cuda")
    inp.q.zero_()
    err, _, sel = run_prefill(gsa, inp, cfg, queries=[(i, j) for i in range(0, cfg.n_q, 7) for j in (0, 1)])
    t = cfg.q_start + np.arange(cfg.n_q)
    elig = np.minimum(t // cfg.chunk, cfg.M)
    want = np.where(np.arange(topk)[None, :] < elig[:, None], np.arange(topk)[None, :], -1)
    np.testing.assert_array_equal(to_np(sel), np.broadcast_to(want, (cfg.n_kv_heads,) + want.shape))
    say(f"  max err / rms = {err:.2e}")
