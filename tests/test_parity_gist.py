"""GPU parity of the cache-building step against the fp64 oracle.

  * gsa_gist_prefill: gist tokens under the gist causal mask (own chunk's raw
    tokens and the earlier gists), every (query, kv-head) against
    oracle.gist_query;
  * a gist token at decode time is gsa_decode with topk = 0 and tail = C on
    the cache before its gist row exists;
  * gsa_cache_append: every row of the grown cache bit for bit against the
    placement of oracle.cache_row, untouched rows unchanged;
  * row_capacity: every reader on a cache sized for more rows than it holds
    gives bit for bit the result it gives on the exactly sized cache (same
    kernels, only the stride between blocks differs);
  * a batch of sequences grown token by token (raw rows, a gist every C
    tokens, each gist's attention checked) ends in a decode step that matches
    the oracle on the densely built cache.
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


def with_capacity(x, extra, fill=3.0):
    """Copy of a cache [..., R, D] inside a larger [..., R + extra, D] buffer
    whose spare rows hold `fill`."""
    big = torch.full((*x.shape[:-2], x.shape[-2] + extra, x.shape[-1]), fill, dtype=x.dtype,
                     device=x.device)
    big[..., :x.shape[-2], :] = x
    return big


# ------------------------------------------------------------ gist prefill ---

GIST_CASES = [
    dict(Hq=8, Hkv=2, C=16, M=150, r=7, m_start=0, n_q=150),     # 3 blocks, ragged last block
    dict(Hq=2, Hkv=2, C=16, M=100, r=16, m_start=0, n_q=101),    # g = 1; chunk M complete, no gist yet
    dict(Hq=8, Hkv=2, C=4, M=300, r=0, m_start=37, n_q=200),     # C = 4, later start
    dict(Hq=4, Hkv=1, C=64, M=70, r=10, m_start=5, n_q=65),      # C = 64
    dict(Hq=4, Hkv=1, C=1, M=200, r=1, m_start=0, n_q=130),      # C = 1: one raw token per gist
    dict(Hq=8, Hkv=2, C=16, M=64, r=0, m_start=63, n_q=1),       # one query
    dict(Hq=16, Hkv=2, C=16, M=150, r=7, m_start=0, n_q=150),    # g = 8
]


def check_gist(gsa, c, seed, capacity=0):
    N = c["M"] * c["C"] + c["r"]
    q, k, v = gi.make_gist(c["Hq"], c["Hkv"], 128, N, c["M"], c["n_q"], seed, device="cuda")
    out = gsa.gsa_gist_prefill(q, k, v, chunk=c["C"], m_start=c["m_start"], n_gist=c["M"])
    torch.cuda.synchronize()
    g = c["Hq"] // c["Hkv"]
    qn, kn, vn, on = to_np(q), to_np(k), to_np(v), to_np(out)
    got, ref = [], []
    for i in range(c["n_q"]):
        for j in range(c["Hkv"]):
            r = oracle.gist_query(qn[j * g:(j + 1) * g, i], kn[j], vn[j], m=c["m_start"] + i, n_raw=N,
                                  n_gist=c["M"], chunk=c["C"])
            got.append(on[j * g:(j + 1) * g, i])
            ref.append(r["out"])
    err = check_out(np.stack(got), np.stack(ref), "bf16", f"gist {c}")
    if capacity:
        o2 = gsa.gsa_gist_prefill(q, with_capacity(k, capacity), with_capacity(v, capacity), chunk=c["C"],
                                  m_start=c["m_start"], n_gist=c["M"], n_raw=N)
        torch.cuda.synchronize()
        assert torch.equal(o2, out), "row_capacity changed the gist attention"
    return err


@pytest.mark.parametrize("c", GIST_CASES, ids=[f"case{i}" for i in range(len(GIST_CASES))])
def test_gist_prefill_matches_oracle(gsa, c):
    say(f"gist prefill {c}")
    err = check_gist(gsa, c, 4100 + GIST_CASES.index(c), capacity=37 if c is GIST_CASES[0] else 0)
    say(f"  max err / rms = {err:.2e}")


def test_gist_prefill_prompt_64k(gsa):
    """Every gist of a 64K-token prompt (4096 chunks of 16, Hq 32 / Hkv 8):
    sampled queries (first, block edges, last) against the oracle."""
    C, M, Hq, Hkv = 16, 4096, 32, 8
    N = M * C
    say("gist prefill 64k prompt")
    q, k, v = gi.make_gist(Hq, Hkv, 128, N, M, M, 4200, device="cuda")
    out = gsa.gsa_gist_prefill(q, k, v, chunk=C, m_start=0, n_gist=M)
    torch.cuda.synchronize()
    g = Hq // Hkv
    got, ref = [], []
    for i, j in [(0, 0), (1, 7), (63, 3), (64, 2), (2047, 5), (4032, 1), (4095, 6)]:
        kj, vj = to_np(k[j]), to_np(v[j])
        r = oracle.gist_query(to_np(q[j * g:(j + 1) * g, i]), kj, vj, m=i, n_raw=N, n_gist=M, chunk=C)
        got.append(to_np(out[j * g:(j + 1) * g, i]))
        ref.append(r["out"])
    err = check_out(np.stack(got), np.stack(ref), "bf16", "gist 64k")
    say(f"  max err / rms = {err:.2e}")


@pytest.mark.parametrize("B,Hq,Hkv,C,M", [(2, 8, 2, 16, 40), (32, 32, 8, 16, 100), (4, 32, 8, 8, 500)])
def test_gist_token_at_decode_is_decode_with_tail_c(gsa, B, Hq, Hkv, C, M):
    """Chunk M just completed (N = (M + 1) C), its gist not yet in the cache:
    the gist token's attention is gsa_decode with topk = 0 and tail = C."""
    N = (M + 1) * C
    say(f"gist at decode B={B} Hq={Hq} Hkv={Hkv} C={C} M={M}")
    q, k, v = gi.make_gist(B * Hq, B * Hkv, 128, N, M, 1, 4300 + M, device="cuda")
    q, k, v = q.view(B, Hq, 128), k.view(B, Hkv, N + M, 128), v.view(B, Hkv, N + M, 128)
    out, _, _ = gsa.gsa_decode(q, k, v, chunk=C, topk=0, tail=C, n_gist=M, want_sel=False)
    torch.cuda.synchronize()
    g = Hq // Hkv
    got, ref = [], []
    for b in range(B):
        for j in range(Hkv):
            r = oracle.gist_query(to_np(q[b, j * g:(j + 1) * g]), to_np(k[b, j]), to_np(v[b, j]), m=M,
                                  n_raw=N, n_gist=M, chunk=C)
            got.append(to_np(out[b, j * g:(j + 1) * g]))
            ref.append(r["out"])
    err = check_out(np.stack(got), np.stack(ref), "bf16", "gist at decode")
    say(f"  max err / rms = {err:.2e}")


# ------------------------------------------------------------ cache append ---

def dense_cache(raw, gist, C):
    """[lead..., N + M, D] cache with raw row p at oracle.cache_row(p) and gist
    m at oracle.cache_row(m, gist)."""
    N, M = raw.shape[-2], gist.shape[-2]
    out = np.full((*raw.shape[:-2], N + M, raw.shape[-1]), np.nan, dtype=raw.dtype)
    for p in range(N):
        out[..., oracle.cache_row(p, C, False), :] = raw[..., p, :]
    for m in range(M):
        out[..., oracle.cache_row(m, C, True), :] = gist[..., m, :]
    assert not np.isnan(out).any()
    return out


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("bf16", 64), ("f32", 128)])
def test_cache_append_places_every_row(gsa, dtype, D):
    """A prompt's raw rows, then its gists, then token-by-token appends (with a
    gist row as each chunk completes, sometimes in the same call): the grown
    cache equals the dense interleaved layout bit for bit and the spare rows
    keep their fill."""
    B, Hkv, C, cap = 2, 3, 8, 160
    say(f"cache append {dtype} D={D}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    s = gi.make_token_stream(B, Hkv, Hkv, D, 120, C, 4400 + D, device="cuda", dtype=dtype)
    rk, rv = s.raw_k.permute(1, 2, 0, 3).contiguous(), s.raw_v.permute(1, 2, 0, 3).contiguous()
    gk, gv = s.gist_k.permute(1, 2, 0, 3).contiguous(), s.gist_v.permute(1, 2, 0, 3).contiguous()
    kc = torch.full((B, Hkv, cap, D), 5.0, dtype=tdt, device="cuda")
    vc = torch.full((B, Hkv, cap, D), -5.0, dtype=tdt, device="cuda")
    N, M = 0, 0

    def rows(x, a, b):
        return x[:, :, a:b].contiguous()
    gsa.gsa_cache_append(kc, vc, chunk=C, n_raw=N, n_gist=M, k_raw=rows(rk, 0, 50), v_raw=rows(rv, 0, 50))
    N = 50
    gsa.gsa_cache_append(kc, vc, chunk=C, n_raw=N, n_gist=M, k_gist=rows(gk, 0, 6), v_gist=rows(gv, 0, 6))
    M = 6
    while N < 120:
        if N % C == C - 1 and N // C % 2 == 0:      # completes a chunk: raw and gist in one call
            gsa.gsa_cache_append(kc, vc, chunk=C, n_raw=N, n_gist=M, k_raw=rows(rk, N, N + 1),
                                 v_raw=rows(rv, N, N + 1), k_gist=rows(gk, M, M + 1), v_gist=rows(gv, M, M + 1))
            N, M = N + 1, M + 1
            continue
        gsa.gsa_cache_append(kc, vc, chunk=C, n_raw=N, n_gist=M, k_raw=rows(rk, N, N + 1),
                             v_raw=rows(rv, N, N + 1))
        N += 1
        if N % C == 0:
            gsa.gsa_cache_append(kc, vc, chunk=C, n_raw=N, n_gist=M, k_gist=rows(gk, M, M + 1),
                                 v_gist=rows(gv, M, M + 1))
            M += 1
    torch.cuda.synchronize()
    assert (N, M) == (120, 15)
    for cache, raw, gist, fill in ((kc, rk, gk, 5.0), (vc, rv, gv, -5.0)):
        want = dense_cache(to_np(raw), to_np(gist), C)
        got = to_np(cache)
        np.testing.assert_array_equal(got[:, :, :N + M], want)
        assert (got[:, :, N + M:] == fill).all()


def test_cache_append_rejects_a_gist_before_its_chunk(gsa):
    """A gist row for a chunk with 7 of its 8 raw tokens is refused on the
    host, the cache untouched."""
    kc = torch.zeros(1, 1, 64, 128, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    rows = torch.ones(1, 1, 7, 128, dtype=torch.bfloat16, device="cuda")
    gist = torch.ones(1, 1, 1, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gsa.GsaError):
        gsa.gsa_cache_append(kc, vc, chunk=8, n_raw=0, n_gist=0, k_raw=rows, v_raw=rows, k_gist=gist,
                             v_gist=gist)
    torch.cuda.synchronize()
    assert not kc.any() and not vc.any()


# ------------------------------------------------------------ row_capacity ---

def test_decode_on_capacity_cache_is_bit_identical(gsa):
    """Decode (one-workgroup-per-unit launch and the split launch), two-level
    decode and prefill on caches with spare rows: bit-identical results."""
    extra = 41
    for name, kw in (("unit", dict(n_raw=4096)), ("split", dict(batch=2, n_raw=4096 + 9, n_gist=256))):
        cfg = dataclasses.replace(gi.CONFIGS["gqa_32k"], **kw)
        say(f"capacity decode {name}")
        inp = gi.make_decode(cfg, 4500, device="cuda")
        a = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=cfg.chunk, topk=cfg.topk, tail=cfg.tail,
                           n_gist=cfg.M)
        b = gsa.gsa_decode(inp.q, with_capacity(inp.k_cache, extra), with_capacity(inp.v_cache, extra),
                           chunk=cfg.chunk, topk=cfg.topk, tail=cfg.tail, n_gist=cfg.M, n_raw=cfg.n_raw)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y), name
    say("capacity decode hier")
    hcfg = gi.HierConfig(dataclasses.replace(gi.CONFIGS["hier_1m"].base, batch=2, n_raw=16 * 16 * 40), 16, 6)
    h = gi.make_hier(hcfg, 4600, device="cuda")
    a = gsa.gsa_decode_hier(h.q, h.k_cache, h.v_cache, h.k_l2, h.v_l2, chunk=16, fanout=16, topk1=16,
                            topk2=6, tail=64, n_gist=hcfg.base.M)
    b = gsa.gsa_decode_hier(h.q, with_capacity(h.k_cache, extra), with_capacity(h.v_cache, extra), h.k_l2,
                            h.v_l2, chunk=16, fanout=16, topk1=16, topk2=6, tail=64, n_gist=hcfg.base.M,
                            n_raw=hcfg.base.n_raw)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y), "hier"
    say("capacity prefill")
    pcfg = dataclasses.replace(gi.CONFIGS["prefill_64k"], n_raw=4096, n_q=200, n_kv_heads=2, n_q_heads=8,
                               topk=8)
    p = gi.make_prefill(pcfg, 4700, device="cuda")
    a = gsa.gsa_prefill_blocksparse(p.q, p.k_cache, p.v_cache, chunk=16, topk=8, window=64,
                                    q_start=pcfg.q_start, n_gist=pcfg.M)
    b = gsa.gsa_prefill_blocksparse(p.q, with_capacity(p.k_cache, extra), with_capacity(p.v_cache, extra),
                                    chunk=16, topk=8, window=64, q_start=pcfg.q_start, n_gist=pcfg.M,
                                    n_raw=pcfg.n_raw)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y), "prefill"


# ------------------------------------------------- a cache grown in place ---

@pytest.mark.parametrize("B,Hq,Hkv,C,steps,topk", [(2, 8, 2, 8, 100, 4), (32, 32, 8, 16, 300, 8)])
def test_decode_loop_grows_the_cache_in_place(gsa, B, Hq, Hkv, C, steps, topk):
    """Token by token: append the raw row; when a chunk completes, run its gist
    token (gsa_decode, topk = 0, tail = C) and check it against the oracle,
    then append the gist row. The last step decodes with top-k on the grown
    cache and matches the oracle on the densely built one."""
    say(f"decode loop B={B} Hq={Hq} Hkv={Hkv} C={C} steps={steps} k={topk}")
    D, g = 128, Hq // Hkv
    cap = steps + steps // C + 16
    s = gi.make_token_stream(B, Hq, Hkv, D, steps, C, 4800 + B, device="cuda")
    kc = torch.zeros(B, Hkv, cap, D, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    N, M = 0, 0
    gist_got, gist_ref = [], []
    for p in range(steps):
        gsa.gsa_cache_append(kc, vc, chunk=C, n_raw=N, n_gist=M, k_raw=s.raw_k[p].unsqueeze(2).contiguous(),
                             v_raw=s.raw_v[p].unsqueeze(2).contiguous())
        N += 1
        if N % C == 0:
            o, _, _ = gsa.gsa_decode(s.gist_q[M], kc, vc, chunk=C, topk=0, tail=C, n_gist=M, n_raw=N,
                                     want_sel=False)
            if M % 5 == 0 or M == steps // C - 1:
                torch.cuda.synchronize()
                kn, vn = to_np(kc[:, :, :N + M]), to_np(vc[:, :, :N + M])
                for b, j in ((0, 0), (B - 1, Hkv - 1)):
                    r = oracle.gist_query(to_np(s.gist_q[M, b, j * g:(j + 1) * g]), kn[b, j], vn[b, j], m=M,
                                          n_raw=N, n_gist=M, chunk=C)
                    gist_got.append(to_np(o[b, j * g:(j + 1) * g]))
                    gist_ref.append(r["out"])
            gsa.gsa_cache_append(kc, vc, chunk=C, n_raw=N, n_gist=M, k_gist=s.gist_k[M].unsqueeze(2).contiguous(),
                                 v_gist=s.gist_v[M].unsqueeze(2).contiguous())
            M += 1
    torch.cuda.synchronize()
    check_out(np.stack(gist_got), np.stack(gist_ref), "bf16", "gist tokens in the loop")
    raw = to_np(s.raw_k.permute(1, 2, 0, 3))
    want_k = dense_cache(raw, to_np(s.gist_k.permute(1, 2, 0, 3)), C)
    want_v = dense_cache(to_np(s.raw_v.permute(1, 2, 0, 3)), to_np(s.gist_v.permute(1, 2, 0, 3)), C)
    np.testing.assert_array_equal(to_np(kc[:, :, :N + M]), want_k)
    np.testing.assert_array_equal(to_np(vc[:, :, :N + M]), want_v)
    tail = max(C, N - M * C)
    out, lse, sel = gsa.gsa_decode(s.q, kc, vc, chunk=C, topk=topk, tail=tail, n_gist=M, n_raw=N)
    torch.cuda.synchronize()
    ref = oracle.decode(to_np(s.q), want_k, want_v, chunk=C, topk=topk, tail=tail, n_gist=M)
    np.testing.assert_array_equal(to_np(sel), ref[2])
    err = check_out(to_np(out), ref[0], "bf16", "decode on the grown cache")
    say(f"  max err / rms = {err:.2e}")
