"""GPU parity of gsa_prefill_varlen (causal block-sparse prefill of several
sequences of different lengths in one call) against the fp64 oracle's
prefill_query, sequence by sequence on its own rows.

Cache rows past a sequence's own N_b + M_b hold a constant the attention
would notice, so a read beyond them shows; output rows past a sequence's
queries start as NaN and must stay so. Integer-valued cases ({-2..2}) keep
every group score exact (selections decided by the scores and the index tie
rule alone).
"""
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


def make_case(c, seed):
    """Per sequence (n_raw, n_gist, q_start, n_q); caches [B, Hkv, R, D] and
    queries [B, Hq, n_q_max, D]."""
    B, Hq, Hkv, C = c["B"], c["Hq"], c["Hkv"], c["C"]
    rng = np.random.default_rng(seed)
    n, m = gi.varlen_lengths(B, c["n_min"], c["n_max"], C, seed)
    rows = []
    for b in range(B):
        nq = int(rng.integers(1, min(n[b], c["nq_max"]) + 1)) if b % 3 else min(n[b], c["nq_max"])
        qs = int(rng.integers(0, n[b] - nq + 1)) if b % 2 else n[b] - nq
        rows.append([n[b], m[b], qs, nq])
    nq_max = max(r[3] for r in rows)
    N, M = max(n), max(m)
    R = N + M + 3
    g = torch.Generator(device="cuda").manual_seed(seed)
    if c.get("values", "int") == "int":
        draw = lambda *s: torch.randint(-2, 3, s, generator=g, device="cuda").to(torch.bfloat16)
    else:
        draw = lambda *s: torch.randn(*s, generator=g, device="cuda").to(torch.bfloat16)
    q = draw(B, Hq, nq_max, 128)
    k = draw(B, Hkv, R, 128)
    v = draw(B, Hkv, R, 128)
    for b, (nb, mb, _, _) in enumerate(rows):
        k[b, :, nb + mb:] = 3.0
        v[b, :, nb + mb:] = 3.0
    return q, k, v, rows


def check(c, q, k, v, rows, out, sel, per_seq=None):
    g = c["Hq"] // c["Hkv"]
    rng = np.random.default_rng(1)
    qn, on = to_np(q), to_np(out)
    sn = to_np(sel) if c["k"] > 0 else None
    got, ref = [], []
    for b, (nb, mb, qs, nq) in enumerate(rows):
        assert np.isnan(on[b, :, nq:]).all(), f"sequence {b}: rows past its queries were written"
        K = [to_np(k[b, j, :nb + mb]) for j in range(c["Hkv"])]
        V = [to_np(v[b, j, :nb + mb]) for j in range(c["Hkv"])]
        pick = range(nq) if per_seq is None or nq <= per_seq else sorted(
            set(rng.choice(nq, per_seq, replace=False).tolist()) | {0, nq - 1})
        for i in pick:
            for j in range(c["Hkv"]):
                r = oracle.prefill_query(qn[b, j * g:(j + 1) * g, i], K[j], V[j], t=qs + i, n_raw=nb, n_gist=mb,
                                         chunk=c["C"], topk=c["k"], window=c["W"])
                if c["k"] > 0:
                    np.testing.assert_array_equal(sn[b, j, i], r["sel"], err_msg=f"sequence {b} query {i} kv {j}")
                got.append(on[b, j * g:(j + 1) * g, i])
                ref.append(r["out"])
    return check_out(np.stack(got), np.stack(ref), "bf16", str(c))


CASES = [
    dict(B=3, Hq=8, Hkv=2, C=16, k=8, W=64, n_min=600, n_max=4096, nq_max=700),
    dict(B=4, Hq=16, Hkv=2, C=8, k=16, W=20, n_min=300, n_max=3000, nq_max=400, values="gauss"),   # g = 8
    dict(B=2, Hq=4, Hkv=1, C=4, k=48, W=10, n_min=500, n_max=1200, nq_max=300),                    # k = 48
    dict(B=5, Hq=4, Hkv=2, C=16, k=0, W=32, n_min=100, n_max=2000, nq_max=200),                    # k = 0
]


@pytest.mark.parametrize("i", range(len(CASES)), ids=[f"case{i}" for i in range(len(CASES))])
def test_prefill_varlen_matches_oracle_per_sequence(gsa, i):
    c = CASES[i]
    say(f"prefill varlen {c}")
    q, k, v, rows = make_case(c, 8100 + i)
    out = torch.full((c["B"], c["Hq"], q.shape[2], 128), float("nan"), device="cuda")
    out, sel = gsa.gsa_prefill_varlen(q, k, v, seqs=rows, chunk=c["C"], topk=c["k"], window=c["W"], out=out)
    torch.cuda.synchronize()
    err = check(c, q, k, v, rows, out, sel, per_seq=40)
    say(f"  rows {rows}: max err / rms = {err:.2e}")


def test_prefill_varlen_one_sequence_is_blocksparse(gsa):
    """A batch of one: bit-identical to gsa_prefill_blocksparse on the same
    sequence."""
    c = CASES[0]
    q, k, v, rows = make_case(c, 8200)
    nb, mb, qs, nq = rows[0]
    say("prefill varlen = one sequence")
    q1 = q[0:1, :, :nq].contiguous()
    a_out, a_sel = gsa.gsa_prefill_varlen(q1, k[0:1], v[0:1], seqs=[rows[0]], chunk=c["C"], topk=c["k"],
                                          window=c["W"])
    b_out, b_sel = gsa.gsa_prefill_blocksparse(q1[0], k[0], v[0], chunk=c["C"], topk=c["k"], window=c["W"],
                                               q_start=qs, n_gist=mb, n_raw=nb)
    torch.cuda.synchronize()
    assert torch.equal(a_out[0], b_out) and torch.equal(a_sel[0], b_sel)


def test_prefill_varlen_device_seqs_and_rule_breaker(gsa):
    """seqs as a device array is used as given; a sequence whose row breaks
    the rules (queries past its raw tokens) gets no work: its output rows stay
    as they were."""
    c = CASES[0]
    q, k, v, rows = make_case(c, 8300)
    N, M = max(r[0] for r in rows), max(r[1] for r in rows)
    bad = 1
    rows2 = [list(r) for r in rows]
    rows2[bad][2] = rows2[bad][0] - rows2[bad][3] + 1          # q_start + n_q = n + 1
    sd = torch.tensor(rows2, dtype=torch.int32, device="cuda")
    out = torch.full((c["B"], c["Hq"], q.shape[2], 128), float("nan"), device="cuda")
    say("prefill varlen device seqs")
    out, sel = gsa.gsa_prefill_varlen(q, k, v, seqs=sd, n_raw=N, n_gist=M, chunk=c["C"], topk=c["k"],
                                      window=c["W"], out=out)
    torch.cuda.synchronize()
    assert torch.isnan(out[bad]).all()
    keep = [b for b in range(c["B"]) if b != bad]
    sub = dict(c, B=len(keep))
    check(sub, q[keep], k[keep], v[keep], [rows[b] for b in keep], out[keep], sel[keep], per_seq=20)
