"""GPU parity of gsa_decode_paged (caches in shuffled pages of a shared pool,
per-sequence lengths, rows attended directly) against the fp64 oracle's
decode_paged_unit, and bit for bit against gsa_decode_varlen on the dense
layout the pages spell out.

Integer-valued entries ({-2..2}) keep every group score exact, so the
selections are decided by the scores and the index tie rule alone.
"""
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


def dense_case(B, Hq, Hkv, C, n_min, n_max, seed, values="int"):
    n, m = gi.varlen_lengths(B, n_min, n_max, C, seed)
    N, M = max(n), max(m)
    cap = N + M + 5
    q, k, v, _, _ = gi.make_levels(B, Hq, Hkv, 128, cap - (cap // (C + 1)), cap // (C + 1), C, 2, 2, seed,
                                   device="cuda", values=values)
    return q, k[:, :, :cap].contiguous(), v[:, :, :cap].contiguous(), n, m


CASES = [  # B, Hq, Hkv, C, n_min, n_max, k, T, P
    (32, 32, 8, 16, 1000, 4000, 16, 64, 16),     # 256 units: one workgroup each
    (32, 32, 8, 16, 1000, 4000, 16, 64, 1),      # pages of one chunk
    (2, 8, 2, 16, 20000, 40000, 16, 64, 4),      # several workgroups per unit, candidates
    (2, 8, 2, 8, 20000, 40000, 40, 64, 8),       # k > 16: every score handed on
    (2, 8, 2, 16, 3000, 9000, 0, 40, 2),         # k = 0
    (3, 12, 3, 32, 5000, 12000, 8, 33, 64),      # g = 4, C = 32, 64-chunk pages
]


@pytest.mark.parametrize("case", range(len(CASES)), ids=[f"paged{i}" for i in range(len(CASES))])
def test_paged_equals_varlen_and_oracle(gsa, case):
    B, Hq, Hkv, C, n_min, n_max, k, T, P = CASES[case]
    say(f"paged {CASES[case]}")
    q, kc, vc, n, m = dense_case(B, Hq, Hkv, C, n_min, n_max, 7000 + case)
    rows = [a + b for a, b in zip(n, m)]
    kp, vp, table = gi.to_pages(kc, vc, rows, P, C, 7100 + case)
    out, lse, sel = gsa.gsa_decode_paged(q, kp, vp, block_table=table, seq_n_raw=n, seq_n_gist=m, chunk=C,
                                         topk=k, tail=T, page_chunks=P)
    ro, rl, rs = gsa.gsa_decode_varlen(q, kc, vc, seq_n_raw=n, seq_n_gist=m, chunk=C, topk=k, tail=T)
    torch.cuda.synchronize()
    # same rows in the same order through the same kernels: identical results
    assert torch.equal(out, ro) and torch.equal(lse, rl)
    if k > 0:
        assert torch.equal(sel, rs)
    g = Hq // Hkv
    units = [(b, j) for b in range(B) for j in range(Hkv)]
    pick = units if len(units) <= 8 else [units[i] for i in np.random.default_rng(case).choice(len(units), 8, False)]
    got, ref = [], []
    for b, j in pick:
        r = oracle.decode_paged_unit(to_np(q[b, j * g:(j + 1) * g]), to_np(kp[:, j]), to_np(vp[:, j]),
                                     [int(x) for x in table[b]], page_chunks=P, n_raw=n[b], n_gist=m[b],
                                     chunk=C, topk=k, tail=T)
        if k > 0:
            np.testing.assert_array_equal(to_np(sel[b, j]), r["sel"], err_msg=f"unit {(b, j)}")
        got.append(to_np(out[b, j * g:(j + 1) * g]))
        ref.append(r["out"])
        check_lse(to_np(lse[b, j * g:(j + 1) * g]), r["lse"], "bf16", f"unit {(b, j)}")
    err = check_out(np.stack(got), np.stack(ref), "bf16", "paged")
    say(f"  max err / rms = {err:.2e}, {gsa.gsa_profile_marks() - 1} launches")


@pytest.mark.parametrize("many", [False, True], ids=["one-wg", "split"])
def test_paged_extra_rows(gsa, many):
    """Rows listed as extra (some in spare pages, some in the sequence's own
    pages) join the attention set of their sequence's query heads."""
    B, Hq, Hkv, C, P, k, T = (2, 8, 2, 16, 4, 16, 64) if many else (32, 32, 8, 16, 4, 16, 64)
    n_min, n_max = (20000, 40000) if many else (1000, 3000)
    q, kc, vc, n, m = dense_case(B, Hq, Hkv, C, n_min, n_max, 7200 + many)
    rows = [a + b for a, b in zip(n, m)]
    kp, vp, table = gi.to_pages(kc, vc, rows, P, C, 7300, spare=6)
    n_pages, rpp = kp.shape[0], kp.shape[2]
    rng = np.random.default_rng(7400)
    max_extra = 12
    extra = np.full((B, max_extra, 2), -1, dtype=np.int32)
    counts = rng.integers(0, max_extra + 1, size=B)
    for b in range(B):
        for e in range(counts[b]):
            extra[b, e] = (rng.integers(n_pages), rng.integers(rpp))
    out, lse, sel = gsa.gsa_decode_paged(q, kp, vp, block_table=table, seq_n_raw=n, seq_n_gist=m, chunk=C,
                                         topk=k, tail=T, page_chunks=P, extra_rows=extra)
    torch.cuda.synchronize()
    g = Hq // Hkv
    units = [(b, j) for b in range(B) for j in range(Hkv)]
    pick = units if len(units) <= 8 else [units[i] for i in rng.choice(len(units), 10, False)]
    got, ref = [], []
    for b, j in pick:
        xs = [(int(p_), int(r_)) for p_, r_ in extra[b] if p_ >= 0][:counts[b]]
        r = oracle.decode_paged_unit(to_np(q[b, j * g:(j + 1) * g]), to_np(kp[:, j]), to_np(vp[:, j]),
                                     [int(x) for x in table[b]], page_chunks=P, n_raw=n[b], n_gist=m[b],
                                     chunk=C, topk=k, tail=T, extra_rows=xs)
        np.testing.assert_array_equal(to_np(sel[b, j]), r["sel"], err_msg=f"unit {(b, j)}")
        got.append(to_np(out[b, j * g:(j + 1) * g]))
        ref.append(r["out"])
        check_lse(to_np(lse[b, j * g:(j + 1) * g]), r["lse"], "bf16", f"unit {(b, j)}")
    err = check_out(np.stack(got), np.stack(ref), "bf16", "paged extra rows")
    say(f"  max err / rms = {err:.2e}")


def test_reused_documents_ending_mid_chunk(gsa):
    """Three document caches built apart (pages of one chunk), the first two
    ending mid-chunk, reused by two sequences in different orders; each
    sequence routes among every document's gists, and a gist of one document
    planted along a sequence's mean query is chosen. Checked against the
    oracle unit by unit."""
    C, D, Hq, Hkv = 16, 128, 8, 2
    g = Hq // Hkv
    lens = [7 * C + 5, 5 * C + 9, 9 * C + 3]
    gen = torch.Generator(device="cpu").manual_seed(7500)
    docs = []
    for L in lens:
        M = L // C
        R = L + M
        kd = torch.randint(-2, 3, (Hkv, R, D), generator=gen).to(torch.bfloat16)
        vd = torch.randint(-2, 3, (Hkv, R, D), generator=gen).to(torch.bfloat16)
        docs.append((L, M, kd, vd))
    n_pages = sum(M + 1 for L, M, _, _ in docs) + 4
    rng = np.random.default_rng(7501)
    slots = rng.permutation(n_pages)
    kp = torch.randint(-2, 3, (n_pages, Hkv, C + 1, D), generator=gen).to(torch.bfloat16)
    vp = torch.randint(-2, 3, (n_pages, Hkv, C + 1, D), generator=gen).to(torch.bfloat16)
    pages_of, nxt = [], 0
    for L, M, kd, vd in docs:
        ps = []
        for i in range(M + 1):                  # M full chunk pages, one page with the last raw rows
            pg = int(slots[nxt]); nxt += 1
            r0, r1 = i * (C + 1), min(L + M, (i + 1) * (C + 1))
            if r1 > r0:
                kp[pg, :, :r1 - r0] = kd[:, r0:r1]
                vp[pg, :, :r1 - r0] = vd[:, r0:r1]
            ps.append(pg)
        pages_of.append(ps)
    orders = [[0, 1, 2], [1, 2, 0]]
    B = len(orders)
    max_pages = sum(M for _, M, _, _ in docs) + 1
    table = np.full((B, max_pages), -1, dtype=np.int32)
    extra = np.full((B, 16, 2), -1, dtype=np.int32)
    n, m = [], []
    for b, order in enumerate(orders):
        tbl, ex = [], []
        for d in order[:-1]:                     # reused documents: their chunks, their last tokens as extras
            L, M, _, _ = docs[d]
            tbl += pages_of[d][:M]
            ex += [(pages_of[d][M], r) for r in range(L - M * C)]
        L, M, _, _ = docs[order[-1]]             # the sequence's own document, with its trailing rows
        tbl += pages_of[order[-1]][:M + 1]
        table[b, :len(tbl)] = tbl
        extra[b, :len(ex)] = ex
        n.append(sum(docs[d][1] for d in order[:-1]) * C + L)
        m.append(sum(docs[d][1] for d in order))
    q = torch.randint(-2, 3, (B, Hq, D), generator=gen).to(torch.bfloat16)
    # plant: sequence b routes to chunk 2 of its first document
    for b, order in enumerate(orders):
        d = order[0]
        for j in range(Hkv):
            kp[pages_of[d][2], j, C] = (q[b, j * g:(j + 1) * g].float().sum(0).sign() * 2).to(torch.bfloat16)
    q, kp, vp = q.cuda(), kp.cuda(), vp.cuda()
    T = 16
    out, lse, sel = gsa.gsa_decode_paged(q, kp, vp, block_table=table, seq_n_raw=n, seq_n_gist=m, chunk=C,
                                         topk=1, tail=T, page_chunks=1, extra_rows=extra)
    torch.cuda.synchronize()
    got, ref = [], []
    for b in range(B):
        xs = [(int(p_), int(r_)) for p_, r_ in extra[b] if p_ >= 0]
        for j in range(Hkv):
            r = oracle.decode_paged_unit(to_np(q[b, j * g:(j + 1) * g]), to_np(kp[:, j]), to_np(vp[:, j]),
                                         [int(x) for x in table[b]], page_chunks=1, n_raw=n[b], n_gist=m[b],
                                         chunk=C, topk=1, tail=T, extra_rows=xs)
            assert r["sel"].tolist() == [2], r["sel"]
            np.testing.assert_array_equal(to_np(sel[b, j]), r["sel"])
            got.append(to_np(out[b, j * g:(j + 1) * g]))
            ref.append(r["out"])
            check_lse(to_np(lse[b, j * g:(j + 1) * g]), r["lse"], "bf16", f"seq {b}")
    check_out(np.stack(got), np.stack(ref), "bf16", "reused documents")


@pytest.mark.parametrize("gist_set", ["selected", "none"])
@pytest.mark.parametrize("many", [False, True], ids=["one-wg", "split"])
def test_paged_selection_rules(gsa, many, gist_set):
    """The slide 17 rules over paged caches with extra rows: the gists' K rows
    are scored through the block table, then the set (chosen raw rows, their
    gists under rule 1, the tail and the extra rows) is attended; against the
    oracle with the same rule, unit by unit."""
    B, Hq, Hkv, C, P, k, T = (2, 8, 2, 16, 4, 16, 64) if many else (32, 32, 8, 16, 4, 16, 64)
    n_min, n_max = (20000, 40000) if many else (1000, 3000)
    q, kc, vc, n, m = dense_case(B, Hq, Hkv, C, n_min, n_max, 7600 + many)
    rows = [a + b for a, b in zip(n, m)]
    kp, vp, table = gi.to_pages(kc, vc, rows, P, C, 7700, spare=6)
    n_pages, rpp = kp.shape[0], kp.shape[2]
    rng = np.random.default_rng(7800 + many)
    max_extra = 8
    extra = np.full((B, max_extra, 2), -1, dtype=np.int32)
    counts = rng.integers(0, max_extra + 1, size=B)
    for b in range(B):
        for e in range(counts[b]):
            extra[b, e] = (rng.integers(n_pages), rng.integers(rpp))
    say(f"paged {gist_set} many={many}")
    out, lse, sel = gsa.gsa_decode_paged(q, kp, vp, block_table=table, seq_n_raw=n, seq_n_gist=m, chunk=C,
                                         topk=k, tail=T, page_chunks=P, extra_rows=extra, gist_set=gist_set)
    torch.cuda.synchronize()
    g = Hq // Hkv
    units = [(b, j) for b in range(B) for j in range(Hkv)]
    pick = units if len(units) <= 8 else [units[i] for i in rng.choice(len(units), 10, False)]
    got, ref = [], []
    for b, j in pick:
        xs = [(int(p_), int(r_)) for p_, r_ in extra[b] if p_ >= 0][:counts[b]]
        r = oracle.decode_paged_unit(to_np(q[b, j * g:(j + 1) * g]), to_np(kp[:, j]), to_np(vp[:, j]),
                                     [int(x) for x in table[b]], page_chunks=P, n_raw=n[b], n_gist=m[b],
                                     chunk=C, topk=k, tail=T, extra_rows=xs, gist_set=gist_set)
        np.testing.assert_array_equal(to_np(sel[b, j]), r["sel"], err_msg=f"unit {(b, j)}")
        got.append(to_np(out[b, j * g:(j + 1) * g]))
        ref.append(r["out"])
        check_lse(to_np(lse[b, j * g:(j + 1) * g]), r["lse"], "bf16", f"unit {(b, j)}")
    err = check_out(np.stack(got), np.stack(ref), "bf16", f"paged {gist_set}")
    say(f"  max err / rms = {err:.2e}, {gsa.gsa_profile_marks() - 1} launches")
