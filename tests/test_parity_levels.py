"""GPU parity of gsa_decode_levels (L-level gist-of-gist decode) against the
fp64 oracle: every level's selection bit for bit, outputs and lse within the
stated tolerance.

Integer-valued inputs (entries in {-2..2}) make every group score exact on
both sides, so the selections are decided by the scores and the index tie
rule alone, with many ties among the candidates.
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


def run_levels(gsa, c, seed, units=None, values="int"):
    B, Hq, Hkv, D, C, M, r, G, topks, T = (c[k] for k in ("B", "Hq", "Hkv", "D", "C", "M", "r", "G", "topks", "T"))
    dtype = c.get("dtype", "bf16")
    L = len(topks)
    N = M * C + r
    q, k, v, ku, vu = gi.make_levels(B, Hq, Hkv, D, N, M, C, G, L, seed, device="cuda", dtype=dtype,
                                     values=values)
    out, lse, sels = gsa.gsa_decode_levels(q, k, v, ku, vu, chunk=C, fanout=G, topks=topks, tail=T, n_gist=M)
    torch.cuda.synchronize()
    c["_launches"] = gsa.gsa_profile_marks() - 1
    g = Hq // Hkv
    us = [(b, j) for b in range(B) for j in range(Hkv)] if units is None else units
    got, ref, got_l, ref_l = [], [], [], []
    for b, j in us:
        r_ = oracle.decode_levels_unit(to_np(q[b, j * g:(j + 1) * g]), to_np(k[b, j]), to_np(v[b, j]),
                                       [(to_np(ku[i][b, j]), to_np(vu[i][b, j])) for i in range(L - 1)],
                                       n_raw=N, n_gist=M, chunk=C, fanout=G, topks=topks, tail=T)
        for lvl in range(L):
            if topks[lvl] > 0:
                np.testing.assert_array_equal(to_np(sels[lvl][b, j]), r_["sels"][lvl],
                                              err_msg=f"unit {(b, j)} level {lvl + 1}")
        got.append(to_np(out[b, j * g:(j + 1) * g]))
        ref.append(r_["out"])
        got_l.append(to_np(lse[b, j * g:(j + 1) * g]))
        ref_l.append(r_["lse"])
    err = check_out(np.stack(got), np.stack(ref), dtype, str(c))
    check_lse(np.stack(got_l), np.stack(ref_l), dtype, str(c))
    return err, (q, k, v, ku, vu, out, lse, sels, N)


CASES = [
    # three levels, ragged raw tail (sizes 640, 160, 40)
    dict(B=2, Hq=8, Hkv=2, D=128, C=16, M=640, r=5, G=4, topks=[8, 6, 4], T=64),
    # four levels with ungrouped gists at levels 1 and 3 (sizes 1010, 336, 112, 37), fp32, D = 64
    dict(B=1, Hq=16, Hkv=4, D=64, C=8, M=1010, r=0, G=3, topks=[16, 10, 5, 3], T=8, dtype="f32"),
    # two levels through the L-level chain, g = 8
    dict(B=2, Hq=16, Hkv=2, D=128, C=16, M=512, r=16, G=8, topks=[12, 5], T=16),
    # six levels, fanout 2 (sizes 4096 .. 128)
    dict(B=1, Hq=4, Hkv=2, D=128, C=4, M=4096, r=3, G=2, topks=[30, 30, 30, 30, 30, 30], T=3),
    # k_1 = 0: the level-1 pass merges
    dict(B=2, Hq=8, Hkv=2, D=128, C=16, M=640, r=0, G=4, topks=[0, 6, 4], T=16),
    # nothing chosen at the top: only ungrouped gists go down (sizes 650, 162, 40)
    dict(B=1, Hq=8, Hkv=2, D=128, C=16, M=650, r=9, G=4, topks=[2, 2, 0], T=9),
    # every candidate chosen at every level
    dict(B=1, Hq=4, Hkv=1, D=128, C=4, M=100, r=0, G=3, topks=[100, 33, 11], T=0),
    # bf16 with k_1 > 64: the per-level passes
    dict(B=2, Hq=8, Hkv=2, D=128, C=16, M=640, r=5, G=4, topks=[70, 20, 8], T=64),
]


# bf16, D = 128, every k <= 64, a top level of at most 4096 gists: one
# workgroup per unit streams the top level and walks the levels down (one
# launch); otherwise one pass per level + unfold
FUSED = {0, 2, 3, 4, 5}


@pytest.mark.parametrize("i", range(len(CASES)), ids=[f"case{i}" for i in range(len(CASES))])
def test_levels_small(gsa, i):
    c = dict(CASES[i])
    say(f"levels {c}")
    err, _ = run_levels(gsa, c, 6000 + i)
    L = len(c["topks"])
    want = 1 if i in FUSED else L + (1 if c["topks"][0] > 0 else 0)
    say(f"  max err / rms = {err:.2e}, {c['_launches']} launches")
    assert c["_launches"] == want


def test_levels_gaussian_values(gsa):
    """Continuous values (no ties) on a small three-level case."""
    c = dict(B=2, Hq=8, Hkv=2, D=128, C=16, M=96, r=4, G=4, topks=[6, 3, 2], T=20)
    say("levels gaussian")
    err, _ = run_levels(gsa, c, 6100, values="gauss")
    say(f"  max err / rms = {err:.2e}")


def test_levels_capacity_and_repeat(gsa):
    """A cache with spare rows gives bit-identical results; so does a second
    call with the same (reused) workspace."""
    c = dict(CASES[0])
    say("levels capacity")
    _, (q, k, v, ku, vu, out, lse, sels, N) = run_levels(gsa, c, 6200)
    big_k = torch.zeros(c["B"], c["Hkv"], k.shape[2] + 19, c["D"], dtype=k.dtype, device="cuda")
    big_v = torch.zeros_like(big_k)
    big_k[:, :, :k.shape[2]] = k
    big_v[:, :, :k.shape[2]] = v
    import decode_gsa_amd as g
    base = g.decode_params(c["B"], c["Hq"], c["Hkv"], c["D"], N, c["M"], c["C"], c["topks"][0], c["T"])
    ws = g.new_workspace(g.levels_workspace_size(g.levels_params(base, c["G"], c["topks"][1:])))
    for _ in range(2):
        o2, l2, s2 = gsa.gsa_decode_levels(q, big_k, big_v, ku, vu, chunk=c["C"], fanout=c["G"], topks=c["topks"],
                                           tail=c["T"], n_gist=c["M"], n_raw=N, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o2, out) and torch.equal(l2, lse)
        assert all(torch.equal(a, b) for a, b in zip(s2, sels))


def test_levels_1m_three_levels_sampled(gsa):
    """The 1M-token two-level workload with a third level (4 sequences, Hq 32 /
    Hkv 8, C 16, G 16: 65536, 4096, 256 gists; k = 16, 8, 4), sampled units."""
    c = dict(B=4, Hq=32, Hkv=8, D=128, C=16, M=65536, r=0, G=16, topks=[16, 8, 4], T=64)
    say("levels 1m")
    err, _ = run_levels(gsa, c, 6300, units=[(0, 0), (1, 3), (3, 7)])
    say(f"  max err / rms = {err:.2e}")


# ------------------------------------------------ variable lengths ---

def levels_varlen_case(c, seed):
    """Per-sequence lengths and the level arrays of the batch's largest M;
    rows past a sequence's own rows (cache and every level) hold a constant
    the attention would notice."""
    B, Hq, Hkv, C, G, L = c["B"], c["Hq"], c["Hkv"], c["C"], c["G"], len(c["topks"])
    n, m = gi.varlen_lengths(B, c["n_min"], c["n_max"], C, seed)
    N, M = max(n), max(m)
    q, k, v, ku, vu = gi.make_levels(B, Hq, Hkv, 128, N + 3, M, C, G, L, seed, device="cuda", values="int")
    cap = N + M + 3
    for b in range(B):
        k[b, :, n[b] + m[b]:] = 3.0
        v[b, :, n[b] + m[b]:] = 3.0
        ml = m[b]
        for i in range(L - 1):
            ml //= G
            ku[i][b, :, ml:] = 3.0
            vu[i][b, :, ml:] = 3.0
    return q, k[:, :, :cap].contiguous(), v[:, :, :cap].contiguous(), ku, vu, n, m


VARLEN_CASES = [
    # three levels, lengths 8K-40K (top level at most 156 gists)
    dict(B=4, Hq=8, Hkv=2, C=16, G=4, topks=[8, 6, 4], T=64, n_min=8000, n_max=40000),
    # four levels, G = 2, 256 units
    dict(B=32, Hq=32, Hkv=8, C=16, G=2, topks=[8, 6, 4, 3], T=32, n_min=2000, n_max=9000),
]


@pytest.mark.parametrize("i", range(len(VARLEN_CASES)), ids=[f"varlen{i}" for i in range(len(VARLEN_CASES))])
def test_levels_varlen_matches_oracle_per_sequence(gsa, i):
    c = VARLEN_CASES[i]
    say(f"levels varlen {c}")
    q, k, v, ku, vu, n, m = levels_varlen_case(c, 9100 + i)
    topks, G, L = c["topks"], c["G"], len(c["topks"])
    out, lse, sels = gsa.gsa_decode_levels_varlen(q, k, v, ku, vu, seq_n_raw=n, seq_n_gist=m, chunk=c["C"],
                                                  fanout=G, topks=topks, tail=c["T"])
    torch.cuda.synchronize()
    assert gsa.gsa_profile_marks() == 2
    g = c["Hq"] // c["Hkv"]
    got, ref, got_l, ref_l = [], [], [], []
    for b in range(c["B"]):
        sizes = [m[b]]
        for _ in range(L - 1):
            sizes.append(sizes[-1] // G)
        for j in range(c["Hkv"]):
            r_ = oracle.decode_levels_unit(to_np(q[b, j * g:(j + 1) * g]), to_np(k[b, j, :n[b] + m[b]]),
                                           to_np(v[b, j, :n[b] + m[b]]),
                                           [(to_np(ku[l][b, j, :sizes[l + 1]]), to_np(vu[l][b, j, :sizes[l + 1]]))
                                            for l in range(L - 1)],
                                           n_raw=n[b], n_gist=m[b], chunk=c["C"], fanout=G, topks=topks,
                                           tail=c["T"])
            for lvl in range(L):
                np.testing.assert_array_equal(to_np(sels[lvl][b, j]), r_["sels"][lvl],
                                              err_msg=f"sequence {b} kv {j} level {lvl + 1}")
            got.append(to_np(out[b, j * g:(j + 1) * g]))
            ref.append(r_["out"])
            got_l.append(to_np(lse[b, j * g:(j + 1) * g]))
            ref_l.append(r_["lse"])
    err = check_out(np.stack(got), np.stack(ref), "bf16", str(c))
    check_lse(np.stack(got_l), np.stack(ref_l), "bf16", str(c))
    say(f"  max err / rms = {err:.2e}")


def test_levels_varlen_equal_lengths_is_levels(gsa):
    """Every sequence at the call's largest lengths: bit-identical to
    gsa_decode_levels."""
    c = dict(VARLEN_CASES[0])
    B, C, G, L = c["B"], c["C"], c["G"], len(c["topks"])
    M = 1500
    N = M * C + 7
    q, k, v, ku, vu = gi.make_levels(B, c["Hq"], c["Hkv"], 128, N, M, C, G, L, 9200, device="cuda", values="int")
    kw = dict(chunk=C, fanout=G, topks=c["topks"], tail=c["T"])
    a = gsa.gsa_decode_levels(q, k, v, ku, vu, n_gist=M, **kw)
    b = gsa.gsa_decode_levels_varlen(q, k, v, ku, vu, seq_n_raw=[N] * B, seq_n_gist=[M] * B, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    for x, y in zip(a[2], b[2]):
        assert torch.equal(x, y)


# ------------------------------------------------------ selection rules ---

@pytest.mark.parametrize("gist_set", ["selected", "none"])
@pytest.mark.parametrize("i", [0, 1, 2, 4, 7, 8])
def test_levels_selection_rules(gsa, i, gist_set):
    """The slide 17 rules on L-level decode (R20: every level's gists route,
    the rule picks which gists are attended): one launch (top level in LDS),
    the two-launch path (top level above 4096 gists) and the per-level split
    path (fp32 with D = 64, k_1 > 64, k_1 = 0), against the oracle with the
    same rule."""
    c = CASES[i] if i < len(CASES) else None
    if i == 4:
        # three levels with a top level of 5000 gists: the stream launch, then the descent
        c = dict(B=1, Hq=8, Hkv=2, D=128, C=4, M=5000 * 16, r=2, G=4, topks=[8, 6, 4], T=16)
    if i == 8:
        # the split path with k_1 = 0: the levels only route, the set is the tail
        c = dict(CASES[1], topks=[0, 10, 5, 3])
    B, Hq, Hkv, D, C, M, r, G, topks, T = (c[k] for k in ("B", "Hq", "Hkv", "D", "C", "M", "r", "G", "topks", "T"))
    dtype = c.get("dtype", "bf16")
    split = i in (1, 7, 8)
    say(f"levels {gist_set} {c}")
    L = len(topks)
    N = M * C + r
    q, k, v, ku, vu = gi.make_levels(B, Hq, Hkv, D, N, M, C, G, L, 9300 + i, device="cuda", dtype=dtype,
                                     values="int")
    out, lse, sels = gsa.gsa_decode_levels(q, k, v, ku, vu, chunk=C, fanout=G, topks=topks, tail=T, n_gist=M,
                                           gist_set=gist_set)
    torch.cuda.synchronize()
    if split:   # one pass per level, then the set's pass
        assert gsa.gsa_profile_marks() - 1 == L + 1
    g = Hq // Hkv
    got, ref = [], []
    units = [(b, j) for b in range(B) for j in range(Hkv)]
    for b, j in units:
        r_ = oracle.decode_levels_unit(to_np(q[b, j * g:(j + 1) * g]), to_np(k[b, j]), to_np(v[b, j]),
                                       [(to_np(ku[l][b, j]), to_np(vu[l][b, j])) for l in range(L - 1)],
                                       n_raw=N, n_gist=M, chunk=C, fanout=G, topks=topks, tail=T, gist_set=gist_set)
        for lvl in range(L):
            if topks[lvl] > 0:
                np.testing.assert_array_equal(to_np(sels[lvl][b, j]), r_["sels"][lvl],
                                              err_msg=f"unit {(b, j)} level {lvl + 1}")
        got.append(to_np(out[b, j * g:(j + 1) * g]))
        ref.append(r_["out"])
        check_lse(to_np(lse[b, j * g:(j + 1) * g]), r_["lse"], dtype, f"unit {(b, j)}")
    err = check_out(np.stack(got), np.stack(ref), dtype, str(c))
    say(f"  max err / rms = {err:.2e}, {gsa.gsa_profile_marks() - 1} launches")


@pytest.mark.parametrize("gist_set", ["selected", "none"])
def test_levels_varlen_selection_rules(gsa, gist_set):
    c = VARLEN_CASES[0]
    say(f"levels varlen {gist_set} {c}")
    q, k, v, ku, vu, n, m = levels_varlen_case(c, 9400)
    topks, G, L = c["topks"], c["G"], len(c["topks"])
    out, lse, sels = gsa.gsa_decode_levels_varlen(q, k, v, ku, vu, seq_n_raw=n, seq_n_gist=m, chunk=c["C"],
                                                  fanout=G, topks=topks, tail=c["T"], gist_set=gist_set)
    torch.cuda.synchronize()
    g = c["Hq"] // c["Hkv"]
    got, ref = [], []
    for b in range(c["B"]):
        sizes = [m[b]]
        for _ in range(L - 1):
            sizes.append(sizes[-1] // G)
        for j in range(c["Hkv"]):
            r_ = oracle.decode_levels_unit(to_np(q[b, j * g:(j + 1) * g]), to_np(k[b, j, :n[b] + m[b]]),
                                           to_np(v[b, j, :n[b] + m[b]]),
                                           [(to_np(ku[l][b, j, :sizes[l + 1]]), to_np(vu[l][b, j, :sizes[l + 1]]))
                                            for l in range(L - 1)],
                                           n_raw=n[b], n_gist=m[b], chunk=c["C"], fanout=G, topks=topks,
                                           tail=c["T"], gist_set=gist_set)
            for lvl in range(L):
                np.testing.assert_array_equal(to_np(sels[lvl][b, j]), r_["sels"][lvl])
            got.append(to_np(out[b, j * g:(j + 1) * g]))
            ref.append(r_["out"])
    err = check_out(np.stack(got), np.stack(ref), "bf16", str(c))
    say(f"  max err / rms = {err:.2e}")
