"""GPU parity of gsa_decode_hier_varlen (two-level decode of sequences of
different lengths in one batch) against the fp64 oracle's decode_hier_unit,
sequence by sequence on its own rows and its own level-2 gists.

Cache rows past a sequence's own N_b + M_b and level-2 rows past its own
M2_b = floor(M_b / G) hold a constant the attention would notice, so a read
beyond them shows. Integer-valued entries ({-2..2}) keep every group score
exact, so the selections at both levels are decided by the scores and the
index tie rule alone.
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


def make_case(c, seed):
    B, Hq, Hkv, C, G = c["B"], c["Hq"], c["Hkv"], c["C"], c["G"]
    n, m = gi.varlen_lengths(B, c["n_min"], c["n_max"], C, seed)
    N, M = max(n), max(m)
    cap = N + M + 5
    q, k, v, ku, vu = gi.make_levels(B, Hq, Hkv, 128, cap - (cap // (C + 1)), cap // (C + 1), C, G, 2, seed,
                                     device="cuda", values="int")
    k, v = k[:, :, :cap].contiguous(), v[:, :, :cap].contiguous()
    M2 = M // G
    k2, v2 = ku[0][:, :, :M2].contiguous(), vu[0][:, :, :M2].contiguous()
    for b in range(B):                       # past the sequence's own rows
        k[b, :, n[b] + m[b]:] = 3.0
        v[b, :, n[b] + m[b]:] = 3.0
        k2[b, :, m[b] // G:] = 3.0
        v2[b, :, m[b] // G:] = 3.0
    return q, k, v, k2, v2, n, m


def check(c, q, k, v, k2, v2, n, m, out, lse, sel2, sel1, seqs=None, gist_set="all"):
    g = c["Hq"] // c["Hkv"]
    got, ref, got_l, ref_l = [], [], [], []
    for b in (range(c["B"]) if seqs is None else seqs):
        R, m2 = n[b] + m[b], m[b] // c["G"]
        for j in range(c["Hkv"]):
            r = oracle.decode_hier_unit(to_np(q[b, j * g:(j + 1) * g]), to_np(k[b, j, :R]), to_np(v[b, j, :R]),
                                        to_np(k2[b, j, :m2]), to_np(v2[b, j, :m2]), n_raw=n[b], n_gist=m[b],
                                        chunk=c["C"], fanout=c["G"], topk1=c["k1"], topk2=c["k2"], tail=c["T"],
                                        gist_set=gist_set)
            np.testing.assert_array_equal(to_np(sel2[b, j]), r["sel2"], err_msg=f"level 2, sequence {b} kv-head {j}")
            np.testing.assert_array_equal(to_np(sel1[b, j]), r["sel1"], err_msg=f"level 1, sequence {b} kv-head {j}")
            got.append(to_np(out[b, j * g:(j + 1) * g]))
            ref.append(r["out"])
            got_l.append(to_np(lse[b, j * g:(j + 1) * g]))
            ref_l.append(r["lse"])
    err = check_out(np.stack(got), np.stack(ref), "bf16", str(c))
    check_lse(np.stack(got_l), np.stack(ref_l), "bf16", str(c))
    return err


CASES = [
    # 64 units, lengths 20K-70K, G = 16: several workgroups per unit
    dict(B=8, Hq=32, Hkv=8, C=16, G=16, k1=16, k2=8, T=64, n_min=20000, n_max=70000),
    # short sequences, C = 8, G = 4, orphans in most sequences
    dict(B=4, Hq=8, Hkv=2, C=8, G=4, k1=8, k2=4, T=16, n_min=300, n_max=5000),
    # g = 8, 256 units
    dict(B=32, Hq=64, Hkv=8, C=16, G=8, k1=8, k2=6, T=32, n_min=2000, n_max=9000),
]


@pytest.mark.parametrize("i", range(len(CASES)), ids=[f"case{i}" for i in range(len(CASES))])
def test_hier_varlen_matches_oracle_per_sequence(gsa, i):
    c = CASES[i]
    say(f"hier varlen {c}")
    q, k, v, k2, v2, n, m = make_case(c, 7600 + i)
    out, lse, sel2, sel1 = gsa.gsa_decode_hier_varlen(q, k, v, k2, v2, seq_n_raw=n, seq_n_gist=m, chunk=c["C"],
                                                      fanout=c["G"], topk1=c["k1"], topk2=c["k2"], tail=c["T"])
    torch.cuda.synchronize()
    err = check(c, q, k, v, k2, v2, n, m, out, lse, sel2, sel1)
    say(f"  max err / rms = {err:.2e}, {gsa.gsa_profile_marks() - 1} launches")


def test_hier_varlen_equal_lengths_is_hier(gsa):
    """Every sequence at the call's largest length: bit-identical to
    gsa_decode_hier."""
    c = CASES[0]
    q, k, v, k2, v2, n, m = make_case(c, 7700)
    N, M = max(n), max(m)
    kk, vv = k[:, :, :N + M].contiguous(), v[:, :, :N + M].contiguous()
    say("hier varlen = uniform")
    kw = dict(chunk=c["C"], fanout=c["G"], topk1=c["k1"], topk2=c["k2"], tail=c["T"])
    # fresh level-2 rows everywhere (the per-sequence filler would be read now)
    k2u = torch.randint(-2, 3, k2.shape, device="cuda").to(k2.dtype)
    v2u = torch.randint(-2, 3, v2.shape, device="cuda").to(v2.dtype)
    kk[:] = torch.randint(-2, 3, kk.shape, device="cuda").to(kk.dtype)
    vv[:] = torch.randint(-2, 3, vv.shape, device="cuda").to(vv.dtype)
    a = gsa.gsa_decode_hier(q, kk, vv, k2u, v2u, n_gist=M, **kw)
    b = gsa.gsa_decode_hier_varlen(q, kk, vv, k2u, v2u, seq_n_raw=[N] * c["B"], seq_n_gist=[M] * c["B"], **kw)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_hier_varlen_device_lengths_and_fallback(gsa):
    """Lengths given as device arrays are used as given; a sequence whose
    lengths break the two-level rules (here fewer level-2 gists than topk2)
    runs with the call's largest lengths, reading only its own slabs."""
    c = CASES[1]
    q, k, v, k2, v2, n, m = make_case(c, 7800)
    N, M = max(n), max(m)
    bad = int(np.argmin(m))
    n2, m2 = list(n), list(m)
    n2[bad], m2[bad] = 3 * c["C"], 3          # 0 level-2 gists < topk2
    sn = torch.tensor(n2, dtype=torch.int32, device="cuda")
    sm = torch.tensor(m2, dtype=torch.int32, device="cuda")
    say("hier varlen device lengths")
    out, lse, sel2, sel1 = gsa.gsa_decode_hier_varlen(q, k, v, k2, v2, seq_n_raw=sn, seq_n_gist=sm, n_raw=N,
                                                      n_gist=M, chunk=c["C"], fanout=c["G"], topk1=c["k1"],
                                                      topk2=c["k2"], tail=c["T"])
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    n3, m3 = list(n), list(m)
    n3[bad], m3[bad] = N, M
    keep = [b for b in range(c["B"]) if b != bad]
    check(c, q, k, v, k2, v2, n3, m3, out, lse, sel2, sel1, seqs=keep)
    # the sequence that broke the rules: the call's maxima over its own slabs
    g = c["Hq"] // c["Hkv"]
    for j in range(c["Hkv"]):
        r = oracle.decode_hier_unit(to_np(q[bad, j * g:(j + 1) * g]), to_np(k[bad, j, :N + M]),
                                    to_np(v[bad, j, :N + M]), to_np(k2[bad, j]), to_np(v2[bad, j]), n_raw=N,
                                    n_gist=M, chunk=c["C"], fanout=c["G"], topk1=c["k1"], topk2=c["k2"],
                                    tail=c["T"])
        np.testing.assert_array_equal(to_np(sel1[bad, j]), r["sel1"])
        check_out(to_np(out[bad, j * g:(j + 1) * g]), r["out"], "bf16", f"sequence {bad}")


@pytest.mark.parametrize("gist_set", ["selected", "none"])
@pytest.mark.parametrize("i", [0, 1])
def test_hier_selection_rules(gsa, gist_set, i):
    """The slide 17 rules on the two-level decode (the rule picks which gists
    are attended; the routing is unchanged): uniform lengths through
    gsa_decode_hier and different lengths through gsa_decode_hier_varlen,
    both against the oracle with the same rule."""
    c = CASES[i]
    say(f"hier {gist_set} {c}")
    q, k, v, k2, v2, n, m = make_case(c, 7900 + i)
    kw = dict(chunk=c["C"], fanout=c["G"], topk1=c["k1"], topk2=c["k2"], tail=c["T"], gist_set=gist_set)
    out, lse, s2, s1 = gsa.gsa_decode_hier_varlen(q, k, v, k2, v2, seq_n_raw=n, seq_n_gist=m, **kw)
    torch.cuda.synchronize()
    err = check(c, q, k, v, k2, v2, n, m, out, lse, s2, s1, gist_set=gist_set)
    # the longest sequence's cache for every sequence: the uniform entry point
    b = int(np.argmax(n))
    N, M = n[b], m[b]
    nn, mm = [N] * c["B"], [M] * c["B"]
    kk = k[b:b + 1].expand(c["B"], -1, -1, -1)[:, :, :N + M].contiguous()
    vv = v[b:b + 1].expand(c["B"], -1, -1, -1)[:, :, :N + M].contiguous()
    k2u = k2[b:b + 1].expand(c["B"], -1, -1, -1)[:, :, :M // c["G"]].contiguous()
    v2u = v2[b:b + 1].expand(c["B"], -1, -1, -1)[:, :, :M // c["G"]].contiguous()
    out, lse, s2, s1 = gsa.gsa_decode_hier(q, kk, vv, k2u, v2u, n_gist=M, **kw)
    torch.cuda.synchronize()
    err2 = check(c, q, kk, vv, k2u, v2u, nn, mm, out, lse, s2, s1, gist_set=gist_set)
    say(f"  max err / rms = {err:.2e} (varlen), {err2:.2e} (uniform)")
