"""GPU parity of gsa_decode_varlen (sequences of different lengths in one
batch) against the fp64 oracle, sequence by sequence on its own rows.

Rows past a sequence's own N_b + M_b hold a constant the attention would
notice, so a read beyond them shows. Integer-valued entries ({-2..2}) keep
every group score exact (selections decided by the scores and the index tie
rule alone).
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
    B, Hq, Hkv, D, C = c["B"], c["Hq"], c["Hkv"], c["D"], c["C"]
    dtype = c.get("dtype", "bf16")
    n, m = gi.varlen_lengths(B, c["n_min"], c["n_max"], C, seed)
    N, M = max(n), max(m)
    cap = N + M + 5
    q, k, v, _, _ = gi.make_levels(B, Hq, Hkv, D, cap - (cap // (C + 1)), cap // (C + 1), C, 2, 2, seed,
                                   device="cuda", dtype=dtype, values="int")
    k, v = k[:, :, :cap].contiguous(), v[:, :, :cap].contiguous()
    for b in range(B):                       # past the sequence's own rows
        k[b, :, n[b] + m[b]:] = 3.0
        v[b, :, n[b] + m[b]:] = 3.0
    return q, k, v, n, m


def check(gsa, c, q, k, v, n, m, out, lse, sel, gist_set="all"):
    g = c["Hq"] // c["Hkv"]
    dtype = c.get("dtype", "bf16")
    got, ref, got_l, ref_l = [], [], [], []
    for b in range(c["B"]):
        R = n[b] + m[b]
        for j in range(c["Hkv"]):
            r = oracle.decode_unit(to_np(q[b, j * g:(j + 1) * g]), to_np(k[b, j, :R]), to_np(v[b, j, :R]),
                                   n_raw=n[b], n_gist=m[b], chunk=c["C"], topk=c["k"], tail=c["T"],
                                   gist_set=gist_set)
            if c["k"] > 0:
                np.testing.assert_array_equal(to_np(sel[b, j]), r["sel"], err_msg=f"sequence {b} kv-head {j}")
            got.append(to_np(out[b, j * g:(j + 1) * g]))
            ref.append(r["out"])
            got_l.append(to_np(lse[b, j * g:(j + 1) * g]))
            ref_l.append(r["lse"])
    err = check_out(np.stack(got), np.stack(ref), dtype, str(c))
    check_lse(np.stack(got_l), np.stack(ref_l), dtype, str(c))
    return err


CASES = [
    # 256 units: one workgroup per unit
    dict(B=32, Hq=32, Hkv=8, D=128, C=16, k=16, T=64, n_min=300, n_max=8192),
    # 16 units: several workgroups per unit, then the selecting unfold launch
    dict(B=2, Hq=32, Hkv=8, D=128, C=16, k=16, T=64, n_min=1000, n_max=20000),
    # split path: fp32, D = 64
    dict(B=3, Hq=4, Hkv=2, D=64, C=8, k=8, T=8, n_min=80, n_max=3000, dtype="f32"),
    # split path in bf16: k above 64
    dict(B=4, Hq=8, Hkv=2, D=128, C=16, k=80, T=32, n_min=1300, n_max=6000),
    # k = 0
    dict(B=32, Hq=32, Hkv=8, D=128, C=16, k=0, T=16, n_min=16, n_max=4000),
]


@pytest.mark.parametrize("i", range(len(CASES)), ids=[f"case{i}" for i in range(len(CASES))])
def test_varlen_matches_oracle_per_sequence(gsa, i):
    c = CASES[i]
    say(f"varlen {c}")
    q, k, v, n, m = make_case(c, 7100 + i)
    out, lse, sel = gsa.gsa_decode_varlen(q, k, v, seq_n_raw=n, seq_n_gist=m, chunk=c["C"], topk=c["k"],
                                          tail=c["T"])
    torch.cuda.synchronize()
    err = check(gsa, c, q, k, v, n, m, out, lse, sel)
    say(f"  max err / rms = {err:.2e}, {gsa.gsa_profile_marks() - 1} launches")


def test_varlen_equal_lengths_is_gsa_decode(gsa):
    """Every sequence at the call's largest length: bit-identical to gsa_decode."""
    c = CASES[0]
    q, k, v, n, m = make_case(c, 7200)
    N, M = max(n), max(m)
    say("varlen = uniform")
    kk = k[:, :, :N + M].contiguous()
    vv = v[:, :, :N + M].contiguous()
    a = gsa.gsa_decode(q, kk, vv, chunk=c["C"], topk=c["k"], tail=c["T"], n_gist=M)
    b = gsa.gsa_decode_varlen(q, kk, vv, seq_n_raw=[N] * c["B"], seq_n_gist=[M] * c["B"], chunk=c["C"],
                              topk=c["k"], tail=c["T"])
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_varlen_device_lengths_and_fallback(gsa):
    """Lengths given as device arrays are used as given; a sequence whose pair
    breaks the rules (here fewer gists than k) runs with the call's largest
    lengths, reading only its own slab."""
    c = CASES[0]
    q, k, v, n, m = make_case(c, 7300)
    N, M = max(n), max(m)
    bad = 5
    n2, m2 = list(n), list(m)
    m2[bad] = c["k"] - 1
    sn = torch.tensor(n2, dtype=torch.int32, device="cuda")
    sm = torch.tensor(m2, dtype=torch.int32, device="cuda")
    say("varlen device lengths")
    out, lse, sel = gsa.gsa_decode_varlen(q, k, v, seq_n_raw=sn, seq_n_gist=sm, n_raw=N, n_gist=M, chunk=c["C"],
                                          topk=c["k"], tail=c["T"])
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    n3, m3 = list(n), list(m)
    n3[bad], m3[bad] = N, M
    keep = [b for b in range(c["B"]) if b != bad]
    g = c["Hq"] // c["Hkv"]
    for b in keep[:4] + [bad]:
        R = n3[b] + m3[b]
        for j in (0, c["Hkv"] - 1):
            r = oracle.decode_unit(to_np(q[b, j * g:(j + 1) * g]), to_np(k[b, j, :R]), to_np(v[b, j, :R]),
                                   n_raw=n3[b], n_gist=m3[b], chunk=c["C"], topk=c["k"], tail=c["T"])
            np.testing.assert_array_equal(to_np(sel[b, j]), r["sel"])
            check_out(to_np(out[b, j * g:(j + 1) * g]), r["out"], "bf16", f"sequence {b}")


@pytest.mark.parametrize("gist_set", ["selected", "none"])
@pytest.mark.parametrize("i", [0, 1, 2], ids=["units256", "units16", "split_f32"])
def test_varlen_selection_rules(gsa, i, gist_set):
    """The slide 17 rules with sequences of different lengths: one workgroup
    per unit, several per unit (scoring launch, then the set's launch) and
    the split path, each sequence against the oracle with the same rule."""
    c = CASES[i]
    say(f"varlen {gist_set} {c}")
    q, k, v, n, m = make_case(c, 7400 + i)
    out, lse, sel = gsa.gsa_decode_varlen(q, k, v, seq_n_raw=n, seq_n_gist=m, chunk=c["C"], topk=c["k"],
                                          tail=c["T"], gist_set=gist_set)
    torch.cuda.synchronize()
    err = check(gsa, c, q, k, v, n, m, out, lse, sel, gist_set=gist_set)
    say(f"  max err / rms = {err:.2e}, {gsa.gsa_profile_marks() - 1} launches")
