"""Cross-document routing over reused document caches (GPU).

Each document's K/V rows (raw tokens and gists, built for the document on
its own) are appended one document after another into one cache with
gsa_cache_append; every document ends on a chunk boundary, so the result is
one interleaved cache whose chunk ids run across the documents. A decode
step then picks its top-k chunks among every document's gists. One
document's gists are aligned with the query, so the chosen chunks must all
come from it; the output is checked against the fp64 oracle on the densely
built cache.
"""
import numpy as np
import pytest
import torch

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


def test_routing_across_appended_documents(gsa):
    C, Hq, Hkv, D, k, T = 16, 8, 2, 128, 8, 16
    chunks = [96, 40, 200, 64]              # chunks per document
    relevant = 2
    g = Hq // Hkv
    gen = torch.Generator(device="cuda")
    gen.manual_seed(8100)
    q = torch.randn(1, Hq, D, generator=gen, device="cuda").to(torch.bfloat16)
    docs = []
    for d, m in enumerate(chunks):
        raw_k = torch.randn(1, Hkv, m * C, D, generator=gen, device="cuda")
        raw_v = torch.randn(1, Hkv, m * C, D, generator=gen, device="cuda")
        gist_k = torch.randn(1, Hkv, m, D, generator=gen, device="cuda")
        gist_v = torch.randn(1, Hkv, m, D, generator=gen, device="cuda")
        if d == relevant:                   # this document's gists point at the query
            for j in range(Hkv):
                qbar = q[0, j * g:(j + 1) * g].float().mean(0)
                gist_k[0, j] += 3.0 * qbar / qbar.norm() * D ** 0.5 / 2
        docs.append([x.to(torch.bfloat16).contiguous() for x in (raw_k, raw_v, gist_k, gist_v)])
    N, M = sum(chunks) * C, sum(chunks)
    cap = N + M + 7
    kc = torch.zeros(1, Hkv, cap, D, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    n, m = 0, 0
    for raw_k, raw_v, gist_k, gist_v in docs:
        gsa.gsa_cache_append(kc, vc, chunk=C, n_raw=n, n_gist=m, k_raw=raw_k, v_raw=raw_v, k_gist=gist_k,
                             v_gist=gist_v)
        n, m = n + raw_k.shape[2], m + gist_k.shape[2]
    say(f"documents {chunks}: N={N}, M={M}")
    out, lse, sel = gsa.gsa_decode(q, kc, vc, chunk=C, topk=k, tail=T, n_gist=M, n_raw=N)
    torch.cuda.synchronize()
    # the dense concatenation, row by row from the documents
    K = np.zeros((Hkv, N + M, D))
    V = np.zeros((Hkv, N + M, D))
    p0, m0 = 0, 0
    for raw_k, raw_v, gist_k, gist_v in docs:
        for p in range(raw_k.shape[2]):
            r = oracle.cache_row(p0 + p, C, False)
            K[:, r], V[:, r] = to_np(raw_k[0, :, p]), to_np(raw_v[0, :, p])
        for mm in range(gist_k.shape[2]):
            r = oracle.cache_row(m0 + mm, C, True)
            K[:, r], V[:, r] = to_np(gist_k[0, :, mm]), to_np(gist_v[0, :, mm])
        p0, m0 = p0 + raw_k.shape[2], m0 + gist_k.shape[2]
    np.testing.assert_array_equal(to_np(kc[0, :, :N + M]), K)
    lo = sum(chunks[:relevant])
    hi = lo + chunks[relevant]
    got, ref = [], []
    for j in range(Hkv):
        r = oracle.decode_unit(to_np(q[0, j * g:(j + 1) * g]), K[j], V[j], n_raw=N, n_gist=M, chunk=C, topk=k,
                               tail=T)
        np.testing.assert_array_equal(to_np(sel[0, j]), r["sel"])
        assert all(lo <= c < hi for c in r["sel"]), "routing left the relevant document"
        got.append(to_np(out[0, j * g:(j + 1) * g]))
        ref.append(r["out"])
    err = check_out(np.stack(got), np.stack(ref), "bf16", "documents")
    say(f"  chosen chunks {to_np(sel[0, 0]).tolist()} in document {relevant} [{lo}, {hi}); max err / rms = {err:.2e}")
