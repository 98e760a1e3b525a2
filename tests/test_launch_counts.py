"""The launch-count queries (gsa_*_launches) against what the calls do: after a
call, gsa_profile_marks reports its launches + 1, on every decode, two-level,
L-level and prefill path."""
import numpy as np
import pytest
import torch

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_gsa_amd
    decode_gsa_amd.lib()
    return decode_gsa_amd


def cache(B, Hkv, N, M, D, dtype, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    k = torch.randn(B, Hkv, N + M, D, generator=g).to(dtype).cuda()
    v = torch.randn(B, Hkv, N + M, D, generator=g).to(dtype).cuda()
    return k, v


DECODE = [  # B, Hq, Hkv, D, dtype, N, C, k, T (, gist_set)
    (32, 32, 8, 128, torch.bfloat16, 1024, 16, 8, 64),     # one workgroup per unit
    (1, 8, 2, 128, torch.bfloat16, 8192, 16, 8, 64),       # several per unit + select/unfold
    (1, 8, 2, 128, torch.bfloat16, 8192, 16, 0, 64),
    (1, 4, 1, 64, torch.float32, 4096, 16, 8, 16),         # split path, candidate pass
    (2, 4, 2, 128, torch.float32, 1024, 16, 4, 16),        # split path
    (2, 4, 2, 64, torch.float32, 1024, 16, 0, 16),
    (1, 4, 1, 128, torch.bfloat16, 4096, 16, 80, 64),      # k > 64: split path
    (1, 4, 1, 64, torch.float32, 4096, 16, 8, 16, 1),      # split path, selection rule 1
    (2, 4, 2, 128, torch.float32, 1024, 16, 4, 16, 2),     # split path, selection rule 2
    (2, 4, 2, 64, torch.float32, 1024, 16, 0, 16, 2),      # k = 0: the tail alone
]


@pytest.mark.parametrize("case", DECODE)
def test_decode_marks(gsa, case):
    B, Hq, Hkv, D, dt, N, C, k, T = case[:9]
    rule = case[9] if len(case) > 9 else 0
    M = N // C
    say("decode launches", case)
    kc, vc = cache(B, Hkv, N, M, D, dt, 1)
    q = torch.randn(B, Hq, D).to(dt).cuda()
    gsa.gsa_decode(q, kc, vc, chunk=C, topk=k, tail=T, gist_set=["all", "selected", "none"][rule])
    torch.cuda.synchronize()
    p = gsa.decode_params(B, Hq, Hkv, D, N, M, C, k, T, 0.0,
                          gsa.GSA_BF16 if dt == torch.bfloat16 else gsa.GSA_F32)
    p.gist_set = rule
    assert gsa.gsa_profile_marks() == gsa.launches(p) + 1


HIER = [  # D, dtype, N, G, k1, k2, gist_set
    (128, torch.bfloat16, 65536, 16, 8, 4, 0),
    (64, torch.float32, 65536, 16, 8, 4, 0),
    (64, torch.float32, 65536, 16, 0, 4, 0),
    (64, torch.float32, 65536, 16, 8, 4, 1),
    (64, torch.float32, 65536, 16, 0, 4, 2),   # the selection rules: the set's pass runs with k1 = 0
]


@pytest.mark.parametrize("case", HIER)
def test_hier_marks(gsa, case):
    D, dt, N, G, k1, k2, rule = case
    C, T, Hq, Hkv = 16, 64, 4, 1
    M = N // C
    say("hier launches", case)
    kc, vc = cache(1, Hkv, N, M, D, dt, 2)
    k2a = torch.randn(1, Hkv, M // G, D).to(dt).cuda()
    q = torch.randn(1, Hq, D).to(dt).cuda()
    gsa.gsa_decode_hier(q, kc, vc, k2a, k2a, chunk=C, fanout=G, topk1=k1, topk2=k2, tail=T,
                        gist_set=["all", "selected", "none"][rule])
    torch.cuda.synchronize()
    base = gsa.decode_params(1, Hq, Hkv, D, N, M, C, k1, T, 0.0,
                             gsa.GSA_BF16 if dt == torch.bfloat16 else gsa.GSA_F32, gist_set=rule)
    assert gsa.gsa_profile_marks() == gsa.launches(gsa.hier_params(base, G, k2)) + 1


LEVELS = [  # D, dtype, N, G, topks
    (128, torch.bfloat16, 65536, 16, [8, 4, 2]),     # top level of 16 gists: one launch
    (128, torch.bfloat16, 160000, 2, [8, 4]),        # top level of 5000 gists: two
    (64, torch.float32, 65536, 16, [8, 4, 2]),       # split path
    (64, torch.float32, 65536, 16, [0, 4, 2]),
]


@pytest.mark.parametrize("case", LEVELS)
def test_levels_marks(gsa, case):
    D, dt, N, G, topks = case
    C, T, Hq, Hkv = 16, 64, 4, 1
    M = N // C
    say("levels launches", case)
    kc, vc = cache(1, Hkv, N, M, D, dt, 3)
    sizes, m = [], M
    for _ in topks[1:]:
        m //= G
        sizes.append(m)
    ups = [torch.randn(1, Hkv, s, D).to(dt).cuda() for s in sizes]
    q = torch.randn(1, Hq, D).to(dt).cuda()
    gsa.gsa_decode_levels(q, kc, vc, ups, ups, chunk=C, fanout=G, topks=topks, tail=T)
    torch.cuda.synchronize()
    base = gsa.decode_params(1, Hq, Hkv, D, N, M, C, topks[0], T, 0.0,
                             gsa.GSA_BF16 if dt == torch.bfloat16 else gsa.GSA_F32)
    assert gsa.gsa_profile_marks() == gsa.launches(gsa.levels_params(base, G, topks[1:])) + 1


@pytest.mark.parametrize("k,n_q", [(8, 128), (0, 128), (8, 0)])
def test_prefill_marks(gsa, k, n_q):
    N, C, Hq, Hkv, D = 4096, 16, 8, 2, 128
    M = N // C
    kc, vc = cache(1, Hkv, N, M, D, torch.bfloat16, 4)
    kc, vc = kc[0].contiguous(), vc[0].contiguous()
    q = torch.randn(Hq, n_q, D).to(torch.bfloat16).cuda()
    gsa.gsa_prefill_blocksparse(q, kc, vc, chunk=C, topk=k, window=64, q_start=N - max(n_q, 1))
    torch.cuda.synchronize()
    p = gsa.prefill_params(Hq, Hkv, D, C, k, 64, N, M, N - max(n_q, 1), n_q)
    assert gsa.gsa_profile_marks() == gsa.launches(p) + 1
