"""A decode call captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
the library launches only kernels on the caller's stream (no allocation, no
memset, no synchronization), and its completion counters return to zero at
the end of every call, so each replay reproduces the eager call bit for bit.
Replays alternate with eager work (clearing the outputs) and synchronizations.
"""
import dataclasses

import pytest
import torch

import gsa_inputs as gi
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_gsa_amd
    decode_gsa_amd.lib()          # raises if the library is missing: no fallback
    return decode_gsa_amd


CASES = [
    ("gqa_32k", dict(n_raw=4096)),                       # one workgroup per unit
    ("gqa_32k", dict(batch=2, n_raw=16384)),             # several per unit + the unfold launch
    ("tiny_f32", dict()),                                # fp32, D = 64: gist, candidate and unfold passes
]


@pytest.mark.parametrize("case", range(len(CASES)), ids=[c[0] + str(i) for i, c in enumerate(CASES)])
def test_decode_graph_replays_match_eager(gsa, case):
    name, kw = CASES[case]
    cfg = dataclasses.replace(gi.CONFIGS[name], **kw)
    say(f"graph capture {cfg}")
    inp = gi.make_decode(cfg, 4400 + case, device="cuda")
    B, Hq, D = inp.q.shape
    out = torch.empty(B, Hq, D, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
    sel = torch.empty(B, cfg.n_kv_heads, cfg.topk, dtype=torch.int32, device="cuda")
    p = gsa.decode_params(B, Hq, cfg.n_kv_heads, D, cfg.n_raw, cfg.M, cfg.chunk, cfg.topk, cfg.tail, 0.0,
                          gsa.GSA_BF16 if cfg.dtype == "bf16" else gsa.GSA_F32)
    ws = gsa.new_workspace(gsa.decode_workspace_size(p), "cuda")

    def call(st):
        gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=cfg.chunk, topk=cfg.topk, tail=cfg.tail,
                       n_gist=cfg.M, out=out, lse=lse, sel_idx=sel, workspace=ws, stream=st)

    call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, sel)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for r in range(4):
        for t in (out, lse, sel):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((out, lse, sel), ref):
            assert torch.equal(a, b), f"replay {r} differs from the eager call"
    del g
