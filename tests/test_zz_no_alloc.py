"""gsa_decode_noalloc (no device allocation: the library's own scratch array as
the workspace) against gsa_decode on the same inputs, through the C ABI: a
one-workgroup-per-unit call, then three calls in a row on shapes that use the
scratch (several workgroups per unit: arrival counters, hand-off of partial
states and candidates), each smaller than the one before, so a later call
runs on what the earlier one left in the array."""
import ctypes
import dataclasses

import numpy as np
import pytest
import torch

import gsa_inputs as gi
from gpu_util import LSE_TOL, TOL, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_gsa_amd
    decode_gsa_amd.lib()
    return decode_gsa_amd


CASES = [  # (config, overrides): each scratch-using case smaller than the one before
    ("gqa_32k", dict(n_raw=2048)),                                  # 256 units, one workgroup each
    ("c32_131k", dict(batch=2, n_kv_heads=2, n_q_heads=8, n_raw=65536)),
    ("gqa_32k", dict(batch=1, n_kv_heads=2, n_q_heads=8, n_raw=16384)),
    ("gqa_32k", dict(batch=1, n_kv_heads=1, n_q_heads=4, n_raw=4096, topk=8)),
]


def test_noalloc_matches_gsa_decode(gsa):
    L = gsa.lib()
    stream = torch.cuda.current_stream()
    for i, (name, kw) in enumerate(CASES):
        cfg = dataclasses.replace(gi.CONFIGS[name], **kw)
        say(f"noalloc call {i}: {name} {kw}")
        inp = gi.make_decode(cfg, 3100 + i, device="cuda")
        B, Hq, D = inp.q.shape
        ref_out, ref_lse, ref_sel = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=cfg.chunk,
                                                   topk=cfg.topk, tail=cfg.tail, n_gist=cfg.M)
        out = torch.full((B, Hq, D), float("nan"), device="cuda")
        lse = torch.full((B, Hq), float("nan"), device="cuda")
        sel = torch.full((B, cfg.n_kv_heads, cfg.topk), -7, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        p = gsa.decode_params(B, Hq, cfg.n_kv_heads, D, cfg.n_raw, cfg.M, cfg.chunk, cfg.topk,
                              cfg.tail)
        st = L.gsa_decode_noalloc(ctypes.byref(p), inp.q.data_ptr(), inp.k_cache.data_ptr(),
                                  inp.v_cache.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                  sel.data_ptr(), stream.cuda_stream)
        assert st == 0, L.gsa_last_error()
        torch.cuda.synchronize()
        assert torch.equal(sel, ref_sel), f"call {i}: selections differ"
        ro = ref_out.double().cpu().numpy()
        rms = float(np.sqrt(np.mean(ro ** 2)))
        err = float((out.double().cpu() - ref_out.double().cpu()).abs().max())
        assert err <= TOL["bf16"] * rms, f"call {i}: out err {err:.3e} vs rms {rms:.3e}"
        lerr = float((lse - ref_lse).abs().max())
        assert lerr <= LSE_TOL["bf16"], f"call {i}: lse err {lerr:.3e}"
        say(f"  ok: max err {err / rms:.2e} x rms")


def test_noalloc_rejects_oversize_and_launches_nothing(gsa):
    """A shape whose workspace exceeds the scratch is rejected before any launch."""
    L = gsa.lib()
    p = gsa.decode_params(32, 32, 8, 128, 131072, 16384, 8, 64, 64)
    buf = torch.zeros(16, device="cuda")
    st = L.gsa_decode_noalloc(ctypes.byref(p), buf.data_ptr(), buf.data_ptr(), buf.data_ptr(),
                              buf.data_ptr(), None, None, None)
    assert st == 3, L.gsa_last_error()
    assert gsa.gsa_profile_marks() == 1
