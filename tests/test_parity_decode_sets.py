"""GPU parity of gsa_decode's selection-rule variants (slide deck, slide 17
'Selective Rules Comparison'): the attention set keeps the selected chunks'
gists with their raw tokens (gist_set "selected", SG+SR) or the selected raw
tokens alone ("none", SR-only), plus the tail. They run on the bf16,
head_dim 128, topk <= 64 launches: with one workgroup per unit (256 or more
units, at most 4096 gists) the gist keys are read for the scores only, then
the chosen chunks' rows, their gists and the tail are attended; with several
workgroups per unit (fewer units or more gists) a scoring launch hands on
candidates or scores and a second launch selects and attends the set.
Checked against the fp64 oracle with the same rule: bit-exact selections,
outputs and lse within the stated tolerance (tests/gpu_util.py).
"""
import dataclasses

import numpy as np
import pytest
import torch

import gsa_inputs as gi
from conftest import to_np
from gpu_util import say
from test_parity_decode import run_decode, sample_units

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_gsa_amd
    decode_gsa_amd.lib()          # raises if the library is missing: no fallback
    return decode_gsa_amd


def cfg_of(name, **kw):
    return dataclasses.replace(gi.CONFIGS[name], **kw)


# (config, units compared: None = every unit, else that many sampled)
CASES = [
    (cfg_of("gqa_32k", n_raw=4096), None),                                  # 256 units, g = 4, k = 16
    (cfg_of("gqa_32k", n_q_heads=8, n_raw=3000, n_gist=187, tail=40), 64),  # g = 1, ragged, partial chunk
    (cfg_of("gqa_32k", n_q_heads=64, n_raw=2048), 64),                      # g = 8
    (cfg_of("c8_131k", batch=32, n_raw=8192), 48),                          # C = 8, k = 64
    (cfg_of("c32_131k", batch=32, n_raw=8192, tail=5), 48),                 # C = 32, short tail
    (cfg_of("gqa_32k", n_raw=2048, topk=0, plant="none"), 64),              # k = 0: the tail alone
    (cfg_of("gqa_32k", n_raw=1024, topk=64, plant="none"), 64),             # every chunk selected
    (cfg_of("gqa_32k", n_raw=65536, tail=300), 12),                         # 4096 gists
    # several workgroups per unit
    (cfg_of("c8_131k", n_raw=32768), 24),                                   # 64 units x 4, C = 8, k = 64
    (cfg_of("c32_131k", n_raw=65536), 24),                                  # 64 units, C = 32, k = 16
    (cfg_of("gqa_32k", batch=2, n_raw=8192, tail=70), None),                # 16 units, candidates
    (cfg_of("gqa_32k", batch=1, n_kv_heads=1, n_q_heads=4, n_raw=16 * 5000, tail=64), None),   # 5000 gists
    (cfg_of("gqa_32k", batch=2, n_raw=4096, topk=0, plant="none"), None),   # k = 0: the tail alone
    (cfg_of("gqa_32k", batch=1, n_kv_heads=2, n_q_heads=8, n_raw=1024, topk=64, plant="none"), None),   # k = M
    # the split path: a scoring pass, then one pass over the set
    (cfg_of("tiny_f32"), None),                                             # fp32, D = 64, per-split candidates
    (cfg_of("tiny_f32", n_raw=4000, n_gist=250, tail=20, topk=5), None),    # ragged, partial chunk
    (cfg_of("gqa_32k", batch=2, n_raw=4096, head_dim=64), None),            # bf16, D = 64
    (cfg_of("gqa_32k", batch=2, n_raw=8192, topk=80, plant="none"), None),  # bf16, D = 128, k > 64
    (cfg_of("tiny_f32", topk=0, plant="none"), None),                       # k = 0: the tail alone
]


@pytest.mark.parametrize("gist_set", ["selected", "none"])
@pytest.mark.parametrize("case", range(len(CASES)), ids=[f"set{i}" for i in range(len(CASES))])
def test_decode_gist_set(gsa, case, gist_set):
    cfg, n = CASES[case]
    say(f"decode gist_set={gist_set} {cfg} units={'all' if n is None else n}")
    inp = gi.make_decode(cfg, 5000 + case, device="cuda")
    units = None if n is None else sample_units(cfg, n=n, seed=case)
    err = run_decode(gsa, inp, cfg, units=units, gist_set=gist_set)
    say(f"  max err / rms = {err:.2e}")


@pytest.mark.parametrize("gist_set", ["selected", "none"])
def test_decode_gist_set_ties_and_tail_overlap(gsa, gist_set):
    """q = 0: every score ties, so chunks 0..k-1 are chosen; the tail starts
    inside chunk k-1, whose rows (and, for "selected", gist) are attended
    once."""
    C, M, k = 16, 128, 16
    T = M * C - ((k - 1) * C + 8)
    cfg = cfg_of("gqa_32k", n_raw=M * C, topk=k, tail=T, plant="none")
    say(f"decode gist_set={gist_set} ties {cfg}")
    inp = gi.make_decode(cfg, 5100, device="cuda")
    inp.q.zero_()
    out, lse, sel = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=C, topk=k, tail=T,
                                   gist_set=gist_set)
    torch.cuda.synchronize()
    assert (to_np(sel) == np.arange(k)[None, None, :]).all()
    run_decode(gsa, inp, cfg, units=sample_units(cfg, n=16, seed=5), gist_set=gist_set)


def test_decode_gist_set_rejections(gsa):
    """An empty set is refused before any launch."""
    cfg = cfg_of("gqa_32k", n_raw=1024)
    inp = gi.make_decode(cfg, 5201, device="cuda")
    with pytest.raises(gsa.GsaError) as e:
        gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, chunk=16, topk=0, tail=0, gist_set="none")
    assert e.value.status == gsa.GSA_ERR_INVALID_ARG


@pytest.mark.parametrize("gist_set,want_k", [("all", 10), ("selected", 40), ("none", 42)])
def test_decode_token_budget(gsa, gist_set, want_k):
    """Fixed-token-budget mode: one budget of 744 tokens over 512 gists, C = 16,
    T = 64 unfolds 10 chunks when every gist stays in the set, 40 with only
    the chosen gists and 42 with none (slide 17's argument for dropping the
    unselected gists); each k then runs through gsa_decode and matches the
    oracle."""
    budget = 744
    cfg = cfg_of("gqa_32k", n_raw=8192, plant="none")
    k = gsa.topk_for_budget(budget, cfg.M, cfg.chunk, cfg.tail, gist_set)
    assert k == want_k
    cfg = dataclasses.replace(cfg, topk=k)
    say(f"decode budget {budget} gist_set={gist_set} -> k={k}")
    inp = gi.make_decode(cfg, 5300, device="cuda")
    run_decode(gsa, inp, cfg, units=sample_units(cfg, n=16, seed=6), gist_set=gist_set)
