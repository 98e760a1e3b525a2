"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, the ctypes structs match the C layout, and every invalid
argument is rejected on the host with the documented status before any launch.

None of these calls passes validation, so no kernel is ever launched here.
"""
import ctypes
import os
import re
import subprocess

import pytest

import decode_gsa_amd as gsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gsa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 1 << 20            # 16-byte aligned, never dereferenced (validation fails first)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gsa.LIB_PATH):
        pytest.skip("libgsa.so not built")
    return gsa.lib()


def test_every_declared_symbol_is_exported(L):
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:gsa_status_t|const char\*)\s+(gsa_\w+)\s*\(", text, re.M))
    assert declared == set(gsa.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(L, name), name


def test_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "gsa.h"
#define F(T, m) printf(#T "." #m " %zu\n", offsetof(T, m))
int main(void) {
  printf("gsa_decode_params %zu\n", sizeof(gsa_decode_params));
  printf("gsa_hier_params %zu\n", sizeof(gsa_hier_params));
  printf("gsa_prefill_params %zu\n", sizeof(gsa_prefill_params));
  printf("gsa_gist_params %zu\n", sizeof(gsa_gist_params));
  printf("gsa_levels_params %zu\n", sizeof(gsa_levels_params));
  printf("gsa_paged_params %zu\n", sizeof(gsa_paged_params));
  printf("gsa_prefill_varlen_params %zu\n", sizeof(gsa_prefill_varlen_params));
  F(gsa_prefill_varlen_params, batch);
  F(gsa_paged_params, page_chunks); F(gsa_paged_params, max_pages); F(gsa_paged_params, n_pages);
  F(gsa_paged_params, max_extra);
  printf("GSA_MAX_LEVELS %d\n", GSA_MAX_LEVELS);
  F(gsa_levels_params, n_levels); F(gsa_levels_params, fanout); F(gsa_levels_params, topk_up);
  printf("gsa_append_params %zu\n", sizeof(gsa_append_params));
  F(gsa_decode_params, row_capacity); F(gsa_prefill_params, row_capacity);
  F(gsa_gist_params, n_raw); F(gsa_gist_params, n_gist); F(gsa_gist_params, m_start);
  F(gsa_gist_params, n_q); F(gsa_gist_params, scale); F(gsa_gist_params, dtype);
  F(gsa_gist_params, row_capacity);
  F(gsa_append_params, chunk); F(gsa_append_params, n_raw); F(gsa_append_params, n_gist);
  F(gsa_append_params, raw_new); F(gsa_append_params, gist_new);
  F(gsa_append_params, row_capacity); F(gsa_append_params, dtype);
  F(gsa_decode_params, n_raw); F(gsa_decode_params, n_gist); F(gsa_decode_params, chunk);
  F(gsa_decode_params, scale); F(gsa_decode_params, dtype); F(gsa_decode_params, gist_set);
  printf("GSA_GISTS_ALL %d\nGSA_GISTS_SELECTED %d\nGSA_GISTS_NONE %d\n", GSA_GISTS_ALL,
         GSA_GISTS_SELECTED, GSA_GISTS_NONE);
  F(gsa_hier_params, fanout); F(gsa_hier_params, topk2);
  F(gsa_prefill_params, n_raw); F(gsa_prefill_params, q_start); F(gsa_prefill_params, n_q);
  F(gsa_prefill_params, scale); F(gsa_prefill_params, dtype);
  return 0;
}
''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                 check=True).stdout.splitlines())
    assert int(got["gsa_decode_params"]) == ctypes.sizeof(gsa.DecodeParams)
    assert int(got["gsa_hier_params"]) == ctypes.sizeof(gsa.HierParams)
    assert int(got["gsa_prefill_params"]) == ctypes.sizeof(gsa.PrefillParams)
    assert int(got["gsa_gist_params"]) == ctypes.sizeof(gsa.GistParams)
    assert int(got["gsa_levels_params"]) == ctypes.sizeof(gsa.LevelsParams)
    assert int(got["gsa_paged_params"]) == ctypes.sizeof(gsa.PagedParams)
    assert int(got["gsa_prefill_varlen_params"]) == ctypes.sizeof(gsa.PrefillVarlenParams)
    assert int(got["GSA_MAX_LEVELS"]) == gsa.MAX_LEVELS
    assert int(got["gsa_append_params"]) == ctypes.sizeof(gsa.AppendParams)
    assert [int(got[f"GSA_GISTS_{n}"]) for n in ("ALL", "SELECTED", "NONE")] == \
        [gsa.GIST_SETS[n] for n in ("all", "selected", "none")]
    for key, val in got.items():
        if "." in key and not key.startswith("GSA_"):
            t, m = key.split(".")
            cls = {"gsa_decode_params": gsa.DecodeParams, "gsa_hier_params": gsa.HierParams,
                   "gsa_prefill_params": gsa.PrefillParams, "gsa_gist_params": gsa.GistParams,
                   "gsa_append_params": gsa.AppendParams, "gsa_levels_params": gsa.LevelsParams,
                   "gsa_paged_params": gsa.PagedParams,
                   "gsa_prefill_varlen_params": gsa.PrefillVarlenParams}[t]
            assert getattr(cls, m).offset == int(val), key


def good_decode(**kw):
    p = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_raw=1024, n_gist=64, chunk=16,
             topk=4, tail=32, scale=0.0, dtype=gsa.GSA_BF16)
    p.update(kw)
    return gsa.DecodeParams(**p)


def ws_size(L, p):
    n = ctypes.c_size_t(0)
    st = L.gsa_decode_workspace_size(ctypes.byref(p), ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,status", [
    ({}, OK),
    ({"batch": 0}, INVALID),
    ({"n_q_heads": 7}, INVALID),              # not a multiple of n_kv_heads
    ({"n_q_heads": 6, "n_kv_heads": 2}, UNSUPPORTED),   # g = 3
    ({"head_dim": 96}, UNSUPPORTED),
    ({"dtype": 7}, INVALID),
    ({"chunk": 0}, INVALID),
    ({"n_raw": 0, "n_gist": 0}, INVALID),
    ({"n_gist": 65}, INVALID),                # more gists than chunks
    ({"n_gist": 62}, INVALID),                # 32 raw tokens after the last gist > C
    ({"n_gist": -1}, INVALID),
    ({"topk": -1}, INVALID),
    ({"topk": 65}, INVALID),                  # k > M
    ({"topk": 64}, OK),                       # k = M allowed
    ({"topk": 0}, OK),
    ({"n_raw": 1030, "tail": 5}, INVALID),    # 6 gist-less raw tokens need tail >= 6
    ({"n_raw": 1030, "tail": 6}, OK),
    ({"tail": 1025}, INVALID),                # tail > n_raw
    ({"scale": float("nan")}, INVALID),
    ({"gist_set": 3}, INVALID),
    ({"gist_set": -1}, INVALID),
    ({"gist_set": 1}, OK),                    # 4 units: several workgroups per unit
    ({"gist_set": 1, "head_dim": 64}, OK),    # the split path (D = 64)
    ({"gist_set": 2, "topk": 65, "n_raw": 16 * 128, "n_gist": 128}, OK),   # k > 64: the split path
    ({"gist_set": 2, "batch": 128}, OK),      # 256 units
    ({"gist_set": 1, "batch": 128, "topk": 0, "tail": 0}, INVALID),   # nothing to attend
    ({"gist_set": 2, "batch": 128, "dtype": gsa.GSA_F32}, OK),        # fp32: the split path
    ({"row_capacity": 1088}, OK),              # exactly N + M
    ({"row_capacity": 4096}, OK),
    ({"row_capacity": 1087}, INVALID),         # below N + M
    ({"row_capacity": -1}, INVALID),
])
def test_decode_param_validation(L, kw, status):
    st, n = ws_size(L, good_decode(**kw))
    assert st == status, L.gsa_last_error()
    if status == OK:
        assert n > 0 and n % 256 == 0


def test_decode_rejects_bad_pointers_and_workspace(L):
    p = good_decode()
    st, need = ws_size(L, p)
    assert st == OK
    args = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, sel=None, ws=FAKE, nws=need)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return L.gsa_decode(ctypes.byref(p), a["q"], a["k"], a["v"], a["out"], a["lse"], a["sel"],
                            a["ws"], a["nws"], None)
    assert call(q=None) == INVALID
    assert call(k=None) == INVALID
    assert call(v=FAKE + 4) == INVALID          # misaligned
    assert call(out=None) == INVALID
    assert call(lse=FAKE + 8) == INVALID
    assert call(ws=None) == WORKSPACE
    assert call(nws=need - 1) == WORKSPACE
    assert call(ws=FAKE + 16) == INVALID        # workspace must be 256-byte aligned
    assert b"aligned" in L.gsa_last_error()


def test_hier_param_validation(L):
    base = good_decode(n_raw=16 * 16 * 10 + 16 * 3, n_gist=16 * 10 + 3, topk=8, tail=64)
    # M = 163, G = 16 -> M2 = 10 groups, 3 orphan gists
    n = ctypes.c_size_t(0)

    def st(fanout, k2, k1=None):
        b = gsa.DecodeParams.from_buffer_copy(base)
        if k1 is not None:
            b.topk = k1
        return L.gsa_decode_hier_workspace_size(ctypes.byref(gsa.HierParams(b, fanout, k2)),
                                                ctypes.byref(n))
    assert st(16, 2) == OK
    assert st(0, 2) == INVALID
    assert st(16, 11) == INVALID                # k2 > M2
    assert st(16, 10) == OK
    assert st(16, 1, 19) == OK                  # 16 children + 3 orphans
    assert st(16, 1, 20) == INVALID             # more than the candidates
    assert st(16, 0, 3) == OK                   # orphans only
    assert st(16, 0, 4) == INVALID


def good_prefill(**kw):
    p = dict(n_q_heads=8, n_kv_heads=2, head_dim=128, chunk=16, topk=4, window=64, n_raw=4096,
             n_gist=256, q_start=3072, n_q=1024, scale=0.0, dtype=gsa.GSA_BF16)
    p.update(kw)
    return gsa.PrefillParams(**p)


@pytest.mark.parametrize("kw,status", [
    ({}, OK),
    ({"head_dim": 64}, UNSUPPORTED),
    ({"dtype": gsa.GSA_F32}, UNSUPPORTED),
    ({"window": 0}, INVALID),
    ({"topk": -1}, INVALID),
    ({"q_start": -1}, INVALID),
    ({"n_q": 1025}, INVALID),                   # runs past n_raw
    ({"n_q": (1 << 63) - 1}, INVALID),          # q_start + n_q would wrap below n_raw
    ({"n_gist": 257}, INVALID),
    ({"n_q_heads": 12, "n_kv_heads": 4}, UNSUPPORTED),
    ({"n_q_heads": 16, "n_kv_heads": 2}, OK),            # g = 8
    ({"n_q_heads": 32, "n_kv_heads": 2}, UNSUPPORTED),   # g = 16
    ({"topk": 32}, OK),
    ({"topk": 33}, OK),                          # longer candidate lists
    ({"topk": 64}, OK),
    ({"topk": 65}, UNSUPPORTED),                  # above the per-block union bound
    ({"n_raw": 16 * 65537, "n_gist": 65537, "q_start": 0, "n_q": 64}, OK),
    ({"n_raw": 16 * 262144, "n_gist": 262144, "q_start": 0, "n_q": 64}, OK),
    ({"n_raw": 16 * 262145, "n_gist": 262145, "q_start": 0, "n_q": 64}, UNSUPPORTED),
    ({"n_q": 0}, OK),
    ({"row_capacity": 4352}, OK),              # exactly N + M
    ({"row_capacity": 8192}, OK),
    ({"row_capacity": 4351}, INVALID),
])
def test_prefill_param_validation(L, kw, status):
    n = ctypes.c_size_t(0)
    assert L.gsa_prefill_workspace_size(ctypes.byref(good_prefill(**kw)), ctypes.byref(n)) == status


def test_prefill_workspace_holds_the_selection(L):
    n = ctypes.c_size_t(0)
    assert L.gsa_prefill_workspace_size(ctypes.byref(good_prefill()), ctypes.byref(n)) == OK
    assert n.value >= 2 * 1024 * 4 * 4                # [Hkv, n_q, k] int32
    assert L.gsa_prefill_workspace_size(ctypes.byref(good_prefill(topk=0)), ctypes.byref(n)) == OK
    assert n.value == 0


def test_profile_events_validation(L):
    arr = (ctypes.c_void_p * 9)(*([ctypes.c_void_p(16)] * 9))
    assert L.gsa_profile_events(arr, -1) == INVALID
    assert L.gsa_profile_events(arr, 9) == INVALID
    assert L.gsa_profile_events(None, 2) == INVALID
    nul = (ctypes.c_void_p * 2)(ctypes.c_void_p(16), None)
    assert L.gsa_profile_events(nul, 2) == INVALID
    assert L.gsa_profile_events(None, 0) == OK     # disarm


def test_profile_marks_validation(L):
    assert L.gsa_profile_marks(None) == INVALID
    n = ctypes.c_int32(-1)
    assert L.gsa_profile_marks(ctypes.byref(n)) == OK
    assert n.value >= 0


def test_status_strings(L):
    for s in range(5):
        assert L.gsa_status_string(s).startswith(b"GSA_")
    assert L.gsa_status_string(99) == b"unknown gsa_status_t"


def test_python_binding_raises_without_gpu_tensors():
    import torch
    with pytest.raises((ValueError, gsa.GsaError)):
        q = torch.zeros(1, 1, 64)
        k = torch.zeros(1, 1, 17, 64)
        gsa.gsa_decode(q, k, k, chunk=16, topk=1, tail=0)


@pytest.mark.parametrize("gist_set", ["all", "selected", "none"])
def test_topk_for_budget_matches_the_oracle(L, gist_set):
    """Host-only budget mode: the library's k equals the oracle's for a grid of
    budgets and shapes; a budget below the k = 0 set is rejected."""
    import oracle
    for M, C, T in [(10, 4, 6), (0, 16, 3), (7, 1, 0), (100, 32, 64)]:
        for budget in list(range(0, 60)) + [M * (C + 1) + T, 10 ** 7]:
            want = oracle.topk_for_budget(budget, M, C, T, gist_set)
            k = ctypes.c_int32(-5)
            st = L.gsa_topk_for_budget(budget, M, C, T, gsa.GIST_SETS[gist_set], ctypes.byref(k))
            if want < 0:
                assert st == INVALID
            else:
                assert st == OK and k.value == want, (M, C, T, budget)
    k = ctypes.c_int32(0)
    assert L.gsa_topk_for_budget(100, 10, 0, 0, 0, ctypes.byref(k)) == INVALID    # chunk < 1
    assert L.gsa_topk_for_budget(100, 10, 4, 0, 3, ctypes.byref(k)) == INVALID    # gist_set
    assert L.gsa_topk_for_budget(100, 10, 4, 0, 0, None) == INVALID
    # the largest chunk with the chosen gists: no 32-bit wrap in tokens per chunk
    assert L.gsa_topk_for_budget(1 << 40, 10, 2**31 - 1, 0, 1, ctypes.byref(k)) == OK and k.value == 10
    assert L.gsa_topk_for_budget(2**31 - 1, 10, 2**31 - 1, 0, 1, ctypes.byref(k)) == OK and k.value == 0


# ------------------------------------------------ gist prefill, cache append ---

def good_gist(**kw):
    p = dict(n_q_heads=8, n_kv_heads=2, head_dim=128, chunk=16, n_raw=1024, n_gist=64, m_start=0,
             n_q=64, scale=0.0, dtype=gsa.GSA_BF16)
    p.update(kw)
    return gsa.GistParams(**p)


@pytest.mark.parametrize("kw,status", [
    ({}, "ok"),
    ({"m_start": -1}, INVALID),
    ({"n_q": -1}, INVALID),
    ({"m_start": 1}, INVALID),                  # chunk 64 does not exist (1024 = 64 chunks)
    ({"n_raw": 1030, "m_start": 1}, INVALID),   # chunk 64 incomplete (6 of 16 tokens)
    ({"n_raw": 1040, "n_gist": 64, "m_start": 1}, "ok"),   # chunk 64 complete, gists 0..63 present
    ({"n_raw": 1040, "n_gist": 64, "m_start": 2}, INVALID),
    ({"n_gist": 62, "n_raw": 1008, "n_q": 63}, "ok"),    # 63 complete chunks, gist 62 is the last needed
    ({"n_gist": 61, "n_raw": 992, "n_q": 62}, "ok"),
    ({"head_dim": 64}, UNSUPPORTED),
    ({"dtype": gsa.GSA_F32}, UNSUPPORTED),
    ({"n_q_heads": 16, "n_kv_heads": 2}, "ok"),             # g = 8
    ({"n_q_heads": 32, "n_kv_heads": 2}, UNSUPPORTED),      # g = 16
    ({"chunk": 0}, INVALID),
    ({"row_capacity": 1000}, INVALID),
    ({"n_q": 0}, OK),                   # nothing to launch: NULL q and out are allowed
    # ranges whose end overflows 64 bits are rejected, not wrapped
    ({"n_raw": 1 << 62, "m_start": 1 << 61, "n_q": 1 << 62}, UNSUPPORTED),
    ({"m_start": (1 << 63) - 1, "n_q": 1}, INVALID),
])
def test_gist_prefill_validation(L, kw, status):
    """Shape errors come back with their status; shapes that pass validation
    fail on the NULL q instead, so nothing launches."""
    st = L.gsa_gist_prefill(ctypes.byref(good_gist(**kw)), None, FAKE, FAKE, FAKE, None)
    msg = L.gsa_last_error().decode()
    if status == "ok":
        assert st == INVALID and msg.startswith("q "), msg
    else:
        assert st == status and not msg.startswith("q "), msg


def good_append(**kw):
    p = dict(batch=2, n_kv_heads=4, head_dim=128, chunk=16, n_raw=32, n_gist=2, raw_new=1,
             gist_new=0, row_capacity=4096, dtype=gsa.GSA_BF16)
    p.update(kw)
    return gsa.AppendParams(**p)


@pytest.mark.parametrize("kw,status", [
    ({"n_raw": 32, "n_gist": 2, "raw_new": 0}, OK),      # empty append: nothing to do
    ({"n_raw": 0, "n_gist": 0, "raw_new": 0}, OK),
    ({"batch": 0}, INVALID),
    ({"head_dim": 96}, UNSUPPORTED),
    ({"dtype": 5}, INVALID),
    ({"chunk": 0}, INVALID),
    ({"raw_new": -1}, INVALID),
    ({"n_raw": 32, "n_gist": 3}, INVALID),       # start state: gist 2 of an incomplete chunk
    ({"n_raw": 32, "n_gist": 2, "gist_new": 1, "raw_new": 0}, INVALID),   # gist 2 before chunk 2
    ({"n_raw": 32, "n_gist": 2, "gist_new": 1, "raw_new": 15}, INVALID),  # chunk 2 one token short
    ({"n_raw": 32, "n_gist": 2, "gist_new": 1, "raw_new": 16}, "ok"),
    ({"n_raw": 48, "n_gist": 1}, "ok"),          # raw rows ahead of the gists: slots wait
    ({"n_raw": 0, "n_gist": 0, "raw_new": 50, "row_capacity": 53}, "ok"),   # raw 49 -> row 3 * 17 + 1
    ({"n_raw": 0, "n_gist": 0, "raw_new": 50, "row_capacity": 52}, INVALID),
    ({"n_raw": 32, "n_gist": 0, "gist_new": 2, "raw_new": 0, "row_capacity": 34}, "ok"),  # gist 1 -> row 33
    ({"n_raw": 32, "n_gist": 0, "gist_new": 2, "raw_new": 0, "row_capacity": 33}, INVALID),
    ({"row_capacity": 35}, "ok"),                # raw 32 -> row 34
    ({"row_capacity": 34}, INVALID),
])
def test_cache_append_validation(L, kw, status):
    p = good_append(**kw)
    st = L.gsa_cache_append(ctypes.byref(p), None, None, None, None, None, None, None)
    msg = L.gsa_last_error().decode()
    if status == "ok":
        assert st == INVALID and msg.startswith("k_cache"), msg   # shape fine, NULL cache
    else:
        assert st == status and not msg.startswith("k_cache"), msg


def test_cache_append_rejects_overlap(L):
    """A source inside a cache, and K and V caches that overlap, are refused
    before any launch."""
    p = good_append()
    cache = 2 * 4 * 4096 * 256
    assert L.gsa_cache_append(ctypes.byref(p), FAKE + 256, FAKE + cache + 4096, None, None, FAKE,
                              FAKE + cache, None) == INVALID
    assert "overlap" in L.gsa_last_error().decode()
    assert L.gsa_cache_append(ctypes.byref(p), FAKE + 3 * cache, FAKE + 4 * cache, None, None, FAKE,
                              FAKE + 256, None) == INVALID
    assert "overlap" in L.gsa_last_error().decode()


# ---------------------------------------------------------------- L levels ---

def good_levels(n_levels=3, fanout=4, topk_up=(6, 4), **kw):
    # M = 640 gists: level sizes 640, 160, 40 (L = 3)
    kw = {"topk": 8, **kw}
    base = good_decode(n_raw=16 * 640, n_gist=640, tail=64, **kw)
    return gsa.levels_params(base, fanout, list(topk_up)[:n_levels - 1]) if n_levels >= 2 else None


def levels_ws(L, p):
    n = ctypes.c_size_t(0)
    return L.gsa_decode_levels_workspace_size(ctypes.byref(p), ctypes.byref(n)), n.value


@pytest.mark.parametrize("make,status", [
    (lambda: good_levels(), OK),
    (lambda: good_levels(n_levels=2, topk_up=(6,)), OK),
    (lambda: good_levels(topk_up=(40, 40)), OK),                 # k_3 = M_3 = 40, k_2 = 160 candidates max
    (lambda: good_levels(topk_up=(6, 41)), INVALID),             # k_3 > M_3
    (lambda: good_levels(topk_up=(25, 6)), INVALID),             # 6 groups of 4 = 24 level-2 candidates
    (lambda: good_levels(topk_up=(24, 6)), OK),
    (lambda: good_levels(topk_up=(1, 6)), INVALID),              # k_1 = 8 > 4 level-1 candidates
    (lambda: good_levels(topk_up=(2, 6)), OK),
    (lambda: good_levels(fanout=1), INVALID),
    (lambda: good_levels(gist_set=2, batch=128), OK),              # the selection rules (unit path)
    (lambda: good_levels(gist_set=1, head_dim=64), OK),            # the split path
    (lambda: good_levels(gist_set=2, head_dim=64, topk=0), OK),    # the tail only
    (lambda: gsa.LevelsParams(good_decode(), 1, 4), INVALID),    # one level
    (lambda: gsa.LevelsParams(good_decode(), 7, 4), INVALID),    # above GSA_MAX_LEVELS
    (lambda: gsa.levels_params(good_decode(n_raw=16 * 4096, n_gist=4096, topk=8, tail=64), 2,
                               [1025]), UNSUPPORTED),            # k_2 above 1024
    (lambda: gsa.levels_params(good_decode(n_raw=16 * 4096, n_gist=4096, topk=8, tail=64), 2,
                               [30, 30, 30, 30, 30]), OK),       # six levels
])
def test_levels_param_validation(L, make, status):
    st, n = levels_ws(L, make())
    assert st == status, L.gsa_last_error()
    if status == OK:
        assert n > 0 and n % 256 == 0


def test_levels_rejects_null_arrays(L):
    p = good_levels()
    st, need = levels_ws(L, p)
    arr = (ctypes.c_void_p * 2)(FAKE, FAKE)
    nul = (ctypes.c_void_p * 2)(FAKE, None)
    call = lambda k, v: L.gsa_decode_levels(ctypes.byref(p), FAKE, FAKE, FAKE, k, v, FAKE, None, None, None,
                                            FAKE, need, None)
    assert call(None, arr) == INVALID
    assert call(arr, nul) == INVALID and "v_up[1]" in L.gsa_last_error().decode()
    assert L.gsa_decode_levels(ctypes.byref(p), FAKE, FAKE, FAKE, arr, arr, FAKE, None, None, None, FAKE,
                               need - 256, None) == WORKSPACE


# ------------------------------------------------------- variable lengths ---

def varlen_params(**kw):
    p = dict(batch=3, n_raw=1024, n_gist=64, topk=2, tail=32)
    p.update(kw)
    return good_decode(**p)


# C = 16, k = 2, tail = 32: 1 <= n <= 1024, 2 <= m <= 64, 16 m <= n <= 16 m + 16, 32 <= n
@pytest.mark.parametrize("n,m,status", [
    ([1024, 500, 40], [64, 31, 2], OK),
    ([1024, 512, 48], [64, 32, 3], OK),
    ([1024, 512, 48], [64, 31, 3], OK),           # 512 - 31*16 = 16: a full chunk without its gist
    ([1024, 512, 48], [64, 33, 3], INVALID),      # gist 32 of an incomplete chunk
    ([1024, 500, 31], [64, 31, 1], INVALID),      # n = 31 below the tail
    ([1024, 500, 40], [64, 31, 3], INVALID),      # 3 gists need 48 raw tokens
    ([1024, 500, 40], [64, 30, 2], INVALID),      # 500 - 30*16 = 20 > C
    ([1025, 500, 40], [64, 31, 2], INVALID),      # above the call's n_raw
    ([1024, 500, 40], [65, 31, 2], INVALID),      # above the call's n_gist
    ([1024, 500, 40], [64, 31, 1], INVALID),      # m = 1 below topk = 2
    ([1024, 500, 36], [64, 31, 2], OK),
])
def test_check_seq_lens(L, n, m, status):
    p = varlen_params()
    arr = lambda v: (ctypes.c_int32 * 3)(*v)
    st = L.gsa_check_seq_lens(ctypes.byref(p), arr(n), arr(m))
    assert st == status, L.gsa_last_error()


def test_decode_varlen_rejections(L):
    p = varlen_params()
    st, need = ws_size(L, p)
    call = lambda pp, sn, sm: L.gsa_decode_varlen(ctypes.byref(pp), sn, sm, FAKE, FAKE, FAKE, FAKE, None, None,
                                                  FAKE, need, None)
    assert call(p, None, FAKE) == INVALID and "seq_n_raw" in L.gsa_last_error().decode()
    assert call(p, FAKE, FAKE + 4) == INVALID                       # misaligned



def hier_varlen_params(**kw):
    """batch 3, N 1024, M 64, C 16, k1 4, G 8, k2 2: M2 = 8, candidates 16."""
    base = varlen_params(topk=kw.pop("topk", 4), **{k: kw.pop(k) for k in list(kw) if k in ("head_dim", "dtype")})
    return gsa.hier_params(base, kw.pop("fanout", 8), kw.pop("topk2", 2))


# the varlen rules, plus topk2 = 2 <= floor(m / 8) and topk = 4 <= 2*8 + m mod 8
@pytest.mark.parametrize("n,m,status", [
    ([1024, 500, 260], [64, 31, 16], OK),
    ([1024, 500, 256], [64, 31, 15], INVALID),     # 15 gists: one level-2 gist < topk2
    ([1024, 500, 40], [64, 31, 2], INVALID),       # no level-2 gist
    ([1024, 1024, 300], [64, 64, 18], OK),         # 2 level-2 gists and 2 orphans
    ([1025, 500, 260], [64, 31, 16], INVALID),     # the varlen rules still hold
])
def test_check_hier_seq_lens(L, n, m, status):
    p = hier_varlen_params()
    arr = lambda v: (ctypes.c_int32 * 3)(*v)
    st = L.gsa_check_hier_seq_lens(ctypes.byref(p), arr(n), arr(m))
    assert st == status, L.gsa_last_error()


def test_decode_hier_varlen_rejections(L):
    p = hier_varlen_params()
    need = ctypes.c_size_t(0)
    assert L.gsa_decode_hier_workspace_size(ctypes.byref(p), ctypes.byref(need)) == OK
    call = lambda pp, sn, sm: L.gsa_decode_hier_varlen(ctypes.byref(pp), sn, sm, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                       FAKE, None, None, None, FAKE, need.value, None)
    assert call(p, None, FAKE) == INVALID and "seq_n_raw" in L.gsa_last_error().decode()
    assert call(p, FAKE, FAKE + 4) == INVALID                       # misaligned
    assert call(hier_varlen_params(dtype=gsa.GSA_F32), FAKE, FAKE) == UNSUPPORTED
    assert call(hier_varlen_params(head_dim=64), FAKE, FAKE) == UNSUPPORTED


@pytest.mark.parametrize("kw,status", [
    ({"gist_set": 1}, OK),
    ({"gist_set": 2}, OK),
    ({"gist_set": 2, "dtype": gsa.GSA_F32}, OK),              # the split path
    ({"gist_set": 1, "head_dim": 64}, OK),
    ({"gist_set": 2, "dtype": gsa.GSA_F32, "topk": 0}, OK),   # the tail only
    ({"gist_set": 3}, INVALID),
    ({"gist_set": 1, "topk": 0, "tail": 0}, INVALID),         # nothing to attend
])
def test_hier_gist_set_validation(L, kw, status):
    p = gsa.HierParams(good_decode(**kw), 4, 2)
    n = ctypes.c_size_t(0)
    assert L.gsa_decode_hier_workspace_size(ctypes.byref(p), ctypes.byref(n)) == status, L.gsa_last_error()


def prefill_varlen_params(batch=3, **kw):
    p = good_prefill(q_start=0, n_q=512, **kw)
    return gsa.PrefillVarlenParams(p, batch)


# N 4096, M 256, C 16, n_q 512: 1 <= n <= 4096, m <= 256, 16 m <= n <= 16 m + 16,
# 0 <= q_start, 0 <= n_q <= 512, q_start + n_q <= n
@pytest.mark.parametrize("rows,status", [
    ([[4096, 256, 3584, 512], [1000, 62, 900, 100], [17, 1, 0, 17]], OK),
    ([[4096, 256, 3584, 512], [1000, 62, 900, 100], [16, 1, 0, 0]], OK),     # no queries
    ([[4096, 256, 3584, 512], [1000, 62, 901, 100], [17, 1, 0, 17]], INVALID),   # runs past n
    ([[4096, 256, 3584, 512], [1000, 63, 900, 100], [17, 1, 0, 17]], INVALID),   # gist of an incomplete chunk
    ([[4096, 256, 3000, 513], [1000, 62, 900, 100], [17, 1, 0, 17]], INVALID),   # more than base.n_q
    ([[4097, 256, 3584, 512], [1000, 62, 900, 100], [17, 1, 0, 17]], INVALID),   # above base.n_raw
    ([[4096, 256, -1, 5], [1000, 62, 900, 100], [17, 1, 0, 17]], INVALID),
])
def test_check_prefill_seqs(L, rows, status):
    p = prefill_varlen_params()
    flat = [x for r in rows for x in r]
    st = L.gsa_check_prefill_seqs(ctypes.byref(p), (ctypes.c_int32 * len(flat))(*flat))
    assert st == status, L.gsa_last_error()


def test_prefill_varlen_validation(L):
    n = ctypes.c_size_t(0)
    assert L.gsa_prefill_varlen_workspace_size(ctypes.byref(prefill_varlen_params()), ctypes.byref(n)) == OK
    assert n.value >= 3 * 2 * 512 * 4 * 4                     # [B, Hkv, n_q, k] int32
    assert L.gsa_prefill_varlen_workspace_size(ctypes.byref(prefill_varlen_params(batch=0)),
                                               ctypes.byref(n)) == INVALID
    bad = gsa.PrefillVarlenParams(good_prefill(q_start=1, n_q=512), 3)
    assert L.gsa_prefill_varlen_workspace_size(ctypes.byref(bad), ctypes.byref(n)) == INVALID
    assert L.gsa_prefill_varlen_workspace_size(ctypes.byref(prefill_varlen_params(head_dim=64)),
                                               ctypes.byref(n)) == UNSUPPORTED
    p = prefill_varlen_params()
    assert L.gsa_prefill_varlen_workspace_size(ctypes.byref(p), ctypes.byref(n)) == OK
    call = lambda seqs: L.gsa_prefill_varlen(ctypes.byref(p), seqs, FAKE, FAKE, FAKE, FAKE, None, FAKE, n.value,
                                             None)
    assert call(None) == INVALID and "seqs" in L.gsa_last_error().decode()
    assert call(FAKE + 4) == INVALID                          # misaligned


# ------------------------------------------- documented sets vs validation ---

def _block(text, start, end):
    i = text.index(start)
    return text[i:text.index(end, i)]


def test_documented_head_and_type_sets_match_validation(L):
    """The g / head_dim / dtype sets the header documents for each entry point
    are exactly the ones host validation accepts (everything else is
    GSA_ERR_UNSUPPORTED), and the header still states those sets."""
    text = open(HEADER).read()
    dec = _block(text, "typedef struct {\n  int32_t batch;", "} gsa_decode_params;")
    assert "g = Hq/Hkv must be 1, 2, 4 or 8" in dec and "D: 64 or 128" in dec
    pre = _block(text, "typedef struct {\n  int32_t n_q_heads;", "} gsa_prefill_params;")
    assert "g = Hq/Hkv in {1, 2, 4, 8}" in pre and "D: 128" in pre and "GSA_BF16 (GSA_F32" in pre
    gis = _block(text, "gsa_status_t gsa_prefill_blocksparse(", "gsa_status_t gsa_gist_prefill(")
    assert "g in {1, 2, 4, 8}" in gis
    n = ctypes.c_size_t(0)
    for g in range(1, 10):
        for D in (32, 64, 96, 128, 256):
            for dt in (gsa.GSA_F32, gsa.GSA_BF16):
                want = OK if g in (1, 2, 4, 8) and D in (64, 128) else UNSUPPORTED
                p = good_decode(n_q_heads=2 * g, n_kv_heads=2, head_dim=D, dtype=dt)
                assert L.gsa_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == want, (g, D, dt)
                h = gsa.HierParams(p, 4, 2)
                assert L.gsa_decode_hier_workspace_size(ctypes.byref(h), ctypes.byref(n)) == want
                lv = gsa.levels_params(p, 4, [2, 1])
                assert L.gsa_decode_levels_workspace_size(ctypes.byref(lv), ctypes.byref(n)) == want
                want_p = OK if g in (1, 2, 4, 8) and D == 128 and dt == gsa.GSA_BF16 else UNSUPPORTED
                pp = good_prefill(n_q_heads=2 * g, n_kv_heads=2, head_dim=D, dtype=dt)
                assert L.gsa_prefill_workspace_size(ctypes.byref(pp), ctypes.byref(n)) == want_p, (g, D, dt)
                gp = gsa.gist_params(2 * g, 2, D, 16, 1024, 64, 0, 8, dtype=dt)
                # validation runs before the NULL-pointer checks: a rejected shape
                # reports its status, an accepted one fails on the NULL q
                st = L.gsa_gist_prefill(ctypes.byref(gp), None, None, None, None, None)
                assert st == (INVALID if want_p == OK else UNSUPPORTED), (g, D, dt)


def test_prefill_documented_limits(L):
    n = ctypes.c_size_t(0)
    for k, want in ((64, OK), (65, UNSUPPORTED)):
        assert L.gsa_prefill_workspace_size(ctypes.byref(good_prefill(topk=k)), ctypes.byref(n)) == want
    big = good_prefill(n_raw=16 * 262145, n_gist=262145, q_start=0, n_q=64)
    assert L.gsa_prefill_workspace_size(ctypes.byref(big), ctypes.byref(n)) == UNSUPPORTED
    ok = good_prefill(n_raw=16 * 262144, n_gist=262144, q_start=0, n_q=64)
    assert L.gsa_prefill_workspace_size(ctypes.byref(ok), ctypes.byref(n)) == OK


def _launches(L, fn, p):
    n = ctypes.c_int32(-1)
    st = getattr(L, fn)(ctypes.byref(p), ctypes.byref(n))
    return st, n.value


def test_launch_counts_follow_the_documented_rules(L):
    """gsa_*_launches against the counts the header documents per path."""
    assert L.gsa_decode_launches(ctypes.byref(good_decode()), None) == INVALID
    # unit path, one workgroup per unit: 256 units, <= 4096 gists
    one = gsa.decode_params(32, 32, 8, 128, 32768, 2048, 16, 16, 64)
    assert _launches(L, "gsa_decode_launches", one) == (OK, 1)
    # unit path, several workgroups per unit: a stream and a select-unfold launch
    few = gsa.decode_params(8, 32, 8, 128, 131072, 4096, 32, 16, 64)
    assert _launches(L, "gsa_decode_launches", few) == (OK, 2)
    few0 = gsa.decode_params(8, 32, 8, 128, 131072, 4096, 32, 0, 64)
    assert _launches(L, "gsa_decode_launches", few0) == (OK, 1)
    many = gsa.decode_params(32, 32, 8, 128, 5000 * 16, 5000, 16, 16, 64)   # > 4096 gists
    assert _launches(L, "gsa_decode_launches", many) == (OK, 2)
    # split path (fp32 / D = 64 / k > 64): 1 with k = 0, else 2 or 3
    for kw in (dict(dtype=gsa.GSA_F32), dict(head_dim=64), dict(topk=80)):
        st, n = _launches(L, "gsa_decode_launches", good_decode(n_raw=4096, n_gist=256, **kw))
        assert st == OK and n in (2, 3), kw
        st, n = _launches(L, "gsa_decode_launches", good_decode(n_raw=4096, n_gist=256, **{**kw, "topk": 0}))
        assert (st, n) == (OK, 1), kw
    # a split path with many gists per unit takes the candidate pass
    st, n = _launches(L, "gsa_decode_launches", gsa.decode_params(1, 4, 1, 128, 1 << 20, 1 << 16, 16, 16, 64,
                                                                  dtype=gsa.GSA_F32))
    assert (st, n) == (OK, 3)
    tiny = gsa.decode_params(1, 1, 1, 64, 4096, 256, 16, 8, 16, dtype=gsa.GSA_F32)
    assert _launches(L, "gsa_decode_launches", tiny) == (OK, 3)   # 4 splits of 64 gists, k = 8
    # two-level
    hb = gsa.decode_params(4, 32, 8, 128, 1 << 20, 1 << 16, 16, 16, 64)
    assert _launches(L, "gsa_decode_hier_launches", gsa.HierParams(hb, 16, 8)) == (OK, 1)
    hf = gsa.decode_params(2, 8, 2, 64, 1 << 16, 1 << 12, 16, 16, 64, dtype=gsa.GSA_F32)
    st, n = _launches(L, "gsa_decode_hier_launches", gsa.HierParams(hf, 16, 8))
    assert st == OK and n in (3, 4)
    hf0 = gsa.decode_params(2, 8, 2, 64, 1 << 16, 1 << 12, 16, 0, 64, dtype=gsa.GSA_F32)
    st, n = _launches(L, "gsa_decode_hier_launches", gsa.HierParams(hf0, 16, 8))
    assert st == OK and n in (2, 3)
    hf0.gist_set = 2   # the selection rules: the set's pass runs with k1 = 0 too
    st, m = _launches(L, "gsa_decode_hier_launches", gsa.HierParams(hf0, 16, 8))
    assert st == OK and m == n + 1
    # L levels
    lb = gsa.decode_params(1, 32, 8, 128, 1 << 21, 1 << 17, 16, 16, 64)
    small_top = gsa.levels_params(lb, 16, [8, 8, 8])      # top level 32 gists
    assert _launches(L, "gsa_decode_levels_launches", small_top) == (OK, 1)
    big_top = gsa.levels_params(lb, 16, [8])              # top level 8192 gists
    assert _launches(L, "gsa_decode_levels_launches", big_top) == (OK, 2)
    lf = gsa.decode_params(1, 4, 1, 64, 1 << 16, 1 << 12, 16, 4, 64, dtype=gsa.GSA_F32)
    assert _launches(L, "gsa_decode_levels_launches", gsa.levels_params(lf, 4, [4, 2])) == (OK, 4)
    lf0 = gsa.decode_params(1, 4, 1, 64, 1 << 16, 1 << 12, 16, 0, 64, dtype=gsa.GSA_F32)
    assert _launches(L, "gsa_decode_levels_launches", gsa.levels_params(lf0, 4, [4, 2])) == (OK, 3)
    # prefill
    assert _launches(L, "gsa_prefill_launches", good_prefill()) == (OK, 2)
    assert _launches(L, "gsa_prefill_launches", good_prefill(topk=0)) == (OK, 1)
    assert _launches(L, "gsa_prefill_launches", good_prefill(n_q=0)) == (OK, 0)
    assert _launches(L, "gsa_prefill_launches", good_prefill(topk=33)) == (OK, 2)
    assert _launches(L, "gsa_prefill_launches", good_prefill(topk=65)) == (UNSUPPORTED, -1)


def test_decode_noalloc_host_rejections(L):
    """gsa_decode_noalloc validates on the host before it touches the device:
    bad shapes, NULL pointers and a workspace beyond the library's scratch."""
    big = gsa.decode_params(32, 32, 8, 128, 131072, 16384, 8, 64, 64)   # 16+ MiB of scores
    assert L.gsa_decode_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, None, None, None) == WORKSPACE
    assert b"scratch" in L.gsa_last_error()
    assert L.gsa_decode_noalloc(ctypes.byref(good_decode(batch=0)), FAKE, FAKE, FAKE, FAKE, None, None,
                                None) == INVALID
    assert L.gsa_decode_noalloc(ctypes.byref(good_decode()), None, FAKE, FAKE, FAKE, None, None,
                                None) == INVALID
    n = ctypes.c_int32(-1)
    assert L.gsa_profile_marks(ctypes.byref(n)) == OK and n.value == 1   # nothing launched


# ---------------------------------------------------------------- paged ---

def good_paged(base_kw=None, **kw):
    b = dict(batch=4, n_q_heads=8, n_kv_heads=2, head_dim=128, n_raw=4096, n_gist=256, chunk=16, topk=8,
             tail=64, scale=0.0, dtype=gsa.GSA_BF16)
    b.update(base_kw or {})
    p = dict(page_chunks=4, max_pages=64, n_pages=300, max_extra=8)
    p.update(kw)
    return gsa.PagedParams(gsa.DecodeParams(**b), **p)


@pytest.mark.parametrize("base_kw,kw,status", [
    ({}, {}, OK),
    ({}, {"page_chunks": 3}, INVALID),                 # not a power of two
    ({}, {"page_chunks": 128}, INVALID),
    ({}, {"max_pages": 63}, INVALID),                  # 4352 rows need 64 pages of 68
    ({}, {"max_pages": 4096}, UNSUPPORTED),
    ({}, {"n_pages": 0}, INVALID),
    ({}, {"max_extra": -1}, INVALID),
    ({}, {"max_extra": 65}, UNSUPPORTED),
    ({"dtype": gsa.GSA_F32}, {}, UNSUPPORTED),         # split path shapes
    ({"head_dim": 64}, {}, UNSUPPORTED),
    ({"topk": 80, "n_raw": 4096 * 4, "n_gist": 1024}, {"max_pages": 256}, UNSUPPORTED),
    ({"row_capacity": 9000}, {}, INVALID),
    ({"gist_set": 1}, {}, OK),                         # the selection rules
    ({"gist_set": 2, "topk": 0, "tail": 0}, {}, INVALID),   # nothing to attend
])
def test_paged_param_validation(L, base_kw, kw, status):
    n = ctypes.c_size_t(0)
    assert L.gsa_decode_paged_workspace_size(ctypes.byref(good_paged(base_kw, **kw)), ctypes.byref(n)) == status


def test_check_pages(L):
    import numpy as np
    p = good_paged()
    B, P, C = 4, 4, 16
    rpp = P * (C + 1)
    n = np.array([4096, 1000, 2048, 200], dtype=np.int32)
    m = np.array([256, 62, 127, 12], dtype=np.int32)
    table = np.full((B, 64), -1, dtype=np.int32)
    for b in range(B):
        need = -(-(int(n[b]) + int(m[b])) // rpp)
        table[b, :need] = np.arange(need) + 70 * b
    extra = np.full((B, 8, 2), -1, dtype=np.int32)
    extra[1, 0] = (299, rpp - 1)
    extra[2, :3] = [(0, 0), (5, 3), (7, 9)]
    def chk(t=table, e=extra, nn=n, mm=m):
        return L.gsa_check_pages(ctypes.byref(p), t.ctypes.data, nn.ctypes.data, mm.ctypes.data, e.ctypes.data)
    assert chk() == OK
    bad = table.copy(); bad[0, 63] = 300                 # outside the pool
    assert chk(t=bad) == INVALID and b"sequence 0" in L.gsa_last_error()
    short = table.copy(); short[3, 0] = -1               # a page the sequence reads
    assert chk(t=short) == INVALID
    past = table.copy(); past[3, 5] = 999                # past the sequence's pages: not read
    assert chk(t=past) == OK
    e2 = extra.copy(); e2[1, 0] = (299, rpp)             # row outside the page
    assert chk(e=e2) == INVALID and b"extra row" in L.gsa_last_error()
    e3 = extra.copy(); e3[2, 1] = (-1, 0); e3[2, 2] = (5000, 0)   # after the list's end: not read
    assert chk(e=e3) == OK
    nn = n.copy(); nn[1] = 5000                          # longer than n_raw
    assert chk(nn=nn) == INVALID
