"""Plain fp64 CPU oracle for Gist Sparse Attention (GSA) decode and prefill.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this file: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` use it. It shares no code, table or helper with
the HIP library; the two meet only through the seeded inputs.

What is computed follows the pages' description of the method, step by step,
in float64 on the exact input values (bf16 inputs are widened exactly):

  * interleaved cache -- the sequence is cut into chunks of C raw tokens and
    one gist token follows every chunk (gist.science explainer "Forget, Then
    Recall", section 2 'Key Concepts: Interleaved Gist Tokens'; Taki-lab
    slide deck, slide 3);
  * routing -- the current query scores every gist key by a dot product
    (same section, 'Gist as Routing Signals'; German gist.science explainer,
    'Methodik', step 2);
  * selection -- the k chunks whose gists score highest are chosen (same
    section, 'Selective Unfolding'; slide deck, slide 10 worked example);
  * unfolding + hybrid attention -- softmax attention over the raw tokens of
    the chosen chunks, their gists and the gists of the chunks not chosen
    (same section, 'Hybrid Attention'), plus the trailing raw tokens that
    have no gist yet or that form the uncompressed suffix (slide deck,
    slide 9, prefix/suffix split);
  * selection-rule variants -- the slide deck's slide 17 ('Selective Rules
    Comparison') compares the set above (all gists + selected raw tokens)
    with the selected chunks' gists + their raw tokens, and with the selected
    raw tokens alone; ``gist_set`` picks one of the three;
  * two-level variant -- meta-gists are scored first, then the gists inside
    the chosen meta-gist groups, then raw chunks are unfolded (gist.science
    explainer, 'Hierarchical Extension (H-GSA)', 'Coarse-to-Fine Selection');
    the same descent over L levels of gists-of-gists (``decode_levels_unit``);
  * prefill -- the same rule applied per query position under causality, i.e.
    the forward pass of the top-k attention mask of selective finetuning
    (gist.science explainer, 'Training Procedure: Selective Finetuning');
  * gist tokens -- the gist token of chunk m attends to its own chunk's raw
    tokens and to the gist tokens before it (the gist causal mask: explainer
    section 2 'Interleaved Gist Tokens'; slide deck, slide 7), and the cache
    grows by one row per token, the gist row following its chunk
    (``cache_row``).

Readings where the pages are silent (each also listed in the design notes):
  R1 score = scale * (q . k_gist), scale = 1/sqrt(D) unless given;
  R2 with grouped-query attention one selection is made per (batch, kv-head):
     the group score is the mean over the group's query heads of the scaled
     per-head scores;
  R3 ties: larger score first, then smaller chunk index; selections are
     reported in ascending chunk order;
  R4 every row enters the attention set once (set union) -- a selected chunk
     that overlaps the tail or window is not counted twice;
  R5 the tail is the last T raw positions; raw rows past the last gist
     (0..C of them) must lie inside the tail;
  R6 prefill eligibility: query t may use gist m only if m < floor(t / C);
     the window is raw positions [t - W + 1, t];
  R7 two-level: level-2 gists live in their own array; group i covers chunks
     [i G, (i + 1) G); the level-1 gists that no full group covers are always
     candidates; the attention set holds every level-2 gist, every candidate
     level-1 gist, the raw rows of the selected chunks and the tail;
  R8 the default attention set keeps every gist (all gists + selected raw +
     tail); R12 the slide 17 variants keep the chosen chunks' gists or none;
  R13 gist causal mask: the listed rows are the chunk's C raw tokens and the
     earlier gists; the gist token's own key is not among them (slide 7
     lists g1 -> x1, x2 and g2 -> g1, x3, x4; its third line, which reads
     g3 -> g1, g2, x5, g3, is taken as g3 -> g1, g2, x5, x6: one garbled
     symbol, where a literal self-key would also break the first two lines'
     pattern and leave chunk 3 without its second raw token);
  R18 paged caches: a sequence's interleaved cache may live in pages of P
     chunk slots (P (C + 1) rows each) taken from a shared pool, in the
     order its block table lists them; the computation is that of the cache
     the pages spell out (``gather_pages``);
  R19 reused documents that end mid-chunk: a document of length M_d C + r_d
     contributes its M_d gisted chunks to the routing and its last r_d raw
     tokens, which no gist summarises, are attended directly like the tail
     (``decode_unit(extra=...)``);
  R15 L levels: level l >= 2 has M_l = floor(M_{l-1} / G) gists in its own
     array, gist i of level l summarising gists [i G, (i + 1) G) of level
     l - 1; top-down, every level's candidates are the children of the
     level above's selection plus that level's ungrouped gists (every gist at
     the top); the set holds every top-level gist, every candidate of the
     levels below, the raw rows of the selected chunks and the tail. L = 2 is
     R7.
  R20 the slide 17 rules under the hierarchy: the rule decides which gists
     join the attention set, the routing is unchanged. "selected" keeps the
     chosen level-1 chunks' gists only (level-2 and candidate gists route
     but are not attended), "none" keeps no gist; both attend the chosen
     chunks' raw rows and the tail as R7 does.

Parity pins for every function here live in tests/test_oracle.py.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "gist_row_index", "raw_row_index", "topk_ascending",
    "decode_unit", "decode", "decode_hier_unit", "decode_hier", "decode_levels_unit", "topk_for_budget", "GIST_SETS",
    "prefill_query", "prefill", "cache_row", "gist_query",
    "page_slot", "gather_pages", "decode_paged_unit",
]


# ---------------------------------------------------------------- layout ---

def gist_row_index(m: int, C: int) -> int:
    """Row of gist g_m: the C raw tokens of chunk m come first, then g_m."""
    return m * (C + 1) + C


def raw_row_index(p: int, C: int, M: int) -> int:
    """Row of raw token at position p (0-based).

    Positions inside the M gisted chunks sit at slot p mod C of chunk p div C;
    the (at most C) positions after the last gisted chunk follow the last gist.
    """
    if p < M * C:
        return (p // C) * (C + 1) + (p % C)
    return M * (C + 1) + (p - M * C)


# ------------------------------------------------------------- selection ---

def topk_ascending(scores: Sequence[float], ids: Sequence[int], k: int) -> List[int]:
    """The k ids with the largest score; ties go to the smaller id (R3).

    Returned in ascending id order. If fewer than k ids exist, all are returned.
    """
    order = sorted(range(len(ids)), key=lambda i: (-float(scores[i]), int(ids[i])))
    chosen = [int(ids[i]) for i in order[:k]]
    return sorted(chosen)


def _group_scores(qg: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """S = mean over the group's heads of scale * (q_h . key)  (R1, R2).

    Written as (scale / g) * sum_h (q_h . key): the same value, with one
    rounding after the head sum, so that equal dot-product sums (exact for
    small-integer inputs) give exactly equal scores and the tie rule decides.
    """
    g = qg.shape[0]
    dots = keys @ qg.T                        # [n, g]
    return (scale / g) * dots.sum(axis=1)


# ------------------------------------------------------------- attention ---

def _softmax_attend(qg: np.ndarray, keys: np.ndarray, vals: np.ndarray,
                    scale: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Exact softmax attention of each query head over the given rows.

    Returns out [g, D], lse [g] (natural log of sum exp of the scaled logits)
    and the sum of the softmax weights [g] (1 up to rounding).
    """
    g, D = qg.shape
    out = np.zeros((g, vals.shape[1] if vals.ndim == 2 else D))
    lse = np.full(g, -np.inf)
    wsum = np.zeros(g)
    if keys.shape[0] == 0:
        out[:] = np.nan
        return out, lse, wsum
    for h in range(g):
        logits = scale * (keys @ qg[h])
        mx = logits.max()
        e = np.exp(logits - mx)
        z = e.sum()
        w = e / z
        out[h] = w @ vals
        lse[h] = mx + math.log(z)
        wsum[h] = w.sum()
    return out, lse, wsum


def _f64(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _check_common(n_raw: int, n_gist: int, C: int, R: int) -> None:
    if C <= 0:
        raise ValueError("chunk must be positive")
    if not (0 <= n_raw - n_gist * C <= C):
        raise ValueError("n_gist must leave 0..C raw tokens after the last gist")
    if R != n_raw + n_gist:
        raise ValueError(f"cache has {R} rows, expected {n_raw + n_gist}")


# ---------------------------------------------------------------- decode ---

GIST_SETS = ("all", "selected", "none")


def topk_for_budget(budget: int, n_gist: int, chunk: int, tail: int, gist_set: str = "all") -> int:
    """Fixed-token-budget mode (slide deck, slide 17: under one token budget,
    leaving out the unselected chunks' gists frees room for more unfolded
    chunks): the largest k <= n_gist whose attention set holds at most
    ``budget`` tokens, counting every kept gist, C raw tokens per selected
    chunk and the T tail tokens with no overlap (k is fixed before the
    selection, so the count is the most the set can hold). -1 if even k = 0
    exceeds the budget."""
    if gist_set not in GIST_SETS:
        raise ValueError(f"gist_set must be one of {GIST_SETS}")
    best = -1
    for k in range(n_gist + 1):
        gists = n_gist if gist_set == "all" else (k if gist_set == "selected" else 0)
        if gists + k * chunk + tail <= budget:
            best = k
    return best


def decode_unit(qg: np.ndarray, K: np.ndarray, V: np.ndarray, *, n_raw: int,
                n_gist: int, chunk: int, topk: int, tail: int,
                scale: Optional[float] = None, gist_set: str = "all",
                extra: Optional[Tuple[np.ndarray, np.ndarray]] = None) -> Dict[str, np.ndarray]:
    """One (batch, kv-head) unit of single-level GSA decode.

    qg: [g, D] query heads sharing this kv-head.  K, V: [R, D] interleaved
    cache of the unit, R = n_raw + n_gist.  gist_set: which gist rows join
    the attention set -- "all" (every gist; the hybrid attention of section 2),
    "selected" (the selected chunks' gists) or "none" (raw tokens only); the
    last two are slide 17's SG+SR and SR-only rules.  extra: (K_x, V_x)
    [x, D] rows outside the cache that join the attention set as they are
    (R19: the ungisted last tokens of reused documents).  Returns out [g, D],
    lse [g], wsum [g], sel [k] (ascending chunk ids), rows (sorted
    attention-set rows of the cache) and scores [M] (group scores of every
    gist).
    """
    qg = _f64(qg)
    g, D = qg.shape
    C, M, N, T = chunk, n_gist, n_raw, tail
    _check_common(N, M, C, K.shape[0])
    if not (0 <= topk <= M):
        raise ValueError("need 0 <= topk <= n_gist")
    if not (N - M * C <= T <= N):
        raise ValueError("tail must cover the raw tokens after the last gist")
    if gist_set not in GIST_SETS:
        raise ValueError(f"gist_set must be one of {GIST_SETS}")
    if gist_set != "all" and topk == 0 and T == 0:
        raise ValueError("the attention set would be empty")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)

    # 1. routing: score every gist
    gist_rows = [gist_row_index(m, C) for m in range(M)]
    S = _group_scores(qg, _f64(K[gist_rows]), scale) if M else np.zeros(0)
    # 2. top-k chunks
    sel = topk_ascending(S, list(range(M)), topk)
    # 3. unfold: attention set = the gists of the rule + raw of selected
    #    chunks + tail
    if gist_set == "all":
        A = set(gist_rows)
    elif gist_set == "selected":
        A = {gist_rows[m] for m in sel}
    else:
        A = set()
    for m in sel:
        for j in range(C):
            A.add(raw_row_index(m * C + j, C, M))
    for p in range(N - T, N):
        A.add(raw_row_index(p, C, M))
    rows = np.array(sorted(A), dtype=np.int64)
    keys, vals = _f64(K[rows]), _f64(V[rows])
    if extra is not None and len(extra[0]):
        keys = np.concatenate([keys, _f64(extra[0])])
        vals = np.concatenate([vals, _f64(extra[1])])
    # 4. hybrid softmax attention
    out, lse, wsum = _softmax_attend(qg, keys, vals, scale)
    return {"out": out, "lse": lse, "wsum": wsum,
            "sel": np.array(sel, dtype=np.int64), "rows": rows, "scores": S}


def _units(B: int, Hkv: int, units: Optional[Iterable[Tuple[int, int]]]):
    if units is None:
        return [(b, j) for b in range(B) for j in range(Hkv)]
    return [(int(b), int(j)) for b, j in units]


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, *, chunk: int,
           topk: int, tail: int, n_gist: Optional[int] = None,
           scale: Optional[float] = None,
           units: Optional[Iterable[Tuple[int, int]]] = None, gist_set: str = "all"):
    """Batched single-level decode. q [B, Hq, D]; caches [B, Hkv, R, D].

    Returns out [B, Hq, D], lse [B, Hq], sel [B, Hkv, k] (units not listed in
    ``units`` are left as NaN / -1).
    """
    B, Hq, D = q.shape
    Hkv, R = k_cache.shape[1], k_cache.shape[2]
    g = Hq // Hkv
    if n_gist is None:
        n_gist = R // (chunk + 1)
    n_raw = R - n_gist
    out = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    sel = np.full((B, Hkv, topk), -1, dtype=np.int64)
    for b, j in _units(B, Hkv, units):
        r = decode_unit(q[b, j * g:(j + 1) * g], k_cache[b, j], v_cache[b, j],
                        n_raw=n_raw, n_gist=n_gist, chunk=chunk, topk=topk, tail=tail,
                        scale=scale, gist_set=gist_set)
        out[b, j * g:(j + 1) * g] = r["out"]
        lse[b, j * g:(j + 1) * g] = r["lse"]
        sel[b, j] = r["sel"]
    return out, lse, sel


# ----------------------------------------------------- two-level decode ---

# ---------------------------------------------------------------- paging ---

def page_slot(r: int, page_chunks: int, chunk: int) -> Tuple[int, int]:
    """(i, s): logical cache row r of a sequence sits at row s of the i-th page
    its block table lists, pages holding page_chunks chunk slots of C + 1
    rows (R18). A chunk (its C raw rows and its gist) never straddles two
    pages."""
    rows_per_page = page_chunks * (chunk + 1)
    return r // rows_per_page, r % rows_per_page


def gather_pages(pool: np.ndarray, pages: Sequence[int], *, page_chunks: int, chunk: int,
                 n_rows: int) -> np.ndarray:
    """Rows 0 .. n_rows - 1 of a sequence's interleaved cache (one kv-head),
    read page by page: pool [n_pages, P (C + 1), D] holds that kv-head's rows
    of every page, pages the sequence's block table."""
    out = []
    for r in range(n_rows):
        i, s = page_slot(r, page_chunks, chunk)
        out.append(pool[pages[i], s])
    return np.stack(out) if out else np.zeros((0, pool.shape[-1]))


def decode_paged_unit(qg: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, pages: Sequence[int], *,
                      page_chunks: int, n_raw: int, n_gist: int, chunk: int, topk: int, tail: int,
                      extra_rows: Sequence[Tuple[int, int]] = (), scale: Optional[float] = None,
                      gist_set: str = "all"):
    """One (sequence, kv-head) unit of decode over a paged cache (R18): the
    cache the pages spell out, plus the rows extra_rows lists as (page, row in
    page) attended directly (R19), under the selection rule gist_set (R12).
    k_pool, v_pool: [n_pages, P (C + 1), D] of this kv-head."""
    R = n_raw + n_gist
    K = gather_pages(k_pool, pages, page_chunks=page_chunks, chunk=chunk, n_rows=R)
    V = gather_pages(v_pool, pages, page_chunks=page_chunks, chunk=chunk, n_rows=R)
    xk = np.stack([k_pool[pg, r] for pg, r in extra_rows]) if len(extra_rows) else np.zeros((0, K.shape[1]))
    xv = np.stack([v_pool[pg, r] for pg, r in extra_rows]) if len(extra_rows) else np.zeros((0, K.shape[1]))
    return decode_unit(qg, K, V, n_raw=n_raw, n_gist=n_gist, chunk=chunk, topk=topk, tail=tail, scale=scale,
                       extra=(xk, xv), gist_set=gist_set)


def decode_hier_unit(qg: np.ndarray, K: np.ndarray, V: np.ndarray, K2: np.ndarray,
                     V2: np.ndarray, *, n_raw: int, n_gist: int, chunk: int,
                     fanout: int, topk1: int, topk2: int, tail: int,
                     scale: Optional[float] = None, gist_set: str = "all") -> Dict[str, np.ndarray]:
    """One unit of two-level (gist-of-gist) decode (R7; gist_set: R20).

    K2, V2: [M2, D] level-2 gists, M2 = floor(M / G).
    Returns out, lse, wsum, sel2 [k2], sel1 [k1] (ascending), cand1 (sorted
    candidate chunk ids), rows (level-1 cache rows attended).
    """
    qg = _f64(qg)
    g, D = qg.shape
    C, M, N, T, G = chunk, n_gist, n_raw, tail, fanout
    _check_common(N, M, C, K.shape[0])
    if G <= 0:
        raise ValueError("fanout must be positive")
    M2 = M // G
    if K2.shape[0] != M2:
        raise ValueError(f"level-2 array has {K2.shape[0]} rows, expected {M2}")
    if not (0 <= topk2 <= M2):
        raise ValueError("need 0 <= topk2 <= M2")
    if not (0 <= topk1 <= topk2 * G + (M - M2 * G)):
        raise ValueError("topk1 exceeds the number of level-1 candidates")
    if not (N - M * C <= T <= N):
        raise ValueError("tail must cover the raw tokens after the last gist")
    if gist_set not in GIST_SETS:
        raise ValueError(f"gist_set must be one of {GIST_SETS}")
    if gist_set != "all" and topk1 == 0 and T == 0:
        raise ValueError("the attention set would be empty")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)

    # level 2: score the meta-gists, keep the top-k2 groups
    S2 = _group_scores(qg, _f64(K2), scale) if M2 else np.zeros(0)
    sel2 = topk_ascending(S2, list(range(M2)), topk2)
    # level 1 candidates: children of the chosen groups + ungrouped gists
    cand = sorted({i * G + c for i in sel2 for c in range(G)} | set(range(M2 * G, M)))
    cand_rows = [gist_row_index(m, C) for m in cand]
    S1 = _group_scores(qg, _f64(K[cand_rows]), scale) if cand else np.zeros(0)
    sel1 = topk_ascending(S1, cand, topk1)
    # attention set: the gists of the rule (all: every level-2 gist and every
    # candidate gist; selected: the chosen chunks' gists; none) + unfolded +
    # tail
    if gist_set == "all":
        A = set(cand_rows)
    elif gist_set == "selected":
        A = {gist_row_index(m, C) for m in sel1}
    else:
        A = set()
    for m in sel1:
        for j in range(C):
            A.add(raw_row_index(m * C + j, C, M))
    for p in range(N - T, N):
        A.add(raw_row_index(p, C, M))
    rows = np.array(sorted(A), dtype=np.int64)
    n2 = M2 if gist_set == "all" else 0
    keys = np.concatenate([_f64(K2[:n2]), _f64(K[rows])], axis=0)
    vals = np.concatenate([_f64(V2[:n2]), _f64(V[rows])], axis=0)
    out, lse, wsum = _softmax_attend(qg, keys, vals, scale)
    return {"out": out, "lse": lse, "wsum": wsum,
            "sel2": np.array(sel2, dtype=np.int64), "sel1": np.array(sel1, dtype=np.int64),
            "cand1": np.array(cand, dtype=np.int64), "rows": rows}


def decode_hier(q, k_cache, v_cache, k_l2, v_l2, *, chunk: int, fanout: int, topk1: int,
                topk2: int, tail: int, n_gist: Optional[int] = None,
                scale: Optional[float] = None, units=None):
    """Batched two-level decode. Returns out, lse, sel2 [B,Hkv,k2], sel1 [B,Hkv,k1]."""
    B, Hq, D = q.shape
    Hkv, R = k_cache.shape[1], k_cache.shape[2]
    g = Hq // Hkv
    if n_gist is None:
        n_gist = R // (chunk + 1)
    n_raw = R - n_gist
    out = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    sel2 = np.full((B, Hkv, topk2), -1, dtype=np.int64)
    sel1 = np.full((B, Hkv, topk1), -1, dtype=np.int64)
    for b, j in _units(B, Hkv, units):
        r = decode_hier_unit(q[b, j * g:(j + 1) * g], k_cache[b, j], v_cache[b, j],
                             k_l2[b, j], v_l2[b, j], n_raw=n_raw, n_gist=n_gist,
                             chunk=chunk, fanout=fanout, topk1=topk1, topk2=topk2,
                             tail=tail, scale=scale)
        out[b, j * g:(j + 1) * g] = r["out"]
        lse[b, j * g:(j + 1) * g] = r["lse"]
        sel2[b, j] = r["sel2"]
        sel1[b, j, :len(r["sel1"])] = r["sel1"]
    return out, lse, sel2, sel1


def decode_levels_unit(qg: np.ndarray, K: np.ndarray, V: np.ndarray, upper, *, n_raw: int,
                       n_gist: int, chunk: int, fanout: int, topks, tail: int,
                       scale: Optional[float] = None, gist_set: str = "all") -> Dict[str, object]:
    """One unit of L-level decode (R15; explainer 'Hierarchical Extension
    (H-GSA)' and 'Coarse-to-Fine Selection', slide 11; gist_set: R20).

    upper: [(K_2, V_2), ..., (K_L, V_L)], K_l: [M_l, D] with
    M_l = floor(M_{l-1} / G), M_1 = n_gist.  topks: [k_1, ..., k_L], k_1 the
    chunks unfolded.  Returns out, lse, wsum, sels [sel_1 .. sel_L]
    (ascending ids), cands [cand_1 .. cand_L] (sorted candidate ids of every
    level; all ids at the top) and rows (level-1 cache rows attended).
    """
    qg = _f64(qg)
    g, D = qg.shape
    C, M, N, T, G = chunk, n_gist, n_raw, tail, fanout
    _check_common(N, M, C, K.shape[0])
    L = len(upper) + 1
    if G <= 0 or L < 2 or len(topks) != L:
        raise ValueError("need fanout > 0, at least two levels and one k per level")
    sizes = [M]
    for l in range(2, L + 1):
        sizes.append(sizes[-1] // G)
        if upper[l - 2][0].shape[0] != sizes[-1]:
            raise ValueError(f"level {l} array has {upper[l - 2][0].shape[0]} rows, expected {sizes[-1]}")
    if not (N - M * C <= T <= N):
        raise ValueError("tail must cover the raw tokens after the last gist")
    if gist_set not in GIST_SETS:
        raise ValueError(f"gist_set must be one of {GIST_SETS}")
    if gist_set != "all" and topks[0] == 0 and T == 0:
        raise ValueError("the attention set would be empty")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)

    def keys_of(l, ids):           # key rows of gists `ids` at level l (1-based)
        if l == 1:
            return _f64(K[[gist_row_index(m, C) for m in ids]])
        return _f64(upper[l - 2][0][list(ids)])

    sels, cands = [None] * (L + 1), [None] * (L + 1)
    cands[L] = list(range(sizes[L - 1]))
    for l in range(L, 0, -1):
        if l < L:
            above = sels[l + 1]
            grouped = sizes[l] * G
            cands[l] = sorted({i * G + c for i in above for c in range(G)} | set(range(grouped, sizes[l - 1])))
        k = topks[l - 1]
        if not (0 <= k <= len(cands[l])):
            raise ValueError(f"k at level {l} exceeds its {len(cands[l])} candidates")
        S = _group_scores(qg, keys_of(l, cands[l]), scale) if cands[l] else np.zeros(0)
        sels[l] = topk_ascending(S, cands[l], k)
    # attention set: the gists of the rule (all: the top level and every
    # lower level's candidates; selected: the chosen chunks' gists; none),
    # the raw rows of the chosen chunks and the tail (rows of the level-1
    # cache)
    if gist_set == "all":
        A = {gist_row_index(m, C) for m in cands[1]}
    elif gist_set == "selected":
        A = {gist_row_index(m, C) for m in sels[1]}
    else:
        A = set()
    for m in sels[1]:
        for j in range(C):
            A.add(raw_row_index(m * C + j, C, M))
    for p in range(N - T, N):
        A.add(raw_row_index(p, C, M))
    rows = np.array(sorted(A), dtype=np.int64)
    up = range(L, 1, -1) if gist_set == "all" else []
    keys = [_f64(upper[l - 2][0][cands[l]]) for l in up] + [_f64(K[rows])]
    vals = [_f64(upper[l - 2][1][cands[l]]) for l in up] + [_f64(V[rows])]
    out, lse, wsum = _softmax_attend(qg, np.concatenate(keys), np.concatenate(vals), scale)
    return {"out": out, "lse": lse, "wsum": wsum,
            "sels": [np.array(sels[l], dtype=np.int64) for l in range(1, L + 1)],
            "cands": [np.array(cands[l], dtype=np.int64) for l in range(1, L + 1)], "rows": rows}


# --------------------------------------------------------------- prefill ---

def prefill_query(qg_t: np.ndarray, K: np.ndarray, V: np.ndarray, *, t: int, n_raw: int,
                  n_gist: int, chunk: int, topk: int, window: int,
                  scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Causal block-sparse prefill for one query position t and one kv-head (R6).

    qg_t: [g, D] the group's query heads at position t.  K, V: [R, D].
    Returns out [g, D], lse [g], wsum [g], sel [k] (ascending, -1 padded),
    rows (sorted attention-set rows).
    """
    qg = _f64(qg_t)
    g, D = qg.shape
    C, M, N, W = chunk, n_gist, n_raw, window
    _check_common(N, M, C, K.shape[0])
    if not (0 <= t < N):
        raise ValueError("query position outside the sequence")
    if topk < 0 or W < 1:
        raise ValueError("need topk >= 0 and window >= 1")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)

    # gists of chunks complete before t (their gist row precedes t's row)
    elig = list(range(min(M, t // C)))
    erows = [gist_row_index(m, C) for m in elig]
    S = _group_scores(qg, _f64(K[erows]), scale) if elig else np.zeros(0)
    sel = topk_ascending(S, elig, topk)
    A = set(erows)
    for m in sel:
        for j in range(C):
            A.add(raw_row_index(m * C + j, C, M))
    for p in range(max(0, t - W + 1), t + 1):
        A.add(raw_row_index(p, C, M))
    rows = np.array(sorted(A), dtype=np.int64)
    out, lse, wsum = _softmax_attend(qg, _f64(K[rows]), _f64(V[rows]), scale)
    padded = np.full(topk, -1, dtype=np.int64)
    padded[:len(sel)] = sel
    return {"out": out, "lse": lse, "wsum": wsum, "sel": padded, "rows": rows}


def prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, *, chunk: int,
            topk: int, window: int, q_start: int, n_gist: Optional[int] = None,
            scale: Optional[float] = None,
            queries: Optional[Iterable[Tuple[int, int]]] = None):
    """Prefill for query positions q_start + i, i < n_q, of one sequence.

    q: [Hq, n_q, D]; caches [Hkv, R, D]. ``queries`` lists (i, kv_head) pairs
    to compute (default: all). Returns out [Hq, n_q, D], sel [Hkv, n_q, k].
    """
    Hq, n_q, D = q.shape
    Hkv, R = k_cache.shape[0], k_cache.shape[1]
    g = Hq // Hkv
    if n_gist is None:
        n_gist = R // (chunk + 1)
    n_raw = R - n_gist
    out = np.full((Hq, n_q, D), np.nan)
    sel = np.full((Hkv, n_q, topk), -1, dtype=np.int64)
    todo = ([(i, j) for j in range(Hkv) for i in range(n_q)] if queries is None
            else [(int(i), int(j)) for i, j in queries])
    for i, j in todo:
        r = prefill_query(q[j * g:(j + 1) * g, i], k_cache[j], v_cache[j], t=q_start + i,
                          n_raw=n_raw, n_gist=n_gist, chunk=chunk, topk=topk,
                          window=window, scale=scale)
        out[j * g:(j + 1) * g, i] = r["out"]
        sel[j, i] = r["sel"]
    return out, sel


# ------------------------------------------------ gist tokens, cache rows ---

def cache_row(position: int, chunk: int, is_gist: bool) -> int:
    """Row written when the cache grows by one token (explainer section 2
    'Interleaved Gist Tokens': a gist token follows every chunk): raw token
    ``position`` goes to its chunk's slot, the gist of chunk ``position`` to
    the slot after the chunk's C raw tokens."""
    if position < 0 or chunk <= 0:
        raise ValueError("need position >= 0 and chunk >= 1")
    if is_gist:
        return gist_row_index(position, chunk)
    m, j = divmod(position, chunk)
    return m * (chunk + 1) + j


def gist_query(qg: np.ndarray, K: np.ndarray, V: np.ndarray, *, m: int, n_raw: int,
               n_gist: int, chunk: int, scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Attention of chunk m's gist token under the gist causal mask (R13): its
    own chunk's C raw tokens and the gists of chunks 0..m-1.

    qg: [g, D] the gist token's query heads of one kv-group.  K, V: [R, D].
    Needs chunk m complete ((m + 1) C <= n_raw) and the gists before it in
    the cache (m <= n_gist).  Returns out [g, D], lse [g], wsum [g], rows.
    """
    qg = _f64(qg)
    g, D = qg.shape
    C, M, N = chunk, n_gist, n_raw
    _check_common(N, M, C, K.shape[0])
    if not (0 <= m and (m + 1) * C <= N and m <= M):
        raise ValueError("chunk m must be complete and the gists before it present")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rows = [raw_row_index(m * C + j, C, M) for j in range(C)]
    rows += [gist_row_index(mm, C) for mm in range(m)]
    rows = np.array(sorted(rows), dtype=np.int64)
    out, lse, wsum = _softmax_attend(qg, _f64(K[rows]), _f64(V[rows]), scale)
    return {"out": out, "lse": lse, "wsum": wsum, "rows": rows}

