// Host-side validation and planning for libgsa (no HIP calls in this file).
#include "gsa_plan.hpp"

#include <algorithm>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

namespace gsa {

namespace {
thread_local char g_last_error[512] = "";

int32_t clamp_i(int64_t v, int64_t lo, int64_t hi) {
  return (int32_t)(v < lo ? lo : (v > hi ? hi : v));
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workgroups per unit for a streaming pass over `rows` rows: enough to put
// about kTargetWGs workgroups on the chip, but never fewer than kMinRows rows
// per workgroup.
constexpr int64_t kTargetWGs = 2048;
constexpr int64_t kMinRows = 64;

// Unfold workgroups get at least this many rows: few rows each keep the
// latency of the pass short (it starts only after the selection).
constexpr int64_t kMinUnfoldRows = 64;
// A gist workgroup gathers its scores in LDS: at most this many items each.
constexpr int64_t kMaxTaskItems = 1024;

// Workgroups per unit of the one-workgroup-per-unit path, 0 if it does not
// apply: bf16, D = 128, k <= kFastSelect, rows addressable in 31 bits; one
// workgroup per unit when there are enough units, else enough splits to fill
// the chip; every split's gists fit its LDS and the selection's scores fit
// kUnitMaxSel.
static int32_t unit_splits(const DecodePlan& d) {
  if (d.dtype != GSA_BF16 || d.D != 128 || d.k > kFastSelect) return 0;
  if (d.R >= ((int64_t)1 << 31) || (int64_t)d.k * d.C + d.M + d.T >= ((int64_t)1 << 31)) return 0;
  if (d.k > 0 && d.M > kUnitMaxSel) return 0;
  const int64_t items = d.M + d.T;
  if (d.units >= kUnitMinWGs && d.M <= kUnitMaxGist) return 1;
  int64_t s = ceil_div(kUnitMinWGs, d.units);
  const int64_t need = ceil_div(items, kUnitWgItems);   // gists + tail per split <= LDS scores
  if (s < need) s = need;
  if (s > kUnitMaxSplits) return 0;
  if (ceil_div(items, s) < 64) s = ceil_div(items, 64);
  return (int32_t)(s < 2 ? 2 : s);
}

int32_t splits_for(int64_t rows, int64_t units, int64_t min_rows = kMinRows) {
  if (rows <= 0) return 1;
  int64_t want = ceil_div(kTargetWGs, units);
  int64_t cap = ceil_div(rows, min_rows);
  return clamp_i(want < cap ? want : cap, 1, 1 << 16);
}

bool g_supported(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8; }
}  // namespace

gsa_status_t fail(gsa_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_last_error[0] = '\0'; }

const char* last_error_message() { return g_last_error; }

gsa_status_t check_ptr(const void* p, const char* name, bool allow_null) {
  if (!p) return allow_null ? GSA_OK : fail(GSA_ERR_INVALID_ARG, "%s is NULL", name);
  if (((uintptr_t)p) % 16 != 0) return fail(GSA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return GSA_OK;
}

gsa_status_t check_workspace(const void* ws, size_t have, size_t need) {
  if (need == 0) return GSA_OK;
  if (!ws) return fail(GSA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  if (have < need)
    return fail(GSA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  if (((uintptr_t)ws) % kAlign != 0)
    return fail(GSA_ERR_INVALID_ARG, "workspace is not %zu-byte aligned", kAlign);
  return GSA_OK;
}

static gsa_status_t check_geometry(int64_t n_raw, int64_t n_gist, int32_t chunk) {
  if (chunk < 1 || chunk > 4096) return fail(GSA_ERR_INVALID_ARG, "chunk=%d outside [1, 4096]", chunk);
  if (n_raw < 1) return fail(GSA_ERR_INVALID_ARG, "n_raw=%lld must be >= 1", (long long)n_raw);
  if (n_gist < 0) return fail(GSA_ERR_INVALID_ARG, "n_gist=%lld is negative", (long long)n_gist);
  if (n_gist > n_raw / chunk)
    return fail(GSA_ERR_INVALID_ARG, "n_gist=%lld exceeds n_raw/chunk", (long long)n_gist);
  int64_t r = n_raw - n_gist * (int64_t)chunk;
  if (r > chunk)
    return fail(GSA_ERR_INVALID_ARG, "%lld raw tokens follow the last gist (at most chunk=%d)",
                (long long)r, chunk);
  if (n_raw > ((int64_t)1 << 40)) return fail(GSA_ERR_UNSUPPORTED, "n_raw too large");
  return GSA_OK;
}

static gsa_status_t check_heads(int32_t hq, int32_t hkv, int32_t d, int32_t dtype) {
  if (hq < 1 || hkv < 1) return fail(GSA_ERR_INVALID_ARG, "head counts must be >= 1");
  if (hq % hkv != 0)
    return fail(GSA_ERR_INVALID_ARG, "n_q_heads=%d is not a multiple of n_kv_heads=%d", hq, hkv);
  if (!g_supported(hq / hkv))
    return fail(GSA_ERR_UNSUPPORTED, "query heads per kv-head %d not in {1,2,4,8}", hq / hkv);
  if (dtype != GSA_F32 && dtype != GSA_BF16) return fail(GSA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (d != 64 && d != 128) return fail(GSA_ERR_UNSUPPORTED, "head_dim=%d not in {64,128}", d);
  return GSA_OK;
}

// Stride in rows between the [rows, D] cache blocks of consecutive
// (sequence, kv-head) pairs: the rows in use, or the caller's capacity.
static gsa_status_t resolve_rows(int64_t rows, int64_t capacity, int64_t* R) {
  if (capacity < 0 || (capacity > 0 && capacity < rows))
    return fail(GSA_ERR_INVALID_ARG, "row_capacity=%lld below the %lld rows of the cache", (long long)capacity,
                (long long)rows);
  if (capacity > ((int64_t)1 << 41)) return fail(GSA_ERR_UNSUPPORTED, "row_capacity too large");
  *R = capacity > 0 ? capacity : rows;
  return GSA_OK;
}

static float resolve_scale(float s, int32_t d) {
  return (s > 0.f && isfinite(s)) ? s : 1.0f / sqrtf((float)d);
}

gsa_status_t plan_decode(const gsa_decode_params* p, DecodePlan* o) {
  if (!p || !o) return fail(GSA_ERR_INVALID_ARG, "params is NULL");
  if (p->batch < 1) return fail(GSA_ERR_INVALID_ARG, "batch=%d must be >= 1", p->batch);
  gsa_status_t s = check_heads(p->n_q_heads, p->n_kv_heads, p->head_dim, p->dtype);
  if (s != GSA_OK) return s;
  if ((s = check_geometry(p->n_raw, p->n_gist, p->chunk)) != GSA_OK) return s;
  if (isnan(p->scale)) return fail(GSA_ERR_INVALID_ARG, "scale is NaN");
  if (p->topk < 0 || p->topk > p->n_gist)
    return fail(GSA_ERR_INVALID_ARG, "topk=%d outside [0, n_gist=%lld]", p->topk, (long long)p->n_gist);
  int64_t r = p->n_raw - p->n_gist * (int64_t)p->chunk;
  if (p->tail < r || p->tail > p->n_raw)
    return fail(GSA_ERR_INVALID_ARG, "tail=%d outside [%lld, n_raw=%lld]", p->tail, (long long)r,
                (long long)p->n_raw);
  int64_t units = (int64_t)p->batch * p->n_kv_heads;
  if (units > (1 << 24)) return fail(GSA_ERR_UNSUPPORTED, "too many (batch, kv-head) units");
  int64_t items = (int64_t)p->topk * p->chunk;
  if (items > (1 << 30) || p->n_gist > (1 << 30))
    return fail(GSA_ERR_UNSUPPORTED, "selection too large");

  DecodePlan d{};
  d.units = (int32_t)units;
  d.Hkv = p->n_kv_heads;
  d.g = p->n_q_heads / p->n_kv_heads;
  d.D = p->head_dim;
  d.M = p->n_gist;
  d.N = p->n_raw;
  if ((s = resolve_rows(cache_rows(p->n_raw, p->n_gist), p->row_capacity, &d.R)) != GSA_OK) return s;
  d.C = p->chunk;
  d.k = p->topk;
  d.T = p->tail;
  d.scale = resolve_scale(p->scale, p->head_dim);
  d.dtype = p->dtype;
  if (p->gist_set < GSA_GISTS_ALL || p->gist_set > GSA_GISTS_NONE)
    return fail(GSA_ERR_INVALID_ARG, "gist_set=%d not in {0, 1, 2}", p->gist_set);
  if (p->gist_set != GSA_GISTS_ALL && p->topk == 0 && p->tail == 0)
    return fail(GSA_ERR_INVALID_ARG, "gist_set=%d with topk = 0 and tail = 0 leaves nothing to attend",
                p->gist_set);
  d.gist_set = p->gist_set;
  d.S = splits_for(d.M, units);
  if (ceil_div(d.M, d.S) > kMaxTaskItems) d.S = (int32_t)ceil_div(d.M, kMaxTaskItems);
  d.gists_per_split = d.M > 0 ? ceil_div(d.M, d.S) : 0;
  d.S = d.M > 0 ? (int32_t)ceil_div(d.M, d.gists_per_split) : 1;
  d.tail_per_split = (int32_t)ceil_div(d.T, d.S);
  d.n_items = (int32_t)items;
  d.S2 = splits_for(items, units, kMinUnfoldRows);
  d.items_per_split = items > 0 ? (int32_t)ceil_div(items, d.S2) : 0;
  d.S2 = items > 0 ? (int32_t)ceil_div(items, d.items_per_split) : 0;
  d.NP = d.S + d.S2;
  d.score_stride = d.k > 0 ? (d.M + 63) / 64 * 64 : 0;
  d.unit_S = unit_splits(d);
  if (d.gist_set != GSA_GISTS_ALL && d.unit_S == 0) {
    // split path, selection-rule variants: the gist pass only scores; the
    // unfold pass attends the whole set (chosen raw rows, the chosen gists
    // with rule 1, the tail) and merges its own partial states alone
    const int64_t set_items = items + (d.gist_set == GSA_GISTS_SELECTED ? d.k : 0) + d.T;
    if (set_items > (1 << 30)) return fail(GSA_ERR_UNSUPPORTED, "selection too large");
    d.n_items = (int32_t)set_items;
    d.S2 = splits_for(set_items, units, kMinUnfoldRows);
    d.items_per_split = (int32_t)ceil_div(set_items, d.S2);
    d.S2 = (int32_t)ceil_div(set_items, d.items_per_split);
    d.NP = d.S + d.S2;
  }
  d.unit_S2 = 0;
  if (d.unit_S > 1) {
    // the unfold launch: the stream's workgroup count, at least 64 rows each
    // (selection-rule variants: its items are the whole set)
    const int64_t set_items = d.gist_set == GSA_GISTS_ALL
                                  ? items
                                  : items + (d.gist_set == GSA_GISTS_SELECTED ? d.k : 0) + d.T;
    d.unit_S2 = set_items > 0 && (d.k > 0 || d.gist_set != GSA_GISTS_ALL)
                    ? (int32_t)std::max<int64_t>(1, std::min<int64_t>(d.unit_S, ceil_div(set_items, 64)))
                    : 0;
    if (d.NP < d.unit_S + d.unit_S2) d.NP = d.unit_S + d.unit_S2;   // stream + unfold partials
  }
  size_t off = 0;
  d.off_ctrl = off;
  off = align_up(off + ctrl_bytes(units));
  d.off_scores = off;
  off = align_up(off + sizeof(float) * (size_t)units * (size_t)d.score_stride);
  d.off_sel = off;
  d.sel_stride = line_pad(d.k > 0 ? d.k : 1);
  off = align_up(off + sizeof(int32_t) * (size_t)units * (size_t)d.sel_stride);
  d.off_part = off;
  off = align_up(off + sizeof(float) * (size_t)units * d.NP * (size_t)part_stride(d.g, d.D));
  d.cand_stride = 0;
  if (d.unit_S > 1 && d.k > 0 && d.k <= kUnitCandMaxK) {
    // each stream workgroup's top-k, selected among by the unfold launch: the
    // scores, then the ids, directly after the partial states (the kernels
    // derive the place from the partial region)
    d.cand_stride = line_pad((int64_t)d.unit_S * cand_cap(d.unit_S, d.k));
    d.off_cand = d.off_part + sizeof(float) * (size_t)units * d.NP * (size_t)part_stride(d.g, d.D);
    d.off_cand_ids = d.off_cand + sizeof(float) * (size_t)units * (size_t)d.cand_stride;
    off = align_up(d.off_cand_ids + sizeof(int32_t) * (size_t)units * (size_t)d.cand_stride);
  } else if (d.unit_S == 0 && d.k > 0 && d.k <= kFastSelect && d.S >= 4 && (int64_t)d.S * d.k * 2 <= d.M) {
    d.cand_stride = line_pad((int64_t)d.S * d.k);
    d.off_cand = off;
    off = align_up(off + sizeof(float) * (size_t)units * (size_t)d.cand_stride);
    d.off_cand_ids = off;
    off = align_up(off + sizeof(int32_t) * (size_t)units * (size_t)d.cand_stride);
  }
  d.total = off;
  *o = d;
  return GSA_OK;
}

gsa_status_t plan_paged(const gsa_paged_params* p, DecodePlan* o) {
  if (!p || !o) return fail(GSA_ERR_INVALID_ARG, "params is NULL");
  if (p->base.row_capacity != 0)
    return fail(GSA_ERR_INVALID_ARG, "paged decode: base.row_capacity must be 0 (pages hold the rows)");
  gsa_status_t s = plan_decode(&p->base, o);
  if (s != GSA_OK) return s;
  const int32_t P = p->page_chunks;
  if (P < 1 || P > 64 || (P & (P - 1)) != 0)
    return fail(GSA_ERR_INVALID_ARG, "page_chunks=%d must be a power of two in [1, 64]", P);
  const int64_t rpp = (int64_t)P * (p->base.chunk + 1);
  const int64_t need = (o->N + o->M + rpp - 1) / rpp;   // pages of the longest sequence
  if (p->max_pages < need || p->max_pages < 1)
    return fail(GSA_ERR_INVALID_ARG, "max_pages=%d below the %lld pages of n_raw + n_gist rows", p->max_pages,
                (long long)need);
  if (p->max_pages > kPagedMaxPages)
    return fail(GSA_ERR_UNSUPPORTED, "max_pages=%d above %d", p->max_pages, kPagedMaxPages);
  if (p->n_pages < 1 || p->n_pages > ((int64_t)1 << 31) - 1)
    return fail(GSA_ERR_INVALID_ARG, "n_pages=%lld must be in [1, 2^31)", (long long)p->n_pages);
  if (p->max_extra < 0 || p->max_extra > kPagedMaxExtra)
    return fail(p->max_extra < 0 ? GSA_ERR_INVALID_ARG : GSA_ERR_UNSUPPORTED, "max_extra=%d outside [0, %d]",
                p->max_extra, kPagedMaxExtra);
  if (o->unit_S == 0)
    return fail(GSA_ERR_UNSUPPORTED,
                "paged decode runs on the bf16, head_dim 128, topk <= 64 path (n_gist <= 16384 when topk > 0)");
  if (o->N + o->M + (int64_t)p->max_extra >= ((int64_t)1 << 30))
    return fail(GSA_ERR_UNSUPPORTED, "paged decode: sequences up to 2^30 rows");
  o->pg_P = P;
  o->pg_max = p->max_pages;
  o->pg_max_extra = p->max_extra;
  o->pg_count = p->n_pages;
  return GSA_OK;
}

gsa_status_t plan_hier(const gsa_hier_params* p, HierPlan* o) {
  if (!p || !o) return fail(GSA_ERR_INVALID_ARG, "params is NULL");
  gsa_status_t s = plan_decode(&p->base, &o->base);
  if (s != GSA_OK) return s;
  HierPlan h{};
  h.base = o->base;
  const DecodePlan& d = h.base;
  if (p->fanout < 1) return fail(GSA_ERR_INVALID_ARG, "fanout=%d must be >= 1", p->fanout);
  h.G = p->fanout;
  h.M2 = d.M / h.G;
  h.k2 = p->topk2;
  if (h.k2 < 0 || h.k2 > h.M2)
    return fail(GSA_ERR_INVALID_ARG, "topk2=%d outside [0, M2=%lld]", h.k2, (long long)h.M2);
  h.n_orphan = (int32_t)(d.M - h.M2 * h.G);
  int64_t n_cand = (int64_t)h.k2 * h.G + h.n_orphan;
  if (n_cand > (1 << 30)) return fail(GSA_ERR_UNSUPPORTED, "too many level-1 candidates");
  h.n_cand = (int32_t)n_cand;
  if (d.k > h.n_cand)
    return fail(GSA_ERR_INVALID_ARG, "topk=%d exceeds the %d level-1 candidates", d.k, h.n_cand);
  if (h.k2 > kMaxTopk2) return fail(GSA_ERR_UNSUPPORTED, "topk2=%d above %d", h.k2, kMaxTopk2);
  int64_t units = d.units;
  h.S_l2 = splits_for(h.M2, units);
  if (ceil_div(h.M2, h.S_l2) > kMaxTaskItems) h.S_l2 = (int32_t)ceil_div(h.M2, kMaxTaskItems);
  h.l2_per_split = h.M2 > 0 ? ceil_div(h.M2, h.S_l2) : 0;
  h.S_l2 = h.M2 > 0 ? (int32_t)ceil_div(h.M2, h.l2_per_split) : 1;
  h.S_c = splits_for(h.n_cand, units);
  if (ceil_div(h.n_cand, h.S_c) > kMaxTaskItems) h.S_c = (int32_t)ceil_div(h.n_cand, kMaxTaskItems);
  h.cand_per_split = h.n_cand > 0 ? (int32_t)ceil_div(h.n_cand, h.S_c) : 0;
  h.S_c = h.n_cand > 0 ? (int32_t)ceil_div(h.n_cand, h.cand_per_split) : 1;
  h.tail_per_split = (int32_t)ceil_div(d.T, h.S_l2);
  h.NP = h.S_l2 + h.S_c + d.S2;
  h.unit_S = 0;
  if (d.dtype == GSA_BF16 && d.D == 128 && d.k <= kFastSelect && h.k2 <= kFastSelect &&
      h.M2 <= kUnitMaxSel && h.n_cand <= kUnitMaxGist && d.R < ((int64_t)1 << 31) &&
      (int64_t)d.k * d.C + h.n_cand + h.M2 + d.T < ((int64_t)1 << 31)) {
    const int64_t items = h.M2 + d.T;
    int64_t s = ceil_div(kUnitMinWGs, units);
    if (s < ceil_div(items, kUnitWgItems)) s = ceil_div(items, kUnitWgItems);
    if (ceil_div(items, s) < 64) s = ceil_div(items, 64);
    if (s < 1) s = 1;
    if (s <= kUnitMaxSplits) {
      h.unit_S = (int32_t)s;
      if (h.NP < h.unit_S + 1) h.NP = h.unit_S + 1;   // level-2 stream partials + the rest's
    }
  }
  if (d.gist_set != GSA_GISTS_ALL && h.unit_S == 0) {
    // split path, selection rules: the level-2 and candidate passes only
    // score; the unfold pass attends the whole set (chosen raw rows, their
    // gists with rule 1, the tail) and merges its own partial states alone
    const int64_t set_items = (int64_t)d.k * d.C + (d.gist_set == GSA_GISTS_SELECTED ? d.k : 0) + d.T;
    if (set_items > (1 << 30)) return fail(GSA_ERR_UNSUPPORTED, "selection too large");
    h.base.n_items = (int32_t)set_items;
    h.base.S2 = splits_for(set_items, units, kMinUnfoldRows);
    h.base.items_per_split = (int32_t)ceil_div(set_items, h.base.S2);
    h.base.S2 = (int32_t)ceil_div(set_items, h.base.items_per_split);
    h.NP = h.S_l2 + h.S_c + h.base.S2;
  }
  h.s2_stride = (h.M2 + 63) / 64 * 64;
  h.sc_stride = d.k > 0 ? (h.n_cand + 63) / 64 * 64 : 0;
  size_t off = 0;
  h.off_ctrl = off;
  off = align_up(off + ctrl_bytes(units));
  h.off_s2 = off;
  off = align_up(off + sizeof(float) * (size_t)units * (size_t)h.s2_stride);
  h.off_sc = off;
  off = align_up(off + sizeof(float) * (size_t)units * (size_t)h.sc_stride);
  h.off_sel2 = off;
  h.sel2_stride = line_pad(h.k2 > 0 ? h.k2 : 1);
  off = align_up(off + sizeof(int32_t) * (size_t)units * (size_t)h.sel2_stride);
  h.off_sel1 = off;
  off = align_up(off + sizeof(int32_t) * (size_t)units * (size_t)d.sel_stride);
  h.off_part = off;
  off = align_up(off + sizeof(float) * (size_t)units * h.NP * (size_t)part_stride(d.g, d.D));
  h.cand2_stride = 0;
  if (h.unit_S == 0 && h.k2 > 0 && h.k2 <= kFastSelect && h.S_l2 >= 4 && (int64_t)h.S_l2 * h.k2 * 2 <= h.M2) {
    h.cand2_stride = line_pad((int64_t)h.S_l2 * h.k2);
    h.off_cand2 = off;
    off = align_up(off + sizeof(float) * (size_t)units * (size_t)h.cand2_stride);
    h.off_cand2_ids = off;
    off = align_up(off + sizeof(int32_t) * (size_t)units * (size_t)h.cand2_stride);
  }
  h.total = off;
  *o = h;
  return GSA_OK;
}

gsa_status_t plan_prefill(const gsa_prefill_params* p, PrefillPlan* o) {
  if (!p || !o) return fail(GSA_ERR_INVALID_ARG, "params is NULL");
  gsa_status_t s = check_heads(p->n_q_heads, p->n_kv_heads, p->head_dim, p->dtype);
  if (s != GSA_OK) return s;
  if ((s = check_geometry(p->n_raw, p->n_gist, p->chunk)) != GSA_OK) return s;
  if (isnan(p->scale)) return fail(GSA_ERR_INVALID_ARG, "scale is NaN");
  if (p->topk < 0) return fail(GSA_ERR_INVALID_ARG, "topk=%d is negative", p->topk);
  if (p->window < 1) return fail(GSA_ERR_INVALID_ARG, "window=%d must be >= 1", p->window);
  if (p->q_start < 0 || p->n_q < 0 || p->q_start > p->n_raw || p->n_q > p->n_raw - p->q_start)
    return fail(GSA_ERR_INVALID_ARG, "query range of %lld from %lld outside [0, n_raw=%lld)",
                (long long)p->n_q, (long long)p->q_start, (long long)p->n_raw);
  if (p->head_dim != 128) return fail(GSA_ERR_UNSUPPORTED, "prefill needs head_dim=128");
  if (p->dtype != GSA_BF16) return fail(GSA_ERR_UNSUPPORTED, "prefill needs bf16 inputs");
  const int32_t g = p->n_q_heads / p->n_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(GSA_ERR_UNSUPPORTED, "prefill: %d query heads per kv-head not in {1, 2, 4, 8}", g);
  if (p->topk > kPrefillMaxK)
    return fail(GSA_ERR_UNSUPPORTED, "prefill: topk=%d above %d", p->topk, kPrefillMaxK);
  if (p->n_gist > kPrefillMaxGist)
    return fail(GSA_ERR_UNSUPPORTED, "prefill: n_gist=%lld above %d", (long long)p->n_gist, kPrefillMaxGist);
  if (p->n_raw + p->n_gist >= ((int64_t)1 << 31) || p->window > (1 << 30))
    return fail(GSA_ERR_UNSUPPORTED, "prefill: sequence too long for 32-bit positions");
  PrefillPlan d{};
  d.Hq = p->n_q_heads;
  d.Hkv = p->n_kv_heads;
  d.g = g;
  d.D = p->head_dim;
  d.C = p->chunk;
  d.k = p->topk;
  d.W = p->window;
  d.N = p->n_raw;
  d.M = p->n_gist;
  if ((s = resolve_rows(cache_rows(d.N, d.M), p->row_capacity, &d.R)) != GSA_OK) return s;
  d.q_start = p->q_start;
  d.q_stride = 1;
  d.n_q = p->n_q;
  d.scale = resolve_scale(p->scale, p->head_dim);
  d.n_blocks = (int32_t)ceil_div(d.n_q, kQBlock);
  if ((int64_t)d.n_blocks * d.Hkv > (1 << 30)) return fail(GSA_ERR_UNSUPPORTED, "prefill: too many blocks");
  // workspace: the selection [Hkv][n_q][k] handed from the select to the attend kernel
  d.total = align_up(sizeof(int32_t) * (size_t)d.Hkv * (size_t)d.n_q * (size_t)d.k);
  d.B = 1;
  d.seqs = nullptr;
  *o = d;
  return GSA_OK;
}

gsa_status_t plan_prefill_varlen(const gsa_prefill_varlen_params* p, PrefillPlan* o) {
  if (!p || !o) return fail(GSA_ERR_INVALID_ARG, "params is NULL");
  if (p->batch < 1) return fail(GSA_ERR_INVALID_ARG, "batch=%d must be >= 1", p->batch);
  if (p->base.q_start != 0)
    return fail(GSA_ERR_INVALID_ARG, "base.q_start=%lld must be 0 (each sequence's start is in its lengths)",
                (long long)p->base.q_start);
  gsa_status_t s = plan_prefill(&p->base, o);
  if (s != GSA_OK) return s;
  const int64_t wgs = (int64_t)o->n_blocks * o->Hkv * (o->g == 8 ? 2 : 1);
  if ((int64_t)p->batch * wgs > (1 << 30)) return fail(GSA_ERR_UNSUPPORTED, "prefill: too many blocks");
  o->B = p->batch;
  o->total = align_up(sizeof(int32_t) * (size_t)p->batch * (size_t)o->Hkv * (size_t)o->n_q * (size_t)o->k);
  return GSA_OK;
}

gsa_status_t plan_levels(const gsa_levels_params* p, LevelsPlan* o) {
  if (!p || !o) return fail(GSA_ERR_INVALID_ARG, "params is NULL");
  if (p->n_levels < 2 || p->n_levels > GSA_MAX_LEVELS)
    return fail(GSA_ERR_INVALID_ARG, "n_levels=%d outside [2, %d]", p->n_levels, GSA_MAX_LEVELS);
  if (p->fanout < 2) return fail(GSA_ERR_INVALID_ARG, "fanout=%d must be >= 2", p->fanout);
  gsa_status_t s = plan_decode(&p->base, &o->base);
  if (s != GSA_OK) return s;
  LevelsPlan h{};
  h.base = o->base;
  const DecodePlan& d = h.base;
  const int L = p->n_levels, G = p->fanout;
  h.L = L;
  h.G = G;
  h.Ml[1] = d.M;
  h.kl[1] = d.k;
  for (int l = 2; l <= L; ++l) {
    h.Ml[l] = h.Ml[l - 1] / G;
    h.kl[l] = p->topk_up[l - 2];
  }
  // candidates top-down
  h.items[L] = h.Ml[L];
  for (int l = L; l >= 1; --l) {
    if (l < L) {
      h.orphan0[l] = h.Ml[l + 1] * G;
      h.items[l] = (int64_t)h.kl[l + 1] * G + (h.Ml[l] - h.orphan0[l]);
    }
    if (h.kl[l] < 0 || h.kl[l] > h.items[l])
      return fail(GSA_ERR_INVALID_ARG, "k at level %d is %d, outside [0, %lld candidates]", l, h.kl[l],
                  (long long)h.items[l]);
    if (l >= 2 && h.kl[l] > kMaxTopk2)
      return fail(GSA_ERR_UNSUPPORTED, "k at level %d is %d, above %d", l, h.kl[l], kMaxTopk2);
    if (h.items[l] > (1 << 30)) return fail(GSA_ERR_UNSUPPORTED, "too many candidates at level %d", l);
  }
  const int64_t units = d.units;
  h.NP = 0;
  for (int l = L; l >= 1; --l) {
    int32_t S = splits_for(h.items[l], units);
    if (ceil_div(h.items[l], S) > kMaxTaskItems) S = (int32_t)ceil_div(h.items[l], kMaxTaskItems);
    h.per_split[l] = h.items[l] > 0 ? ceil_div(h.items[l], S) : 0;
    h.S[l] = h.items[l] > 0 ? (int32_t)ceil_div(h.items[l], h.per_split[l]) : 1;
    h.NP += h.S[l];
  }
  h.tail_per_split = (int32_t)ceil_div(d.T, h.S[L]);
  h.NP += d.S2;
  h.unit_S = 0;
  {
    bool ok = d.dtype == GSA_BF16 && d.D == 128 && d.k <= kFastSelect && h.Ml[L] >= 1 && h.Ml[L] <= kUnitMaxSel &&
              d.R < ((int64_t)1 << 31);
    int64_t rows = (int64_t)d.k * d.C + h.Ml[L] + d.T;
    for (int l = 1; l < L; ++l) {
      ok = ok && h.kl[l + 1] <= kFastSelect && h.items[l] <= kUnitMaxGist;
      rows += h.items[l];
    }
    ok = ok && rows < ((int64_t)1 << 31);
    if (ok) {
      const int64_t items = h.Ml[L] + d.T;
      int64_t s = ceil_div(kUnitMinWGs, units);
      if (s < ceil_div(items, kUnitWgItems)) s = ceil_div(items, kUnitWgItems);
      if (ceil_div(items, s) < 64) s = ceil_div(items, 64);
      if (s < 1) s = 1;
      if (s <= kUnitMaxSplits) {
        h.unit_S = (int32_t)s;
        if (h.NP < h.unit_S + 1) h.NP = h.unit_S + 1;   // top-level stream partials + the descent's
      }
    }
  }
  if (d.gist_set != GSA_GISTS_ALL && h.unit_S == 0) {
    // split path, selection rules: the level passes only score; the unfold
    // pass attends the set (chosen raw rows, their gists with rule 1, the
    // tail) and merges its own partial states alone
    const int64_t set_items = (int64_t)d.k * d.C + (d.gist_set == GSA_GISTS_SELECTED ? d.k : 0) + d.T;
    if (set_items > (1 << 30)) return fail(GSA_ERR_UNSUPPORTED, "selection too large");
    const int32_t S2_all = d.S2;
    h.base.n_items = (int32_t)set_items;
    h.base.S2 = splits_for(set_items, units, kMinUnfoldRows);
    h.base.items_per_split = (int32_t)ceil_div(set_items, h.base.S2);
    h.base.S2 = (int32_t)ceil_div(set_items, h.base.items_per_split);
    h.NP = h.NP - S2_all + h.base.S2;
  }
  size_t off = 0;
  h.off_ctrl = off;
  off = align_up(off + ctrl_bytes(units));
  for (int l = 1; l <= L; ++l) {
    h.score_stride[l] = (h.items[l] + 63) / 64 * 64;
    // the one-workgroup-per-unit descent reuses level 1's region for every
    // lower level's selection fallback
    if (l == 1) {
      for (int j = 2; j < L; ++j) h.score_stride[1] = std::max(h.score_stride[1], (h.items[j] + 63) / 64 * 64);
      h.score_stride[1] = std::max(h.score_stride[1], (h.Ml[L] + 63) / 64 * 64);   // the top level, selected in LDS
    }
    h.off_scores[l] = off;
    off = align_up(off + sizeof(float) * (size_t)units * (size_t)h.score_stride[l]);
    if (l >= 2) {
      h.sel_stride[l] = line_pad(h.kl[l] > 0 ? h.kl[l] : 1);
      h.off_sel[l] = off;
      off = align_up(off + sizeof(int32_t) * (size_t)units * (size_t)h.sel_stride[l]);
    }
  }
  h.off_sel1 = off;
  off = align_up(off + sizeof(int32_t) * (size_t)units * (size_t)d.sel_stride);
  h.off_part = off;
  off = align_up(off + sizeof(float) * (size_t)units * h.NP * (size_t)part_stride(d.g, d.D));
  h.total = off;
  *o = h;
  return GSA_OK;
}

gsa_status_t plan_gist(const gsa_gist_params* p, PrefillPlan* o) {
  if (!p || !o) return fail(GSA_ERR_INVALID_ARG, "params is NULL");
  if (p->chunk < 1) return fail(GSA_ERR_INVALID_ARG, "chunk=%d must be >= 1", p->chunk);
  if (p->m_start < 0 || p->n_q < 0 || p->m_start > p->n_raw || p->n_q > p->n_raw)
    return fail(GSA_ERR_INVALID_ARG, "gist queries [%lld, +%lld) outside the sequence", (long long)p->m_start,
                (long long)p->n_q);
  if (p->n_raw > ((int64_t)1 << 40)) return fail(GSA_ERR_UNSUPPORTED, "n_raw too large");
  const int64_t m_end = p->m_start + p->n_q;
  if (p->n_q > 0 && m_end > p->n_raw / p->chunk)
    return fail(GSA_ERR_INVALID_ARG, "chunk %lld is not complete (n_raw=%lld, chunk=%d)", (long long)(m_end - 1),
                (long long)p->n_raw, p->chunk);
  if (p->n_q > 0 && m_end - 1 > p->n_gist)
    return fail(GSA_ERR_INVALID_ARG, "the gist of chunk %lld needs gists 0..%lld, the cache holds %lld",
                (long long)(m_end - 1), (long long)(m_end - 2), (long long)p->n_gist);
  // The attention of a raw query at the chunk's last position, k = 0, W = C,
  // one query every C positions.
  gsa_prefill_params pp{};
  pp.n_q_heads = p->n_q_heads;
  pp.n_kv_heads = p->n_kv_heads;
  pp.head_dim = p->head_dim;
  pp.chunk = p->chunk;
  pp.topk = 0;
  pp.window = p->chunk;
  pp.n_raw = p->n_raw;
  pp.n_gist = p->n_gist;
  pp.q_start = p->n_q > 0 ? p->m_start * p->chunk + p->chunk - 1 : 0;
  pp.n_q = p->n_q > 0 ? 1 : 0;
  pp.scale = p->scale;
  pp.dtype = p->dtype;
  pp.row_capacity = p->row_capacity;
  gsa_status_t s = plan_prefill(&pp, o);
  if (s != GSA_OK) return s;
  // positions of the last block's padding queries stay in 32 bits
  if (p->n_raw + (int64_t)kQBlock * p->chunk >= ((int64_t)1 << 31))
    return fail(GSA_ERR_UNSUPPORTED, "gist prefill: sequence too long for 32-bit positions");
  o->n_q = p->n_q;
  o->q_stride = p->chunk;
  o->n_blocks = (int32_t)ceil_div(p->n_q, kQBlock);
  if ((int64_t)o->n_blocks * o->Hkv > (1 << 30)) return fail(GSA_ERR_UNSUPPORTED, "gist prefill: too many blocks");
  o->total = 0;
  return GSA_OK;
}

gsa_status_t plan_append(const gsa_append_params* p, AppendPlan* o) {
  if (!p || !o) return fail(GSA_ERR_INVALID_ARG, "params is NULL");
  if (p->batch < 1 || p->n_kv_heads < 1)
    return fail(GSA_ERR_INVALID_ARG, "batch=%d and n_kv_heads=%d must be >= 1", p->batch, p->n_kv_heads);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(GSA_ERR_UNSUPPORTED, "head_dim=%d not in {64,128}", p->head_dim);
  if (p->dtype != GSA_F32 && p->dtype != GSA_BF16) return fail(GSA_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
  if (p->chunk < 1 || p->chunk > 4096) return fail(GSA_ERR_INVALID_ARG, "chunk=%d outside [1, 4096]", p->chunk);
  if (p->n_raw < 0 || p->n_gist < 0 || p->raw_new < 0 || p->gist_new < 0 || p->n_raw > ((int64_t)1 << 40) ||
      p->raw_new > ((int64_t)1 << 40) || p->n_gist > p->n_raw || p->gist_new > p->raw_new + p->n_raw)
    return fail(GSA_ERR_INVALID_ARG, "token counts must be >= 0 and within range");
  const int64_t C = p->chunk;
  // a gist exists only for a complete chunk; raw rows may run ahead of the
  // gists (their slots are fixed), the readers need the gists caught up
  if (p->n_gist * C > p->n_raw)
    return fail(GSA_ERR_INVALID_ARG, "cache state n_gist=%lld has gists of incomplete chunks (n_raw=%lld)",
                (long long)p->n_gist, (long long)p->n_raw);
  const int64_t N1 = p->n_raw + p->raw_new, M1 = p->n_gist + p->gist_new;
  if (M1 * C > N1)
    return fail(GSA_ERR_INVALID_ARG, "the append adds gists of incomplete chunks (n_raw=%lld, n_gist=%lld after it)",
                (long long)N1, (long long)M1);
  // one past the highest slot written: the last raw row, or the last gist row
  const int64_t raw_end = N1 > 0 ? (N1 - 1) / C * (C + 1) + (N1 - 1) % C + 1 : 0;
  const int64_t need = raw_end > M1 * (C + 1) ? raw_end : M1 * (C + 1);
  if (p->row_capacity < need)
    return fail(GSA_ERR_INVALID_ARG, "row_capacity=%lld below the %lld rows the append reaches",
                (long long)p->row_capacity, (long long)need);
  const int64_t units = (int64_t)p->batch * p->n_kv_heads;
  if (units > (1 << 24)) return fail(GSA_ERR_UNSUPPORTED, "too many (batch, kv-head) units");
  AppendPlan d{};
  d.units = units;
  d.C = p->chunk;
  d.N = p->n_raw;
  d.M = p->n_gist;
  d.raw_new = p->raw_new;
  d.gist_new = p->gist_new;
  d.R = p->row_capacity;
  d.row_bytes = (int32_t)(p->head_dim * (p->dtype == GSA_BF16 ? 2 : 4));
  *o = d;
  return GSA_OK;
}

int32_t decode_launches(const DecodePlan& d) {
  if (d.unit_S > 1 && d.gist_set != GSA_GISTS_ALL) return (d.k > 0 ? 1 : 0) + 1;
  if (d.unit_S > 0) return 1 + (d.unit_S2 > 0 ? 1 : 0);
  if (d.gist_set != GSA_GISTS_ALL)   // split path: scoring pass (k > 0), candidates, the set's pass
    return (d.k > 0 ? 1 : 0) + (d.cand_stride > 0 ? 1 : 0) + 1;
  return 1 + (d.cand_stride > 0 ? 1 : 0) + (d.k > 0 ? 1 : 0);
}

int32_t hier_launches(const HierPlan& h) {
  if (h.unit_S > 0) return 1;
  return 2 + (h.cand2_stride > 0 ? 1 : 0) + (h.base.k > 0 || h.base.gist_set != GSA_GISTS_ALL ? 1 : 0);
}

int32_t levels_launches(const LevelsPlan& l) {
  if (l.unit_S > 0) return levels_top_in_lds(l) ? 1 : 2;
  return l.L + (l.base.k > 0 || l.base.gist_set != GSA_GISTS_ALL ? 1 : 0);
}

int32_t prefill_launches(const PrefillPlan& p) {
  if (p.n_q == 0) return 0;
  return (p.k > 0 ? 1 : 0) + 1;
}

}  // namespace gsa

extern "C" gsa_status_t gsa_check_seq_lens(const gsa_decode_params* p, const int32_t* seq_n_raw,
                                           const int32_t* seq_n_gist) {
  gsa::clear_error();
  gsa::DecodePlan d;
  gsa_status_t s = gsa::plan_decode(p, &d);
  if (s != GSA_OK) return s;
  if (!seq_n_raw || !seq_n_gist) return gsa::fail(GSA_ERR_INVALID_ARG, "length arrays are NULL");
  const int64_t C = p->chunk;
  for (int32_t b = 0; b < p->batch; ++b) {
    const int64_t n = seq_n_raw[b], m = seq_n_gist[b];
    const bool ok = n >= 1 && n <= p->n_raw && m >= p->topk && m <= p->n_gist && m * C <= n && n <= m * C + C &&
                    n - m * C <= p->tail && p->tail <= n;
    if (!ok)
      return gsa::fail(GSA_ERR_INVALID_ARG,
                       "sequence %d: n_raw=%lld, n_gist=%lld break 1 <= n <= %lld, %d <= m <= %lld, "
                       "0 <= n - m*C <= C, n - m*C <= tail=%d <= n",
                       b, (long long)n, (long long)m, (long long)p->n_raw, p->topk, (long long)p->n_gist, p->tail);
  }
  return GSA_OK;
}

extern "C" gsa_status_t gsa_check_prefill_seqs(const gsa_prefill_varlen_params* p, const int32_t* seqs) {
  gsa::clear_error();
  gsa::PrefillPlan d;
  gsa_status_t s = gsa::plan_prefill_varlen(p, &d);
  if (s != GSA_OK) return s;
  if (!seqs) return gsa::fail(GSA_ERR_INVALID_ARG, "seqs is NULL");
  const int64_t C = p->base.chunk;
  for (int32_t b = 0; b < p->batch; ++b) {
    const int64_t n = seqs[4 * b], m = seqs[4 * b + 1], qs = seqs[4 * b + 2], nq = seqs[4 * b + 3];
    const bool ok = n >= 1 && n <= p->base.n_raw && m >= 0 && m <= p->base.n_gist && m * C <= n && n <= m * C + C &&
                    qs >= 0 && nq >= 0 && nq <= p->base.n_q && qs + nq <= n;
    if (!ok)
      return gsa::fail(GSA_ERR_INVALID_ARG,
                       "sequence %d: (n_raw=%lld, n_gist=%lld, q_start=%lld, n_q=%lld) break 1 <= n <= %lld, "
                       "m <= %lld, 0 <= n - m*C <= C, 0 <= q_start, 0 <= n_q <= %lld, q_start + n_q <= n",
                       b, (long long)n, (long long)m, (long long)qs, (long long)nq, (long long)p->base.n_raw,
                       (long long)p->base.n_gist, (long long)p->base.n_q);
  }
  return GSA_OK;
}

extern "C" gsa_status_t gsa_check_levels_seq_lens(const gsa_levels_params* p, const int32_t* seq_n_raw,
                                                  const int32_t* seq_n_gist) {
  gsa::clear_error();
  gsa::LevelsPlan lp;
  gsa_status_t s = gsa::plan_levels(p, &lp);
  if (s != GSA_OK) return s;
  if ((s = gsa_check_seq_lens(&p->base, seq_n_raw, seq_n_gist)) != GSA_OK) return s;
  const int32_t L = p->n_levels, G = p->fanout;
  for (int32_t b = 0; b < p->base.batch; ++b) {
    int64_t cnt[GSA_MAX_LEVELS + 2];
    cnt[1] = seq_n_gist[b];
    for (int l = 2; l <= L + 1; ++l) cnt[l] = cnt[l - 1] / G;
    bool ok = lp.kl[L] <= cnt[L];
    for (int l = 1; l < L; ++l) ok = ok && lp.kl[l] <= (int64_t)lp.kl[l + 1] * G + cnt[l] - cnt[l + 1] * G;
    if (!ok)
      return gsa::fail(GSA_ERR_INVALID_ARG,
                       "sequence %d: n_gist=%lld leaves a level with fewer gists or candidates than its k", b,
                       (long long)seq_n_gist[b]);
  }
  return GSA_OK;
}

extern "C" gsa_status_t gsa_check_hier_seq_lens(const gsa_hier_params* p, const int32_t* seq_n_raw,
                                                const int32_t* seq_n_gist) {
  gsa::clear_error();
  gsa::HierPlan h;
  gsa_status_t s = gsa::plan_hier(p, &h);
  if (s != GSA_OK) return s;
  if ((s = gsa_check_seq_lens(&p->base, seq_n_raw, seq_n_gist)) != GSA_OK) return s;
  for (int32_t b = 0; b < p->base.batch; ++b) {
    const int64_t m = seq_n_gist[b], m2 = m / p->fanout;
    const int64_t nc = (int64_t)p->topk2 * p->fanout + (m - m2 * p->fanout);
    if (p->topk2 > m2 || p->base.topk > nc)
      return gsa::fail(GSA_ERR_INVALID_ARG,
                       "sequence %d: n_gist=%lld gives %lld level-2 gists and %lld level-1 candidates: need "
                       "topk2=%d <= level-2 gists and topk=%d <= candidates",
                       b, (long long)m, (long long)m2, (long long)nc, p->topk2, p->base.topk);
  }
  return GSA_OK;
}

extern "C" gsa_status_t gsa_check_pages(const gsa_paged_params* p, const int32_t* block_table,
                                        const int32_t* seq_n_raw, const int32_t* seq_n_gist,
                                        const int32_t* extra_rows) {
  gsa::clear_error();
  gsa::DecodePlan d;
  gsa_status_t s = gsa::plan_paged(p, &d);
  if (s != GSA_OK) return s;
  if ((s = gsa_check_seq_lens(&p->base, seq_n_raw, seq_n_gist)) != GSA_OK) return s;
  if (!block_table) return gsa::fail(GSA_ERR_INVALID_ARG, "block_table is NULL");
  if (p->max_extra > 0 && !extra_rows) return gsa::fail(GSA_ERR_INVALID_ARG, "extra_rows is NULL");
  const int64_t rpp = (int64_t)p->page_chunks * (p->base.chunk + 1);
  for (int32_t b = 0; b < p->base.batch; ++b) {
    const int64_t rows = (int64_t)seq_n_raw[b] + seq_n_gist[b];
    const int64_t pages = (rows + rpp - 1) / rpp;
    for (int64_t i = 0; i < pages; ++i) {
      const int32_t pg = block_table[(size_t)b * p->max_pages + i];
      if (pg < 0 || pg >= p->n_pages)
        return gsa::fail(GSA_ERR_INVALID_ARG, "sequence %d: page %lld of its table is %d, outside [0, %lld)", b,
                         (long long)i, pg, (long long)p->n_pages);
    }
    for (int32_t e = 0; e < p->max_extra; ++e) {
      const int32_t pg = extra_rows[((size_t)b * p->max_extra + e) * 2], r = extra_rows[((size_t)b * p->max_extra + e) * 2 + 1];
      if (pg < 0) break;
      if (pg >= p->n_pages || r < 0 || r >= rpp)
        return gsa::fail(GSA_ERR_INVALID_ARG, "sequence %d: extra row %d is (%d, %d), outside the pool", b, e, pg, r);
    }
  }
  return GSA_OK;
}

extern "C" gsa_status_t gsa_topk_for_budget(int64_t budget, int64_t n_gist, int32_t chunk, int32_t tail,
                                            int32_t gist_set, int32_t* topk) {
  gsa::clear_error();
  if (!topk) return gsa::fail(GSA_ERR_INVALID_ARG, "topk is NULL");
  if (n_gist < 0 || n_gist > (1 << 30) || chunk < 1 || tail < 0)
    return gsa::fail(GSA_ERR_INVALID_ARG, "need n_gist >= 0, chunk >= 1, tail >= 0");
  if (gist_set < GSA_GISTS_ALL || gist_set > GSA_GISTS_NONE)
    return gsa::fail(GSA_ERR_INVALID_ARG, "gist_set=%d not in {0, 1, 2}", gist_set);
  const int64_t fixed = (gist_set == GSA_GISTS_ALL ? n_gist : 0) + tail;   // tokens with k = 0
  const int64_t per = (int64_t)chunk + (gist_set == GSA_GISTS_SELECTED ? 1 : 0);   // tokens per chosen chunk
  if (budget < fixed)
    return gsa::fail(GSA_ERR_INVALID_ARG, "budget %lld is below the %lld tokens of the set with k = 0",
                     (long long)budget, (long long)fixed);
  const int64_t k = (budget - fixed) / per;
  *topk = (int32_t)(k < n_gist ? k : n_gist);
  return GSA_OK;
}

extern "C" const char* gsa_status_string(gsa_status_t s) {
  switch (s) {
    case GSA_OK: return "GSA_OK";
    case GSA_ERR_INVALID_ARG: return "GSA_ERR_INVALID_ARG: an argument is outside its documented range";
    case GSA_ERR_UNSUPPORTED: return "GSA_ERR_UNSUPPORTED: valid arguments this build does not run";
    case GSA_ERR_WORKSPACE: return "GSA_ERR_WORKSPACE: workspace missing or too small";
    case GSA_ERR_HIP: return "GSA_ERR_HIP: a HIP call or kernel launch failed";
  }
  return "unknown gsa_status_t";
}

extern "C" const char* gsa_last_error(void) { return gsa::last_error_message(); }

extern "C" gsa_status_t gsa_decode_launches(const gsa_decode_params* p, int32_t* n) {
  gsa::clear_error();
  if (!n) return gsa::fail(GSA_ERR_INVALID_ARG, "n is NULL");
  gsa::DecodePlan d;
  gsa_status_t s = gsa::plan_decode(p, &d);
  if (s != GSA_OK) return s;
  *n = gsa::decode_launches(d);
  return GSA_OK;
}

extern "C" gsa_status_t gsa_decode_hier_launches(const gsa_hier_params* p, int32_t* n) {
  gsa::clear_error();
  if (!n) return gsa::fail(GSA_ERR_INVALID_ARG, "n is NULL");
  gsa::HierPlan h;
  gsa_status_t s = gsa::plan_hier(p, &h);
  if (s != GSA_OK) return s;
  *n = gsa::hier_launches(h);
  return GSA_OK;
}

extern "C" gsa_status_t gsa_decode_levels_launches(const gsa_levels_params* p, int32_t* n) {
  gsa::clear_error();
  if (!n) return gsa::fail(GSA_ERR_INVALID_ARG, "n is NULL");
  gsa::LevelsPlan l;
  gsa_status_t s = gsa::plan_levels(p, &l);
  if (s != GSA_OK) return s;
  *n = gsa::levels_launches(l);
  return GSA_OK;
}

extern "C" gsa_status_t gsa_prefill_launches(const gsa_prefill_params* p, int32_t* n) {
  gsa::clear_error();
  if (!n) return gsa::fail(GSA_ERR_INVALID_ARG, "n is NULL");
  gsa::PrefillPlan pl;
  gsa_status_t s = gsa::plan_prefill(p, &pl);
  if (s != GSA_OK) return s;
  *n = gsa::prefill_launches(pl);
  return GSA_OK;
}
