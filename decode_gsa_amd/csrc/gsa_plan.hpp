// Host-side argument validation, work splitting and workspace layout for libgsa.
// Pure C++ (no HIP calls): every check runs before any launch.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "gsa.h"

namespace gsa {

// Record the reason for a failure on this thread; returns `s` for chaining.
gsa_status_t fail(gsa_status_t s, const char* fmt, ...);
void clear_error();
const char* last_error_message();

constexpr size_t kAlign = 256;

// Selections of at most this many items use wave-level bit-serial selects;
// larger ones a block-wide radix select.
constexpr int32_t kFastSelect = 64;
// One-workgroup-per-unit decode (bf16, D = 128, k <= kFastSelect): a unit is
// cut into unit_S workgroups, enough of them to fill the chip (kUnitMinWGs);
// each keeps at most kUnitMaxGist group scores in LDS, and the unit's
// selection reads at most kUnitMaxSel scores.
constexpr int32_t kUnitMinWGs = 256;
constexpr int64_t kUnitMaxGist = 4096;     // one workgroup per unit: gists kept in LDS
constexpr int64_t kUnitWgItems = 5120;     // several per unit: gist + tail rows per workgroup
constexpr int64_t kUnitMaxSel = 16384;
constexpr int32_t kUnitMaxSplits = 256;
// A two-level call's level-2 selection is staged in LDS: topk2 at most this.
constexpr int32_t kMaxTopk2 = 1024;
inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Phases of one fused decode launch (gist pass(es), then unfold).
constexpr int kMaxPhases = 3;

// Control words at the start of every decode workspace: per (phase, unit) a
// finished-task count and a ready flag. They must be zero before the first
// call; every call leaves them zero again.
// Each unit owns one 256-byte block of control words (a finished-task count
// per phase at word p, a ready flag per phase at word 8 + p), so waiting
// workgroups of different units poll different lines and memory channels.
constexpr size_t kCtrlUnitWords = 64;
inline size_t ctrl_words(int64_t units) { return kCtrlUnitWords * (size_t)units; }
// The control words live in a fixed 1 MiB area at offset 0 (room for 4096
// units), so calls of different shapes can share one workspace: no shape's
// data ever lands on another shape's control words.
constexpr size_t kCtrlBytes = (size_t)1 << 20;
inline size_t ctrl_bytes(int64_t units) {
  const size_t need = (sizeof(uint32_t) * ctrl_words(units) + 255) / 256 * 256;
  return need > kCtrlBytes ? need : kCtrlBytes;
}

#ifdef __HIP__
#define GSA_HD __host__ __device__
#else
#define GSA_HD
#endif

// Candidate hand-off of the several-workgroups-per-unit launches: each of the
// S stream workgroups of a unit writes `cand_cap` (score, id) slots, the
// scores at or above a bound on its kk-th largest (2 kk slots), or its exact
// top kk when 2 kk slots per split would make the unit's list longer than
// kUnitMaxSel. The kernels and the plan both use this.
// Paged caches (gsa_decode_paged): a sequence's block table and extra rows
// are staged in LDS, so they hold at most this many entries.
constexpr int32_t kPagedMaxPages = 2048;
constexpr int32_t kPagedMaxExtra = 64;

// The several-workgroups-per-unit launch hands candidates on for k up to
// this; above it every group score.
constexpr int32_t kUnitCandMaxK = 64;
GSA_HD inline int32_t cand_cap(int32_t S, int32_t kk) {
  return (int64_t)S * 2 * kk <= kUnitMaxSel ? 2 * kk : kk;
}

// Per-unit strides of workspace regions that other workgroups read back are
// whole 128-byte lines, so no two units (or partial slots) share a line.
inline int64_t line_pad(int64_t n_words) { return (n_words + 31) / 32 * 32; }
// floats per partial slot: g heads x (m, l, acc[D])
inline int64_t part_stride(int32_t g, int32_t D) { return line_pad((int64_t)g * (D + 2)); }

// Number of rows of the interleaved cache of one unit.
inline int64_t cache_rows(int64_t n_raw, int64_t n_gist) { return n_raw + n_gist; }

// Workspace layout and launch shape of one single-level decode call.
struct DecodePlan {
  int32_t units;        // B * Hkv
  int32_t g;            // query heads per kv-head
  int32_t D;
  int64_t M, R, N;      // R: rows between (sequence, kv-head) blocks (>= N + M)
  int32_t C, k, T;
  float scale;          // resolved (> 0)
  int32_t dtype;
  int32_t gist_set;     // GSA_GISTS_*
  // gist pass: S workgroups per unit, each over a contiguous gist range
  int32_t S;
  int64_t gists_per_split;
  int32_t tail_per_split;   // tail rows per gist workgroup (the gist pass attends the tail)
  // unfold pass (k > 0 only): S2 workgroups per unit over the k*C raw rows of
  // the selected chunks
  int32_t S2;
  int32_t items_per_split;
  int32_t n_items;      // k*C (selection-rule variants on the split path: the whole set)
  int32_t NP;           // partial states per unit = S (+ S2 when k > 0)
  // byte offsets inside the workspace (control words first)
  size_t off_ctrl, off_scores, off_sel, off_part, total;
  int64_t score_stride; // floats per unit in the score region (read by the unfold pass)
  // one-workgroup-per-unit path: workgroups per unit, 0 when the shape takes
  // the gist + unfold passes instead; with unit_S > 1 a second launch of
  // unit_S2 workgroups per unit selects and unfolds (k > 0)
  int32_t unit_S, unit_S2;
  int64_t sel_stride;   // ints per unit in the selection region (large k only)
  int32_t Hkv;
  // split path with many gists per unit (k <= 64): each gist workgroup hands
  // its own top-k (score, id) candidates on, and the unit's last workgroup
  // selects among S k of them; cand_stride = 0 when it selects among all M
  int64_t cand_stride;
  size_t off_cand, off_cand_ids;
  // variable-length batches (gsa_decode_varlen): device arrays of each
  // sequence's raw tokens and gists, null for uniform lengths
  const int32_t* seq_n;
  const int32_t* seq_m;
  // paged caches (gsa_decode_paged): block tables [B][pg_max], extra rows
  // [B][pg_max_extra][2], pages of pg_P chunk slots; null otherwise
  const int32_t* pg_table;
  const int32_t* pg_extra;
  int64_t pg_count;
  int32_t pg_P, pg_max, pg_max_extra;
};

gsa_status_t plan_decode(const gsa_decode_params* p, DecodePlan* out);
// Paged decode: plan_decode of the base, then the paging checks; the launch
// must be the one-workgroup-per-unit path (bf16, D = 128, k <= 64).
gsa_status_t plan_paged(const gsa_paged_params* p, DecodePlan* out);

// Two-level plan: level-2 gist pass, candidate level-1 gist pass, unfold.
struct HierPlan {
  DecodePlan base;      // level-1 geometry (k = k1); base.S is unused
  int32_t G, k2;
  int64_t M2;
  int32_t n_orphan;     // M - M2*G
  int32_t n_cand;       // k2*G + n_orphan
  int32_t S_l2;         // workgroups per unit over the level-2 gists
  int64_t l2_per_split;
  int32_t S_c;          // workgroups per unit over the level-1 candidates
  int32_t cand_per_split;
  int32_t tail_per_split;   // tail rows per level-2 workgroup
  int32_t NP;           // S_l2 + S_c (+ S2 when k1 > 0)
  size_t off_ctrl, off_s2, off_sc, off_sel2, off_sel1, off_part, total;
  int64_t s2_stride, sc_stride, sel2_stride;
  // one-workgroup-per-unit path (bf16, D = 128, k1, k2 <= 64, at most 16384
  // level-2 gists and 4096 candidates): workgroups per unit over the level-2
  // gists and the tail, then one workgroup per unit for the rest; 0 when the
  // gist passes run instead
  int32_t unit_S;
  // split path, k2 <= 64 and many level-2 gists: the level-2 workgroups'
  // top-k2 candidates (cand_kernel) replace the M2 scores in the candidate
  // pass's selection; cand2_stride = 0 otherwise
  int64_t cand2_stride;
  size_t off_cand2, off_cand2_ids;
};

gsa_status_t plan_hier(const gsa_hier_params* p, HierPlan* out);

// L-level plan (split path only): pass L over the top level + tail, one
// candidate pass per lower level, unfold. Index l = 1..L.
struct LevelsPlan {
  DecodePlan base;      // level 1 (k = k_1); base.S unused
  int32_t L, G;
  int64_t Ml[GSA_MAX_LEVELS + 1];        // gists at level l
  int32_t kl[GSA_MAX_LEVELS + 1];        // chosen at level l
  int64_t items[GSA_MAX_LEVELS + 1];     // items of pass l: M_L at the top, candidates below
  int64_t orphan0[GSA_MAX_LEVELS + 1];   // l < L: first level-l gist no group covers (M_{l+1} G)
  int32_t S[GSA_MAX_LEVELS + 1];         // workgroups per unit of pass l
  int64_t per_split[GSA_MAX_LEVELS + 1];
  int32_t tail_per_split;                // tail rows per top-level workgroup
  int32_t NP;                            // sum of S + S2 (k_1 > 0)
  size_t off_ctrl, off_part, off_sel1, total;
  size_t off_scores[GSA_MAX_LEVELS + 1]; // scores of pass l (read by the pass below)
  int64_t score_stride[GSA_MAX_LEVELS + 1];
  size_t off_sel[GSA_MAX_LEVELS + 1];    // l >= 2: chosen ids of level l
  int64_t sel_stride[GSA_MAX_LEVELS + 1];
  // one-workgroup-per-unit path (bf16, D = 128, every k <= 64, at most 16384
  // top-level gists and 4096 candidates per lower level): workgroups per unit
  // over the top level and the tail, then one workgroup per unit for the
  // descent; 0 when the per-level passes run instead
  int32_t unit_S;
};

gsa_status_t plan_levels(const gsa_levels_params* p, LevelsPlan* out);

// One-workgroup-per-unit L-level path: the top level fits one workgroup's LDS
// scores, so the descent's workgroup streams it itself (one launch per call).
inline bool levels_top_in_lds(const LevelsPlan& l) {
  return l.Ml[l.L] <= kUnitMaxGist && l.Ml[l.L] + l.base.T <= kUnitWgItems;
}

// Prefill plan.
struct PrefillPlan {
  int32_t Hq, Hkv, g, D, C, k, W;
  int64_t N, M, R, q_start, n_q;   // R: rows between kv-head blocks (>= N + M)
  int32_t q_stride;     // positions between consecutive queries (1; C for gist tokens)
  float scale;
  int32_t n_blocks;     // query blocks of kQBlock queries
  size_t total;
  // a batch of sequences (gsa_prefill_varlen): B sequences, each with its
  // lengths at seqs[4 b ..] (device); n_q (the rows per head of q, out and
  // the selection) and N, M are the batch's largest. B = 1, seqs = null for
  // one sequence.
  int32_t B;
  const int32_t* seqs;
};

constexpr int kQBlock = 64;
// Prefill limits: chunks a query block can select are tracked in an LDS
// bitmap (n_gist <= kPrefillMaxGist), and the union of a block's selections
// holds at most 64 * kPrefillMaxK chunks.
constexpr int32_t kPrefillMaxGist = 262144;
constexpr int32_t kPrefillMaxK = 64;

gsa_status_t plan_prefill(const gsa_prefill_params* p, PrefillPlan* out);
gsa_status_t plan_prefill_varlen(const gsa_prefill_varlen_params* p, PrefillPlan* out);
// Gist-token queries as prefill queries at positions mC + C - 1 (stride C),
// k = 0, W = C.
gsa_status_t plan_gist(const gsa_gist_params* p, PrefillPlan* out);

struct AppendPlan {
  int64_t units;        // B * Hkv
  int32_t C, row_bytes;
  int64_t N, M, raw_new, gist_new, R;
};
gsa_status_t plan_append(const gsa_append_params* p, AppendPlan* out);

// Kernel launches a call with this plan makes (what gsa_profile_marks reports,
// minus one). Each matches the launch sequence of the entry point's runner.
int32_t decode_launches(const DecodePlan& d);
int32_t hier_launches(const HierPlan& h);
int32_t levels_launches(const LevelsPlan& l);
int32_t prefill_launches(const PrefillPlan& p);

// Pointer checks shared by the entry points.
gsa_status_t check_ptr(const void* p, const char* name, bool allow_null = false);
gsa_status_t check_workspace(const void* ws, size_t have, size_t need);

}  // namespace gsa
