/*
 * gsa.h -- C ABI of libgsa: Gist Sparse Attention (GSA) decode and prefill
 * on AMD Instinct MI355X (gfx950).
 *
 * The method (gist.science explainer "Forget, Then Recall: Learnable
 * Compression and Selective Unfolding via Gist Sparse Attention", section 2
 * 'Key Concepts'; Taki-lab slide deck on the same paper, slides 3 and 6-10):
 * a sequence is cut into chunks of C raw tokens and one gist token follows
 * every chunk. At each step the query scores every gist key by a dot
 * product, keeps the k best chunks, restores ("unfolds") their raw K/V, and
 * runs softmax attention over all gists, the unfolded raw tokens and the
 * trailing raw tokens that have no gist yet.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor arguments are DEVICE pointers, dense and row-major as stated,
 *    16-byte aligned. The caller owns every buffer; the library allocates no
 *    memory and never synchronizes.
 *  - q, K and V share one element type (gsa_dtype_t). out and lse are fp32.
 *  - Interleaved cache of one (batch, kv-head) unit: R = n_raw + n_gist rows
 *    of head_dim elements. Row m*(C+1)+j (j < C) holds raw token m*C+j; row
 *    m*(C+1)+C holds the gist of chunk m; the 0..C raw tokens after the last
 *    gisted chunk follow in rows n_gist*(C+1) onwards.
 *  - scale <= 0 selects 1/sqrt(head_dim). Logits are scale * (q . k).
 *  - With grouped-query attention (g = n_q_heads / n_kv_heads query heads per
 *    kv-head) one selection is made per (batch, kv-head): the group score of
 *    a gist is the mean over the g heads of their scaled logits.
 *  - Ties in a top-k go to the smaller chunk index; selections are written in
 *    ascending chunk order.
 *  - Every row enters the attention set once even when a selected chunk
 *    overlaps the tail (decode) or the window (prefill).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = default
 *    stream). Results are valid after the caller synchronizes the stream.
 *  - Every argument is validated on the host before any launch; a rejected
 *    call returns a non-zero status, launches nothing and writes nothing.
 *    A launch failure returns GSA_ERR_HIP. gsa_last_error() gives a
 *    human-readable reason for the last failure on the calling thread.
 *  - Calls keep no state between them (re-entrant). The workspace of a call
 *    must not be used by another call that runs concurrently.
 */
#ifndef GSA_H_
#define GSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GSA_OK = 0,
  GSA_ERR_INVALID_ARG = 1, /* argument out of its documented range / NULL */
  GSA_ERR_UNSUPPORTED = 2, /* valid, but a shape or type this build does not run */
  GSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  GSA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} gsa_status_t;

typedef enum { GSA_F32 = 0, GSA_BF16 = 1 } gsa_dtype_t;

/* ------------------------------------------------------------------------
 * Single-level decode: one new query per sequence.
 * Source: gist.science explainer, section 2 'Key Concepts' (gist as routing
 * signal; selective unfolding; hybrid attention) and the slide deck's
 * slide 10 worked example (scores 0.1/0.8/0.7/0.2, k=2 -> chunks 2 and 3).
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t batch;       /* B >= 1 */
  int32_t n_q_heads;   /* Hq >= 1, multiple of n_kv_heads */
  int32_t n_kv_heads;  /* Hkv >= 1; g = Hq/Hkv must be 1, 2, 4 or 8 */
  int32_t head_dim;    /* D: 64 or 128 */
  int64_t n_raw;       /* N >= 1 raw tokens per sequence (same for all) */
  int64_t n_gist;      /* M gisted chunks; 0 <= N - M*C <= C */
  int32_t chunk;       /* C >= 1 raw tokens per chunk */
  int32_t topk;        /* 0 <= k <= M chunks to unfold */
  int32_t tail;        /* T: the last T raw tokens are always attended;
                          N - M*C <= T <= N */
  float scale;         /* <= 0: 1/sqrt(D) */
  int32_t dtype;       /* gsa_dtype_t of q, K, V */
  int32_t gist_set;    /* which gist rows the attention set holds (the slide
                          deck's slide 17, 'Selective Rules Comparison'):
                          GSA_GISTS_ALL (0, the default: every gist, the
                          explainer's hybrid attention), GSA_GISTS_SELECTED
                          (1, the chosen chunks' gists: SG+SR) or
                          GSA_GISTS_NONE (2, raw tokens only: SR-only).
                          1 and 2 need k > 0 or T > 0 (a non-empty set);
                          gsa_decode and gsa_decode_noalloc run them on
                          every shape they accept; so do
                          gsa_decode_hier and gsa_decode_levels, the rule
                          deciding which gists are attended while the
                          routing stays the same; gsa_decode_varlen,
                          gsa_decode_hier_varlen and
                          gsa_decode_levels_varlen on every shape they
                          accept; gsa_decode_paged on every
                          shape it accepts. */
  int64_t row_capacity; /* rows allocated per (sequence, kv-head) in the
                          caches, the stride between their [R, D] blocks:
                          0 means exactly R = N + M; else it must be
                          >= N + M, so a cache sized once for its final
                          length grows in place (gsa_cache_append) */
} gsa_decode_params;

enum { GSA_GISTS_ALL = 0, GSA_GISTS_SELECTED = 1, GSA_GISTS_NONE = 2 };

/* Bytes of device workspace gsa_decode needs for these parameters. */
gsa_status_t gsa_decode_workspace_size(const gsa_decode_params* p, size_t* bytes);

/*
 * q        [B, Hq, D]        query of the new token, per head
 * k_cache  [B, Hkv, R, D]    interleaved key cache, R = N + M (R =
 *                            row_capacity when that is set; rows past N + M
 *                            are never read)
 * v_cache  [B, Hkv, R, D]    interleaved value cache
 * out      [B, Hq, D] fp32   attention output (written)
 * lse      [B, Hq]    fp32   natural-log sum-exp of the attended logits, or NULL
 * sel_idx  [B, Hkv, k] int32 selected chunk ids, ascending, or NULL
 * workspace / workspace_bytes: device scratch of at least
 *          gsa_decode_workspace_size() bytes, 256-byte aligned. Its first
 *          1 MiB holds task counters: the buffer must be zero-filled once
 *          before its first use, and every call that runs to completion leaves
 *          the counters zero again, so one buffer serves any number of later
 *          calls of any shape that fits it (batch * n_kv_heads <= 4096; above
 *          that, zero it again when the shape changes), one call at a time.
 */
gsa_status_t gsa_decode(const gsa_decode_params* p, const void* q, const void* k_cache,
                        const void* v_cache, float* out, float* lse, int32_t* sel_idx,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * gsa_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, hosts that
 * forbid hipMalloc). It allocates nothing: its workspace is a 16 MiB device
 * array inside the library, one copy per GPU, held until the process ends.
 * Arguments, results and launches are gsa_decode's; the first call on a
 * device also clears the array's control words (one more launch, outside the
 * timing hook's count). Every call on a GPU shares that GPU's array and
 * leaves its control words zero: calls that overlap on one GPU (on different
 * streams, or from several threads) race and give wrong results; serialize
 * them. GSA_ERR_WORKSPACE when gsa_decode_workspace_size exceeds 16 MiB (see
 * that call's size), GSA_ERR_UNSUPPORTED above 4096 (batch, kv-head) units;
 * nothing is launched then.
 * ---------------------------------------------------------------------- */
gsa_status_t gsa_decode_noalloc(const gsa_decode_params* p, const void* q, const void* k_cache,
                                const void* v_cache, float* out, float* lse, int32_t* sel_idx,
                                void* stream);

/* ------------------------------------------------------------------------
 * Variable-length batch: the same step as gsa_decode, for sequences of
 * different lengths (each (sequence, kv-head) block holds its own raw tokens
 * and gists, read only up to its own N_b + M_b rows).
 * Source: the decode rule of gsa_decode (explainer section 2 'Key
 * Concepts'), applied per sequence; serving batches of documents of several
 * lengths is the use the explainer's reuse of cached documents implies.
 * p->n_raw and p->n_gist are the batch's largest values (they size the
 * workspace and the launch: gsa_decode_workspace_size(p) applies);
 * p->row_capacity (or N + M of those maxima) is the slab stride.
 * seq_n_raw, seq_n_gist: device arrays [B] int32, 16-byte aligned: sequence
 * b holds N_b raw tokens and M_b gists with 1 <= N_b <= N, topk <= M_b <= M,
 * 0 <= N_b - M_b*C <= C and N_b - M_b*C <= tail <= N_b. They stay on the
 * device (read by the kernels); gsa_check_seq_lens validates a host copy.
 * A sequence that breaks these rules is run with (N, M) instead, so no read
 * leaves its slab. gist_set: the selection rules, as gsa_decode (every
 * shape).
 * ---------------------------------------------------------------------- */
gsa_status_t gsa_decode_varlen(const gsa_decode_params* p, const int32_t* seq_n_raw,
                               const int32_t* seq_n_gist, const void* q, const void* k_cache,
                               const void* v_cache, float* out, float* lse, int32_t* sel_idx,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Paged caches: gsa_decode_varlen's step over caches that live in pages of a
 * shared pool, plus rows attended directly.
 * Source: the explainer's section 4 'Experimental Results' (KV-cache reuse:
 * document caches computed once and reused, the query routed among their
 * gists) with the decode rule of section 2 'Key Concepts'. A page holds P
 * chunk slots of C + 1 rows (C raw rows and the chunk's gist), so no chunk
 * straddles two pages. Sequence b's interleaved cache (gsa_decode's layout)
 * is its block table's pages in order: logical row r is row r mod P(C+1) of
 * page block_table[b][r / (P(C+1))]. Documents reused from separate caches
 * concatenate by listing their pages (P = 1 concatenates at any chunk); a
 * document that ends mid-chunk lists its complete chunks, and its last raw
 * tokens, which no gist summarises, go in extra_rows: they are attended
 * directly, like the tail.
 * ---------------------------------------------------------------------- */
typedef struct {
  gsa_decode_params base; /* as gsa_decode_varlen: n_raw / n_gist are the
                             batch's largest; bf16, head_dim 128, topk <= 64
                             (n_gist <= 16384 when topk > 0), row_capacity
                             0; else GSA_ERR_UNSUPPORTED /
                             GSA_ERR_INVALID_ARG. gist_set as gsa_decode:
                             the extra rows are attended under every rule */
  int32_t page_chunks;    /* P: chunk slots per page, a power of two in [1, 64] */
  int32_t max_pages;      /* columns of block_table, >= the pages of
                             n_raw + n_gist rows, <= 2048 */
  int64_t n_pages;        /* pages in each pool, >= 1 */
  int32_t max_extra;      /* columns of extra_rows, 0..64 */
} gsa_paged_params;

/* Bytes of device workspace gsa_decode_paged needs (as gsa_decode's). */
gsa_status_t gsa_decode_paged_workspace_size(const gsa_paged_params* p, size_t* bytes);

/*
 * block_table  [B, max_pages] int32 (device): page ids of each sequence's
 *              logical pages; entries past its rows are not read
 * seq_n_raw, seq_n_gist  [B] int32 (device): as gsa_decode_varlen
 * extra_rows   [B, max_extra, 2] int32 (device) (page, row within the page)
 *              pairs attended by every query head of the sequence's kv-heads
 *              (the same row of each kv-head's slab of the page); a
 *              sequence's list ends at its first entry with a negative page;
 *              NULL when max_extra = 0
 * q            [B, Hq, D]
 * k_pool, v_pool [n_pages, Hkv, P(C+1), D]: page p's rows of kv-head j
 * out, lse, sel_idx, workspace: as gsa_decode (zero-filled once).
 * The kernels clamp page ids and rows into the pools (a bad table gives a
 * wrong result, never a read outside them); gsa_check_pages validates host
 * copies. Launches as gsa_decode_varlen of the same base parameters.
 */
gsa_status_t gsa_decode_paged(const gsa_paged_params* p, const int32_t* block_table, const int32_t* seq_n_raw,
                              const int32_t* seq_n_gist, const int32_t* extra_rows, const void* q,
                              const void* k_pool, const void* v_pool, float* out, float* lse, int32_t* sel_idx,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Host check of paged inputs (host arrays): the lengths as
 * gsa_check_seq_lens, every page id a sequence reads in [0, n_pages), every
 * extra row's page in [0, n_pages) and row in [0, P(C+1)). GSA_OK or
 * GSA_ERR_INVALID_ARG naming the first bad entry (gsa_last_error). */
gsa_status_t gsa_check_pages(const gsa_paged_params* p, const int32_t* block_table, const int32_t* seq_n_raw,
                             const int32_t* seq_n_gist, const int32_t* extra_rows);

/* Host check of per-sequence lengths (host arrays [p->batch]) against the
 * rules above: GSA_OK, or GSA_ERR_INVALID_ARG naming the first sequence that
 * breaks one (gsa_last_error). */
gsa_status_t gsa_check_seq_lens(const gsa_decode_params* p, const int32_t* seq_n_raw,
                                const int32_t* seq_n_gist);

/* ------------------------------------------------------------------------
 * Two-level (gist-of-gist) decode.
 * Source: gist.science explainer, 'Hierarchical Extension (H-GSA)': meta-gists
 * summarise groups of gists; selection scores the meta-gists, then the gists
 * inside the chosen groups, then unfolds raw chunks (also the slide deck,
 * slide 11, and the authors' abstract on multi-resolution access).
 * Level-2 gist i summarises level-1 gists [i*G, (i+1)*G); M2 = floor(M/G).
 * The M - M2*G level-1 gists no group covers are always candidates.
 * Attention set: every level-2 gist, every candidate level-1 gist (all G
 * children of each chosen group, plus the ungrouped ones), the raw rows of
 * the k1 chosen chunks and the tail. With base.gist_set 1 (2) the set is the
 * chosen chunks' gists (no gist), their raw rows and the tail: the level-2
 * and candidate gists only route (every dtype and head_dim).
 * ---------------------------------------------------------------------- */
typedef struct {
  gsa_decode_params base; /* level-1 cache; base.topk = k1 */
  int32_t fanout;         /* G >= 1 */
  int32_t topk2;          /* 0 <= k2 <= M2; k1 <= k2*G + (M - M2*G) */
} gsa_hier_params;

gsa_status_t gsa_decode_hier_workspace_size(const gsa_hier_params* p, size_t* bytes);

/*
 * q, k_cache, v_cache, out, lse: as gsa_decode.
 * k_l2, v_l2 [B, Hkv, M2, D]  level-2 gist keys / values (dense rows)
 * sel2 [B, Hkv, k2] int32     chosen level-2 groups, ascending, or NULL
 * sel1 [B, Hkv, k1] int32     chosen chunks, ascending, or NULL
 */
gsa_status_t gsa_decode_hier(const gsa_hier_params* p, const void* q, const void* k_cache,
                             const void* v_cache, const void* k_l2, const void* v_l2,
                             float* out, float* lse, int32_t* sel2, int32_t* sel1,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Variable-length two-level decode: gsa_decode_hier's step for sequences of
 * different lengths.
 * Source: the two-level rule of gsa_decode_hier (explainer 'Hierarchical
 * Extension (H-GSA)'), applied per sequence, as gsa_decode_varlen applies
 * gsa_decode's.
 * p->base.n_raw and p->base.n_gist are the batch's largest values N, M
 * (they size the workspace: gsa_decode_hier_workspace_size(p) applies, and
 * the launches); p->base.row_capacity (or N + M) is the cache slab stride
 * and M2 = floor(M / G) the level-2 slab stride: sequence b's M2_b =
 * floor(M_b / G) level-2 gists are the first rows of its [M2, D] slab.
 * seq_n_raw, seq_n_gist: device arrays [B] int32 (16-byte aligned), the
 * rules of gsa_decode_varlen plus topk2 <= M2_b and base.topk <= topk2*G +
 * (M_b - M2_b*G); gsa_check_hier_seq_lens validates a host copy. A sequence
 * that breaks them runs with (N, M) instead, so no read leaves its slabs.
 * Other arguments as gsa_decode_hier. Runs on the bf16, head_dim 128 path
 * (topk, topk2 <= 64, at most 4096 level-1 candidates; else
 * GSA_ERR_UNSUPPORTED); gist_set as gsa_decode_hier. One launch.
 * ---------------------------------------------------------------------- */
gsa_status_t gsa_decode_hier_varlen(const gsa_hier_params* p, const int32_t* seq_n_raw,
                                    const int32_t* seq_n_gist, const void* q, const void* k_cache,
                                    const void* v_cache, const void* k_l2, const void* v_l2, float* out,
                                    float* lse, int32_t* sel2, int32_t* sel1, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* Host check of per-sequence lengths (host arrays [p->base.batch]) against
 * gsa_decode_hier_varlen's rules: GSA_OK, or GSA_ERR_INVALID_ARG naming the
 * first sequence that breaks one (gsa_last_error). */
gsa_status_t gsa_check_hier_seq_lens(const gsa_hier_params* p, const int32_t* seq_n_raw,
                                     const int32_t* seq_n_gist);

/* ------------------------------------------------------------------------
 * L-level decode (gists of gists of gists ...).
 * Source: gist.science explainer, 'Hierarchical Extension (H-GSA)' and
 * 'Coarse-to-Fine Selection' (multi-resolution access: the selection walks
 * down from the coarsest summaries), slide deck slide 11.
 * Level 1 is the interleaved cache's M gists; level l >= 2 holds
 * M_l = floor(M_{l-1} / G) gists in its own [B, Hkv, M_l, D] array, gist i
 * of level l summarising gists [i*G, (i+1)*G) of level l - 1. Top-down: the
 * top level's gists are all candidates; each level's top-k_l candidates (by
 * group score, ties to the smaller id) make their G children candidates of
 * the level below, together with that level's M_l - M_{l+1}*G gists no group
 * covers. Attention set: every top-level gist, every candidate of the
 * levels below, the raw rows of the k_1 chosen chunks and the tail.
 * L = 2 is gsa_decode_hier's rule.
 * ---------------------------------------------------------------------- */
#define GSA_MAX_LEVELS 6

typedef struct {
  gsa_decode_params base; /* level 1 and the step: base.topk = k_1 chunks
                             unfolded; base.gist_set 1 or 2 (the chosen
                             chunks' gists, or none, attended; every
                             level's gists only route) */
  int32_t n_levels;       /* L, 2 <= L <= GSA_MAX_LEVELS */
  int32_t fanout;         /* G >= 2 */
  int32_t topk_up[GSA_MAX_LEVELS - 1]; /* topk_up[i] = k_{i+2}, for levels
                             2..L: 0 <= k_L <= M_L, and k_l at most the
                             candidates of level l (k_{l+1}*G + M_l -
                             M_{l+1}*G), k_l <= 1024; k_1 likewise */
} gsa_levels_params;

gsa_status_t gsa_decode_levels_workspace_size(const gsa_levels_params* p, size_t* bytes);

/*
 * q, k_cache, v_cache, out, lse: as gsa_decode (row_capacity honoured).
 * k_up, v_up   host arrays of L - 1 device pointers: k_up[i] is level i+2's
 *              [B, Hkv, M_{i+2}, D] key array (v_up its values), dense rows
 * sel_up       host array of L - 1 device pointers or NULL: sel_up[i]
 *              [B, Hkv, k_{i+2}] int32 gets level i+2's chosen ids
 *              (ascending); an entry may be NULL
 * sel1         [B, Hkv, k_1] int32 chosen chunk ids (ascending) or NULL
 * workspace    as gsa_decode (zero-filled once; left zero by each call)
 * The work is a pass over the top level and the tail, then per lower level a
 * selection among the level above's scores and a pass over its candidates,
 * then the unfold. gsa_decode_levels_launches gives the launch count.
 * GSA_ERR_INVALID_ARG for out-of-range sizes or NULL arrays;
 * GSA_ERR_UNSUPPORTED for g outside {1, 2, 4, 8}, D outside {64, 128}.
 */
gsa_status_t gsa_decode_levels(const gsa_levels_params* p, const void* q, const void* k_cache,
                               const void* v_cache, const void* const* k_up,
                               const void* const* v_up, float* out, float* lse,
                               int32_t* const* sel_up, int32_t* sel1, void* workspace,
                               size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Variable-length L-level decode: gsa_decode_levels' step for sequences of
 * different lengths.
 * Source: the L-level rule above applied per sequence, as gsa_decode_varlen
 * applies gsa_decode's.
 * p->base.n_raw, p->base.n_gist are the batch's largest N, M; they size the
 * workspace (gsa_decode_levels_workspace_size(p)) and the slabs: the cache
 * slabs hold base.row_capacity (or N + M) rows, level l's slabs M_l =
 * floor(M / G^(l-1)) rows, and sequence b's level l has M_l(b) =
 * floor(M_b / G^(l-1)) gists, the first rows of its slab.
 * seq_n_raw, seq_n_gist: device arrays [B] int32 (16-byte aligned), the
 * rules of gsa_decode_varlen plus k_L <= M_L(b) and each k_l at most
 * sequence b's candidates of level l; gsa_check_levels_seq_lens validates a
 * host copy. A sequence that breaks them runs with (N, M) instead, so no
 * read leaves its slabs. Runs on the one-launch path only (bf16, head_dim
 * 128, every k <= 64, at most 4096 top-level gists and 4096 candidates per
 * level; else GSA_ERR_UNSUPPORTED). Other arguments as gsa_decode_levels.
 * ---------------------------------------------------------------------- */
gsa_status_t gsa_decode_levels_varlen(const gsa_levels_params* p, const int32_t* seq_n_raw,
                                      const int32_t* seq_n_gist, const void* q, const void* k_cache,
                                      const void* v_cache, const void* const* k_up,
                                      const void* const* v_up, float* out, float* lse,
                                      int32_t* const* sel_up, int32_t* sel1, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* Host check of per-sequence lengths (host arrays [p->base.batch]) against
 * gsa_decode_levels_varlen's rules: GSA_OK, or GSA_ERR_INVALID_ARG naming
 * the first sequence that breaks one (gsa_last_error). */
gsa_status_t gsa_check_levels_seq_lens(const gsa_levels_params* p, const int32_t* seq_n_raw,
                                       const int32_t* seq_n_gist);

/* ------------------------------------------------------------------------
 * Causal block-sparse prefill of query positions [q_start, q_start + n_q)
 * of one sequence.
 * Source: gist.science explainer, 'Training Procedure: Selective Finetuning'
 * (the attention mask admits only the top-k chunks and their raw tokens),
 * with the gist causal order of section 2 'Key Concepts' (a gist sees its
 * own chunk and earlier gists; slide deck slide 7).
 * Query t may use gist m only when m < floor(t/C) (the chunk is complete
 * before t). It selects the top-k of those by group score (all of them when
 * fewer than k, the rest of sel padded with -1) and attends to every
 * eligible gist, the raw rows of its chosen chunks, and the raw tokens in
 * [t - W + 1, t].
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t n_q_heads;   /* Hq, multiple of n_kv_heads; g = Hq/Hkv in {1, 2, 4, 8}
                          (other g: GSA_ERR_UNSUPPORTED) */
  int32_t n_kv_heads;  /* Hkv >= 1 */
  int32_t head_dim;    /* D: 128 (others: GSA_ERR_UNSUPPORTED) */
  int32_t chunk;       /* C >= 1 */
  int32_t topk;        /* 0 <= k <= 64 (k > 64: GSA_ERR_UNSUPPORTED) */
  int32_t window;      /* W >= 1 */
  int64_t n_raw;       /* N raw tokens in the cache */
  int64_t n_gist;      /* M; 0 <= N - M*C <= C; M <= 262144 (above:
                          GSA_ERR_UNSUPPORTED) */
  int64_t q_start;     /* first query position, 0 <= q_start */
  int64_t n_q;         /* queries; q_start + n_q <= N */
  float scale;         /* <= 0: 1/sqrt(D) */
  int32_t dtype;       /* GSA_BF16 (GSA_F32: GSA_ERR_UNSUPPORTED) */
  int64_t row_capacity; /* rows per kv-head in the caches (their stride);
                           0: R = N + M, else >= N + M */
} gsa_prefill_params;

gsa_status_t gsa_prefill_workspace_size(const gsa_prefill_params* p, size_t* bytes);

/*
 * q       [Hq, n_q, D]        queries (row i is position q_start + i)
 * k_cache [Hkv, R, D]         interleaved cache of the sequence, R = N + M
 *                             (R = row_capacity when that is set)
 * v_cache [Hkv, R, D]
 * out     [Hq, n_q, D] fp32   attention output (written)
 * sel     [Hkv, n_q, k] int32 chosen chunks per query, ascending, -1 padded,
 *                             or NULL
 * With n_q = 0 nothing is launched and q, out may be NULL.
 */
gsa_status_t gsa_prefill_blocksparse(const gsa_prefill_params* p, const void* q,
                                     const void* k_cache, const void* v_cache, float* out,
                                     int32_t* sel, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* ------------------------------------------------------------------------
 * Batched prefill of sequences of different lengths: gsa_prefill_blocksparse
 * for B sequences in one call.
 * Source: the selection rule of 'Training Procedure: Selective Finetuning'
 * (explainer) applied to each sequence on its own, as gsa_decode_varlen
 * applies the decode rule per sequence.
 * base.n_raw / base.n_gist are the batch's largest N, M (the cache slabs
 * hold base.row_capacity rows, or N + M); base.n_q is the most queries of
 * any sequence and the row stride of q, out and sel; base.q_start must be
 * 0. Other base fields as gsa_prefill_blocksparse (the same limits).
 * seqs: device array [B][4] int32, 16-byte aligned: sequence b's (N_b, M_b,
 * q_start_b, n_q_b) with 1 <= N_b <= N, M_b <= M, 0 <= N_b - M_b*C <= C,
 * 0 <= q_start_b, 0 <= n_q_b <= base.n_q, q_start_b + n_q_b <= N_b. A
 * sequence that breaks these gets no work (its rows of out and sel are not
 * written); gsa_check_prefill_seqs validates a host copy.
 * q       [B, Hq, n_q, D]      sequence b's query i (position q_start_b + i) in row i
 * k_cache [B, Hkv, R, D]       sequence b's interleaved cache
 * v_cache [B, Hkv, R, D]
 * out     [B, Hq, n_q, D] fp32 (rows past a sequence's n_q_b are not written)
 * sel     [B, Hkv, n_q, k] int32 or NULL (rows past n_q_b not written)
 * workspace: gsa_prefill_varlen_workspace_size bytes (no zero-fill needed).
 * GSA_ERR_INVALID_ARG / GSA_ERR_UNSUPPORTED as gsa_prefill_blocksparse, and
 * for batch < 1 or base.q_start != 0. Launches as gsa_prefill_blocksparse.
 * ---------------------------------------------------------------------- */
typedef struct {
  gsa_prefill_params base; /* the batch's largest lengths, q_start = 0 */
  int32_t batch;           /* B >= 1 */
} gsa_prefill_varlen_params;

gsa_status_t gsa_prefill_varlen_workspace_size(const gsa_prefill_varlen_params* p, size_t* bytes);
gsa_status_t gsa_prefill_varlen(const gsa_prefill_varlen_params* p, const int32_t* seqs, const void* q,
                                const void* k_cache, const void* v_cache, float* out, int32_t* sel,
                                void* workspace, size_t workspace_bytes, void* stream);
/* Host check of the per-sequence lengths (host array [B][4]): GSA_OK, or
 * GSA_ERR_INVALID_ARG naming the first sequence that breaks a rule. */
gsa_status_t gsa_check_prefill_seqs(const gsa_prefill_varlen_params* p, const int32_t* seqs);

/* ------------------------------------------------------------------------
 * Gist-token attention of one sequence (the step that builds the cache).
 * Source: gist.science explainer, section 2 'Key Concepts: Interleaved Gist
 * Tokens' and 'Technical Innovations' (the gist causal mask), slide deck
 * slide 7: the gist token of chunk m attends to the C raw tokens of chunk m
 * and to the gists of chunks 0..m-1 (not to its own key). This is what a
 * raw query at position mC + C - 1 of gsa_prefill_blocksparse sees with
 * topk = 0 and window = C, and it runs on the same attention kernel.
 * One gist token at decode time (batch of sequences, chunk M just complete,
 * gist M not yet appended) is gsa_decode with topk = 0 and tail = C.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t n_q_heads;   /* Hq, multiple of n_kv_heads; g in {1, 2, 4, 8} */
  int32_t n_kv_heads;  /* Hkv >= 1 */
  int32_t head_dim;    /* D: 128 */
  int32_t chunk;       /* C >= 1 */
  int64_t n_raw;       /* N raw tokens in the cache */
  int64_t n_gist;      /* M gists in the cache; 0 <= N - M*C <= C */
  int64_t m_start;     /* first query's chunk */
  int64_t n_q;         /* gist queries, chunks [m_start, m_start + n_q):
                          each chunk complete ((m_start + n_q) * C <= N) and
                          the gists before it present (m_start + n_q - 1 <= M) */
  float scale;         /* <= 0: 1/sqrt(D) */
  int32_t dtype;       /* GSA_BF16 */
  int64_t row_capacity; /* rows per kv-head in the caches; 0: R = N + M */
} gsa_gist_params;

/*
 * q       [Hq, n_q, D]        gist-token queries (row i is chunk m_start + i)
 * k_cache [Hkv, R, D]         interleaved cache of the sequence
 * v_cache [Hkv, R, D]
 * out     [Hq, n_q, D] fp32   attention output (written)
 * No workspace. With n_q = 0 nothing is launched and q, out may be NULL.
 * GSA_ERR_INVALID_ARG for a NULL pointer or a query range the
 * cache cannot serve; GSA_ERR_UNSUPPORTED for shapes the kernel does not
 * run (as gsa_prefill_blocksparse: bf16, D = 128, g in {1, 2, 4, 8},
 * M <= 262144, N + M < 2^31).
 */
gsa_status_t gsa_gist_prefill(const gsa_gist_params* p, const void* q, const void* k_cache,
                              const void* v_cache, float* out, void* stream);

/* ------------------------------------------------------------------------
 * Cache append: place new tokens' K and V rows at their interleaved slots.
 * Source: gist.science explainer, section 2 'Interleaved Gist Tokens' (a
 * gist token follows every C raw tokens); slide deck slide 7. Raw token p
 * goes to row (p / C) * (C + 1) + p % C, the gist of chunk m to row
 * m * (C + 1) + C, in every (sequence, kv-head) block of row_capacity rows.
 * In time order the tokens fill rows N + M, N + M + 1, ... (a decode step
 * appends one raw row, and one gist row every C steps), but raw and gist
 * rows are given apart and may be appended in any split, e.g. a whole
 * prompt's raw rows and then its gists.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t batch;        /* B >= 1 sequences */
  int32_t n_kv_heads;   /* Hkv >= 1 */
  int32_t head_dim;     /* D: 64 or 128 */
  int32_t chunk;        /* C >= 1 */
  int64_t n_raw;        /* N raw tokens already in the cache */
  int64_t n_gist;       /* M gists already in the cache */
  int64_t raw_new;      /* raw tokens appended: positions [N, N + raw_new) */
  int64_t gist_new;     /* gists appended: chunks [M, M + gist_new) */
  int64_t row_capacity; /* rows per (sequence, kv-head) block, past the
                           highest slot written */
  int32_t dtype;        /* gsa_dtype_t of all rows */
} gsa_append_params;

/*
 * k_raw, v_raw     [B, Hkv, raw_new, D]    rows of the new raw tokens
 * k_gist, v_gist   [B, Hkv, gist_new, D]   rows of the new gists
 * k_cache, v_cache [B, Hkv, row_capacity, D]   written at the new slots only
 * Inputs and caches are device memory and must not overlap (checked).
 * Gists only of complete chunks: M * C <= N before and M' * C <= N' after,
 * with N' = N + raw_new, M' = M + gist_new; raw rows may run ahead of the
 * gists, their slots waiting. row_capacity must reach the highest slot
 * written. Else GSA_ERR_INVALID_ARG. The readers (gsa_decode, the prefills)
 * need the gists caught up, 0 <= N - M*C <= C. Empty appends return
 * GSA_OK; pointers of an empty side may be NULL.
 */
gsa_status_t gsa_cache_append(const gsa_append_params* p, const void* k_raw, const void* v_raw,
                              const void* k_gist, const void* v_gist, void* k_cache, void* v_cache,
                              void* stream);

/* ------------------------------------------------------------------------
 * Timing hook (not part of the method): arm this thread with n caller-owned
 * hipEvent_t handles (passed as void*). Every later call on this thread
 * attaches them to its kernel launches (hipExtLaunchKernel): events[0] takes
 * the start of the call's first kernel and events[i] the end of its i-th
 * kernel, for as many events as there are. The launch count of a call comes
 * from the gsa_*_launches queries below (gsa_gist_prefill: 1 launch when
 * n_q > 0; gsa_cache_append: 1 when anything is appended; 0 otherwise).
 * The library never creates, waits on or destroys the events. n = 0 disarms.
 * Returns GSA_ERR_INVALID_ARG for n outside [0, 8] or a NULL handle.
 * ---------------------------------------------------------------------- */
gsa_status_t gsa_profile_events(void* const* events, int32_t n);

/* Number of marks (kernel launches + 1) the last call of a launching entry
 * point on this thread made, armed or not (a rejected call launched nothing:
 * 1); 0 before any such call. GSA_ERR_INVALID_ARG for a NULL n. */
gsa_status_t gsa_profile_marks(int32_t* n);

/* Host-only queries: *n = the number of kernel launches a call with these
 * parameters makes (the timing hook takes *n + 1 events), after the same
 * validation as the call itself (its status on failure). The counts:
 *   gsa_decode / gsa_decode_varlen / gsa_decode_paged (its base) on the
 *     bf16, D = 128, topk <= 64 path
 *     (n_gist <= 16384 when topk > 0): 1 when each (batch, kv-head) unit
 *     takes one workgroup (B*Hkv >= 256 and n_gist <= 4096) or topk = 0,
 *     else 2 (a stream launch, then a select-unfold-merge launch); with
 *     gist_set 1 or 2 and several workgroups per unit: a scoring launch
 *     (none when topk = 0), then the launch that selects and attends;
 *     other shapes: 1 when topk = 0, else 2 or 3 (a gist pass, a pass that
 *     takes each split's top-k when there are many gists per unit, an
 *     unfold pass); with gist_set 1 or 2: a scoring pass (none when
 *     topk = 0), the split top-k pass when there is one, and the pass that
 *     attends the set;
 *   gsa_decode_hier on the bf16, D = 128, k1, k2 <= 64 path: 1 (the
 *     level-2 stream, whose last workgroup per unit runs the descent);
 *     other shapes: 2 to 4 (a level-2
 *     pass, possibly a pass over its splits' top-k2, a level-1 candidate
 *     pass, and an unfold pass when topk1 > 0 or base.gist_set is 1 or 2);
 *   gsa_decode_levels on the bf16, D = 128, every k <= 64 path: 1 when the
 *     top level holds <= 4096 gists and top + tail <= 5120 rows, else 2;
 *     other shapes: one pass per level and an unfold pass when k_1 > 0 or
 *     base.gist_set is 1 or 2;
 *   gsa_prefill_blocksparse: 0 when n_q = 0, else a selection launch when
 *     topk > 0 and an attention launch.
 * GSA_ERR_INVALID_ARG for a NULL n. */
gsa_status_t gsa_decode_launches(const gsa_decode_params* p, int32_t* n);
gsa_status_t gsa_decode_hier_launches(const gsa_hier_params* p, int32_t* n);
gsa_status_t gsa_decode_levels_launches(const gsa_levels_params* p, int32_t* n);
gsa_status_t gsa_prefill_launches(const gsa_prefill_params* p, int32_t* n);

/* ------------------------------------------------------------------------
 * Fixed-token-budget mode (slide deck, slide 17: under one token budget,
 * leaving out the unselected chunks' gists leaves room for more unfolded
 * chunks). Host only.
 * *topk = the largest k <= n_gist whose attention set under gist_set holds at
 * most `budget` tokens, counting n_gist gists (GSA_GISTS_ALL) or k gists
 * (GSA_GISTS_SELECTED) or none, plus k * chunk raw tokens and `tail` tail
 * tokens with no overlap (k is fixed before the selection, so this is the
 * most the set can hold).
 * GSA_ERR_INVALID_ARG for n_gist < 0, chunk < 1, tail < 0, an unknown
 * gist_set, a NULL topk, or a budget below the k = 0 set.
 * ---------------------------------------------------------------------- */
gsa_status_t gsa_topk_for_budget(int64_t budget, int64_t n_gist, int32_t chunk, int32_t tail,
                                 int32_t gist_set, int32_t* topk);

/* Static description of a status code. */
const char* gsa_status_string(gsa_status_t s);

/* Reason for the last non-OK status returned on the calling thread ("" if none). */
const char* gsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GSA_H_ */
