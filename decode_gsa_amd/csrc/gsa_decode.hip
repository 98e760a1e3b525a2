// GSA decode on gfx950: gist scoring + online softmax over every gist, exact
// top-k chunk selection, unfolding of the chosen chunks' raw rows, the tail,
// and a log-sum-exp merge, per (batch, kv-head) unit.
//
// Method: gist.science explainer "Forget, Then Recall", section 2 'Key
// Concepts' (routing by gist scores, top-k selection, selective unfolding,
// hybrid attention) and 'Hierarchical Extension (H-GSA)' for the two-level
// entry point (score the meta-gists, then the gists of the chosen groups,
// then unfold raw chunks).
//
// Launch shapes:
//   unit path (bf16, D = 128, k <= 64): a workgroup's four waves stream rows
//                 on MFMA through direct-to-LDS rings, keep the group scores
//                 in LDS and run an exact top-k in LDS.
//     unit_kernel alone (>= 256 units, <= 4096 gists): one workgroup runs a
//                 unit's whole step -- gists and tail, the top-k, the chosen
//                 chunks' raw rows, the merge of its four waves' softmax
//                 states. Nothing is handed off through memory.
//     unit_kernel + unit_unfold_kernel (fewer units or more gists): S
//                 workgroups per unit stream shares of the gists and tail and
//                 hand on their partial states and either the scores at or
//                 above a bound on their own k-th best (k <= 16) or all
//                 their group scores; S2 workgroups per unit then each make
//                 the unit's selection among those, stream a share of the
//                 chosen raw rows, and the last one merges every partial
//                 (k = 0: the stream launch's last workgroup merges).
//     unit_kernel<HIER> (two-level decode, one launch): S workgroups per
//                 unit stream the level-2 gists and the tail and hand on
//                 their partial states and level-2 scores; the unit's last
//                 one then selects the level-2 groups, streams the candidate
//                 level-1 gists, selects the chunks, unfolds them and merges.
//   gist_kernel + unfold_kernel (every other shape: fp32, D = 64, k > 64, ...)
//                 split-K over gists: each gist workgroup streams a range of
//                 gist rows (and a share of the tail), keeps its group scores
//                 and writes one online-softmax partial (m, l, acc[D]) per
//                 query head; the unit's last workgroup to finish (an atomic
//                 counter) selects the unit's top-k from the scores. The
//                 unfold launch streams the chosen chunks' raw rows (rows the
//                 tail owns are skipped) and the unit's last workgroup merges
//                 every partial into out and lse. Two-level decode runs
//                 level-2 gists, then the candidate level-1 gists, then the
//                 unfold.
//
// In the split path memory-bound work stays on the VALU: 16 lanes cover one
// 256-byte row with one 16-byte load each, q.k uses v_dot2_f32_bf16, the
// 16-lane sum uses DPP, and the softmax weights stay fp32. Hand-off data
// between workgroups (scores, partials) is written with device-scope stores
// and read with device-scope loads: the XCDs' L2s are not coherent.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>
#include <type_traits>

#include "gsa.h"
#include "gsa_device.hpp"
#include "gsa_plan.hpp"
#include "gsa_profile.hpp"

// Phase stamps: a diagnostic build of the library (-DGSA_PHASE_STAMPS,
// libgsa_stamps.so; the product build has none of it). Thread 0 of a
// workgroup of the unit-path decode kernels records the chip's 100 MHz
// real-time counter at the edges of its phases, in slot [blockIdx][slot]:
//   unit_kernel: 0 start, 1 its wave's gists + tail streamed, then with one
//     workgroup per unit 2 selection made, 3 chosen rows unfolded, 4 output
//     written; with several (and two-level): 5 partial state written,
//     6 candidates or scores handed on;
//   unit_unfold_kernel: 8 start, 9 selection made, 10 its rows unfolded,
//     11 partial state written, 12 merged (the unit's last workgroup);
//   two-level descent (the unit's last stream workgroup): 8 start, 9 level-2
//     choice, 10 candidates streamed, 11 level-1 choice, 12 unfolded,
//     13 partial state written, 14 merged.
// gsa_debug_phase_stamps copies [workgroups][kStampSlots] out and clears it.
#ifdef GSA_PHASE_STAMPS
constexpr int kStampSlots = 16;
constexpr int kStampWGs = 32768;
__device__ unsigned long long g_phase_stamps[kStampWGs * kStampSlots];
#define GSA_STAMP(slot)                                                                               \
  do {                                                                                                \
    if (threadIdx.x == 0 && blockIdx.x < kStampWGs)                                                   \
      g_phase_stamps[(size_t)blockIdx.x * kStampSlots + (slot)] = __builtin_amdgcn_s_memrealtime();   \
  } while (0)
extern "C" int gsa_debug_phase_stamps(void* host, size_t bytes) {
  if (bytes > sizeof(g_phase_stamps)) bytes = sizeof(g_phase_stamps);
  hipError_t e = hipMemcpyFromSymbol(host, HIP_SYMBOL(g_phase_stamps), bytes, 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return (int)e;
  static std::vector<unsigned long long> zeros(sizeof(g_phase_stamps) / sizeof(unsigned long long), 0ull);
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(g_phase_stamps), zeros.data(), sizeof(g_phase_stamps), 0,
                                hipMemcpyHostToDevice);
}
#else
#define GSA_STAMP(slot) ((void)0)
#endif

namespace gsa {
namespace {

using namespace dev;

constexpr int kThreads = 256;   // 4 waves per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kU = 2;           // rows per lane group per batch (two batches in flight)
constexpr int kTaskScores = 1024;        // scores a gist workgroup gathers in LDS
constexpr int kSelLds = 1024;   // selected chunk ids staged in LDS by unfold tasks

template <bool BF16, int D>
struct Geo {
  static constexpr int VEC = Slice<BF16>::N;        // elements per lane
  static constexpr int LPR = D / VEC;               // lanes per row
  static constexpr int SLOTS = 64 / LPR;            // rows per wave instruction
  static constexpr int NS = SLOTS * kWaves;         // row slots per workgroup
  static constexpr int ROW_BYTES = D * (BF16 ? 2 : 4);
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "unsupported lane split");
};

// Running online-softmax state of one lane group, per query head.
template <bool BF16, int G>
struct State {
  float m[G], l[G], acc[G][Slice<BF16>::N];
};

// How item i of a gist pass maps to a cache row of the unit.
struct RowMap {
  int32_t kind;          // 0: gist i of the interleaved cache; 1: dense row i;
                         // 2: level-1 candidate i of a two-level call
  int32_t C;
  const int32_t* sel2;   // kind 2: chosen level-2 groups, sel2_stride ints per unit
  int32_t G, k2;
  int64_t orphan0;       // kind 2: first level-1 gist no group covers
  int64_t sel2_stride;
};

// sel2 was written by an earlier launch: plain loads see it.
__device__ __forceinline__ int64_t map_row(const RowMap& rm, int unit, int64_t i) {
  if (rm.kind == 0) return i * (rm.C + 1) + rm.C;
  if (rm.kind == 1) return i;
  const int64_t kg = (int64_t)rm.k2 * rm.G;
  int64_t m;
  if (i < kg) {
    int64_t grp = rm.sel2[(int64_t)unit * rm.sel2_stride + i / rm.G];
    if (grp < 0 || grp * rm.G >= rm.orphan0) grp = 0;   // keeps reads in bounds; never taken
    m = grp * rm.G + i % rm.G;
  } else {
    m = rm.orphan0 + (i - kg);
  }
  return m * (rm.C + 1) + rm.C;
}

// Id reported for item i of a selection.
struct IdMap {
  const int32_t* sel2;  // nullptr: id = item index; else level-1 candidate ids
  int32_t G, k2;
  int64_t orphan0;
  int64_t sel2_stride;
};

__device__ __forceinline__ int32_t map_id(const IdMap& im, int unit, int32_t i) {
  if (im.sel2 == nullptr) return i;
  const int32_t kg = im.k2 * im.G;
  return i < kg ? im.sel2[(size_t)unit * im.sel2_stride + i / im.G] * im.G + i % im.G
                : (int32_t)(im.orphan0 + (i - kg));
}

// Variable-length batches: sequence b holds seq_n[b] raw tokens and
// seq_m[b] gists (device arrays); N and M of the call are the batch's
// largest. A sequence whose pair breaks the rules a call checks for uniform
// lengths (1 <= n <= N, k <= m <= M, m C <= n <= m C + C, n - m C <= T <= n)
// is run with (N, M) instead: every row read stays inside its slab.
struct SeqLens {
  const int32_t* n;       // [B] or null (every sequence has N, M)
  const int32_t* m;
  int32_t Hkv;
  int32_t k;              // the call's top-k (a sequence needs k <= m)
  int32_t G2, k2;         // two-level decode: fanout and top-k2 (else 0)
};

__device__ __forceinline__ void unit_lengths(const SeqLens& sl, int unit, int64_t N, int64_t M, int32_t C,
                                             int32_t T, int64_t* n_out, int64_t* m_out) {
  *n_out = N;
  *m_out = M;
  if (sl.n == nullptr) return;
  const int k = sl.k;
  const int b = unit / sl.Hkv;
  const int64_t n = sl.n[b], m = sl.m[b];
  const bool ok = n >= 1 && n <= N && m >= k && m <= M && m * C <= n && n <= m * C + C && n - m * C <= T && T <= n;
  if (ok) {
    *n_out = n;
    *m_out = m;
  }
}

// Two-level decode with per-sequence lengths: the sequence's N and M as
// unit_lengths gives them, its level-2 gists M2 = floor(M / G) (the first
// rows of its level-2 slab) and its level-1 candidates k2 G + (M - M2 G). A
// sequence whose lengths break a rule (unit_lengths', k2 <= M2, k1 at most
// its candidates) runs with the call's maxima.
__device__ __forceinline__ void hier_lengths(const SeqLens& sl, int unit, int64_t N, int64_t M, int32_t C,
                                             int32_t T, int64_t M2, int32_t n_cand, int64_t* n_out,
                                             int64_t* m_out, int64_t* m2_out, int32_t* nc_out) {
  *m2_out = M2;
  *nc_out = n_cand;
  unit_lengths(sl, unit, N, M, C, T, n_out, m_out);
  if (sl.n == nullptr || *m_out == M) return;   // maxima (also a sequence at the largest M)
  const int64_t m = *m_out, m2 = m / sl.G2;
  const int64_t nc = (int64_t)sl.k2 * sl.G2 + (m - m2 * sl.G2);
  if (sl.k2 <= m2 && sl.k <= nc) {
    *m2_out = m2;
    *nc_out = (int32_t)nc;
  } else {
    *n_out = N;
    *m_out = M;
  }
}

// Stream items [i0, i1) of one unit through the online softmax. row_of(i)
// gives the cache row of item i; with CAN_SKIP it may return -1 to skip the
// item. When score_out is set (LDS), the group score of item i goes to
// score_out[i - i0]; with score_only the V rows are neither read nor folded
// in (the items only route: their scores are all that is kept).
//
// Rows are double-buffered in registers: the loads of the next batch are in
// flight while the current one is folded in. A batch is kU rows per lane group
// of every wave; the four waves of the workgroup cover consecutive rows.
//
// The running max is raised lazily: only when a new scaled logit exceeds it by
// more than kLazy (log2 units); the softmax weights of the state then stay
// below 2^kLazy, far inside fp32 range, and most batches skip the rescale.
constexpr float kLazy = 8.f;

template <bool BF16, int D, int G, bool CAN_SKIP, class RowOf>
__device__ __forceinline__ void stream_rows(const char* __restrict__ Kb, const char* __restrict__ Vb,
                                            int64_t i0, int64_t i1, RowOf row_of,
                                            const uint4 (&qv)[G], State<BF16, G>& st,
                                            float scale_log2, float* __restrict__ score_out,
                                            float score_mul, bool score_only = false) {
  using Gm = Geo<BF16, D>;
  constexpr int VEC = Gm::VEC, LPR = Gm::LPR, NS = Gm::NS;
  const int lane = threadIdx.x & 63;
  const int lr = lane % LPR;
  const int slot = (threadIdx.x >> 6) * Gm::SLOTS + lane / LPR;
  constexpr int64_t kPer = (int64_t)NS * kU;     // items per batch (whole workgroup)
  const int64_t n = i1 - i0;
  const int64_t iters = n > 0 ? (n + kPer - 1) / kPer : 0;
  const size_t lane_off = (size_t)lr * 16;
  const float c = scale_log2;

  struct Batch {
    uint4 k[kU], v[kU];
    bool ok[kU];
  };
  auto load = [&](int64_t it, Batch& b) {
    const int64_t base = i0 + it * kPer;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t item = base + u * NS + slot;
      const int64_t row = item < i1 ? row_of(item) : -1;
      b.ok[u] = row >= 0;
      if (row >= 0) {
        const size_t off = (size_t)row * Gm::ROW_BYTES + lane_off;
        b.k[u] = load16_stream(Kb + off);
        b.v[u] = score_only ? make_uint4(0u, 0u, 0u, 0u) : load16_stream(Vb + off);
      } else {
        b.k[u] = make_uint4(0u, 0u, 0u, 0u);
        b.v[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  auto fold = [&](int64_t it, const Batch& b) {
    const int64_t base = i0 + it * kPer;
    float s[kU][G];   // raw q.k
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int h = 0; h < G; ++h) s[u][h] = group_sum<LPR>(dot_slice<BF16>(qv[h], b.k[u]));
    if (score_out != nullptr) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (b.ok[u] && lr == 0) {
          float t = 0.f;
#pragma unroll
          for (int h = 0; h < G; ++h) t += s[u][h];
          score_out[base + u * NS + slot - i0] = t * score_mul;
        }
      }
    }
    if (score_only) return;
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int h = 0; h < G; ++h) s[u][h] = b.ok[u] ? s[u][h] : -INFINITY;
    float cand[G];
    bool need = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = s[0][h];
#pragma unroll
      for (int u = 1; u < kU; ++u) mx = fmaxf(mx, s[u][h]);
      cand[h] = mx * c;
      need |= cand[h] > st.m[h] + kLazy;
    }
    if (__ballot(need) != 0ull) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = cand[h] > st.m[h] + kLazy ? cand[h] : st.m[h];
        const float a = fexp2(st.m[h] - mn);
        st.m[h] = mn;
        st.l[h] *= a;
#pragma unroll
        for (int e = 0; e < VEC; ++e) st.acc[h][e] *= a;
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float vf[VEC];
      widen<BF16>(b.v[u], vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = fexp2(fmaf(s[u][h], c, -st.m[h]));
        st.l[h] += p;
#pragma unroll
        for (int e = 0; e < VEC; ++e) st.acc[h][e] = fmaf(p, vf[e], st.acc[h][e]);
      }
    }
  };
  (void)sizeof(CAN_SKIP);

  Batch A, B;
  if (iters > 0) load(0, A);
  for (int64_t it = 0; it < iters; it += 2) {
    if (it + 1 < iters) load(it + 1, B);
    fold(it, A);
    if (it + 1 >= iters) break;
    if (it + 2 < iters) load(it + 2, A);
    fold(it + 1, B);
  }
}

template <int D, int G>
struct PartLds {
  float m[kWaves][G], l[kWaves][G];
  float acc[kWaves][G][D];
};

// Merge the lane groups' states of the workgroup and write one partial
// (m, l, acc[D]) per head to `dst` ([G][D + 2] floats).
template <bool BF16, int D, int G>
__device__ __forceinline__ void write_partial(State<BF16, G>& st, float* __restrict__ dst,
                                              PartLds<D, G>& L, bool poison) {
  using Gm = Geo<BF16, D>;
  constexpr int VEC = Gm::VEC, LPR = Gm::LPR;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane % LPR;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mw = st.m[h];
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) mw = fmaxf(mw, __shfl_xor(mw, off));
    const float f = fexp2(st.m[h] - mw);
    float l = st.l[h] * f;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = st.acc[h][e] * f;
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
      l += __shfl_xor(l, off);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], off);
    }
    if (lane < LPR) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) L.acc[w][h][lr * VEC + e] = acc[e];
      if (lane == 0) {
        L.m[w][h] = mw;
        L.l[w][h] = l;
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    float M = L.m[0][h];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, L.m[ww][h]);
    float S = 0.f, A = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = fexp2(L.m[ww][h] - M);
      S = fmaf(L.l[ww][h], f, S);
      A = fmaf(L.acc[ww][h][d], f, A);
    }
    st_coh(dst + h * (D + 2) + 2 + d, A);
    if (d == 0) {
      st_coh(dst + h * (D + 2), M);
      st_coh(dst + h * (D + 2) + 1, poison ? NAN : S);
    }
  }
}

// ------------------------------------------------------------- top-k -------

constexpr int kSelKeys = 4096;                    // keys staged in LDS by the selector
constexpr int kSub = 4;                           // items per thread per round
constexpr int kRound = kThreads * kSub;           // items per round (1024)
constexpr int kStage = kSelKeys / kThreads;       // staging loads per thread (all in flight)
constexpr int kDigitBits = 8;                     // radix digit; 4 passes cover 32 bits
constexpr int kBins = 1 << kDigitBits;

struct TopkLds {
  uint32_t hist[kBins];
  uint32_t keys[kSelKeys];
  int scan[kWaves];
  int bcast[3];
  int cnt[kSub][kWaves];
};

// Exclusive prefix over threads of v; *total gets the sum over the block.
__device__ __forceinline__ int block_scan_total(int v, int* buf, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) buf[w] = x;
  __syncthreads();
  int base = 0, t = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int b = buf[i];
    base += i < w ? b : 0;
    t += b;
  }
  __syncthreads();
  *total = t;
  return base + x - v;
}

// Keys of items b0 + s*kThreads + tid (s < kSub): from LDS when staged,
// else device-scope loads issued together.
__device__ __forceinline__ void round_keys(const CohBuf& sc, int n, int b0, bool in_lds,
                                           const TopkLds& L, uint32_t (&kr)[kSub]) {
#pragma unroll
  for (int q = 0; q < kSub; ++q) {
    const int i = b0 + q * kThreads + (int)threadIdx.x;
    const uint32_t g = in_lds ? 0u : sc.u32(i);
    kr[q] = i < n ? (in_lds ? L.keys[i] : order_key(__uint_as_float(g))) : 0u;
  }
}

// Block-wide exclusive prefix, in item order (round-major, then thread), of
// one round's per-item flags; `bal` holds this wave's ballots. Writes this
// thread's prefix per item to pre[] and adds the round total to *base.
__device__ __forceinline__ void round_prefix(const uint64_t (&bal)[kSub], int (&pre)[kSub],
                                             int* base, TopkLds& L) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
#pragma unroll
    for (int q = 0; q < kSub; ++q) L.cnt[q][w] = __popcll(bal[q]);
  }
  __syncthreads();
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  int run = *base;
#pragma unroll
  for (int q = 0; q < kSub; ++q) {
    int before = 0, tot = 0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const int c = L.cnt[q][ww];
      before += ww < w ? c : 0;
      tot += c;
    }
    pre[q] = run + before + __popcll(bal[q] & lt);
    run += tot;
  }
  *base = run;
  __syncthreads();
}

// Exact top-k of the n scores sc[0..n) of one unit, written in ascending item
// order (ids through `im`) to dst (device-scope stores) and, if set, dst2.
// Keys are the scores' order-preserving uint32 images; ties go to the smaller
// item index. Radix select, most significant 8-bit digit first:
// each pass histograms the keys that still match the known prefix, finds the
// digit holding the k-th largest key, and stops early once that digit's keys
// are all needed. The result is every key whose prefix is above the found
// prefix plus the first `need` keys equal to it, in item order. Up to 4096
// keys are staged in LDS once (one round trip); more are re-read in rounds.
__device__ void block_topk(const float* __restrict__ scores, int n, int k, const IdMap& im, int unit,
                           int32_t* __restrict__ dst, TopkLds& L) {
  const int tid = threadIdx.x;
  const CohBuf sc(scores, (uint32_t)n * 4u);
  if (k <= 0) return;
  if (k >= n) {
    for (int i = tid; i < n; i += kThreads) dst[i] = map_id(im, unit, i);
    return;
  }
  const bool in_lds = n <= kSelKeys;
  if (in_lds) {   // stage every key with one round of independent loads
    uint32_t kr[kStage];
#pragma unroll
    for (int q = 0; q < kStage; ++q) {
      const int i = q * kThreads + tid;
      const uint32_t g = sc.u32(i);
      kr[q] = i < n ? order_key(__uint_as_float(g)) : 0u;
    }
#pragma unroll
    for (int q = 0; q < kStage; ++q) {
      const int i = q * kThreads + tid;
      if (i < n) L.keys[i] = kr[q];
    }
    __syncthreads();
  }
  uint32_t prefix = 0u, pmask = 0u;
  int need = k;
#pragma unroll 1
  for (int pass = 0; pass < 32 / kDigitBits; ++pass) {
    const int sh = 32 - kDigitBits * (pass + 1);
    const int nb = kBins;
    const uint32_t dm = (uint32_t)nb - 1u;
    for (int b = tid; b < nb; b += kThreads) L.hist[b] = 0u;
    __syncthreads();
    for (int b0 = 0; b0 < n; b0 += kRound) {
      uint32_t kr[kSub];
      round_keys(sc, n, b0, in_lds, L, kr);
#pragma unroll
      for (int q = 0; q < kSub; ++q) {
        const int i = b0 + q * kThreads + tid;
        if (i < n && (kr[q] & pmask) == prefix) atomicAdd(&L.hist[(kr[q] >> sh) & dm], 1u);
      }
    }
    __syncthreads();
    const int per = nb / kThreads;              // digits owned by this thread
    int c = 0;
    for (int j = 0; j < per; ++j) c += (int)L.hist[tid * per + j];
    int total;
    const int excl = block_scan_total(c, L.scan, &total);
    const int above_t = total - excl - c;       // keys in digits owned by higher threads
    if (above_t < need && need <= above_t + c) {
      int acc = above_t;
      for (int j = per - 1; j >= 0; --j) {
        const int h = (int)L.hist[tid * per + j];
        if (acc + h >= need) {
          L.bcast[0] = tid * per + j;
          L.bcast[1] = acc;
          L.bcast[2] = h;
          break;
        }
        acc += h;
      }
    }
    __syncthreads();
    const uint32_t dg = (uint32_t)L.bcast[0];
    const int above = L.bcast[1], inbin = L.bcast[2];
    __syncthreads();
    need -= above;
    prefix |= dg << sh;
    pmask |= dm << sh;
    if (need == inbin) break;                   // every key with this prefix is taken
  }
  // ordered compaction: ranks among equal keys, then output positions
  int eq_base = 0, pos_base = 0;
  for (int b0 = 0; b0 < n; b0 += kRound) {
    uint32_t kr[kSub];
    round_keys(sc, n, b0, in_lds, L, kr);
    uint64_t bal[kSub];
    bool gt[kSub], eq[kSub];
#pragma unroll
    for (int q = 0; q < kSub; ++q) {
      const int i = b0 + q * kThreads + tid;
      const uint32_t mk = kr[q] & pmask;
      gt[q] = i < n && mk > prefix;
      eq[q] = i < n && mk == prefix;
      bal[q] = __ballot(eq[q]);
    }
    int pre[kSub];
    round_prefix(bal, pre, &eq_base, L);
    bool pick[kSub];
#pragma unroll
    for (int q = 0; q < kSub; ++q) {
      pick[q] = gt[q] || (eq[q] && pre[q] < need);
      bal[q] = __ballot(pick[q]);
    }
    round_prefix(bal, pre, &pos_base, L);
#pragma unroll
    for (int q = 0; q < kSub; ++q) {
      const int pos = pre[q];
      if (pick[q] && pos >= 0 && pos < k) dst[pos] = map_id(im, unit, b0 + q * kThreads + tid);
    }
  }
}

// Exact top-k inside one wave, without barriers or LDS. The wave holds up to
// 64*EM items, item (e, lane) = e*64 + lane, in ascending id order; key is the
// order-preserving image of the score (order_key), 0 for "no item". A bit-
// serial radix search (one ballot per slot and bit) finds P, the k-th largest
// key; every key above P is taken and the keys equal to P fill the remaining
// places in item order, so ties go to the smaller id. Returns per slot the
// ballot of taken items; fewer than k valid items are all taken.
template <int EM>
__device__ __forceinline__ void wave_topk(const uint32_t (&key)[EM], int E, int k, uint64_t (&take)[EM]) {
  const int lane = threadIdx.x & 63;
  uint32_t P = 0u;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = P | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < EM; ++e)
      if (e < E) cnt += __popcll(__ballot(key[e] >= c));
    if (cnt >= k) P = c;
  }
  int gt = 0;
#pragma unroll
  for (int e = 0; e < EM; ++e)
    if (e < E) gt += __popcll(__ballot(key[e] > P));
  const int need = k - gt;
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  int eq_before = 0;
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    take[e] = 0ull;
    if (e < E) {
      const uint64_t be = __ballot(key[e] == P && key[e] != 0u);
      const bool eq = (be >> lane) & 1ull;
      take[e] = __ballot(key[e] > P || (eq && eq_before + __popcll(be & lt) < need));
      eq_before += __popcll(be);
    }
  }
}

constexpr int kSlots = 5;           // wave_topk slots: the running selection + 256 items
constexpr int kFastSel = kFastSelect;
static_assert(kFastSel <= 64, "the running selection must fit one slot");

// Position of this lane's item (e) among the taken items, in item order.
template <int EM>
__device__ __forceinline__ int taken_before(const uint64_t (&take)[EM], int e) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  int pos = __popcll(take[e] & lt);
#pragma unroll
  for (int f = 0; f < EM; ++f)
    if (f < e) pos += __popcll(take[f]);
  return pos;
}

// Make this wave's LDS writes visible to its own later reads in other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wave: top-k over n items (key, id) in ascending id order, fetched by
// item(i, &key, &id) (key 0 = no item). Items are taken in blocks of
// 64*(kSlots-1); slot 0 carries the selection so far, whose ids precede the
// block's. xs is this wave's LDS scratch. Afterwards lane j < k holds the j-th
// selected item (ascending id) in run_key / run_id.
template <class Item>
__device__ __forceinline__ void wave_select(int n, int k, Item item, uint32_t (*xs)[64],
                                            uint32_t& run_key, uint32_t& run_id) {
  const int lane = threadIdx.x & 63;
  run_key = 0u;
  run_id = 0u;
  constexpr int kBlock = 64 * (kSlots - 1);
  for (int c0 = 0; c0 < n; c0 += kBlock) {
    uint32_t key[kSlots], id[kSlots];
    key[0] = run_key;
    id[0] = run_id;
#pragma unroll
    for (int e = 1; e < kSlots; ++e) item(c0 + (e - 1) * 64 + lane, key[e], id[e]);
    const int rest = n - c0 < kBlock ? n - c0 : kBlock;
    const int E = 1 + (rest + 63) / 64;
    uint64_t take[kSlots];
    wave_topk<kSlots>(key, E, k, take);
    int total = 0;
#pragma unroll
    for (int e = 0; e < kSlots; ++e) {
      if (e < E && ((take[e] >> lane) & 1ull)) {
        const int pos = taken_before<kSlots>(take, e);
        xs[0][pos] = key[e];
        xs[1][pos] = id[e];
      }
      total += __popcll(take[e]);
    }
    wave_lds_sync();
    run_key = lane < total ? xs[0][lane] : 0u;
    run_id = lane < total ? xs[1][lane] : 0u;
    wave_lds_sync();
  }
}

// ------------------------------------------------------------- merge -------

constexpr int kMergeBatch = 8;   // partials whose loads are in flight together

// out[h][d] = sum_j 2^(m_j - m*) acc_j[d] / sum_j 2^(m_j - m*) l_j over the
// unit's NP partials. One wave per head; each lane owns D/64 output elements;
// the device-scope loads of a batch of partials are issued together (one
// round trip per batch) and folded into a running (max, sum, acc) state.
template <int D, int G>
__device__ void merge_unit(const float* __restrict__ part_u, int NP, uint32_t ps,
                           float* __restrict__ out, float* __restrict__ lse, int waves) {
  constexpr int PL = D / 64;                  // outputs per lane
  const CohBuf P(part_u, (uint32_t)NP * ps * 4u);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int h = w; h < G; h += waves) {
    float mx = kMinus, L = 0.f, acc[PL];
#pragma unroll
    for (int e = 0; e < PL; ++e) acc[e] = 0.f;
    for (int j0 = 0; j0 < NP; j0 += kMergeBatch) {
      float m[kMergeBatch], l[kMergeBatch], a[kMergeBatch][PL];
#pragma unroll
      for (int b = 0; b < kMergeBatch; ++b) {
        // past NP the buffer returns 0: those slots get weight 0 below
        const uint32_t o = (uint32_t)(j0 + b) * ps + (uint32_t)h * (D + 2);
        m[b] = __uint_as_float(P.u32(o));
        l[b] = __uint_as_float(P.u32(o + 1));
#pragma unroll
        for (int e = 0; e < PL; ++e) a[b][e] = __uint_as_float(P.u32(o + 2 + lane + 64 * e));
      }
#pragma unroll
      for (int b = 0; b < kMergeBatch; ++b) m[b] = j0 + b < NP ? m[b] : kMinus;
      float nm = mx;
#pragma unroll
      for (int b = 0; b < kMergeBatch; ++b) nm = fmaxf(nm, m[b]);
      const float r = fexp2(mx - nm);
      L *= r;
#pragma unroll
      for (int e = 0; e < PL; ++e) acc[e] *= r;
#pragma unroll
      for (int b = 0; b < kMergeBatch; ++b) {
        const float f = j0 + b < NP ? fexp2(m[b] - nm) : 0.f;
        L = fmaf(l[b], f, L);
#pragma unroll
        for (int e = 0; e < PL; ++e) acc[e] = fmaf(a[b][e], f, acc[e]);
      }
      mx = nm;
    }
#pragma unroll
    for (int e = 0; e < PL; ++e) out[(size_t)h * D + lane + 64 * e] = acc[e] / L;
    if (lse != nullptr && lane == 0) lse[h] = (mx + log2f(L)) * kLn2;
  }
}

// ---------------------------------------------------------- hand-offs ------

// Every write of a control word is an atomic read-modify-write: those are
// performed at one coherence point for the whole chip, whereas two plain
// stores to one word from different XCDs go through different L2 caches and
// may reach memory in either order.
__device__ __forceinline__ void ctrl_set(uint32_t* w, uint32_t v) {
  (void)__hip_atomic_exchange(w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Count this workgroup finished once its hand-off stores have completed;
// true in the unit's last one, which then resets the counter for the next
// launch. The last one reads the others' data with device-scope loads.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected, uint32_t* s_old) {
  done_stores();
  __syncthreads();
  if (threadIdx.x == 0)
    *s_old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const bool last = *s_old == expected - 1u;
  if (last && threadIdx.x == 0) ctrl_set(counter, 0u);
  return last;
}

template <bool BF16, int D, int G>
__device__ __forceinline__ void load_q(const void* q, int unit, uint4 (&qv)[G]) {
  using Gm = Geo<BF16, D>;
  const int lr = (threadIdx.x & 63) % Gm::LPR;
  const char* qb = reinterpret_cast<const char*>(q) + (size_t)unit * G * Gm::ROW_BYTES;
#pragma unroll
  for (int h = 0; h < G; ++h) qv[h] = load16(qb + (size_t)h * Gm::ROW_BYTES + (size_t)lr * 16);
}

template <bool BF16, int G>
__device__ __forceinline__ void init_state(State<BF16, G>& st) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = kMinus;
    st.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < Slice<BF16>::N; ++e) st.acc[h][e] = 0.f;
  }
}

// -------------------------------------------------------------- tail rows ---

// Cache row of tail item i (position N - T + i) of the interleaved cache.
__device__ __forceinline__ int64_t tail_row(int64_t i, int64_t N, int32_t T, int64_t M, int32_t C) {
  const int64_t pos = N - T + i, MC = M * C;
  return pos < MC ? (pos / C) * (C + 1) + pos % C : M * (C + 1) + (pos - MC);
}

// ------------------------------------------------------------ selection ----

constexpr int kSelLdsMax = 1024;   // selections staged in LDS by the workgroups that use them
constexpr int kCandMax = 64;       // candidates above the threshold: one per lane of a wave

struct SelectLds {
  uint32_t tw[kWaves];             // per-wave lower bounds on the k-th largest key
  uint32_t ck[kCandMax];           // candidates (key, id), in no particular order
  uint32_t ci[kCandMax];
  int cnt;
};


// One compare-exchange step of a bitonic network at distance J within blocks of K.
template <bool DESC, int K, int J, class T>
__device__ __forceinline__ T bitonic_step(T x) {
  const int lane = threadIdx.x & 63;
  const T y = lane_xor<J>(x);
  const bool seg_desc = ((lane & K) == 0) == DESC;
  const bool keep_max = ((lane & J) == 0) == seg_desc;
  return keep_max ? (x > y ? x : y) : (x < y ? x : y);
}
template <bool DESC, int K, int J, class T>
__device__ __forceinline__ T bitonic_stage(T x) {
  x = bitonic_step<DESC, K, J>(x);
  if constexpr (J > 1) x = bitonic_stage<DESC, K, J / 2>(x);
  return x;
}
template <bool DESC, int K, class T>
__device__ __forceinline__ T bitonic_from(T x) {
  x = bitonic_stage<DESC, K, K / 2>(x);
  if constexpr (K < 64) x = bitonic_from<DESC, K * 2>(x);
  return x;
}

// Bitonic sort of one value per lane over the wave's 64 lanes, descending
// (lane 0 largest) or ascending.
template <bool DESC, class T>
__device__ __forceinline__ T wave_sort(T x) {
  return bitonic_from<DESC, 2>(x);
}

// Exact top-k (ties to the smaller id) of the n scores sc[0..n) of one unit,
// written by an earlier launch; ids through im. The k ids go, ascending, to
// dst (LDS or global). Every thread of the workgroup calls it; dst is valid
// after the caller's next barrier.
// k <= kFastSel: thread t owns scores [t*per, (t+1)*per). In each wave the
// k-th largest of its 64 per-thread maxima bounds the unit's k-th largest
// score from below (those maxima are k distinct scores); tau is the largest
// of the four bounds. The scores >= tau (at least k) are gathered and, if at
// most 64, wave 0 sorts them by (score, smaller id first), keeps k and sorts
// their ids. More candidates (heavy ties) or a larger k take the block-wide
// radix select.
__device__ void unit_topk(const float* __restrict__ sc, int n, int k, const IdMap& im, int unit,
                          int32_t* __restrict__ dst, SelectLds& S, TopkLds& T) {
  if (k <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (k >= n) {
    for (int i = tid; i < n; i += kThreads) dst[i] = map_id(im, unit, i);
    return;
  }
  if (k > kFastSel) {
    block_topk(sc, n, k, im, unit, dst, T);
    return;
  }
  const int per = (n + kThreads - 1) / kThreads;
  const int i0 = tid * per, i1 = min(n, i0 + per);
  // this thread's keys, kPer at a time with every load of a round in flight
  // (device-scope loads: the scores may come from other workgroups of this launch)
  constexpr int kPer = 8;
  const CohBuf scb(sc, (uint32_t)n * 4u);
  auto keys_at = [&](int r0, uint32_t (&kv)[kPer]) {
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      kv[j] = r0 + j < i1 ? order_key(__uint_as_float(scb.u32(r0 + j))) : 0u;
  };
  uint32_t kv[kPer];
  keys_at(i0, kv);
  uint32_t mx = 0u;
  for (int r0 = i0;; ) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) mx = max(mx, kv[j]);
    r0 += kPer;
    if (r0 >= i1) break;
    keys_at(r0, kv);
  }
  const uint32_t sorted = wave_sort<true>(mx);
  const uint32_t tw = (uint32_t)__builtin_amdgcn_readlane((int)sorted, k - 1);
  if (lane == 0) S.tw[w] = tw;
  if (tid == 0) S.cnt = 0;
  __syncthreads();
  uint32_t tau = S.tw[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) tau = max(tau, S.tw[i]);
  const bool one_round = per <= kPer;   // then kv still holds every key of this thread
  int c = 0;
  if (one_round) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) c += kv[j] >= tau ? 1 : 0;   // 0 (no item) < tau unless tau = 0
    if (tau == 0u) c = i1 > i0 ? i1 - i0 : 0;
  } else {
    for (int r0 = i0; r0 < i1; r0 += kPer) {
      keys_at(r0, kv);
#pragma unroll
      for (int j = 0; j < kPer; ++j) c += (kv[j] >= tau && r0 + j < i1) ? 1 : 0;
    }
  }
  int pos = c > 0 ? atomicAdd(&S.cnt, c) : 0;
  for (int r0 = i0; r0 < i1; r0 += kPer) {
    if (!one_round) keys_at(r0, kv);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (kv[j] >= tau && r0 + j < i1) {
        if (pos < kCandMax) {
          S.ck[pos] = kv[j];
          S.ci[pos] = (uint32_t)map_id(im, unit, r0 + j);
        }
        ++pos;
      }
    }
  }
  __syncthreads();
  const int total = S.cnt;
  if (total > kCandMax) {   // uniform: heavy ties at the threshold
    __syncthreads();
    block_topk(sc, n, k, im, unit, dst, T);
    return;
  }
  if (w == 0) {
    typedef unsigned long long u64;
    u64 key = lane < total ? (((u64)S.ck[lane] << 32) | (u64)(~S.ci[lane])) : 0ull;
    key = wave_sort<true>(key);                       // best first; equal scores: smaller id first
    uint32_t id = lane < k ? ~(uint32_t)key : 0xFFFFFFFFu;
    id = wave_sort<false>(id);                        // the k ids ascending
    if (lane < k) dst[lane] = (int32_t)id;
  }
}

// ------------------------------------------------------------ kernels ------

// A pass over gist-like rows of every unit: the group score of every item
// (for the selection made by the next launch) and one attention partial per
// workgroup, plus a share of the tail rows (attended, not scored). With out
// set (the call's last pass) the unit's last workgroup merges the partials.
// Candidate passes of a two-level call first select the unit's level-2
// groups from the previous pass's scores.
struct GistArgs {
  const void* q;
  const void* K;
  const void* V;
  int64_t unit_rows;      // rows per unit in K/V
  int64_t n_items;        // items per unit
  int64_t per_task;       // items per workgroup
  int32_t tasks;          // workgroups per unit
  RowMap rm;              // kind 2: rm.sel2 unused (the selection is made here)
  // tail rows, from the interleaved cache Kt/Vt
  const void* Kt;
  const void* Vt;
  int64_t tail_unit_rows;
  int64_t N, M;
  int32_t C, T, tail_per_task;
  float* scores;          // [units][score_stride] or null (no later selection)
  int64_t score_stride;
  // kind 2: level-2 selection from the previous pass's scores
  const float* prev_scores;
  int64_t prev_stride;
  int32_t prev_n, prev_k;
  IdMap prev_im;          // previous pass' score index -> id (identity when it scored every gist)
  int32_t* sel2_ws;       // [units][sel2_stride] (for the unfold pass' ids)
  int64_t sel2_stride;
  int32_t* sel2_out;      // [units][prev_k] or null
  // partial softmax states
  float* part;            // [units][NP][part_stride]
  int64_t part_stride;
  int32_t NP, part_base;
  float* out;             // set: the last workgroup merges into out / lse
  float* lse;
  uint32_t* cnt;          // unit u's counter at cnt[u * kCtrlUnitWords]
  float scale_log2;       // softmax logits in log2 units
  float score_mul;        // group score = sum_h(q_h . k) * score_mul
  // single-level decode with k > 0: the unit's last workgroup selects the
  // top-k chunks from this pass's scores for the unfold launch
  int32_t fuse_k;
  int32_t* sel_ws;        // [units][sel_stride] (k > kSelLdsMax: the selection lives here)
  int64_t sel_stride;
  int32_t* sel_out;       // [units][k] or null
  SeqLens seq;            // single-level decode: per-sequence lengths
  // selection rules: the items only route (scores out, no V read); the
  // partial state written is the empty one and is never merged
  int32_t score_only;
};

template <int D, int G>
struct GistLds {
  float scores[kTaskScores];   // this workgroup's scores
  int32_t sel2[kSelLdsMax];    // kind 2: the unit's level-2 selection; fused: the chunk selection
  union {
    PartLds<D, G> part;
    struct {
      SelectLds s;
      TopkLds t;
    } sel;
  } u;
};

// At least 4 waves per SIMD: the rare selection code must not cost the
// streaming loop its occupancy.
template <bool BF16, int D, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 2, 8)))
void gist_kernel(GistArgs a) {
  using Gm = Geo<BF16, D>;
  __shared__ GistLds<D, G> lds;
  __shared__ uint32_t s_old;
  const int tid = threadIdx.x;
  const int unit = blockIdx.x / a.tasks, split = blockIdx.x % a.tasks;
  RowMap rm = a.rm;
  if (rm.kind == 2) {
    // the unit's level-2 groups (every workgroup of the unit makes the same selection)
    unit_topk(a.prev_scores + (size_t)unit * a.prev_stride, a.prev_n, a.prev_k, a.prev_im, unit, lds.sel2,
              lds.u.sel.s, lds.u.sel.t);
    __syncthreads();
    if (split == 0)
      for (int i = tid; i < a.prev_k; i += kThreads) {
        a.sel2_ws[(size_t)unit * a.sel2_stride + i] = lds.sel2[i];
        if (a.sel2_out) a.sel2_out[(size_t)unit * a.prev_k + i] = lds.sel2[i];
      }
    rm.sel2 = lds.sel2;
    rm.sel2_stride = 0;
    __syncthreads();   // LDS changes role: selection scratch -> partial merge
  }
  uint4 qv[G];
  load_q<BF16, D, G>(a.q, unit, qv);
  State<BF16, G> st;
  init_state<BF16, G>(st);
  // this unit's lengths (single-level decode: the items are its gists)
  int64_t uN = a.N, uM = a.M, n_items = a.n_items;
  if (a.seq.n != nullptr) {
    unit_lengths(a.seq, unit, a.N, a.M, a.C, a.T, &uN, &uM);
    n_items = uM;
  }
  const size_t ub = (size_t)unit * (size_t)a.unit_rows * Gm::ROW_BYTES;
  const int64_t i0 = (int64_t)split * a.per_task;
  const int64_t i1 = i0 + a.per_task < n_items ? i0 + a.per_task : (i0 < n_items ? n_items : i0);
  stream_rows<BF16, D, G, false>(reinterpret_cast<const char*>(a.K) + ub,
                                 reinterpret_cast<const char*>(a.V) + ub, i0, i1,
                                 [&](int64_t i) { return map_row(rm, 0, i); }, qv, st,
                                 a.scale_log2, lds.scores, a.score_mul, a.score_only != 0);
  // this workgroup's share of the tail
  const int64_t t0 = (int64_t)split * a.tail_per_task;
  const int64_t t1 = t0 + a.tail_per_task < a.T ? t0 + a.tail_per_task : a.T;
  if (t0 < t1) {
    const size_t tb = (size_t)unit * (size_t)a.tail_unit_rows * Gm::ROW_BYTES;
    const int64_t N = uN, M = uM;
    const int32_t C = a.C, T = a.T;
    stream_rows<BF16, D, G, false>(reinterpret_cast<const char*>(a.Kt) + tb,
                                   reinterpret_cast<const char*>(a.Vt) + tb, t0, t1,
                                   [&](int64_t i) { return tail_row(i, N, T, M, C); }, qv, st,
                                   a.scale_log2, nullptr, 0.f);
  }
  __syncthreads();
  if (a.scores != nullptr) {
    // scores out for the selection (device-scope stores: the unit's last
    // workgroup or the next launch reads them)
    float* so = a.scores + (size_t)unit * a.score_stride + i0;
    for (int64_t i = tid; i < i1 - i0; i += kThreads) st_coh(so + i, lds.scores[i]);

  }
  float* part_u = a.part + (size_t)unit * a.NP * a.part_stride;
  write_partial<BF16, D, G>(st, part_u + (size_t)(a.part_base + split) * a.part_stride, lds.u.part, false);
  if (a.out == nullptr && a.fuse_k == 0) return;
  if (!arrive_last(a.cnt + (size_t)unit * kCtrlUnitWords, (uint32_t)a.tasks, &s_old)) return;
  if (a.fuse_k > 0) {
    // the unit's selection, for the unfold launch
    __syncthreads();   // LDS changes role: partial merge -> selection
    const int k = a.fuse_k;
    int32_t* us = a.sel_ws + (size_t)unit * a.sel_stride;
    unit_topk(a.scores + (size_t)unit * a.score_stride, (int)n_items, k, IdMap{nullptr, 0, 0, 0, 0}, unit, us,
              lds.u.sel.s, lds.u.sel.t);
    __syncthreads();
    if (a.sel_out)
      for (int i = tid; i < k; i += kThreads) a.sel_out[(size_t)unit * k + i] = us[i];
  }
  if (a.out != nullptr)
    merge_unit<D, G>(part_u, a.NP, (uint32_t)a.part_stride, a.out + (size_t)unit * G * D,
                     a.lse ? a.lse + (size_t)unit * G : nullptr, kWaves);
}

// Split path with many gists per unit: workgroup (unit, split) takes the top-k
// of the split's scores (written by the gist pass) and writes them as (score,
// id) candidates, padded with scores that never win. The unit's top-k (ties to
// the smaller id) lies within the candidates of its splits, so the unfold
// pass selects among S k of them instead of all M scores.
struct CandArgs {
  const float* scores;    // [units][score_stride]
  int64_t score_stride;
  int64_t n_items, per_task;
  int32_t tasks, k;
  int64_t N, M;
  int32_t C, T;
  SeqLens seq;
  float* cand_scores;     // [units][cand_stride]
  int32_t* cand_ids;
  int64_t cand_stride;
};

__global__ __launch_bounds__(kThreads) void cand_kernel(CandArgs a) {
  __shared__ SelectLds sl;
  __shared__ TopkLds tl;
  __shared__ int32_t loc[kFastSel];
  const int tid = threadIdx.x;
  const int unit = blockIdx.x / a.tasks, split = blockIdx.x % a.tasks;
  int64_t uN = a.N, uM = a.M;
  unit_lengths(a.seq, unit, a.N, a.M, a.C, a.T, &uN, &uM);
  const int64_t n_items = a.seq.n != nullptr ? uM : a.n_items;
  const int64_t i0 = (int64_t)split * a.per_task;
  const int64_t i1 = i0 + a.per_task < n_items ? i0 + a.per_task : n_items;
  const int nl = i1 > i0 ? (int)(i1 - i0) : 0;
  const float* su = a.scores + (size_t)unit * a.score_stride;
  unit_topk(su + i0, nl, a.k, IdMap{nullptr, 0, 0, 0, 0}, unit, loc, sl, tl);
  __syncthreads();
  float* cs = a.cand_scores + (size_t)unit * a.cand_stride + (size_t)split * a.k;
  int32_t* ci = a.cand_ids + (size_t)unit * a.cand_stride + (size_t)split * a.k;
  for (int j = tid; j < a.k; j += kThreads) {
    const bool real = j < nl;
    const int li = real ? loc[j] : 0;
    cs[j] = real ? su[i0 + li] : -INFINITY;
    ci[j] = real ? (int32_t)(i0 + li) : 0;
  }
}

// Raw rows of the selected chunks (minus rows the tail owns); every workgroup
// first makes the unit's selection from the previous pass's scores, and the
// unit's last workgroup merges every partial into out and lse.
struct UnfoldArgs {
  const void* q;
  const void* K;
  const void* V;
  int64_t unit_rows;
  const float* scores;    // [units][score_stride] the previous pass's scores, or null:
                          // the selection is ready in sel_ws
  int64_t score_stride;
  int32_t n_cand;         // scores per unit
  IdMap im;               // score index -> chunk id
  int32_t* sel_ws;        // [units][sel_stride] (k > kSelLdsMax: the selection lives here)
  int64_t sel_stride;
  int32_t* sel_out;       // [units][k] or null
  int32_t k;
  int32_t C, T;
  int64_t M, N;
  int64_t n_items, per_task;   // n_items = k * C
  int32_t tasks;
  float* part;
  int64_t part_stride;
  int32_t NP, part_base;
  float* out;
  float* lse;
  uint32_t* cnt;
  float scale_log2;
  SeqLens seq;            // per-sequence lengths (single-level decode)
  // selection-rule variants (gist_set 1 or 2): after the k C raw items come
  // set_kg chosen gists (k with rule 1, else 0) and the T tail rows; the
  // partial states merged are [merge_base, NP) (the scoring pass's are not
  // in the set)
  int32_t set_kg, set_tail, merge_base;
};

template <int D, int G>
struct UnfoldLds {
  int32_t sel[kSelLdsMax];
  union {
    PartLds<D, G> part;
    struct {
      SelectLds s;
      TopkLds t;
    } sel;
  } u;
};

template <bool BF16, int D, int G>
__global__ __launch_bounds__(kThreads) void unfold_kernel(UnfoldArgs a) {
  using Gm = Geo<BF16, D>;
  __shared__ UnfoldLds<D, G> lds;
  __shared__ uint32_t s_old;
  const int tid = threadIdx.x;
  const int unit = blockIdx.x / a.tasks, split = blockIdx.x % a.tasks;
  const bool in_lds = a.k <= kSelLdsMax;
  int32_t* const gsel = a.sel_ws + (size_t)unit * a.sel_stride;
  int32_t* us = in_lds ? lds.sel : gsel;
  int64_t uN = a.N, uM = a.M;
  unit_lengths(a.seq, unit, a.N, a.M, a.C, a.T, &uN, &uM);
  if (a.scores != nullptr) {
    // make the unit's selection from the previous pass's scores
    // a variable-length unit's own gist scores (identity ids); candidate lists keep their size
    const int n_cand = a.seq.n != nullptr && a.im.sel2 == nullptr ? (int)uM : a.n_cand;
    unit_topk(a.scores + (size_t)unit * a.score_stride, n_cand, a.k, a.im, unit, us, lds.u.sel.s, lds.u.sel.t);
    __syncthreads();
    if (split == 0 && a.sel_out)
      for (int i = tid; i < a.k; i += kThreads) a.sel_out[(size_t)unit * a.k + i] = us[i];
  } else if (in_lds) {
    // the previous launch made it
    const int32_t* ws_sel = a.sel_ws + (size_t)unit * a.sel_stride;
    for (int i = tid; i < a.k; i += kThreads) lds.sel[i] = ws_sel[i];
    __syncthreads();
  }
  uint4 qv[G];
  load_q<BF16, D, G>(a.q, unit, qv);
  State<BF16, G> st;
  init_state<BF16, G>(st);
  const size_t ub = (size_t)unit * (size_t)a.unit_rows * Gm::ROW_BYTES;
  const int64_t i0 = (int64_t)split * a.per_task;
  const int64_t i1 = i0 + a.per_task < a.n_items ? i0 + a.per_task : a.n_items;
  // 32-bit index math: items < 2^30
  const uint32_t C = (uint32_t)a.C;
  const int64_t M = uM, tail0 = uN - a.T;
  const int64_t kC = (int64_t)a.k * a.C;
  const int32_t T = a.T;
  // The row lookups read the selection through a pointer of a fixed address
  // space (one stream per place): through a generic pointer into LDS the
  // compiler may fold part of a computed index into the flat access's
  // immediate offset, and a base address below the LDS aperture is rejected
  // by the hardware.
  auto stream = [&](auto sel_id) {
    auto row_of = [&](int64_t i64) -> int64_t {
      if (i64 >= kC) {   // selection-rule variants: the chosen gists, then the tail
        const int64_t j = i64 - kC;
        if (j < a.set_kg) {
          const int64_t m = sel_id(j);
          return m < 0 || m >= M ? -1 : m * (C + 1) + C;
        }
        return tail_row(j - a.set_kg, uN, T, M, (int32_t)C);
      }
      const uint32_t i = (uint32_t)i64;
      const uint32_t ci = i / C, j = i - ci * C;
      const int64_t m = sel_id(ci);
      if (m < 0 || m >= M) return -1;         // never taken for a valid selection
      if (m * C + j >= tail0) return -1;      // the tail attends this row
      return m * (C + 1) + j;
    };
    stream_rows<BF16, D, G, true>(reinterpret_cast<const char*>(a.K) + ub,
                                  reinterpret_cast<const char*>(a.V) + ub, i0, i1, row_of, qv, st,
                                  a.scale_log2, nullptr, 0.f);
  };
  if (in_lds)
    stream([&](int64_t x) -> int64_t { return lds.sel[x]; });
  else
    stream([&](int64_t x) -> int64_t { return gsel[x]; });
  float* part_u = a.part + (size_t)unit * a.NP * a.part_stride;
  __syncthreads();   // LDS changes role: selection scratch -> partial merge
  write_partial<BF16, D, G>(st, part_u + (size_t)(a.part_base + split) * a.part_stride, lds.u.part, false);
  if (arrive_last(a.cnt + (size_t)unit * kCtrlUnitWords, (uint32_t)a.tasks, &s_old))
    merge_unit<D, G>(part_u + (size_t)a.merge_base * a.part_stride, a.NP - a.merge_base, (uint32_t)a.part_stride,
                     a.out + (size_t)unit * G * D, a.lse ? a.lse + (size_t)unit * G : nullptr, kWaves);
}

// ------------------------------------------------------------------ host ---

gsa_status_t launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return GSA_OK;
}

// Counter regions: word p of each unit's control block counts phase p.
inline uint32_t* ctrl_of(char* ws, size_t off_ctrl, int phase) {
  return reinterpret_cast<uint32_t*>(ws + off_ctrl) + phase;
}

template <bool BF16, int D, int G>
gsa_status_t run_decode(const DecodePlan& pl, const void* q, const void* K, const void* V,
                        float* out, float* lse, int32_t* sel_idx, char* ws, hipStream_t st) {
  float* part = reinterpret_cast<float*>(ws + pl.off_part);
  float* scores = reinterpret_cast<float*>(ws + pl.off_scores);
  int32_t* wsel = reinterpret_cast<int32_t*>(ws + pl.off_sel);
  const int64_t ps = part_stride(G, D);
  GistArgs g{};
  g.q = q; g.K = K; g.V = V;
  g.unit_rows = pl.R; g.n_items = pl.M; g.per_task = pl.gists_per_split; g.tasks = pl.S;
  g.rm = RowMap{0, pl.C, nullptr, 0, 0, 0, 0};
  g.Kt = K; g.Vt = V; g.tail_unit_rows = pl.R;
  g.N = pl.N; g.M = pl.M; g.C = pl.C; g.T = pl.T; g.tail_per_task = pl.tail_per_split;
  g.scores = pl.k > 0 ? scores : nullptr; g.score_stride = pl.score_stride;
  g.part = part; g.part_stride = ps; g.NP = pl.NP; g.part_base = 0;
  g.out = pl.k > 0 ? nullptr : out; g.lse = pl.k > 0 ? nullptr : lse;
  g.cnt = ctrl_of(ws, pl.off_ctrl, 0);
  g.scale_log2 = pl.scale * kLog2e; g.score_mul = pl.scale / G;
  const bool cand = pl.cand_stride > 0;
  g.fuse_k = cand ? 0 : pl.k;   // with candidates the unfold pass selects
  g.sel_ws = wsel; g.sel_stride = pl.sel_stride; g.sel_out = sel_idx;
  g.seq = SeqLens{pl.seq_n, pl.seq_m, pl.Hkv, pl.k};
  // selection-rule variants: the gist pass only scores (its partial states
  // are not merged) and leaves the tail to the set's pass; with k = 0 there
  // is nothing to score
  const bool sets = pl.gist_set != GSA_GISTS_ALL;
  if (sets) g.tail_per_task = 0;
  g.score_only = sets ? 1 : 0;
  prof_begin_call();
  if (!sets || pl.k > 0)
    prof_launch((gist_kernel<BF16, D, G>), dim3(pl.units * pl.S), dim3(kThreads), 0, st, g);
  float* cand_s = reinterpret_cast<float*>(ws + pl.off_cand);
  int32_t* cand_i = reinterpret_cast<int32_t*>(ws + pl.off_cand_ids);
  if (cand) {
    CandArgs c{};
    c.scores = scores; c.score_stride = pl.score_stride;
    c.n_items = pl.M; c.per_task = pl.gists_per_split; c.tasks = pl.S; c.k = pl.k;
    c.N = pl.N; c.M = pl.M; c.C = pl.C; c.T = pl.T; c.seq = g.seq;
    c.cand_scores = cand_s; c.cand_ids = cand_i; c.cand_stride = pl.cand_stride;
    prof_launch(cand_kernel, dim3(pl.units * pl.S), dim3(kThreads), 0, st, c);
  }
  if (pl.k > 0 || sets) {
    UnfoldArgs u{};
    u.q = q; u.K = K; u.V = V; u.unit_rows = pl.R;
    u.scores = nullptr;
    if (cand) {
      u.scores = cand_s; u.score_stride = pl.cand_stride; u.n_cand = pl.S * pl.k;
      u.im = IdMap{cand_i, 1, pl.S * pl.k, 0, pl.cand_stride};
      u.sel_out = sel_idx;
    }
    u.sel_ws = wsel; u.sel_stride = pl.sel_stride; u.k = pl.k;
    if (!cand) u.sel_out = nullptr;
    u.C = pl.C; u.T = pl.T; u.M = pl.M; u.N = pl.N;
    u.n_items = pl.n_items; u.per_task = pl.items_per_split; u.tasks = pl.S2;
    u.part = part; u.part_stride = ps; u.NP = pl.NP; u.part_base = pl.S;
    u.out = out; u.lse = lse;
    u.cnt = ctrl_of(ws, pl.off_ctrl, 2);
    u.scale_log2 = pl.scale * kLog2e;
    u.seq = g.seq;
    u.set_kg = pl.gist_set == GSA_GISTS_SELECTED ? pl.k : 0;
    u.set_tail = sets ? pl.T : 0;
    u.merge_base = sets ? pl.S : 0;
    prof_launch((unfold_kernel<BF16, D, G>), dim3(pl.units * pl.S2), dim3(kThreads), 0, st, u);
  }
  return launch_status("gsa_decode launch");
}

template <bool BF16, int D, int G>
gsa_status_t run_hier(const HierPlan& hp, const void* q, const void* K, const void* V,
                      const void* K2, const void* V2, float* out, float* lse, int32_t* sel2,
                      int32_t* sel1, char* ws, hipStream_t st) {
  const DecodePlan& pl = hp.base;
  float* s2 = reinterpret_cast<float*>(ws + hp.off_s2);
  float* sc = reinterpret_cast<float*>(ws + hp.off_sc);
  int32_t* wsel2 = reinterpret_cast<int32_t*>(ws + hp.off_sel2);
  float* part = reinterpret_cast<float*>(ws + hp.off_part);
  const int64_t ps = part_stride(G, D);
  const int64_t orphan0 = hp.M2 * hp.G;
  // level 2: every meta-gist (dense rows of the level-2 array) and the tail
  GistArgs g{};
  g.q = q; g.K = K2; g.V = V2;
  g.unit_rows = hp.M2; g.n_items = hp.M2; g.per_task = hp.l2_per_split; g.tasks = hp.S_l2;
  g.rm = RowMap{1, pl.C, nullptr, 0, 0, 0, 0};
  g.Kt = K; g.Vt = V; g.tail_unit_rows = pl.R;
  // selection rules: every pass before the unfold only scores (their partial
  // states are not merged) and the tail goes to the set's pass
  const bool sets = pl.gist_set != GSA_GISTS_ALL;
  g.N = pl.N; g.M = pl.M; g.C = pl.C; g.T = pl.T; g.tail_per_task = sets ? 0 : hp.tail_per_split;
  g.score_only = sets ? 1 : 0;
  g.scores = s2; g.score_stride = hp.s2_stride;
  g.part = part; g.part_stride = ps; g.NP = hp.NP; g.part_base = 0;
  g.out = nullptr; g.lse = nullptr;
  g.cnt = ctrl_of(ws, hp.off_ctrl, 0);
  g.scale_log2 = pl.scale * kLog2e; g.score_mul = pl.scale / G;
  g.fuse_k = 0;
  prof_begin_call();
  prof_launch((gist_kernel<BF16, D, G>), dim3(pl.units * hp.S_l2), dim3(kThreads), 0, st, g);
  // level 1: select the groups, then score and attend their children and the
  // ungrouped gists
  GistArgs c = g;
  c.K = K; c.V = V;
  c.unit_rows = pl.R; c.n_items = hp.n_cand; c.per_task = hp.cand_per_split; c.tasks = hp.S_c;
  c.rm = RowMap{2, pl.C, nullptr, hp.G, hp.k2, orphan0, 0};
  c.T = 0; c.tail_per_task = 0;
  c.scores = pl.k > 0 ? sc : nullptr; c.score_stride = hp.sc_stride;
  c.prev_scores = s2; c.prev_stride = hp.s2_stride; c.prev_n = (int32_t)hp.M2; c.prev_k = hp.k2;
  c.prev_im = IdMap{nullptr, 0, 0, 0, 0};
  if (hp.cand2_stride > 0) {
    // the level-2 workgroups' own top-k2, then the selection among those
    float* cs = reinterpret_cast<float*>(ws + hp.off_cand2);
    int32_t* ci = reinterpret_cast<int32_t*>(ws + hp.off_cand2_ids);
    CandArgs ca{};
    ca.scores = s2; ca.score_stride = hp.s2_stride;
    ca.n_items = hp.M2; ca.per_task = hp.l2_per_split; ca.tasks = hp.S_l2; ca.k = hp.k2;
    ca.N = pl.N; ca.M = pl.M; ca.C = pl.C; ca.T = pl.T;
    ca.cand_scores = cs; ca.cand_ids = ci; ca.cand_stride = hp.cand2_stride;
    prof_launch(cand_kernel, dim3(pl.units * hp.S_l2), dim3(kThreads), 0, st, ca);
    c.prev_scores = cs; c.prev_stride = hp.cand2_stride; c.prev_n = hp.S_l2 * hp.k2;
    c.prev_im = IdMap{ci, 1, hp.S_l2 * hp.k2, 0, hp.cand2_stride};
  }
  c.sel2_ws = wsel2; c.sel2_stride = hp.sel2_stride; c.sel2_out = sel2;
  c.part_base = hp.S_l2;
  c.out = pl.k > 0 || sets ? nullptr : out; c.lse = pl.k > 0 || sets ? nullptr : lse;
  c.cnt = ctrl_of(ws, hp.off_ctrl, 1);
  prof_launch((gist_kernel<BF16, D, G>), dim3(pl.units * hp.S_c), dim3(kThreads), 0, st, c);
  // unfold the chosen chunks, merge everything (selection rules: attend the
  // set, merge its own partial states)
  if (pl.k > 0 || sets) {
    UnfoldArgs u{};
    u.q = q; u.K = K; u.V = V; u.unit_rows = pl.R;
    u.scores = pl.k > 0 ? sc : nullptr; u.score_stride = hp.sc_stride; u.n_cand = hp.n_cand;
    u.im = IdMap{wsel2, hp.G, hp.k2, orphan0, hp.sel2_stride};
    u.sel_ws = reinterpret_cast<int32_t*>(ws + hp.off_sel1); u.sel_stride = pl.sel_stride;
    u.sel_out = sel1; u.k = pl.k;
    u.C = pl.C; u.T = pl.T; u.M = pl.M; u.N = pl.N;
    u.n_items = pl.n_items; u.per_task = pl.items_per_split; u.tasks = pl.S2;
    u.part = part; u.part_stride = ps; u.NP = hp.NP; u.part_base = hp.S_l2 + hp.S_c;
    u.out = out; u.lse = lse;
    u.cnt = ctrl_of(ws, hp.off_ctrl, 2);
    u.set_kg = pl.gist_set == GSA_GISTS_SELECTED ? pl.k : 0;
    u.set_tail = sets ? pl.T : 0;
    u.merge_base = sets ? hp.S_l2 + hp.S_c : 0;
    u.scale_log2 = pl.scale * kLog2e;
    prof_launch((unfold_kernel<BF16, D, G>), dim3(pl.units * pl.S2), dim3(kThreads), 0, st, u);
  }
  return launch_status("gsa_decode_hier launch");
}


// ===================================================== one workgroup per unit
//
// bf16, D = 128, one workgroup per (batch, kv-head) unit when there are enough
// units to fill the chip: the whole decode step of a unit -- every gist and
// tail row, the selection, the chosen chunks' raw rows and the merge -- with
// no hand-off through memory. Each of the four waves streams its own share of
// rows, 16 at a time, through a private ring of LDS stages filled by
// direct-to-LDS loads up to four stages ahead, and folds them in on MFMA:
//   S^T = K Q^T     16x16x32: A = 16 K rows (LDS, 16-byte reads), B = the g
//                   query heads padded to 16 columns with zeros;
//   O^T += V^T P^T  16x16x16: A = V^T read transposed (ds_read_b64_tr_b16),
//                   B = the softmax weights, split into bf16 hi + lo.
// Lane (h = lane%16, j = lane/16) holds head h's logits of rows 4j..4j+3 of a
// stage, exactly the B operand of the second product; the sum over the 16
// lanes of a row (DPP) is that row's group score (heads past g add 0).

constexpr int kUW = 4;                  // waves per unit workgroup
constexpr int kUBR = 16;                // rows per stage
constexpr int kUNB = 4;                 // stages in a wave's ring
constexpr int kUTile = kUBR * 256;      // one stage's K (or V) rows
constexpr int kUStage = 2 * kUTile;
constexpr int kUMaxGist = (int)kUnitMaxGist;   // gists of a unit selected from LDS (one workgroup)
constexpr int kUWgItems = (int)kUnitWgItems;   // group scores a workgroup keeps in LDS
constexpr int kUMaxSel = (int)kUnitMaxSel;     // scores one unit's selection reads
// cache policy of the row loads: nontemporal (each row is read once per call)
constexpr int kUNt = 2;
static_assert(kUW == kWaves, "the selection helpers assume the workgroup size");
static_assert(kUW == 4, "the merge combines four wave states");
static_assert(kUMaxGist % (16 * kThreads) == 0 && kUMaxSel % (16 * kThreads) == 0 && kCandMax == 64,
              "selection layout: keys in groups of 16 per thread");

typedef __bf16 bf16x8u __attribute__((ext_vector_type(8)));
typedef float f32x4u __attribute__((ext_vector_type(4)));
typedef short i16x4u __attribute__((ext_vector_type(4)));

template <int N>
__device__ __forceinline__ void uwait_vm() {
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16-byte chunk c of stage row r sits in LDS slot uk_slot (K) / uv_slot (V):
// conflict-free K-fragment reads and transposed V reads.
__device__ __forceinline__ int uk_slot(int c, int r) { return c ^ (r & 15); }
__device__ __forceinline__ int uv_slot(int c, int r) { return c ^ (2 * (r & 7)); }

// The K operands of a stage (four 16-byte reads), waiting for them in the same
// asm block: the compiler does not see these LDS reads, so it adds no wait for
// the direct-to-LDS loads still in flight.
__device__ __forceinline__ void u_k_frag(const uint32_t (&addr)[4], bf16x8u (&kf)[4]) {
  uint4 a0, a1, a2, a3;
  __asm__ volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3)
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3])
      : "memory");
  kf[0] = __builtin_bit_cast(bf16x8u, a0);
  kf[1] = __builtin_bit_cast(bf16x8u, a1);
  kf[2] = __builtin_bit_cast(bf16x8u, a2);
  kf[3] = __builtin_bit_cast(bf16x8u, a3);
}

// The V^T operands of a stage for the eight 16-column blocks of d.
// A stage's K fragments (4 x 16-byte reads) and V^T fragments (8 transposed
// reads) in one block with one wait: the V reads' latency hides under the K
// reads' instead of following the score and softmax work.
__device__ __forceinline__ void u_kv_frag(const uint32_t (&ka)[4], const uint32_t (&va)[8], bf16x8u (&kf)[4],
                                          i16x4u (&vf)[8]) {
  uint4 a0, a1, a2, a3;
  __asm__ volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %1, %13\n\t"
      "ds_read_b128 %2, %14\n\t"
      "ds_read_b128 %3, %15\n\t"
      "ds_read_b64_tr_b16 %4, %16\n\t"
      "ds_read_b64_tr_b16 %5, %17\n\t"
      "ds_read_b64_tr_b16 %6, %18\n\t"
      "ds_read_b64_tr_b16 %7, %19\n\t"
      "ds_read_b64_tr_b16 %8, %20\n\t"
      "ds_read_b64_tr_b16 %9, %21\n\t"
      "ds_read_b64_tr_b16 %10, %22\n\t"
      "ds_read_b64_tr_b16 %11, %23\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(vf[0]), "=&v"(vf[1]), "=&v"(vf[2]), "=&v"(vf[3]),
        "=&v"(vf[4]), "=&v"(vf[5]), "=&v"(vf[6]), "=&v"(vf[7])
      : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]),
        "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7])
      : "memory");
  kf[0] = __builtin_bit_cast(bf16x8u, a0);
  kf[1] = __builtin_bit_cast(bf16x8u, a1);
  kf[2] = __builtin_bit_cast(bf16x8u, a2);
  kf[3] = __builtin_bit_cast(bf16x8u, a3);
}

// Exact top-k of the unit's n group scores (k <= 64 < n <= 4096), all in
// LDS: the same result as the radix select (larger score first, equal
// scores: smaller id first), ids written ascending to dst (LDS).
//  1. thread t holds the keys of items t*per .. t*per + per - 1 (per a multiple
//     of 4); each wave's k-th
//     largest per-thread maximum is a lower bound on the k-th largest key,
//     tau = the largest of the four bounds;
//  2. the items with key >= tau are compacted in id order (thread t holds
//     a contiguous id range; a scan of the per-thread counts places them);
//  3. each candidate's rank among the candidates decides; the selected ones
//     keep their id order.
// More than kCandMax candidates (ties at tau) go to the radix select over a
// copy of the scores in gscratch (device memory).
struct UnitSelLds {
  uint32_t tw[kWaves];
  int wsum[kWaves];
  uint32_t top[kWaves][64];               // each wave's 64 largest of the threads' top-4 keys
  uint32_t tau;
  // candidates (key << 32 | ~id) in id order; [kCandMax, 2 kCandMax) takes
  // the writes of the other items
  unsigned long long ck[2 * kCandMax];
  int pr[kWaves][kCandMax];               // partial ranks
};

// One compare-exchange step of a descending bitonic sort of 256 values held
// four per lane (element 4 lane + r): partners at distance J < 4 are in the
// same lane, farther ones J/4 lanes away.
template <int K, int J>
__device__ __forceinline__ void bitonic4_step(uint32_t (&x)[4]) {
  const int lane = threadIdx.x & 63;
  if constexpr (J >= 4) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = 4 * lane + r;
      const uint32_t y = lane_xor<J / 4>(x[r]);
      const bool keep_max = ((e & J) == 0) == ((e & K) == 0);
      x[r] = keep_max ? max(x[r], y) : min(x[r], y);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if ((r & J) == 0) {
        const bool desc = ((4 * lane + r) & K) == 0;
        const uint32_t a = x[r], b = x[r | J];
        x[r] = desc ? max(a, b) : min(a, b);
        x[r | J] = desc ? min(a, b) : max(a, b);
      }
    }
  }
}
template <int K, int J>
__device__ __forceinline__ void bitonic4_stage(uint32_t (&x)[4]) {
  bitonic4_step<K, J>(x);
  if constexpr (J > 1) bitonic4_stage<K, J / 2>(x);
}
template <int K>
__device__ __forceinline__ void bitonic4_from(uint32_t (&x)[4]) {
  bitonic4_stage<K, K / 2>(x);
  if constexpr (K < 256) bitonic4_from<K * 2>(x);
}
// 256 values, four per lane, sorted descending over the wave.
__device__ __forceinline__ void wave_sort4(uint32_t (&x)[4]) { bitonic4_from<2>(x); }

// k-th largest (k <= 64) of the union of every thread's four largest keys: a
// lower bound on the workgroup's k-th largest key (they are distinct items),
// equal to it unless one thread holds more than four of the k largest. Each
// wave sorts its 256 top-4 keys; wave 0 sorts the four waves' 64 largest.
template <int PER>
__device__ __forceinline__ uint32_t tau_top4(const uint32_t (&key)[PER], int k, UnitSelLds& S) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t t[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint32_t v = key[j];
    const uint32_t n1 = max(t[1], min(t[0], v)), n2 = max(t[2], min(t[1], v)), n3 = max(t[3], min(t[2], v));
    t[0] = max(t[0], v);
    t[1] = n1;
    t[2] = n2;
    t[3] = n3;
  }
  wave_sort4(t);
  if (lane < 16) *reinterpret_cast<uint4*>(&S.top[w][4 * lane]) = make_uint4(t[0], t[1], t[2], t[3]);
  __syncthreads();
  if (w == 0) {   // a scalar branch: the whole wave takes it
    const uint4 v = *reinterpret_cast<const uint4*>(&S.top[lane >> 4][4 * (lane & 15)]);
    uint32_t u[4] = {v.x, v.y, v.z, v.w};
    wave_sort4(u);
    const int r = (k - 1) & 3;
    const uint32_t pick = r == 0 ? u[0] : r == 1 ? u[1] : r == 2 ? u[2] : u[3];
    const uint32_t tau = (uint32_t)__builtin_amdgcn_readlane((int)pick, (k - 1) >> 2);
    if (lane == 0) S.tau = tau;
  }
  __syncthreads();
  return S.tau;
}

// Four 16-byte LDS reads that wait for themselves (the compiler does not see
// them, so it adds no wait for loads in flight).
__device__ __forceinline__ void lds_read4x16(const uint32_t (&ad)[4], uint4 (&v)[4]) {
  __asm__ volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
      : "memory");
}

// The steps of the exact top-k below, shared with the candidate hand-off.
// Thread t holds items t*per .. t*per + per - 1 (per a multiple of 4).
__device__ __forceinline__ int select_per(int n) { return (n + 4 * kThreads - 1) / (4 * kThreads) * 4; }

// 1. this thread's keys (order-preserving images of the scores; 0 past its
// nv items), every read in bounds and in flight with the others of its group.
// FROM_LDS: an LDS array of LDS_N floats; otherwise device memory written by
// other workgroups with device-scope stores (gstride floats per row).
template <int PER, bool FROM_LDS, int LDS_N>
__device__ __forceinline__ void select_keys(const float* __restrict__ sc, const float* __restrict__ gscores,
                                            int64_t gstride, int i0, int per, int nv, uint32_t (&key)[PER]) {
  static_assert(PER % 16 == 0, "keys come in groups of 16");
  if constexpr (FROM_LDS) {
    const uint32_t base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) float*)sc;
#pragma unroll
    for (int grp = 0; grp < PER / 16; ++grp) {
      uint32_t ad[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) ad[q] = base + 16u * (uint32_t)min(i0 / 4 + 4 * grp + q, LDS_N / 4 - 1);
      uint4 v[4];
      lds_read4x16(ad, v);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t raw[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 16 * grp + 4 * q + e;
          key[j] = j < nv ? order_key(__uint_as_float(raw[e])) : 0u;
        }
      }
    }
  } else {
    // 16-byte device-scope loads, all issued together; the buffer covers the
    // unit's padded score row (gstride floats, a multiple of 4) and a read
    // past it returns 0 without touching memory: groups past this thread's
    // `per` items are sent there
    const CohBuf P(gscores, (uint32_t)gstride * 4u);
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const uint4 v = P.u128(4 * q < per ? (uint32_t)(i0 + 4 * q) : (uint32_t)gstride);
      const uint32_t raw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) key[4 * q + e] = 4 * q + e < nv ? order_key(__uint_as_float(raw[e])) : 0u;
    }
  }
}

// 2. a lower bound tau >= 1 on the k-th largest key (k <= 64) that keeps few
// keys above it: k <= 16, the k-th largest of every thread's maximum
// (distinct items), each wave's 16 largest merged by one wave; k > 16, the
// k-th largest of the union of the threads' four largest (tau_top4). Items
// that are not there have key 0 (a real item has key 0 only for a NaN score
// with every bit set), so tau >= 1 selects exactly the items.
template <int PER>
__device__ __forceinline__ uint32_t select_tau(const uint32_t (&key)[PER], int k, UnitSelLds& S) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t tau;
  if (k <= 16) {
    uint32_t mx = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j) mx = max(mx, key[j]);
    const uint32_t srt = wave_sort<true>(mx);
    if (lane < 16) S.top[w][lane] = srt;
    __syncthreads();
    if (w == 0) {   // a scalar branch: the whole wave takes it
      const uint32_t v = wave_sort<true>(S.top[lane >> 4][lane & 15]);
      const uint32_t t = (uint32_t)__builtin_amdgcn_readlane((int)v, k - 1);
      if (lane == 0) S.tau = t;
    }
    __syncthreads();
    tau = S.tau;
  } else {
    tau = tau_top4(key, k, S);
  }
  return max(tau, 1u);
}

// 3. this thread's exclusive prefix (in item order) of the per-thread counts
// c over the workgroup; *total gets the sum. DPP row scan, then the totals of
// the rows and waves below.
__device__ __forceinline__ int select_scan(int c, UnitSelLds& S, int* total) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int x = c;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);
  {
    const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
              r2 = __builtin_amdgcn_readlane(x, 47);
    x += (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
  }
  const int wtot = __builtin_amdgcn_readlane(x, 63);
  if (lane == 0) S.wsum[w] = wtot;
  __syncthreads();
  int run = x - c, t = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int v = S.wsum[i];
    run += i < w ? v : 0;
    t += v;
  }
  *total = t;
  return run;
}

// PER: keys per thread at most (n <= PER * kThreads). FROM_LDS: the scores are
// an LDS array of LDS_N floats (n <= LDS_N, a multiple of 4); otherwise
// gscores holds them in device memory, written by other workgroups with
// device-scope stores. The selected item indices go to dst ascending.
template <int PER, bool FROM_LDS, int LDS_N = PER * kThreads>
__device__ __forceinline__ void unit_select(const float* __restrict__ sc, int n, int k, float* __restrict__ gscores,
                                            int64_t gstride, int unit, int32_t* __restrict__ dst, UnitSelLds& S,
                                            TopkLds& T) {
  // Written to keep decisions in vector arithmetic: with one wave per SIMD
  // every vector -> scalar -> vector round trip costs a full pipeline drain.
  typedef unsigned long long u64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (k <= 0) return;
  if (k >= n) {
    for (int i = tid; i < n; i += kThreads) dst[i] = i;
    return;
  }
  const int per = select_per(n);   // <= PER
  const int i0 = tid * per;
  const int nv = max(0, min(per, n - i0));   // this thread's items
  uint32_t key[PER];
  select_keys<PER, FROM_LDS, LDS_N>(sc, gscores, gstride, i0, per, nv, key);
  const uint32_t tau = select_tau(key, k, S);
  // count, scan, compact (candidates in id order)
  int c = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) c += key[j] >= tau ? 1 : 0;
  int total;
  int run = select_scan(c, S, &total);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const bool f = key[j] >= tau;
    const int p = f ? run : kCandMax;
    S.ck[p < kCandMax ? p : kCandMax + lane] = ((u64)key[j] << 32) | (uint32_t)~(uint32_t)(i0 + j);
    run += f ? 1 : 0;
  }
  __syncthreads();
  if (total > kCandMax) {   // uniform: heavy ties at the threshold
    if constexpr (FROM_LDS) {   // the radix select reads device memory
      for (int i = tid; i < n; i += kThreads) gscores[i] = sc[i];
      done_stores();
    }
    __syncthreads();
    block_topk(gscores, n, k, IdMap{nullptr, 0, 0, 0, 0}, unit, dst, T);
    return;
  }
  // rank of candidate `lane` against candidates 16 w .. 16 w + 15: the
  // composite keys are distinct, larger first (equal scores: smaller id)
  {
    const u64 mine = S.ck[lane];
    int r = 0;
#pragma unroll
    for (int q = 0; q < 16; q += 2) {
      const ulonglong2 v = reinterpret_cast<const ulonglong2*>(S.ck)[8 * w + q / 2];
      const u64 o0 = 16 * w + q < total ? v.x : 0ull;
      const u64 o1 = 16 * w + q + 1 < total ? v.y : 0ull;
      r += o0 > mine ? 1 : 0;
      r += o1 > mine ? 1 : 0;
    }
    S.pr[w][lane] = r;
  }
  __syncthreads();
  if (w == 0) {
    const int r = S.pr[0][lane] + S.pr[1][lane] + S.pr[2][lane] + S.pr[3][lane];
    const bool chosen = lane < total && r < k;
    const uint64_t m = __ballot(chosen);
    if (chosen)
      dst[__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] =
          (int32_t)~(uint32_t)S.ck[lane];
  }
}

struct UnitArgs {
  const void* q;          // [B][Hq][D] bf16
  const void* K;          // [B][Hkv][R][D]
  const void* V;
  float* out;             // [B][Hq][D]
  float* lse;             // [B][Hq] or null
  int32_t* sel;           // [B][Hkv][k] or null
  float* scores;          // [units][score_stride] workspace (selection fallback)
  int64_t score_stride;
  int64_t R, N, M;
  int32_t C, k, T;
  float scale_log2;       // softmax logits in log2 units
  float score_mul;        // group score = sum_h(q_h . k) * score_mul
  // several workgroups per unit (S > 1, and S2 in the unfold launch): partial
  // states [units][NP][part_stride] and per-unit arrival counters
  int32_t S, S2, NP;
  int64_t part_stride;
  float* part;
  uint32_t* cnt;
  // two-level decode: level-2 gist arrays [units][M2][D], fanout G2, top-k2,
  // level-1 candidates (k2 G2 children + orphans), level-2 scores and ids
  const void* K2;
  const void* V2;
  int64_t M2;
  int32_t G2, k2, n_cand;
  float* s2;
  int64_t s2_stride;
  int32_t* sel2;
  // which gists the attention set holds: 0 all, 1 the selected chunks', 2 none
  int32_t gist_set;
  SeqLens seq;            // per-sequence lengths (single-level decode)
  // paged caches (read only by the PAGED instantiations): K and V are pools
  // [n_pages][Hkv][rpp][D] of pages of 2^lp chunk slots (rpp = 2^lp (C + 1)
  // rows); sequence b's logical row r is row r mod rpp of page
  // table[b][r / rpp]; extra [B][max_extra][2] (page, row) pairs of rows
  // attended directly, the list ending at the first negative page
  const int32_t* pg_table;
  const int32_t* pg_extra;
  int64_t pg_count;       // pages in the pool
  int64_t pg_bytes;       // bytes between consecutive pages (Hkv rpp 256)
  int64_t pg_head_bytes;  // bytes between a page's kv-heads (rpp 256)
  int32_t pg_max, pg_lp, pg_rpp, pg_max_extra, Hkv;
};

// Several workgroups per unit: each split's top-kk group scores and ids
// (kk = k, or k2 over level-2 gists) follow the partial states in the
// workspace, [units][cand_stride] scores then [units][cand_stride] ids, split
// s at [s kk, (s + 1) kk). (Derived here rather than passed: the kernels'
// arguments already fill the scalar registers.)
struct Cands {
  float* s;
  int32_t* id;
  int32_t stride;
};
__device__ __forceinline__ Cands cands_of(const UnitArgs& a, int units, int kk) {
  Cands c;
  c.stride = (a.S * cand_cap(a.S, kk) + 31) / 32 * 32;
  c.s = a.part + (size_t)units * a.NP * a.part_stride;
  c.id = reinterpret_cast<int32_t*>(c.s + (size_t)units * c.stride);
  return c;
}

struct UnitLds {
  union {
    char ring[kUW][kUNB][kUStage];      // streaming
    struct {                            // selection (rings idle)
      UnitSelLds s;
      TopkLds t;
    } sel;
    struct {                            // merge of the waves' states
      float m[16][kUW], l[16][kUW];     // head-major: one 16-byte read per head
      float o[kUW][16][128];
    } mrg;
  } u;
  float scores[kUWgItems];
  int32_t sel[kFastSel];
  int32_t sel2[kFastSel];
  unsigned long long wtop[kUW][16];     // the waves' best keys (select_small)
  uint32_t s_old;
};

// Paged caches: the sequence's block table and extra rows, staged in LDS at
// the start of the launch (page ids clamped into the pool, so that every read
// stays inside it whatever the tables hold).
constexpr int kMaxPages = (int)kPagedMaxPages;
constexpr int kMaxExtra = (int)kPagedMaxExtra;
struct PagedLds : UnitLds {
  int32_t pages[kMaxPages];
  int32_t extra[2 * kMaxExtra];
  int32_t n_extra;
};
// Logical row of extra row e in the item streams (above every cache row).
constexpr int kExtraRow = 1 << 30;

__device__ __forceinline__ void stage_pages(const UnitArgs& a, int unit, PagedLds& L) {
  const int tid = threadIdx.x;
  const int b = unit / a.Hkv;
  if (tid == 0) L.n_extra = a.pg_max_extra;
  const int32_t* tb = a.pg_table + (size_t)b * a.pg_max;
  for (int i = tid; i < a.pg_max; i += kThreads)
    L.pages[i] = (int32_t)min((int64_t)max(tb[i], 0), a.pg_count - 1);
  __syncthreads();
  const int32_t* ex = a.pg_extra + (size_t)b * a.pg_max_extra * 2;
  for (int i = tid; i < a.pg_max_extra; i += kThreads) {
    const int32_t pg = ex[2 * i], r = ex[2 * i + 1];
    if (pg < 0) atomicMin(&L.n_extra, i);
    L.extra[2 * i] = (int32_t)min((int64_t)max(pg, 0), a.pg_count - 1);
    L.extra[2 * i + 1] = min(max(r, 0), a.pg_rpp - 1);
  }
  __syncthreads();
}

// The staged tables read as LDS (ds_read): through a generic pointer the
// compiler would emit flat loads, which count against the vector-memory
// counter the row streams wait on and would stall the loads in flight.
typedef const __attribute__((address_space(3))) int32_t* lds_i32p;
__device__ __forceinline__ int32_t lds_at(const int32_t* p, unsigned i) {
  return reinterpret_cast<lds_i32p>(reinterpret_cast<uintptr_t>(p) & 0xffffffffu)[i];
}

// Byte offset (from the unit's kv-head base in page 0) of an extra row
// (kExtraRow + e).
__device__ __forceinline__ int64_t paged_off(const UnitArgs& a, const PagedLds& L, int row) {
  const unsigned e = (unsigned)(row - kExtraRow);
  return (int64_t)lds_at(L.extra, 2 * e) * a.pg_bytes + (int64_t)lds_at(L.extra, 2 * e + 1) * 256;
}

// One wave's running softmax state: lane (h, j) holds head h's max and its
// share of the sum, and O^T[16 dt + 4 j + r][h] in o[dt][r].
struct UState {
  f32x4u o[8];
  float m, l;
};

// What unit_stream streams (the scored kinds keep their items' group scores
// in LDS):
//   kUKGists   items below M: the gists; then the tail rows          (scored)
//   kUKUnfold  the raw rows of the chosen chunks (lds_sel: chunk ids),
//              skipping those the tail attends
//   kUKL2      items below M2: level-2 gists (their own arrays); then the
//              tail rows                                             (scored)
//   kUKCand    level-1 candidates: the G children of each chosen level-2
//              group (lds_sel: group ids), then the orphans           (scored)
//   kUKScore   items below M: the gists' K rows only, 32 per stage; group
//              scores, no attention                                   (scored)
//   kUKSet     the raw rows of the chosen chunks (skipping those the tail
//              attends), then the chosen chunks' gists when the set keeps
//              them (gist_set 1), then the tail rows
enum { kUKGists = 0, kUKUnfold = 1, kUKL2 = 2, kUKCand = 3, kUKScore = 4, kUKSet = 5 };

// Stream items [i0, i1) of one kind through the wave's state.
// PAGED: Kb / Vb are the unit's kv-head base in page 0 of the pools, rows are
// translated through the staged block table (pl), and kUKGists streams the
// sequence's extra rows after the tail.
// SCORE_ONLY: the scored items are scored but not attended (the selection
// rules under the hierarchy); kUKL2's tail rows are still attended.
template <int KIND, bool PAGED = false, bool SCORE_ONLY = false>
__device__ __forceinline__ void unit_stream(const char* __restrict__ Kb, const char* __restrict__ Vb, int i0,
                                            int i1, const UnitArgs& a, const bf16x8u (&qf)[4], UState& st,
                                            char* ring, float* lds_scores, const int32_t* lds_sel,
                                            int score_base = 0, const char* K2b = nullptr,
                                            const char* V2b = nullptr, const PagedLds* pl = nullptr) {
  const int n = i1 - i0;
  if (n <= 0) return;
  const int lane = threadIdx.x & 63;
  const int hq = lane & 15, jg = lane >> 4;
  constexpr int kRows = KIND == kUKScore ? 2 * kUBR : kUBR;   // rows per stage (K only: twice as many)
  const int nb = (n + kRows - 1) / kRows;
  const int C = a.C, M = (int)a.M;
  const unsigned tail0 = (unsigned)(a.N - a.T);   // rows and positions fit in 31 bits here
  constexpr bool kScored = KIND != kUKUnfold && KIND != kUKSet;
  const int n_scored = KIND == kUKGists || KIND == kUKScore ? M : KIND == kUKL2 ? (int)a.M2 : i1;
  const int kC = a.k * C;                              // kUKSet: raw items, then gists, then tail
  const int kg = KIND == kUKSet && a.gist_set == 1 ? a.k : 0;
  // cache row of item i; -1 when there is no such item or the tail owns it,
  // -2 - j for level-2 gist j. Raw position p sits in row p + p / C (p + M
  // past the last gist).
  auto row_of = [&](int i) -> int {
    if (i >= i1) return -1;
    if (KIND == kUKScore) return i * (C + 1) + C;
    if (KIND == kUKSet && i >= kC) {
      if (i < kC + kg) return (int)(min((unsigned)lds_sel[i - kC], (unsigned)(M - 1)) * (unsigned)(C + 1) + (unsigned)C);
      if (PAGED && i - kC - kg >= a.T) return kExtraRow + (i - kC - kg - a.T);
      const unsigned pos = tail0 + (unsigned)(i - kC - kg);
      return (int)(pos + min(pos / (unsigned)C, (unsigned)M));
    }
    if (KIND == kUKGists || KIND == kUKL2) {
      const int nf = KIND == kUKGists ? M : (int)a.M2;
      if (i < nf) return KIND == kUKGists ? i * (C + 1) + C : -2 - i;
      if (PAGED && i - nf >= a.T) return kExtraRow + (i - nf - a.T);
      const unsigned pos = tail0 + (unsigned)(i - nf);
      return (int)(pos + min(pos / (unsigned)C, (unsigned)M));
    }
    if (KIND == kUKCand) {
      const int kg = a.k2 * a.G2;
      const unsigned id = i < kg ? (unsigned)lds_sel[i / a.G2] * (unsigned)a.G2 + (unsigned)(i % a.G2)
                                 : (unsigned)(a.M2 * a.G2 + (i - kg));
      return (int)(min(id, (unsigned)(M - 1)) * (unsigned)(C + 1) + (unsigned)C);
    }
    const unsigned ci = (unsigned)i / (unsigned)C, jj = (unsigned)i - ci * (unsigned)C;
    const unsigned m = min((unsigned)lds_sel[ci], (unsigned)(M - 1));   // k <= M, so M >= 1
    const unsigned pos = m * (unsigned)C + jj;
    return pos >= tail0 ? -1 : (int)(pos + m);
  };
  // Paged caches: page-table index and row within the page of item i
  // (whose row_of is row), from its chunk m and slot j, so that no row is
  // divided by C + 1 (masked and extra items: index 0, the address comes
  // from elsewhere).
  auto paged_slot = [&](int i, int row, unsigned& pi, unsigned& slot) {
    unsigned m = 0, j = 0;
    if (row >= 0 && row < kExtraRow) {
      if ((KIND == kUKGists || KIND == kUKScore) && i < M) {
        m = (unsigned)i;
        j = (unsigned)C;
      } else if (KIND == kUKGists || (KIND == kUKSet && i >= kC + kg)) {   // tail position
        const unsigned pos = tail0 + (unsigned)(i - (KIND == kUKGists ? M : kC + kg));
        m = min(pos / (unsigned)C, (unsigned)M);
        j = pos - m * (unsigned)C;
      } else if (KIND == kUKSet && i >= kC) {   // a chosen chunk's gist (rule 1)
        m = min((unsigned)lds_sel[i - kC], (unsigned)(M - 1));
        j = (unsigned)C;
      } else {                         // chosen chunk's raw row
        const unsigned ci = (unsigned)i / (unsigned)C;
        m = min((unsigned)lds_sel[ci], (unsigned)(M - 1));
        j = (unsigned)i - ci * (unsigned)C;
      }
    }
    pi = PAGED ? m >> a.pg_lp : 0;
    slot = PAGED ? (m - (pi << a.pg_lp)) * (unsigned)(C + 1) + j : 0;
  };
  // the unit's level-2 arrays (K2b, V2b), as offsets from the level-1 bases
  const int64_t k2off = KIND == kUKL2 ? K2b - Kb : 0;
  const int64_t v2off = KIND == kUKL2 ? V2b - Vb : 0;
  // Paged caches: a stage's four rows per lane, their page-table entries and
  // slots, read from LDS one stage before the stage's loads go out.
  struct PLook {
    int32_t rw[4], pg[4];
    unsigned slot[4];
  } look;
  auto plook = [&](int b) {
    if constexpr (PAGED) {
      unsigned pi[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + b * kRows + 4 * u + (lane >> 4);
        look.rw[u] = row_of(i);
        paged_slot(i, look.rw[u], pi[u], look.slot[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) look.pg[u] = lds_at(pl->pages, pi[u]);
    }
  };
  // stage b -> ring slot b % kUNB: lane i loads 16 bytes of row 4u + i/16 into
  // LDS slot i%16, K and V alike. Items past the end of the last stage read
  // row 0 (in bounds, masked), so that every stage issues the same eight loads.
  // Paged: stage b's rows are in `look` (plook(b) ran before).
  auto issue = [&](int b) {
    char* kd = ring + (b % kUNB) * kUStage;
    char* vd = kd + kUTile;
    const int sl = lane & 15;
    if constexpr (KIND == kUKScore) {
      // rows 0..15 of the stage into the K tile, rows 16..31 into the V tile's place
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = 4 * (u & 3) + (lane >> 4);
        const int i = i0 + b * kRows + 16 * (u >> 2) + r;
        const int row = row_of(i);
        int64_t koffr = (int64_t)(row >= 0 ? row : 0) * 256;
        if constexpr (PAGED) {
          // gist i of the sequence: its page's slot, through the staged block table
          unsigned pi, slot;
          paged_slot(i, row, pi, slot);
          koffr = row >= 0 ? (int64_t)lds_at(pl->pages, pi) * a.pg_bytes + (int64_t)slot * 256 : 0;
        }
        __builtin_amdgcn_global_load_lds(Kb + koffr + uk_slot(sl, r) * 16, kd + (u >> 2) * kUTile + (u & 3) * 1024, 16,
                                         0, kUNt);
      }
      return;
    }
    if constexpr (PAGED) {
      // the stage's rows were looked up in the page table one stage earlier
      // (plook), so the loads wait for no LDS read here
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * u + (lane >> 4);
        const int rw = look.rw[u];
        const int64_t off = rw < 0 ? 0
                            : rw >= kExtraRow ? paged_off(a, *pl, rw)
                                              : (int64_t)look.pg[u] * a.pg_bytes + (int64_t)look.slot[u] * 256;
        __builtin_amdgcn_global_load_lds(Kb + off + uk_slot(sl, r) * 16, kd + u * 1024, 16, 0, kUNt);
        __builtin_amdgcn_global_load_lds(Vb + off + uv_slot(sl, r) * 16, vd + u * 1024, 16, 0, kUNt);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = 4 * u + (lane >> 4);
      const int row = row_of(i0 + b * kRows + r);
      int64_t koffr, voffr;
      koffr = (int64_t)(row >= 0 ? row : 0) * 256;
      voffr = koffr;
      if (KIND == kUKL2 && row <= -2) {
        koffr = k2off + (int64_t)(-2 - row) * 256;
        voffr = v2off + (int64_t)(-2 - row) * 256;
      }
      __builtin_amdgcn_global_load_lds(Kb + koffr + uk_slot(sl, r) * 16, kd + u * 1024, 16, 0, kUNt);
      __builtin_amdgcn_global_load_lds(Vb + voffr + uv_slot(sl, r) * 16, vd + u * 1024, 16, 0, kUNt);
    }
  };
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)ring;
  // per-lane LDS offsets within a stage
  uint32_t koff[4], voff[8];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) koff[ks] = hq * 256 + uk_slot(4 * ks + jg, hq) * 16;
  {
    // transposed read: lane s of 16-lane group j fetches 4 columns of row
    // 4j + s/4, so that lane m receives column m of rows 4j..4j+3
    const int R = 4 * jg + (hq >> 2);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      voff[dt] = kUTile + R * 256 + uv_slot(2 * dt + ((hq & 3) >> 1), R) * 16 + 8 * (hq & 1);
  }
  auto compute = [&](int b) {
    const uint32_t base = ring_lds + (b % kUNB) * kUStage;
    if constexpr (KIND == kUKScore) {
      // two 16-row halves: group scores only
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t ka[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) ka[ks] = base + h * kUTile + koff[ks];
        bf16x8u kf[4];
        u_k_frag(ka, kf);
        f32x4u s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[ks], s, 0, 0, 0);
        const int i_base = i0 + b * kRows + 16 * h + 4 * jg;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gsum = group_sum<16>(s[r]);
          if (hq == 0 && i_base + r < i1) lds_scores[i_base + r - score_base] = gsum * a.score_mul;
        }
      }
      return;
    }
    uint32_t ka[4], va[8];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) ka[ks] = base + koff[ks];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) va[dt] = base + voff[dt];
    bf16x8u kf[4];
    i16x4u vf[8];
    u_kv_frag(ka, va, kf, vf);
    // two independent chains of two products, then their sum: half the
    // dependent MFMA latency of one chain of four
    f32x4u s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0], qf[0], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1], qf[1], s1, 0, 0, 0);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[2], qf[2], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[3], qf[3], s1, 0, 0, 0);
    f32x4u s;
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = s0[r] + s1[r];
    // s[r]: head hq against stage row 4 jg + r
    const int i_base = i0 + b * kRows + 4 * jg;
    bool ok[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ok[r] = kScored ? i_base + r < i1 : row_of(i_base + r) >= 0;
    if constexpr (SCORE_ONLY) {
#pragma unroll
      for (int r = 0; r < 4; ++r) ok[r] = ok[r] && i_base + r >= n_scored;
    }
    if (kScored) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float g = group_sum<16>(s[r]);
        if (hq == 0 && i_base + r < i1 && i_base + r < n_scored) lds_scores[i_base + r - score_base] = g * a.score_mul;
      }
    }
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = ok[r] ? s[r] * a.scale_log2 : -INFINITY;
    const float cand = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if (__ballot(cand > st.m + kLazy) != 0ull) {
      // raise head h's max on its four lanes (j = 0..3) and rescale
      float c4 = fmaxf(cand, __uint_as_float(lane_xor<16>(__float_as_uint(cand))));
      c4 = fmaxf(c4, __uint_as_float(lane_xor<32>(__float_as_uint(c4))));
      const float mn = c4 > st.m + kLazy ? c4 : st.m;
      const float al = fexp2(st.m - mn);
      st.m = mn;
      st.l *= al;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) st.o[dt][r] *= al;
    }
    i16x4u phi, plo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = fexp2(x[r] - st.m);
      st.l += p;
      const __bf16 hi = (__bf16)p;
      const __bf16 lo = (__bf16)(p - (float)hi);
      phi[r] = __builtin_bit_cast(short, hi);
      plo[r] = __builtin_bit_cast(short, lo);
    }
    // every hi product, then every lo product (no product waits on the one
    // just issued)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf[dt], phi, st.o[dt], 0, 0, 0);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf[dt], plo, st.o[dt], 0, 0, 0);
  };
  // The ring's four slots are free when a stream starts: stages 0..3 go out
  // at once (a stream of at most four stages, such as a chosen chunk's rows,
  // waits for one memory round trip). Step b waits for stage b (the 8 loads
  // of each later stage may still be outstanding), computes it, and issues
  // stage b + 4 into its slot (its reads completed inside their asm blocks).
  for (int b = 0; b < nb && b < 4; ++b) {
    plook(b);
    issue(b);
  }
  if (nb > 4) plook(4);
  for (int b = 0; b < nb; ++b) {
    if (b + 3 < nb) {
      uwait_vm<24>();
    } else if (b + 2 < nb) {
      uwait_vm<16>();
    } else if (b + 1 < nb) {
      uwait_vm<8>();
    } else {
      uwait_vm<0>();   // the last stage: nothing of this stream left in flight
    }
    compute(b);
    if (b + 4 < nb) {
      issue(b + 4);
      if (b + 5 < nb) plook(b + 5);   // its page-table reads land while stage b + 1 computes
    }
  }
}

// The four waves' softmax states combined: into out/lse (slot == nullptr) or
// into one partial (m, l, acc[128] per head) written with device-scope stores.
template <int G>
__device__ __forceinline__ void unit_combine(UnitLds& L, const UState& st, int w, float* __restrict__ out,
                                             float* __restrict__ lse, float* __restrict__ slot) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int hq = lane & 15, jg = lane >> 4;
  __syncthreads();   // LDS changes role: rings -> merge
  float lw = st.l + __uint_as_float(lane_xor<16>(__float_as_uint(st.l)));
  lw += __uint_as_float(lane_xor<32>(__float_as_uint(lw)));
  if (jg == 0) {
    L.u.mrg.m[hq][w] = st.m;
    L.u.mrg.l[hq][w] = lw;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    *reinterpret_cast<f32x4u*>(&L.u.mrg.o[w][hq][16 * dt + 4 * jg]) = st.o[dt];
  __syncthreads();
  // thread (h, 4 columns): G * 32 threads, every read of a thread in flight at once
  if (tid < G * 32) {
    const int h = tid >> 5, d4 = 4 * (tid & 31);
    const float4 mm = *reinterpret_cast<const float4*>(L.u.mrg.m[h]);
    const float4 ll = *reinterpret_cast<const float4*>(L.u.mrg.l[h]);
    float4 ov[kUW];
#pragma unroll
    for (int ww = 0; ww < kUW; ++ww) ov[ww] = *reinterpret_cast<const float4*>(&L.u.mrg.o[ww][h][d4]);
    const float Mx = fmaxf(fmaxf(mm.x, mm.y), fmaxf(mm.z, mm.w));
    const float f[kUW] = {fexp2(mm.x - Mx), fexp2(mm.y - Mx), fexp2(mm.z - Mx), fexp2(mm.w - Mx)};
    const float Sm = ll.x * f[0] + ll.y * f[1] + ll.z * f[2] + ll.w * f[3];
    float4 ac = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int ww = 0; ww < kUW; ++ww) {
      ac.x = fmaf(ov[ww].x, f[ww], ac.x);
      ac.y = fmaf(ov[ww].y, f[ww], ac.y);
      ac.z = fmaf(ov[ww].z, f[ww], ac.z);
      ac.w = fmaf(ov[ww].w, f[ww], ac.w);
    }
    if (slot == nullptr) {
      const float inv = 1.f / Sm;
      *reinterpret_cast<float4*>(out + h * 128 + d4) = make_float4(ac.x * inv, ac.y * inv, ac.z * inv, ac.w * inv);
      if (d4 == 0 && lse) lse[h] = (Mx + log2f(Sm)) * kLn2;
    } else {
      float* hs = slot + h * (128 + 2);
      st_coh(hs + 2 + d4, ac.x);
      st_coh(hs + 3 + d4, ac.y);
      st_coh(hs + 4 + d4, ac.z);
      st_coh(hs + 5 + d4, ac.w);
      if (d4 == 0) {
        st_coh(hs, Mx);
        st_coh(hs + 1, Sm);
      }
    }
  }
}

// A stream workgroup's candidates, written with device-scope stores to its
// cap = cand_cap(S, kk) slots of the unit's candidate rows (scores, ids):
// every one of its n group scores (LDS, items id0 .. id0 + n - 1) at or
// above tau, a lower bound on its kk-th largest (select_tau), in id order,
// padded with -inf scores. The unit's top-kk lies in the union of its splits'
// top-kk (under the total order: larger score, then smaller id), so in the
// union of these lists, whose slots are in id order: a selection over them
// with ties to the earlier slot is the selection over every score. When more
// than cap scores reach tau (ties over a range, or cap = kk), the exact top-kk
// (unit_select) is written instead. gscr: the unit's score row at id0 (the
// radix fallback's copy of the scores).
constexpr int kCandPer = 32;   // keys per thread of a stream workgroup's own selection
// k <= 64: select_tau bounds a workgroup's k-th score (k > 16: from its
// threads' four largest), and the unfold launch selects among S cap
// candidates instead of every score.
constexpr int kCandMaxK = kUnitCandMaxK;
static_assert(kCandMaxK <= kFastSel, "select_tau bounds the k-th score for k <= 64");
static_assert(kCandPer * kThreads >= kUWgItems && kCandPer % 16 == 0, "a workgroup's scores fit the selection");
__device__ __forceinline__ void unit_cands(UnitLds& L, int n, int kk, int id0, float* gscr, float* cs, int32_t* ci,
                                           int S, int split, int unit) {
  __syncthreads();   // the LDS union is free again (the merge is done)
  if (kk <= 0) return;   // uniform
  const int cap = cand_cap(S, kk);
  float* csp = cs + (size_t)split * cap;
  int32_t* cip = ci + (size_t)split * cap;
  const int tid = threadIdx.x;
  int written;
  if (kk >= n) {
    for (int i = tid; i < n; i += kThreads) {
      st_coh(csp + i, L.scores[i]);
      st_coh(cip + i, (int32_t)(id0 + i));
    }
    written = n;
  } else {
    const int per = select_per(n);
    const int i0 = tid * per;
    const int nv = max(0, min(per, n - i0));
    uint32_t key[kCandPer];
    select_keys<kCandPer, true, kUWgItems>(L.scores, nullptr, 0, i0, per, nv, key);
    const uint32_t tau = select_tau(key, kk, L.u.sel.s);
    int c = 0;
#pragma unroll
    for (int j = 0; j < kCandPer; ++j) c += key[j] >= tau ? 1 : 0;
    int total;
    int run = select_scan(c, L.u.sel.s, &total);
    if (total <= cap) {   // uniform
#pragma unroll
      for (int j = 0; j < kCandPer; ++j) {
        if (key[j] >= tau) {
          st_coh(csp + run, L.scores[i0 + j]);
          st_coh(cip + run, (int32_t)(id0 + i0 + j));
          ++run;
        }
      }
      written = total;
    } else {
      __syncthreads();
      unit_select<kCandPer, true, kUWgItems>(L.scores, n, kk, gscr, 0, unit, L.sel, L.u.sel.s, L.u.sel.t);
      __syncthreads();
      for (int i = tid; i < kk; i += kThreads) {
        const int j = L.sel[i];
        st_coh(csp + i, L.scores[j]);
        st_coh(cip + i, (int32_t)(id0 + j));
      }
      written = kk;
    }
  }
  for (int i = written + tid; i < cap; i += kThreads) {
    st_coh(csp + i, -INFINITY);
    st_coh(cip + i, (int32_t)id0);
  }
}

// The unit's top-kk among its S splits' candidate lists, ids ascending, into
// dst (LDS); every thread of the workgroup takes part. The ids travel with
// the scores (staged in the LDS score array when they fit), so the mapping
// from list position to id costs no further round trip.
// Few candidates (nc <= 256, kk <= 16): thread t takes candidate t as the
// composite key order_key(score) << 32 | ~id (equal scores: the smaller id
// ranks first; ids are distinct among real candidates, and the -inf padding
// ranks below every real one), each wave sorts its 64 keys, and one wave
// sorts the four waves' 16 best: two sorts, no threshold, scan or rank pass.
// top: LDS for the waves' 16 best. dst (LDS) gets the kk ids ascending; it is
// valid after the barrier at the end.
__device__ __forceinline__ void select_small_keys(unsigned long long key, int nc, int kk, int32_t* dst,
                                                  unsigned long long (&top)[kUW][16]) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (w * 64 < nc) {   // uniform per wave: a wave past the candidates holds only zeros
    key = wave_sort<true>(key);
  }
  if (lane < 16) top[w][lane] = key;
  __syncthreads();
  if (w == 0) {
    unsigned long long k2 = top[lane >> 4][lane & 15];
    k2 = wave_sort<true>(k2);
    uint32_t id = lane < kk ? ~(uint32_t)k2 : 0xFFFFFFFFu;
    id = wave_sort<false>(id);
    if (lane < kk) dst[lane] = (int32_t)id;
  }
  __syncthreads();
}
// candidates in device memory, written by other workgroups
__device__ __forceinline__ void select_small(const float* cs, const int32_t* ci, int stride, int nc, int kk,
                                             int32_t* dst, unsigned long long (&top)[kUW][16]) {
  const int tid = threadIdx.x;
  const CohBuf sb(cs, (uint32_t)stride * 4u), ib(ci, (uint32_t)stride * 4u);
  unsigned long long key = 0ull;
  if (tid < nc) {
    const uint32_t sv = sb.u32((uint32_t)tid), iv = ib.u32((uint32_t)tid);
    key = ((unsigned long long)order_key(__uint_as_float(sv)) << 32) | (uint32_t)~iv;
  }
  select_small_keys(key, nc, kk, dst, top);
}
// scores in LDS, the id of item i being i
__device__ __forceinline__ void select_small_lds(const float* sc, int nc, int kk, int32_t* dst,
                                                 unsigned long long (&top)[kUW][16]) {
  const int tid = threadIdx.x;
  const unsigned long long key =
      tid < nc ? ((unsigned long long)order_key(sc[tid]) << 32) | (uint32_t)~(uint32_t)tid : 0ull;
  select_small_keys(key, nc, kk, dst, top);
}

__device__ __forceinline__ void select_cands(const Cands& c, int S, int unit, int kk, int32_t* dst, UnitLds& L) {
  if (kk <= 0) return;
  const int nc = S * cand_cap(S, kk);
  float* cs = c.s + (size_t)unit * c.stride;
  if (nc <= kUW * 64 && kk <= 16) {   // uniform
    select_small(cs, c.id + (size_t)unit * c.stride, c.stride, nc, kk, dst, L.wtop);
    return;
  }
  const CohBuf ids(c.id + (size_t)unit * c.stride, (uint32_t)c.stride * 4u);
  const int tid = threadIdx.x;
  const bool staged = nc <= kUWgItems;   // uniform
  int32_t* idl = reinterpret_cast<int32_t*>(L.scores);
  // the id loads go out with the score loads; they land in LDS after them
  constexpr int kIdsPer = kUWgItems / kThreads;
  uint32_t idr[kIdsPer];
#pragma unroll
  for (int q = 0; q < kIdsPer; ++q) {
    const int i = tid + q * kThreads;
    idr[q] = staged && i < nc ? ids.u32((uint32_t)i) : 0u;
  }
  if (nc <= kUMaxGist)   // uniform: fewer keys per thread, a shorter selection
    unit_select<kUMaxGist / kThreads, false>(nullptr, nc, kk, cs, c.stride, unit, dst, L.u.sel.s, L.u.sel.t);
  else
    unit_select<kUMaxSel / kThreads, false>(nullptr, nc, kk, cs, c.stride, unit, dst, L.u.sel.s, L.u.sel.t);
  if (staged) {
#pragma unroll
    for (int q = 0; q < kIdsPer; ++q) {
      const int i = tid + q * kThreads;
      if (i < nc) idl[i] = (int32_t)idr[q];
    }
  }
  __syncthreads();
  const int id = tid < kk ? (staged ? idl[dst[tid]] : (int)ids.u32((uint32_t)dst[tid])) : 0;
  __syncthreads();
  if (tid < kk) dst[tid] = id;
  __syncthreads();
}

template <int G, bool SETS = false>
__device__ __forceinline__ void hier_descent(const UnitArgs& a, UnitLds& L, int unit, const bf16x8u (&qf)[4]);

// HIER (kHierDescend, kHierTop): the level-2 gists (their own arrays) and the
// tail; every workgroup hands its partial state and its top-k2 level-2
// candidates on. kHierDescend (two-level decode): the unit's last workgroup
// then runs the descent. kHierTop (the top level of L-level decode):
// unit_levels_kernel does, in a second launch.
enum { kHierNone = 0, kHierDescend = 1, kHierTop = 2 };
// SPLIT: several workgroups per unit (a.S > 1); the one-workgroup-per-unit
// instantiation carries none of the hand-off code.
// PAGED (with VARLEN): the caches are page pools (gsa_decode_paged).
template <int G, int HIER, bool SETS = false, bool VARLEN = false, bool SPLIT = true, bool PAGED = false>
__global__ __launch_bounds__(kUW * 64) void unit_kernel(UnitArgs args) {
  static_assert(!PAGED || (VARLEN && !HIER), "paged caches: single-level, per-sequence lengths");
  __shared__ __attribute__((aligned(16))) std::conditional_t<PAGED, PagedLds, UnitLds> L;
  UnitArgs a = args;
  // the wave index as a scalar: each wave's item ranges and trip counts are
  // then uniform, and the row loops branch on scalars
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hq = lane & 15, jg = lane >> 4;
  const int S = SPLIT ? a.S : 1;
  const int unit = blockIdx.x / S, split = blockIdx.x - unit * S;
  if constexpr (!SETS) GSA_STAMP(0);
  const int64_t m2_slab = a.M2;   // rows of a level-2 slab (the call's M2)
  if constexpr (VARLEN && HIER)
    hier_lengths(args.seq, unit, args.N, args.M, args.C, args.T, args.M2, args.n_cand, &a.N, &a.M, &a.M2,
                 &a.n_cand);
  else if constexpr (VARLEN)
    unit_lengths(args.seq, unit, args.N, args.M, args.C, args.T, &a.N, &a.M);
  const char* Kb = reinterpret_cast<const char*>(a.K) + (size_t)unit * a.R * 256;
  const char* Vb = reinterpret_cast<const char*>(a.V) + (size_t)unit * a.R * 256;
  const PagedLds* pl = nullptr;
  int n_extra = 0;
  if constexpr (PAGED) {
    stage_pages(a, unit, L);
    pl = &L;
    n_extra = L.n_extra;
    Kb = reinterpret_cast<const char*>(a.K) + (size_t)(unit % a.Hkv) * a.pg_head_bytes;
    Vb = reinterpret_cast<const char*>(a.V) + (size_t)(unit % a.Hkv) * a.pg_head_bytes;
  }
  // query fragments: lane (h, j) holds q_h[32 ks + 8 j .. +8], zero past g heads
  bf16x8u qf[4];
  {
    const char* qb = reinterpret_cast<const char*>(a.q) + ((size_t)unit * G + (hq < G ? hq : 0)) * 256 + 16 * jg;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 v = hq < G ? load16(qb + 64 * ks) : make_uint4(0u, 0u, 0u, 0u);
      qf[ks] = __builtin_bit_cast(bf16x8u, v);
    }
    // settle here: a first use inside the row loop would wait for every load
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) __asm__ volatile("" : "+v"(qf[ks]));
  }
  UState st;
  st.m = kMinus;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.o[dt] = f32x4u{0.f, 0.f, 0.f, 0.f};
  char* ring = L.u.ring[w][0];
  // gists and tail as one item range: S consecutive shares, each in four wave shares
  const int M = (int)a.M;
  const int nf = HIER ? (int)a.M2 : M;   // scored items ahead of the tail
  const int n1 = nf + a.T + n_extra;     // (paged: the extra rows after the tail)
  const int perw = (n1 + S - 1) / S;
  const int w0 = min(n1, split * perw), w1 = min(n1, w0 + perw);
  const int per1 = (w1 - w0 + kUW - 1) / kUW;
  if constexpr (HIER) {
    // level-2 slabs hold the call's M2 rows (a sequence's own first)
    const char* K2b = reinterpret_cast<const char*>(a.K2) + (size_t)unit * m2_slab * 256;
    const char* V2b = reinterpret_cast<const char*>(a.V2) + (size_t)unit * m2_slab * 256;
    // selection rules (SETS): the level-2 gists route but are not attended
    unit_stream<kUKL2, false, SETS>(Kb, Vb, min(w1, w0 + w * per1), min(w1, w0 + (w + 1) * per1), a, qf, st, ring,
                                    L.scores, L.sel, w0, K2b, V2b);
    GSA_STAMP(1);
    float* part_u = a.part + (size_t)unit * a.NP * a.part_stride;
    unit_combine<G>(L, st, w, nullptr, nullptr, part_u + (size_t)split * a.part_stride);
    GSA_STAMP(5);
    float* s2u = a.s2 + (size_t)unit * a.s2_stride;
    for (int i = w0 + tid; i < min(w1, nf); i += kUW * 64) st_coh(s2u + i, L.scores[i - w0]);
    if constexpr (HIER == kHierDescend) {
      if (!arrive_last(a.cnt + (size_t)unit * kCtrlUnitWords, (uint32_t)S, &L.s_old)) return;
      GSA_STAMP(6);
      hier_descent<G, SETS>(a, L, unit, qf);
    }
    return;
  }
  if constexpr (SETS && SPLIT) {
    // selection-rule variants, several workgroups per unit: each scores its
    // share of the gists (K rows only, no attention) and hands on candidates
    // (k <= 16) or its scores; unit_unfold_kernel<SETS> selects and attends
    // the set (chosen raw rows, their gists if the set keeps them, the tail)
    const int perg = (M + S - 1) / S;
    const int g0 = min(M, split * perg), g1 = min(M, g0 + perg);
    const int pw = (g1 - g0 + kUW - 1) / kUW;
    unit_stream<kUKScore, PAGED>(Kb, Vb, min(g1, g0 + w * pw), min(g1, g0 + (w + 1) * pw), a, qf, st, ring,
                                 L.scores, L.sel, g0, nullptr, nullptr, pl);
    float* gs = a.scores + (size_t)unit * a.score_stride;
    __syncthreads();   // every score of the share is in LDS
    if (a.k > kCandMaxK) {
      for (int i = g0 + tid; i < g1; i += kUW * 64) st_coh(gs + i, L.scores[i - g0]);
    } else if (a.k > 0) {
      const Cands c = cands_of(a, (int)(gridDim.x / S), a.k);
      unit_cands(L, g1 - g0, a.k, g0, gs + g0, c.s + (size_t)unit * c.stride, c.id + (size_t)unit * c.stride, S,
                 split, unit);
    }
    return;
  }
  if constexpr (SETS) {
    // selection-rule variants (one workgroup per unit): the gists' K rows for
    // the scores only; then the chosen chunks' raw rows, their gists if the
    // set keeps them, and the tail, all attended
    const int perg = (M + kUW - 1) / kUW;
    unit_stream<kUKScore, PAGED>(Kb, Vb, min(M, w * perg), min(M, (w + 1) * perg), a, qf, st, ring, L.scores, L.sel,
                                 0, nullptr, nullptr, pl);
    __syncthreads();   // every group score is in LDS, every ring idle
    float* gsv = a.scores + (size_t)unit * a.score_stride;
    if (a.k > 0) {
      unit_select<kUMaxGist / kThreads, true>(L.scores, M, a.k, gsv, a.score_stride, unit, L.sel, L.u.sel.s,
                                               L.u.sel.t);
      __syncthreads();
    }
    const int n3 = a.k * a.C + (a.gist_set == 1 ? a.k : 0) + a.T + n_extra;   // (paged: the extra rows last)
    const int per3 = (n3 + kUW - 1) / kUW;
    unit_stream<kUKSet, PAGED>(Kb, Vb, min(n3, w * per3), min(n3, (w + 1) * per3), a, qf, st, ring, L.scores, L.sel,
                               0, nullptr, nullptr, pl);
    unit_combine<G>(L, st, w, a.out + (size_t)unit * G * 128, a.lse ? a.lse + (size_t)unit * G : nullptr, nullptr);
    if (a.sel)
      for (int i = tid; i < a.k; i += kUW * 64) a.sel[(size_t)unit * a.k + i] = L.sel[i];
    return;
  }
  unit_stream<kUKGists, PAGED>(Kb, Vb, min(w1, w0 + w * per1), min(w1, w0 + (w + 1) * per1), a, qf, st, ring,
                               L.scores, L.sel, w0, nullptr, nullptr, pl);
  float* gs = a.scores + (size_t)unit * a.score_stride;
  const int items = a.k * a.C;
  const int per2 = (items + kUW - 1) / kUW;
  if constexpr (!SPLIT) {
    GSA_STAMP(1);
    if (a.k > 0) {
      __syncthreads();   // every group score is in LDS, every ring idle
      unit_select<kUMaxGist / kThreads, true>(L.scores, M, a.k, gs, a.score_stride, unit, L.sel, L.u.sel.s,
                                               L.u.sel.t);
      __syncthreads();
      GSA_STAMP(2);
      unit_stream<kUKUnfold, PAGED>(Kb, Vb, min(items, w * per2), min(items, (w + 1) * per2), a, qf, st, ring,
                                    L.scores, L.sel, 0, nullptr, nullptr, pl);
    }
    GSA_STAMP(3);
    unit_combine<G>(L, st, w, a.out + (size_t)unit * G * 128, a.lse ? a.lse + (size_t)unit * G : nullptr,
                    nullptr);
    GSA_STAMP(4);
  } else {
    // hand the split's partial state (and group scores) on: with k > 0 to the
    // unfold launch, else to the unit's last workgroup, which merges
    // (device-scope stores: the XCDs' L2s are not coherent)
    GSA_STAMP(1);
    float* part_u = a.part + (size_t)unit * a.NP * a.part_stride;
    unit_combine<G>(L, st, w, nullptr, nullptr, part_u + (size_t)split * a.part_stride);
    GSA_STAMP(5);
    if (a.k > kCandMaxK) {   // the unfold launch selects among every score
      for (int i = w0 + tid; i < min(w1, M); i += kUW * 64) st_coh(gs + i, L.scores[i - w0]);
      GSA_STAMP(6);
      return;
    }
    if (a.k > 0) {   // the unfold launch selects among the splits' candidates
      const Cands c = cands_of(a, (int)(gridDim.x / S), a.k);
      unit_cands(L, max(0, min(w1, M) - w0), a.k, w0, gs + w0, c.s + (size_t)unit * c.stride,
                 c.id + (size_t)unit * c.stride, S, split, unit);
      GSA_STAMP(6);
      return;
    }
    if (!arrive_last(a.cnt + (size_t)unit * kCtrlUnitWords, (uint32_t)S, &L.s_old)) return;
    merge_unit<128, G>(part_u, S, (uint32_t)a.part_stride, a.out + (size_t)unit * G * 128,
                       a.lse ? a.lse + (size_t)unit * G : nullptr, kWaves);
    return;
  }
  if (a.sel)
    for (int i = tid; i < a.k; i += kUW * 64) a.sel[(size_t)unit * a.k + i] = L.sel[i];
}


// Second launch of the several-workgroups-per-unit path (k > 0): workgroup
// (unit, p) makes the unit's selection from the group scores the stream
// launch wrote (every workgroup of the unit makes the same one), streams
// share p of the chosen chunks' raw rows, and hands its partial state on; the
// unit's last workgroup merges the S stream and S2 unfold partials.
// SETS: the selection-rule variants, whose stream launch only scored the
// gists: the workgroups attend the set (chosen raw rows, their gists if the
// set keeps them, the tail) and the last merges their S2 partials alone.
template <int G, bool VARLEN = false, bool PAGED = false, bool SETS = false>
__global__ __launch_bounds__(kUW * 64) void unit_unfold_kernel(UnitArgs args) {
  static_assert(!PAGED || VARLEN, "paged caches: per-sequence lengths");

  __shared__ __attribute__((aligned(16))) std::conditional_t<PAGED, PagedLds, UnitLds> L;
  UnitArgs a = args;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hq = lane & 15, jg = lane >> 4;
  const int S2 = a.S2;
  const int unit = blockIdx.x / S2, part = blockIdx.x - unit * S2;
  GSA_STAMP(8);
  if constexpr (VARLEN) unit_lengths(args.seq, unit, args.N, args.M, args.C, args.T, &a.N, &a.M);
  const char* Kb = reinterpret_cast<const char*>(a.K) + (size_t)unit * a.R * 256;
  const char* Vb = reinterpret_cast<const char*>(a.V) + (size_t)unit * a.R * 256;
  const PagedLds* pl = nullptr;
  if constexpr (PAGED) {
    stage_pages(a, unit, L);
    pl = &L;
    Kb = reinterpret_cast<const char*>(a.K) + (size_t)(unit % a.Hkv) * a.pg_head_bytes;
    Vb = reinterpret_cast<const char*>(a.V) + (size_t)(unit % a.Hkv) * a.pg_head_bytes;
  }
  bf16x8u qf[4];
  {
    const char* qb = reinterpret_cast<const char*>(a.q) + ((size_t)unit * G + (hq < G ? hq : 0)) * 256 + 16 * jg;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 v = hq < G ? load16(qb + 64 * ks) : make_uint4(0u, 0u, 0u, 0u);
      qf[ks] = __builtin_bit_cast(bf16x8u, v);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) __asm__ volatile("" : "+v"(qf[ks]));
  }
  UState st;
  st.m = kMinus;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.o[dt] = f32x4u{0.f, 0.f, 0.f, 0.f};
  if (a.k > kCandMaxK) {
    unit_select<kUMaxSel / kThreads, false>(nullptr, (int)a.M, a.k, a.scores + (size_t)unit * a.score_stride,
                                            a.score_stride, unit, L.sel, L.u.sel.s, L.u.sel.t);
    __syncthreads();
  } else {
    select_cands(cands_of(a, (int)(gridDim.x / S2), a.k), a.S, unit, a.k, L.sel, L);
  }
  GSA_STAMP(9);
  // SETS: raw rows of the chosen chunks, their gists (rule 1), then the tail
  // SETS: raw rows, their gists (rule 1), the tail, then (paged) the extra rows
  int items = a.k * a.C + (SETS ? (a.gist_set == 1 ? a.k : 0) + a.T : 0);
  if constexpr (SETS && PAGED) items += L.n_extra;
  const int perp = (items + S2 - 1) / S2;
  const int p0 = min(items, part * perp), p1 = min(items, p0 + perp);
  const int per2 = (p1 - p0 + kUW - 1) / kUW;
  if constexpr (SETS)
    unit_stream<kUKSet, PAGED>(Kb, Vb, min(p1, p0 + w * per2), min(p1, p0 + (w + 1) * per2), a, qf, st, L.u.ring[w][0],
                        L.scores, L.sel, 0, nullptr, nullptr, pl);
  else
    unit_stream<kUKUnfold, PAGED>(Kb, Vb, min(p1, p0 + w * per2), min(p1, p0 + (w + 1) * per2), a, qf, st,
                                  L.u.ring[w][0], L.scores, L.sel, 0, nullptr, nullptr, pl);
  GSA_STAMP(10);
  float* part_u = a.part + (size_t)unit * a.NP * a.part_stride;
  unit_combine<G>(L, st, w, nullptr, nullptr, part_u + (size_t)(a.S + part) * a.part_stride);
  GSA_STAMP(11);
  if (!arrive_last(a.cnt + (size_t)unit * kCtrlUnitWords, (uint32_t)S2, &L.s_old)) return;
  // the stream launch's partials, then these; SETS: these alone
  const int m0 = SETS ? a.S : 0;
  merge_unit<128, G>(part_u + (size_t)m0 * a.part_stride, a.S + S2 - m0, (uint32_t)a.part_stride,
                     a.out + (size_t)unit * G * 128, a.lse ? a.lse + (size_t)unit * G : nullptr, kWaves);
  GSA_STAMP(12);
  if (a.sel)
    for (int i = tid; i < a.k; i += kUW * 64) a.sel[(size_t)unit * a.k + i] = L.sel[i];
}

// Two-level decode, the rest of a unit after its level-2 stream (run by the
// unit's last stream workgroup): the level-2 selection among the splits'
// candidates, the level-1 candidates (group scores kept in LDS), their
// selection, the chosen chunks' raw rows, and the merge of every partial.
// SETS: the selection rules (R20): the candidates are scored only, and the
// set's rows after the routing are the chosen chunks' raw rows and, with
// gist_set 1, their gists (the tail came with the level-2 stream).
template <int G, bool SETS>
__device__ __forceinline__ void hier_descent(const UnitArgs& a, UnitLds& L, int unit, const bf16x8u (&qf)[4]) {
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const char* Kb = reinterpret_cast<const char*>(a.K) + (size_t)unit * a.R * 256;
  const char* Vb = reinterpret_cast<const char*>(a.V) + (size_t)unit * a.R * 256;
  UState st;
  st.m = kMinus;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.o[dt] = f32x4u{0.f, 0.f, 0.f, 0.f};
  char* ring = L.u.ring[w][0];
  // level 2: the chosen groups, ascending, from the stream workgroups' scores
  float* s2u = a.s2 + (size_t)unit * a.s2_stride;
  GSA_STAMP(8);
  if (a.M2 <= kUMaxGist)   // uniform: fewer keys per thread, a shorter selection
    unit_select<kUMaxGist / kThreads, false>(nullptr, (int)a.M2, a.k2, s2u, a.s2_stride, unit, L.sel2, L.u.sel.s,
                                             L.u.sel.t);
  else
    unit_select<kUMaxSel / kThreads, false>(nullptr, (int)a.M2, a.k2, s2u, a.s2_stride, unit, L.sel2, L.u.sel.s,
                                            L.u.sel.t);
  __syncthreads();
  GSA_STAMP(9);
  // level 1: every candidate gist (scored), four wave shares
  const int nc = a.n_cand;
  const int perc = (nc + kUW - 1) / kUW;
  unit_stream<kUKCand, false, SETS>(Kb, Vb, min(nc, w * perc), min(nc, (w + 1) * perc), a, qf, st, ring, L.scores,
                                     L.sel2);
  GSA_STAMP(10);
  if (a.k > 0) {
    __syncthreads();   // every candidate score is in LDS, every ring idle
    float* gsc = a.scores + (size_t)unit * a.score_stride;
    if (nc <= kUW * 64 && a.k <= 16 && a.k < nc) {
      select_small_lds(L.scores, nc, a.k, L.sel, L.wtop);
    } else {
      unit_select<kUMaxGist / kThreads, true>(L.scores, nc, a.k, gsc, a.score_stride, unit, L.sel, L.u.sel.s,
                                              L.u.sel.t);
      __syncthreads();
    }
    GSA_STAMP(11);
    // candidate index -> chunk id (candidates are in chunk order)
    if (tid < a.k) {
      const int c = L.sel[tid], kg = a.k2 * a.G2;
      L.sel[tid] = c < kg ? L.sel2[c / a.G2] * a.G2 + c % a.G2 : (int)(a.M2 * a.G2) + (c - kg);
    }
    __syncthreads();
    if constexpr (SETS) {
      // the chosen chunks' raw rows, then their gists under rule 1 (kUKSet's
      // items before the tail)
      const int items = a.k * a.C + (a.gist_set == 1 ? a.k : 0);
      const int per2 = (items + kUW - 1) / kUW;
      unit_stream<kUKSet>(Kb, Vb, min(items, w * per2), min(items, (w + 1) * per2), a, qf, st, ring, L.scores,
                          L.sel);
    } else {
      const int items = a.k * a.C;
      const int per2 = (items + kUW - 1) / kUW;
      unit_stream<kUKUnfold>(Kb, Vb, min(items, w * per2), min(items, (w + 1) * per2), a, qf, st, ring, L.scores,
                             L.sel);
    }
    GSA_STAMP(12);
  }
  float* part_u = a.part + (size_t)unit * a.NP * a.part_stride;
  unit_combine<G>(L, st, w, nullptr, nullptr, part_u + (size_t)a.S * a.part_stride);
  done_stores();
  __syncthreads();
  GSA_STAMP(13);
  merge_unit<128, G>(part_u, a.S + 1, (uint32_t)a.part_stride, a.out + (size_t)unit * G * 128,
                     a.lse ? a.lse + (size_t)unit * G : nullptr, kWaves);
  GSA_STAMP(14);
  if (a.sel2)
    for (int i = tid; i < a.k2; i += kUW * 64) a.sel2[(size_t)unit * a.k2 + i] = L.sel2[i];
  if (a.sel)
    for (int i = tid; i < a.k; i += kUW * 64) a.sel[(size_t)unit * a.k + i] = L.sel[i];
}

// L-level decode, one workgroup per unit after the top level's stream launch:
// choose among the top level's scores, then for each level below stream its
// candidates (the chosen gists' children and the ungrouped gists: dense rows
// of the level's array, gist rows of the interleaved cache at level 1) into
// the wave states with their scores in LDS, choose among them, and finally
// unfold the chosen chunks and merge. The level-1 part is hier_descent's.
struct LevelArgs {
  int32_t L, G;
  const void* K[GSA_MAX_LEVELS + 1];     // l >= 2: [units][Ml[l]][D]
  const void* V[GSA_MAX_LEVELS + 1];
  int64_t Ml[GSA_MAX_LEVELS + 1];
  int32_t kl[GSA_MAX_LEVELS + 1];
  int32_t items[GSA_MAX_LEVELS + 1];     // candidates of level l < L
  int32_t* sel_out[GSA_MAX_LEVELS + 1];  // l >= 2: [units][kl[l]] chosen ids, or null
};

// TOP: the workgroup also streams the top level and the tail itself (top
// level <= kUMaxGist gists, its scores kept in LDS): one launch per call.
// VARLEN (with TOP): per-sequence lengths; sequence b's level l holds
// floor(M_b / G^(l-1)) gists, the first rows of its slab of that level, and a
// sequence whose lengths break a rule (unit_lengths', k_L at most its top
// level, each k_l at most its candidates) runs with the call's maxima.
// SETS: the selection rules (R20): every level's gists are scored only, and
// after the routing the chosen chunks' raw rows and, with gist_set 1, their
// gists are attended (the tail came with the top level's stream).
template <int G, bool TOP = false, bool VARLEN = false, bool SETS = false>
__global__ __launch_bounds__(kUW * 64) void unit_levels_kernel(UnitArgs a, LevelArgs lv) {
  static_assert(!VARLEN || TOP, "per-sequence lengths: the one-launch path");
  __shared__ __attribute__((aligned(16))) UnitLds L;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hq = lane & 15, jg = lane >> 4;
  const int unit = blockIdx.x;
  // gists of level l (>= 1) and candidates of level l < L of this unit's
  // sequence (the call's, from the plan, for uniform lengths)
  int64_t m_seq = a.M;
  auto count = [&](int l) -> int64_t {
    if constexpr (!VARLEN) return lv.Ml[l];
    int64_t c = m_seq;
    for (int i = 1; i < l; ++i) c /= lv.G;
    return c;
  };
  auto cands = [&](int l) -> int32_t {
    if constexpr (!VARLEN) return lv.items[l];
    return (int32_t)((int64_t)lv.kl[l + 1] * lv.G + count(l) - count(l + 1) * lv.G);
  };
  if constexpr (VARLEN) {
    const int64_t N0 = a.N, M0 = a.M;
    unit_lengths(a.seq, unit, N0, M0, a.C, a.T, &a.N, &m_seq);
    bool ok = lv.kl[lv.L] <= count(lv.L);
    for (int l = 1; l < lv.L; ++l) ok = ok && (l == 1 ? a.k : lv.kl[l]) <= cands(l);
    if (!ok) {   // the call's maxima
      a.N = N0;
      m_seq = M0;
    }
    a.M = m_seq;
  }
  const char* Kb = reinterpret_cast<const char*>(a.K) + (size_t)unit * a.R * 256;
  const char* Vb = reinterpret_cast<const char*>(a.V) + (size_t)unit * a.R * 256;
  bf16x8u qf[4];
  {
    const char* qb = reinterpret_cast<const char*>(a.q) + ((size_t)unit * G + (hq < G ? hq : 0)) * 256 + 16 * jg;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 v = hq < G ? load16(qb + 64 * ks) : make_uint4(0u, 0u, 0u, 0u);
      qf[ks] = __builtin_bit_cast(bf16x8u, v);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) __asm__ volatile("" : "+v"(qf[ks]));
  }
  UState st;
  st.m = kMinus;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.o[dt] = f32x4u{0.f, 0.f, 0.f, 0.f};
  char* ring = L.u.ring[w][0];
  const int Lv = lv.L, Gf = lv.G;
  float* gsc = a.scores + (size_t)unit * a.score_stride;
  // the top level: its chosen gists, ascending
  if constexpr (TOP) {
    // its gists (dense rows of the top array, a.K2) and the tail, four wave shares
    const char* K2b = reinterpret_cast<const char*>(a.K2) + (size_t)unit * a.M2 * 256;   // slabs of the call's M_L
    const char* V2b = reinterpret_cast<const char*>(a.V2) + (size_t)unit * a.M2 * 256;
    if constexpr (VARLEN) a.M2 = count(Lv);
    const int n1 = (int)a.M2 + a.T;
    const int per1 = (n1 + kUW - 1) / kUW;
    unit_stream<kUKL2, false, SETS>(Kb, Vb, min(n1, w * per1), min(n1, (w + 1) * per1), a, qf, st, ring, L.scores,
                                    L.sel, 0, K2b, V2b);
    __syncthreads();   // every top-level score is in LDS, every ring idle
    unit_select<kUMaxGist / kThreads, true>(L.scores, (int)count(Lv), lv.kl[Lv], gsc, a.score_stride, unit, L.sel2,
                                            L.u.sel.s, L.u.sel.t);
  } else {
    unit_select<kUMaxSel / kThreads, false>(nullptr, (int)lv.Ml[Lv], lv.kl[Lv], a.s2 + (size_t)unit * a.s2_stride,
                                            a.s2_stride, unit, L.sel2, L.u.sel.s, L.u.sel.t);
  }
  __syncthreads();
  if (lv.sel_out[Lv])
    for (int i = tid; i < lv.kl[Lv]; i += kUW * 64) lv.sel_out[Lv][(size_t)unit * lv.kl[Lv] + i] = L.sel2[i];
  // the levels between: dense rows of each level's array
  for (int l = Lv - 1; l >= 2; --l) {
    UnitArgs b = a;
    b.C = 0;                 // row of gist id = id
    b.M = count(l);
    b.M2 = count(l + 1);
    b.k2 = lv.kl[l + 1];
    b.G2 = Gf;
    const char* Kl = reinterpret_cast<const char*>(lv.K[l]) + (size_t)unit * lv.Ml[l] * 256;   // the call's slabs
    const char* Vl = reinterpret_cast<const char*>(lv.V[l]) + (size_t)unit * lv.Ml[l] * 256;
    const int nc = cands(l);
    const int perc = (nc + kUW - 1) / kUW;
    unit_stream<kUKCand, false, SETS>(Kl, Vl, min(nc, w * perc), min(nc, (w + 1) * perc), b, qf, st, ring, L.scores,
                                      L.sel2);
    __syncthreads();   // every candidate score is in LDS, every ring idle
    const int k = lv.kl[l];
    unit_select<kUMaxGist / kThreads, true>(L.scores, nc, k, gsc, a.score_stride, unit, L.sel, L.u.sel.s,
                                            L.u.sel.t);
    __syncthreads();
    // candidate index -> id (candidates are in id order), then it is the
    // parent list of the level below
    int id = 0;
    if (tid < k) {
      const int c = L.sel[tid], kg = lv.kl[l + 1] * Gf;
      id = c < kg ? L.sel2[c / Gf] * Gf + c % Gf : (int)(b.M2 * Gf) + (c - kg);
    }
    __syncthreads();
    if (tid < k) {
      L.sel2[tid] = id;
      if (lv.sel_out[l]) lv.sel_out[l][(size_t)unit * k + tid] = id;
    }
    __syncthreads();
  }
  // level 1: gist rows of the interleaved cache, then the chunks
  UnitArgs b = a;
  b.M2 = count(2);
  b.k2 = lv.kl[2];
  b.G2 = Gf;
  const int nc = cands(1);
  const int perc = (nc + kUW - 1) / kUW;
  unit_stream<kUKCand, false, SETS>(Kb, Vb, min(nc, w * perc), min(nc, (w + 1) * perc), b, qf, st, ring, L.scores,
                                    L.sel2);
  if (a.k > 0) {
    __syncthreads();
    unit_select<kUMaxGist / kThreads, true>(L.scores, nc, a.k, gsc, a.score_stride, unit, L.sel, L.u.sel.s,
                                            L.u.sel.t);
    __syncthreads();
    if (tid < a.k) {
      const int c = L.sel[tid], kg = b.k2 * Gf;
      L.sel[tid] = c < kg ? L.sel2[c / Gf] * Gf + c % Gf : (int)(b.M2 * Gf) + (c - kg);
    }
    __syncthreads();
    if constexpr (SETS) {
      // the chosen chunks' raw rows, then their gists under rule 1
      const int items = a.k * a.C + (a.gist_set == 1 ? a.k : 0);
      const int per2 = (items + kUW - 1) / kUW;
      unit_stream<kUKSet>(Kb, Vb, min(items, w * per2), min(items, (w + 1) * per2), a, qf, st, ring, L.scores,
                          L.sel);
    } else {
      const int items = a.k * a.C;
      const int per2 = (items + kUW - 1) / kUW;
      unit_stream<kUKUnfold>(Kb, Vb, min(items, w * per2), min(items, (w + 1) * per2), a, qf, st, ring, L.scores,
                             L.sel);
    }
  }
  if constexpr (TOP) {
    unit_combine<G>(L, st, w, a.out + (size_t)unit * G * 128, a.lse ? a.lse + (size_t)unit * G : nullptr, nullptr);
  } else {
    float* part_u = a.part + (size_t)unit * a.NP * a.part_stride;
    unit_combine<G>(L, st, w, nullptr, nullptr, part_u + (size_t)a.S * a.part_stride);
    done_stores();
    __syncthreads();
    merge_unit<128, G>(part_u, a.S + 1, (uint32_t)a.part_stride, a.out + (size_t)unit * G * 128,
                       a.lse ? a.lse + (size_t)unit * G : nullptr, kWaves);
  }
  if (a.sel)
    for (int i = tid; i < a.k; i += kUW * 64) a.sel[(size_t)unit * a.k + i] = L.sel[i];
}

// seq_n, seq_m: per-sequence lengths (device arrays; the one-launch path
// only), or null.
template <int G>
gsa_status_t run_unit_levels(const LevelsPlan& lp, const void* q, const void* K, const void* V,
                             const void* const* Ku, const void* const* Vu, float* out, float* lse,
                             int32_t* const* sel_up, int32_t* sel1, char* ws, hipStream_t st,
                             const int32_t* seq_n = nullptr, const int32_t* seq_m = nullptr) {
  const DecodePlan& pl = lp.base;
  const int Lv = lp.L;
  const bool sets = lp.base.gist_set != GSA_GISTS_ALL;
  UnitArgs u{};
  u.gist_set = lp.base.gist_set;
  u.q = q; u.K = K; u.V = V; u.out = out; u.lse = lse; u.sel = pl.k > 0 ? sel1 : nullptr;
  u.scores = reinterpret_cast<float*>(ws + lp.off_scores[1]); u.score_stride = lp.score_stride[1];
  u.R = pl.R; u.N = pl.N; u.M = pl.M; u.C = pl.C; u.k = pl.k; u.T = pl.T;
  u.scale_log2 = pl.scale * kLog2e; u.score_mul = pl.scale / G;
  u.S = lp.unit_S; u.S2 = 0; u.NP = lp.NP; u.part_stride = part_stride(G, 128);
  u.part = reinterpret_cast<float*>(ws + lp.off_part);
  u.cnt = nullptr;
  // the stream launch sees the top level as its "level 2"
  u.K2 = Ku[Lv - 2]; u.V2 = Vu[Lv - 2]; u.M2 = lp.Ml[Lv]; u.G2 = lp.G; u.k2 = lp.kl[Lv]; u.n_cand = 0;
  u.s2 = reinterpret_cast<float*>(ws + lp.off_scores[Lv]); u.s2_stride = lp.score_stride[Lv];
  u.sel2 = nullptr;

  LevelArgs lv{};
  lv.L = Lv; lv.G = lp.G;
  for (int l = 1; l <= Lv; ++l) {
    lv.Ml[l] = lp.Ml[l];
    lv.kl[l] = lp.kl[l];
    lv.items[l] = (int32_t)lp.items[l];
    if (l >= 2) {
      lv.K[l] = Ku[l - 2];
      lv.V[l] = Vu[l - 2];
      lv.sel_out[l] = sel_up && lp.kl[l] > 0 ? sel_up[l - 2] : nullptr;
    }
  }
  prof_begin_call();
  if (levels_top_in_lds(lp)) {
    // the top level fits one workgroup's LDS scores: one launch
    const dim3 grid(pl.units), block(kUW * 64);
    if (seq_n != nullptr) u.seq = SeqLens{seq_n, seq_m, pl.Hkv, pl.k};
    if (seq_n != nullptr && sets)
      prof_launch((unit_levels_kernel<G, true, true, true>), grid, block, 0, st, u, lv);
    else if (seq_n != nullptr)
      prof_launch((unit_levels_kernel<G, true, true>), grid, block, 0, st, u, lv);
    else if (sets)
      prof_launch((unit_levels_kernel<G, true, false, true>), grid, block, 0, st, u, lv);
    else
      prof_launch((unit_levels_kernel<G, true>), grid, block, 0, st, u, lv);
  } else {
    if (sets) {
      prof_launch((unit_kernel<G, kHierTop, true>), dim3(pl.units * lp.unit_S), dim3(kUW * 64), 0, st, u);
      prof_launch((unit_levels_kernel<G, false, false, true>), dim3(pl.units), dim3(kUW * 64), 0, st, u, lv);
    } else {
      prof_launch((unit_kernel<G, kHierTop>), dim3(pl.units * lp.unit_S), dim3(kUW * 64), 0, st, u);
      prof_launch((unit_levels_kernel<G>), dim3(pl.units), dim3(kUW * 64), 0, st, u, lv);
    }
  }
  return launch_status("gsa_decode_levels launch");
}

// seq_n, seq_m: per-sequence lengths (device arrays), or null.
template <int G>
gsa_status_t run_unit_hier(const HierPlan& hp, const void* q, const void* K, const void* V, const void* K2,
                           const void* V2, float* out, float* lse, int32_t* sel2, int32_t* sel1, char* ws,
                           hipStream_t st, const int32_t* seq_n = nullptr, const int32_t* seq_m = nullptr) {
  const DecodePlan& pl = hp.base;
  UnitArgs u{};
  u.q = q; u.K = K; u.V = V; u.out = out; u.lse = lse; u.sel = pl.k > 0 ? sel1 : nullptr;
  u.scores = reinterpret_cast<float*>(ws + hp.off_sc); u.score_stride = hp.sc_stride;
  u.R = pl.R; u.N = pl.N; u.M = pl.M; u.C = pl.C; u.k = pl.k; u.T = pl.T;
  u.scale_log2 = pl.scale * kLog2e; u.score_mul = pl.scale / G;
  u.S = hp.unit_S; u.S2 = 0; u.NP = hp.NP; u.part_stride = part_stride(G, 128);
  u.part = reinterpret_cast<float*>(ws + hp.off_part);
  u.cnt = nullptr;
  u.K2 = K2; u.V2 = V2; u.M2 = hp.M2; u.G2 = hp.G; u.k2 = hp.k2; u.n_cand = hp.n_cand;
  u.s2 = reinterpret_cast<float*>(ws + hp.off_s2); u.s2_stride = hp.s2_stride;
  u.sel2 = hp.k2 > 0 ? sel2 : nullptr;
  u.cnt = ctrl_of(ws, hp.off_ctrl, 0);
  u.seq = SeqLens{seq_n, seq_m, pl.Hkv, pl.k, hp.G, hp.k2};
  u.gist_set = pl.gist_set;
  prof_begin_call();
  const bool sets = pl.gist_set != GSA_GISTS_ALL;
  const dim3 grid(pl.units * hp.unit_S), block(kUW * 64);
  if (seq_n != nullptr && sets)
    prof_launch((unit_kernel<G, kHierDescend, true, true>), grid, block, 0, st, u);
  else if (seq_n != nullptr)
    prof_launch((unit_kernel<G, kHierDescend, false, true>), grid, block, 0, st, u);
  else if (sets)
    prof_launch((unit_kernel<G, kHierDescend, true>), grid, block, 0, st, u);
  else
    prof_launch((unit_kernel<G, kHierDescend>), grid, block, 0, st, u);
  return launch_status("gsa_decode_hier launch");
}

template <int G>
gsa_status_t run_unit(const DecodePlan& pl, const void* q, const void* K, const void* V, float* out, float* lse,
                      int32_t* sel, char* ws, hipStream_t st) {
  UnitArgs u{};
  u.q = q; u.K = K; u.V = V; u.out = out; u.lse = lse; u.sel = pl.k > 0 ? sel : nullptr;
  u.scores = reinterpret_cast<float*>(ws + pl.off_scores); u.score_stride = pl.score_stride;
  u.R = pl.R; u.N = pl.N; u.M = pl.M; u.C = pl.C; u.k = pl.k; u.T = pl.T;
  u.scale_log2 = pl.scale * kLog2e; u.score_mul = pl.scale / G;
  u.S = pl.unit_S; u.S2 = pl.unit_S2; u.NP = pl.NP; u.part_stride = part_stride(G, 128);
  u.gist_set = pl.gist_set;
  u.part = reinterpret_cast<float*>(ws + pl.off_part);
  u.cnt = ctrl_of(ws, pl.off_ctrl, 0);
  u.seq = SeqLens{pl.seq_n, pl.seq_m, pl.Hkv, pl.k};
  u.Hkv = pl.Hkv;
  prof_begin_call();
  const bool varlen = pl.seq_n != nullptr;
  if (pl.pg_table != nullptr) {   // paged caches (per-sequence lengths)
    u.pg_table = pl.pg_table; u.pg_extra = pl.pg_extra; u.pg_count = pl.pg_count;
    u.pg_max = pl.pg_max; u.pg_max_extra = pl.pg_max_extra;
    int lp = 0;
    while ((1 << lp) < pl.pg_P) ++lp;
    u.pg_lp = lp;
    u.pg_rpp = pl.pg_P * (pl.C + 1);
    u.pg_bytes = (int64_t)pl.Hkv * u.pg_rpp * 256;
    u.pg_head_bytes = (int64_t)u.pg_rpp * 256;
    const dim3 block(kUW * 64);
    if (pl.gist_set != GSA_GISTS_ALL) {   // the selection rules: score, then attend the set
      if (pl.unit_S == 1) {
        prof_launch((unit_kernel<G, kHierNone, true, true, false, true>), dim3(pl.units), block, 0, st, u);
      } else {
        if (pl.k > 0)
          prof_launch((unit_kernel<G, kHierNone, true, true, true, true>), dim3(pl.units * pl.unit_S), block, 0, st, u);
        prof_launch((unit_unfold_kernel<G, true, true, true>), dim3(pl.units * pl.unit_S2), block, 0, st, u);
      }
      return launch_status("gsa_decode_paged launch");
    }
    if (pl.unit_S == 1)
      prof_launch((unit_kernel<G, kHierNone, false, true, false, true>), dim3(pl.units), block, 0, st, u);
    else
      prof_launch((unit_kernel<G, kHierNone, false, true, true, true>), dim3(pl.units * pl.unit_S), block, 0, st, u);
    if (pl.unit_S2 > 0)
      prof_launch((unit_unfold_kernel<G, true, true>), dim3(pl.units * pl.unit_S2), block, 0, st, u);
    return launch_status("gsa_decode_paged launch");
  }
  if (pl.gist_set != GSA_GISTS_ALL) {
    const dim3 block(kUW * 64);
    if (pl.unit_S == 1) {
      if (varlen)
        prof_launch((unit_kernel<G, kHierNone, true, true, false>), dim3(pl.units), block, 0, st, u);
      else
        prof_launch((unit_kernel<G, kHierNone, true, false, false>), dim3(pl.units), block, 0, st, u);
    } else {
      // the gists' scores (none needed with k = 0), then the set
      if (pl.k > 0 && varlen)
        prof_launch((unit_kernel<G, kHierNone, true, true, true>), dim3(pl.units * pl.unit_S), block, 0, st, u);
      else if (pl.k > 0)
        prof_launch((unit_kernel<G, kHierNone, true, false, true>), dim3(pl.units * pl.unit_S), block, 0, st, u);
      if (varlen)
        prof_launch((unit_unfold_kernel<G, true, false, true>), dim3(pl.units * pl.unit_S2), block, 0, st, u);
      else
        prof_launch((unit_unfold_kernel<G, false, false, true>), dim3(pl.units * pl.unit_S2), block, 0, st, u);
    }
    return launch_status(varlen ? "gsa_decode_varlen launch" : "gsa_decode launch");
  }
  else if (varlen && pl.unit_S == 1)
    prof_launch((unit_kernel<G, kHierNone, false, true, false>), dim3(pl.units), dim3(kUW * 64), 0, st, u);
  else if (varlen)
    prof_launch((unit_kernel<G, kHierNone, false, true, true>), dim3(pl.units * pl.unit_S), dim3(kUW * 64), 0, st, u);
  else if (pl.unit_S == 1)
    prof_launch((unit_kernel<G, kHierNone, false, false, false>), dim3(pl.units), dim3(kUW * 64), 0, st, u);
  else
    prof_launch((unit_kernel<G, kHierNone, false, false, true>), dim3(pl.units * pl.unit_S), dim3(kUW * 64), 0, st, u);
  if (pl.unit_S2 > 0) {
    if (varlen)
      prof_launch((unit_unfold_kernel<G, true>), dim3(pl.units * pl.unit_S2), dim3(kUW * 64), 0, st, u);
    else
      prof_launch((unit_unfold_kernel<G>), dim3(pl.units * pl.unit_S2), dim3(kUW * 64), 0, st, u);
  }
  return launch_status("gsa_decode launch");
}

// Dispatch on (dtype, head_dim, heads per kv-head).
template <template <bool, int, int> class F, class... Args>
gsa_status_t dispatch(int32_t dtype, int32_t D, int32_t G, Args&&... args) {
#define GSA_CASE(B, DD, GG) \
  if ((dtype == GSA_BF16) == B && D == DD && G == GG) return F<B, DD, GG>::run(args...);
#define GSA_CASES(B, DD) GSA_CASE(B, DD, 1) GSA_CASE(B, DD, 2) GSA_CASE(B, DD, 4) GSA_CASE(B, DD, 8)
  GSA_CASES(true, 128)
  GSA_CASES(true, 64)
  GSA_CASES(false, 128)
  GSA_CASES(false, 64)
#undef GSA_CASES
#undef GSA_CASE
  return fail(GSA_ERR_UNSUPPORTED, "no kernel for dtype=%d head_dim=%d g=%d", dtype, D, G);
}

template <bool B, int D, int G>
struct DecodeRunner {
  template <class... A>
  static gsa_status_t run(A&&... a) { return run_decode<B, D, G>(a...); }
};
template <bool B, int D, int G>
struct HierRunner {
  template <class... A>
  static gsa_status_t run(A&&... a) { return run_hier<B, D, G>(a...); }
};

// L levels: the top pass scores and attends every top-level gist and the
// tail; the pass of each lower level l first selects the top k_{l+1} of the
// level above from that pass' scores (mapped to ids), then scores and attends
// its candidates (the chosen gists' children and the ungrouped gists, dense
// rows of the level's array; level 1: gist rows of the interleaved cache);
// the unfold pass selects k_1 chunks among the level-1 candidates and merges.
template <bool BF16, int D, int G>
gsa_status_t run_levels(const LevelsPlan& lp, const void* q, const void* K, const void* V,
                        const void* const* Ku, const void* const* Vu, float* out, float* lse,
                        int32_t* const* sel_up, int32_t* sel1, char* ws, hipStream_t st) {
  const DecodePlan& pl = lp.base;
  const int L = lp.L;
  float* part = reinterpret_cast<float*>(ws + lp.off_part);
  const int64_t ps = part_stride(G, D);
  auto scores = [&](int l) { return reinterpret_cast<float*>(ws + lp.off_scores[l]); };
  auto selws = [&](int l) { return reinterpret_cast<int32_t*>(ws + lp.off_sel[l]); };
  GistArgs g{};
  g.q = q; g.K = Ku[L - 2]; g.V = Vu[L - 2];
  g.unit_rows = lp.Ml[L]; g.n_items = lp.items[L]; g.per_task = lp.per_split[L]; g.tasks = lp.S[L];
  g.rm = RowMap{1, pl.C, nullptr, 0, 0, 0, 0};
  g.Kt = K; g.Vt = V; g.tail_unit_rows = pl.R;
  // selection rules: every level pass only scores (their partial states are
  // not merged) and the tail goes to the set's pass
  const bool sets = pl.gist_set != GSA_GISTS_ALL;
  g.N = pl.N; g.M = pl.M; g.C = pl.C; g.T = pl.T; g.tail_per_task = sets ? 0 : lp.tail_per_split;
  g.score_only = sets ? 1 : 0;
  g.scores = scores(L); g.score_stride = lp.score_stride[L];
  g.part = part; g.part_stride = ps; g.NP = lp.NP; g.part_base = 0;
  g.out = nullptr; g.lse = nullptr;
  g.cnt = ctrl_of(ws, lp.off_ctrl, 0);
  g.scale_log2 = pl.scale * kLog2e; g.score_mul = pl.scale / G;
  g.fuse_k = 0;
  prof_begin_call();
  prof_launch((gist_kernel<BF16, D, G>), dim3(pl.units * lp.S[L]), dim3(kThreads), 0, st, g);
  int32_t base = lp.S[L];
  for (int l = L - 1; l >= 1; --l) {
    GistArgs c = g;
    c.K = l >= 2 ? Ku[l - 2] : K;
    c.V = l >= 2 ? Vu[l - 2] : V;
    c.unit_rows = l >= 2 ? lp.Ml[l] : pl.R;
    c.n_items = lp.items[l]; c.per_task = lp.per_split[l]; c.tasks = lp.S[l];
    // kind 2 with C = 0 gives dense rows of a level array
    c.rm = RowMap{2, l >= 2 ? 0 : pl.C, nullptr, lp.G, lp.kl[l + 1], lp.orphan0[l], 0};
    c.T = 0; c.tail_per_task = 0;
    const bool last = l == 1 && pl.k == 0 && !sets;
    c.scores = l == 1 && pl.k == 0 ? nullptr : scores(l); c.score_stride = lp.score_stride[l];
    c.prev_scores = scores(l + 1); c.prev_stride = lp.score_stride[l + 1];
    c.prev_n = (int32_t)lp.items[l + 1]; c.prev_k = lp.kl[l + 1];
    c.prev_im = l + 1 == L ? IdMap{nullptr, 0, 0, 0, 0}
                           : IdMap{selws(l + 2), lp.G, lp.kl[l + 2], lp.orphan0[l + 1], lp.sel_stride[l + 2]};
    c.sel2_ws = selws(l + 1); c.sel2_stride = lp.sel_stride[l + 1];
    c.sel2_out = sel_up ? sel_up[l - 1] : nullptr;
    c.part_base = base;
    c.out = last ? out : nullptr; c.lse = last ? lse : nullptr;
    c.cnt = ctrl_of(ws, lp.off_ctrl, L - l);
    prof_launch((gist_kernel<BF16, D, G>), dim3(pl.units * lp.S[l]), dim3(kThreads), 0, st, c);
    base += lp.S[l];
  }
  if (pl.k > 0 || sets) {
    UnfoldArgs u{};
    u.q = q; u.K = K; u.V = V; u.unit_rows = pl.R;
    u.scores = pl.k > 0 ? scores(1) : nullptr; u.score_stride = lp.score_stride[1];
    u.n_cand = (int32_t)lp.items[1];
    u.im = IdMap{selws(2), lp.G, lp.kl[2], lp.orphan0[1], lp.sel_stride[2]};
    u.sel_ws = reinterpret_cast<int32_t*>(ws + lp.off_sel1); u.sel_stride = pl.sel_stride;
    u.sel_out = sel1; u.k = pl.k;
    u.C = pl.C; u.T = pl.T; u.M = pl.M; u.N = pl.N;
    u.n_items = pl.n_items; u.per_task = pl.items_per_split; u.tasks = pl.S2;
    u.part = part; u.part_stride = ps; u.NP = lp.NP; u.part_base = base;
    u.out = out; u.lse = lse;
    u.cnt = ctrl_of(ws, lp.off_ctrl, L);
    u.set_kg = pl.gist_set == GSA_GISTS_SELECTED ? pl.k : 0;
    u.set_tail = sets ? pl.T : 0;
    u.merge_base = sets ? base : 0;
    u.scale_log2 = pl.scale * kLog2e;
    prof_launch((unfold_kernel<BF16, D, G>), dim3(pl.units * pl.S2), dim3(kThreads), 0, st, u);
  }
  return launch_status("gsa_decode_levels launch");
}

template <bool B, int D, int G>
struct LevelsRunner {
  template <class... A>
  static gsa_status_t run(A&&... a) { return run_levels<B, D, G>(a...); }
};

}  // namespace
}  // namespace gsa

namespace gsa {
namespace {
// The launches of one single-level decode call, after validation.
gsa_status_t run_decode_plan(const DecodePlan& pl, const void* q, const void* K, const void* V, float* out,
                             float* lse, int32_t* sel_idx, char* ws, hipStream_t hs) {
  if (pl.unit_S > 0) {
    switch (pl.g) {
      case 1: return run_unit<1>(pl, q, K, V, out, lse, sel_idx, ws, hs);
      case 2: return run_unit<2>(pl, q, K, V, out, lse, sel_idx, ws, hs);
      case 4: return run_unit<4>(pl, q, K, V, out, lse, sel_idx, ws, hs);
      case 8: return run_unit<8>(pl, q, K, V, out, lse, sel_idx, ws, hs);
    }
  }
  return dispatch<DecodeRunner>(pl.dtype, pl.D, pl.g, pl, q, K, V, out, lse, sel_idx, ws, hs);
}
}  // namespace
}  // namespace gsa

using namespace gsa;

extern "C" gsa_status_t gsa_decode_workspace_size(const gsa_decode_params* p, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(GSA_ERR_INVALID_ARG, "bytes is NULL");
  DecodePlan pl;
  gsa_status_t s = plan_decode(p, &pl);
  if (s != GSA_OK) return s;
  *bytes = pl.total;
  return GSA_OK;
}

extern "C" gsa_status_t gsa_decode(const gsa_decode_params* p, const void* q, const void* k_cache,
                                   const void* v_cache, float* out, float* lse, int32_t* sel_idx,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  prof_begin_call();
  DecodePlan pl;
  gsa_status_t s = plan_decode(p, &pl);
  if (s != GSA_OK) return s;
  if ((s = check_ptr(q, "q")) != GSA_OK || (s = check_ptr(k_cache, "k_cache")) != GSA_OK ||
      (s = check_ptr(v_cache, "v_cache")) != GSA_OK || (s = check_ptr(out, "out")) != GSA_OK ||
      (s = check_ptr(lse, "lse", true)) != GSA_OK || (s = check_ptr(sel_idx, "sel_idx", true)) != GSA_OK)
    return s;
  if ((s = check_workspace(workspace, workspace_bytes, pl.total)) != GSA_OK) return s;
  return run_decode_plan(pl, q, k_cache, v_cache, out, lse, sel_idx, reinterpret_cast<char*>(workspace),
                         reinterpret_cast<hipStream_t>(stream));
}

extern "C" gsa_status_t gsa_decode_hier_workspace_size(const gsa_hier_params* p, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(GSA_ERR_INVALID_ARG, "bytes is NULL");
  HierPlan hp;
  gsa_status_t s = plan_hier(p, &hp);
  if (s != GSA_OK) return s;
  *bytes = hp.total;
  return GSA_OK;
}

extern "C" gsa_status_t gsa_decode_hier(const gsa_hier_params* p, const void* q, const void* k_cache,
                                        const void* v_cache, const void* k_l2, const void* v_l2,
                                        float* out, float* lse, int32_t* sel2, int32_t* sel1,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  prof_begin_call();
  HierPlan hp;
  gsa_status_t s = plan_hier(p, &hp);
  if (s != GSA_OK) return s;
  const bool need_l2 = hp.M2 > 0;
  if ((s = check_ptr(q, "q")) != GSA_OK || (s = check_ptr(k_cache, "k_cache")) != GSA_OK ||
      (s = check_ptr(v_cache, "v_cache")) != GSA_OK || (s = check_ptr(k_l2, "k_l2", !need_l2)) != GSA_OK ||
      (s = check_ptr(v_l2, "v_l2", !need_l2)) != GSA_OK || (s = check_ptr(out, "out")) != GSA_OK ||
      (s = check_ptr(lse, "lse", true)) != GSA_OK || (s = check_ptr(sel2, "sel2", true)) != GSA_OK ||
      (s = check_ptr(sel1, "sel1", true)) != GSA_OK)
    return s;
  if ((s = check_workspace(workspace, workspace_bytes, hp.total)) != GSA_OK) return s;
  if (hp.unit_S > 0) {
    char* ws = reinterpret_cast<char*>(workspace);
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    switch (hp.base.g) {
      case 1: return run_unit_hier<1>(hp, q, k_cache, v_cache, k_l2, v_l2, out, lse, sel2, sel1, ws, hs);
      case 2: return run_unit_hier<2>(hp, q, k_cache, v_cache, k_l2, v_l2, out, lse, sel2, sel1, ws, hs);
      case 4: return run_unit_hier<4>(hp, q, k_cache, v_cache, k_l2, v_l2, out, lse, sel2, sel1, ws, hs);
      case 8: return run_unit_hier<8>(hp, q, k_cache, v_cache, k_l2, v_l2, out, lse, sel2, sel1, ws, hs);
    }
  }
  return dispatch<HierRunner>(hp.base.dtype, hp.base.D, hp.base.g, hp, q, k_cache, v_cache, k_l2, v_l2,
                              out, lse, sel2, sel1, reinterpret_cast<char*>(workspace),
                              reinterpret_cast<hipStream_t>(stream));
}

extern "C" gsa_status_t gsa_decode_hier_varlen(const gsa_hier_params* p, const int32_t* seq_n_raw,
                                               const int32_t* seq_n_gist, const void* q, const void* k_cache,
                                               const void* v_cache, const void* k_l2, const void* v_l2,
                                               float* out, float* lse, int32_t* sel2, int32_t* sel1,
                                               void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  prof_begin_call();
  HierPlan hp;
  gsa_status_t s = plan_hier(p, &hp);
  if (s != GSA_OK) return s;
  if (hp.unit_S == 0)
    return fail(GSA_ERR_UNSUPPORTED,
                "variable-length two-level decode runs on the bf16, head_dim 128 path (topk, topk2 <= 64, at most "
                "4096 level-1 candidates)");
  const bool need_l2 = hp.M2 > 0;
  if ((s = check_ptr(seq_n_raw, "seq_n_raw")) != GSA_OK || (s = check_ptr(seq_n_gist, "seq_n_gist")) != GSA_OK ||
      (s = check_ptr(q, "q")) != GSA_OK || (s = check_ptr(k_cache, "k_cache")) != GSA_OK ||
      (s = check_ptr(v_cache, "v_cache")) != GSA_OK || (s = check_ptr(k_l2, "k_l2", !need_l2)) != GSA_OK ||
      (s = check_ptr(v_l2, "v_l2", !need_l2)) != GSA_OK || (s = check_ptr(out, "out")) != GSA_OK ||
      (s = check_ptr(lse, "lse", true)) != GSA_OK || (s = check_ptr(sel2, "sel2", true)) != GSA_OK ||
      (s = check_ptr(sel1, "sel1", true)) != GSA_OK)
    return s;
  if ((s = check_workspace(workspace, workspace_bytes, hp.total)) != GSA_OK) return s;
  char* ws = reinterpret_cast<char*>(workspace);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  switch (hp.base.g) {
    case 1: return run_unit_hier<1>(hp, q, k_cache, v_cache, k_l2, v_l2, out, lse, sel2, sel1, ws, hs, seq_n_raw, seq_n_gist);
    case 2: return run_unit_hier<2>(hp, q, k_cache, v_cache, k_l2, v_l2, out, lse, sel2, sel1, ws, hs, seq_n_raw, seq_n_gist);
    case 4: return run_unit_hier<4>(hp, q, k_cache, v_cache, k_l2, v_l2, out, lse, sel2, sel1, ws, hs, seq_n_raw, seq_n_gist);
    case 8: return run_unit_hier<8>(hp, q, k_cache, v_cache, k_l2, v_l2, out, lse, sel2, sel1, ws, hs, seq_n_raw, seq_n_gist);
  }
  return fail(GSA_ERR_UNSUPPORTED, "no kernel for g=%d", hp.base.g);
}

extern "C" gsa_status_t gsa_decode_levels_workspace_size(const gsa_levels_params* p, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(GSA_ERR_INVALID_ARG, "bytes is NULL");
  LevelsPlan lp;
  gsa_status_t s = plan_levels(p, &lp);
  if (s != GSA_OK) return s;
  *bytes = lp.total;
  return GSA_OK;
}

extern "C" gsa_status_t gsa_decode_levels(const gsa_levels_params* p, const void* q, const void* k_cache,
                                          const void* v_cache, const void* const* k_up,
                                          const void* const* v_up, float* out, float* lse,
                                          int32_t* const* sel_up, int32_t* sel1, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  clear_error();
  prof_begin_call();
  LevelsPlan lp;
  gsa_status_t s = plan_levels(p, &lp);
  if (s != GSA_OK) return s;
  if ((s = check_ptr(q, "q")) != GSA_OK || (s = check_ptr(k_cache, "k_cache")) != GSA_OK ||
      (s = check_ptr(v_cache, "v_cache")) != GSA_OK || (s = check_ptr(out, "out")) != GSA_OK ||
      (s = check_ptr(lse, "lse", true)) != GSA_OK || (s = check_ptr(sel1, "sel1", true)) != GSA_OK)
    return s;
  if (!k_up || !v_up) return fail(GSA_ERR_INVALID_ARG, "k_up / v_up is NULL");
  static const char* kNames[] = {"k_up[0]", "k_up[1]", "k_up[2]", "k_up[3]", "k_up[4]"};
  static const char* vNames[] = {"v_up[0]", "v_up[1]", "v_up[2]", "v_up[3]", "v_up[4]"};
  static const char* sNames[] = {"sel_up[0]", "sel_up[1]", "sel_up[2]", "sel_up[3]", "sel_up[4]"};
  for (int i = 0; i + 2 <= lp.L; ++i) {
    const bool need = lp.Ml[i + 2] > 0;
    if ((s = check_ptr(k_up[i], kNames[i], !need)) != GSA_OK || (s = check_ptr(v_up[i], vNames[i], !need)) != GSA_OK)
      return s;
    if (sel_up && (s = check_ptr(sel_up[i], sNames[i], true)) != GSA_OK) return s;
  }
  if ((s = check_workspace(workspace, workspace_bytes, lp.total)) != GSA_OK) return s;
  if (lp.unit_S > 0) {
    char* ws = reinterpret_cast<char*>(workspace);
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    switch (lp.base.g) {
      case 1: return run_unit_levels<1>(lp, q, k_cache, v_cache, k_up, v_up, out, lse, sel_up, sel1, ws, hs);
      case 2: return run_unit_levels<2>(lp, q, k_cache, v_cache, k_up, v_up, out, lse, sel_up, sel1, ws, hs);
      case 4: return run_unit_levels<4>(lp, q, k_cache, v_cache, k_up, v_up, out, lse, sel_up, sel1, ws, hs);
      case 8: return run_unit_levels<8>(lp, q, k_cache, v_cache, k_up, v_up, out, lse, sel_up, sel1, ws, hs);
    }
  }
  return dispatch<LevelsRunner>(lp.base.dtype, lp.base.D, lp.base.g, lp, q, k_cache, v_cache, k_up, v_up, out,
                                lse, sel_up, sel1, reinterpret_cast<char*>(workspace),
                                reinterpret_cast<hipStream_t>(stream));
}

extern "C" gsa_status_t gsa_decode_levels_varlen(const gsa_levels_params* p, const int32_t* seq_n_raw,
                                                 const int32_t* seq_n_gist, const void* q, const void* k_cache,
                                                 const void* v_cache, const void* const* k_up,
                                                 const void* const* v_up, float* out, float* lse,
                                                 int32_t* const* sel_up, int32_t* sel1, void* workspace,
                                                 size_t workspace_bytes, void* stream) {
  clear_error();
  prof_begin_call();
  LevelsPlan lp;
  gsa_status_t s = plan_levels(p, &lp);
  if (s != GSA_OK) return s;
  if (lp.unit_S == 0 || !levels_top_in_lds(lp))
    return fail(GSA_ERR_UNSUPPORTED,
                "variable-length L-level decode runs on the one-launch path (bf16, head_dim 128, every k <= 64, "
                "at most 4096 top-level gists and 4096 candidates per level)");
  if ((s = check_ptr(seq_n_raw, "seq_n_raw")) != GSA_OK || (s = check_ptr(seq_n_gist, "seq_n_gist")) != GSA_OK ||
      (s = check_ptr(q, "q")) != GSA_OK || (s = check_ptr(k_cache, "k_cache")) != GSA_OK ||
      (s = check_ptr(v_cache, "v_cache")) != GSA_OK || (s = check_ptr(out, "out")) != GSA_OK ||
      (s = check_ptr(lse, "lse", true)) != GSA_OK || (s = check_ptr(sel1, "sel1", true)) != GSA_OK)
    return s;
  if (!k_up || !v_up) return fail(GSA_ERR_INVALID_ARG, "k_up / v_up is NULL");
  for (int i = 0; i + 2 <= lp.L; ++i) {
    const bool need = lp.Ml[i + 2] > 0;
    if ((s = check_ptr(k_up[i], "k_up[i]", !need)) != GSA_OK || (s = check_ptr(v_up[i], "v_up[i]", !need)) != GSA_OK)
      return s;
    if (sel_up && (s = check_ptr(sel_up[i], "sel_up[i]", true)) != GSA_OK) return s;
  }
  if ((s = check_workspace(workspace, workspace_bytes, lp.total)) != GSA_OK) return s;
  char* ws = reinterpret_cast<char*>(workspace);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  switch (lp.base.g) {
    case 1: return run_unit_levels<1>(lp, q, k_cache, v_cache, k_up, v_up, out, lse, sel_up, sel1, ws, hs, seq_n_raw, seq_n_gist);
    case 2: return run_unit_levels<2>(lp, q, k_cache, v_cache, k_up, v_up, out, lse, sel_up, sel1, ws, hs, seq_n_raw, seq_n_gist);
    case 4: return run_unit_levels<4>(lp, q, k_cache, v_cache, k_up, v_up, out, lse, sel_up, sel1, ws, hs, seq_n_raw, seq_n_gist);
    case 8: return run_unit_levels<8>(lp, q, k_cache, v_cache, k_up, v_up, out, lse, sel_up, sel1, ws, hs, seq_n_raw, seq_n_gist);
  }
  return fail(GSA_ERR_UNSUPPORTED, "no kernel for g=%d", lp.base.g);
}

extern "C" gsa_status_t gsa_decode_varlen(const gsa_decode_params* p, const int32_t* seq_n_raw,
                                          const int32_t* seq_n_gist, const void* q, const void* k_cache,
                                          const void* v_cache, float* out, float* lse, int32_t* sel_idx,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  prof_begin_call();
  DecodePlan pl;
  gsa_status_t s = plan_decode(p, &pl);
  if (s != GSA_OK) return s;
  if ((s = check_ptr(seq_n_raw, "seq_n_raw")) != GSA_OK || (s = check_ptr(seq_n_gist, "seq_n_gist")) != GSA_OK ||
      (s = check_ptr(q, "q")) != GSA_OK || (s = check_ptr(k_cache, "k_cache")) != GSA_OK ||
      (s = check_ptr(v_cache, "v_cache")) != GSA_OK || (s = check_ptr(out, "out")) != GSA_OK ||
      (s = check_ptr(lse, "lse", true)) != GSA_OK || (s = check_ptr(sel_idx, "sel_idx", true)) != GSA_OK)
    return s;
  if ((s = check_workspace(workspace, workspace_bytes, pl.total)) != GSA_OK) return s;
  pl.seq_n = seq_n_raw;
  pl.seq_m = seq_n_gist;
  char* ws = reinterpret_cast<char*>(workspace);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (pl.unit_S > 0) {
    switch (pl.g) {
      case 1: return run_unit<1>(pl, q, k_cache, v_cache, out, lse, sel_idx, ws, hs);
      case 2: return run_unit<2>(pl, q, k_cache, v_cache, out, lse, sel_idx, ws, hs);
      case 4: return run_unit<4>(pl, q, k_cache, v_cache, out, lse, sel_idx, ws, hs);
      case 8: return run_unit<8>(pl, q, k_cache, v_cache, out, lse, sel_idx, ws, hs);
    }
  }
  return dispatch<DecodeRunner>(pl.dtype, pl.D, pl.g, pl, q, k_cache, v_cache, out, lse, sel_idx, ws, hs);
}


extern "C" gsa_status_t gsa_decode_paged_workspace_size(const gsa_paged_params* p, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(GSA_ERR_INVALID_ARG, "bytes is NULL");
  DecodePlan pl;
  gsa_status_t s = plan_paged(p, &pl);
  if (s != GSA_OK) return s;
  *bytes = pl.total;
  return GSA_OK;
}

extern "C" gsa_status_t gsa_decode_paged(const gsa_paged_params* p, const int32_t* block_table,
                                         const int32_t* seq_n_raw, const int32_t* seq_n_gist,
                                         const int32_t* extra_rows, const void* q, const void* k_pool,
                                         const void* v_pool, float* out, float* lse, int32_t* sel_idx,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  prof_begin_call();
  DecodePlan pl;
  gsa_status_t s = plan_paged(p, &pl);
  if (s != GSA_OK) return s;
  if ((s = check_ptr(block_table, "block_table")) != GSA_OK || (s = check_ptr(seq_n_raw, "seq_n_raw")) != GSA_OK ||
      (s = check_ptr(seq_n_gist, "seq_n_gist")) != GSA_OK ||
      (s = check_ptr(extra_rows, "extra_rows", p->max_extra == 0)) != GSA_OK || (s = check_ptr(q, "q")) != GSA_OK ||
      (s = check_ptr(k_pool, "k_pool")) != GSA_OK || (s = check_ptr(v_pool, "v_pool")) != GSA_OK ||
      (s = check_ptr(out, "out")) != GSA_OK || (s = check_ptr(lse, "lse", true)) != GSA_OK ||
      (s = check_ptr(sel_idx, "sel_idx", true)) != GSA_OK)
    return s;
  if ((s = check_workspace(workspace, workspace_bytes, pl.total)) != GSA_OK) return s;
  pl.seq_n = seq_n_raw;
  pl.seq_m = seq_n_gist;
  pl.pg_table = block_table;
  // no extra rows: an empty list (the pointer is never read)
  pl.pg_extra = extra_rows != nullptr ? extra_rows : block_table;
  if (extra_rows == nullptr) pl.pg_max_extra = 0;
  char* ws = reinterpret_cast<char*>(workspace);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  switch (pl.g) {
    case 1: return run_unit<1>(pl, q, k_pool, v_pool, out, lse, sel_idx, ws, hs);
    case 2: return run_unit<2>(pl, q, k_pool, v_pool, out, lse, sel_idx, ws, hs);
    case 4: return run_unit<4>(pl, q, k_pool, v_pool, out, lse, sel_idx, ws, hs);
    case 8: return run_unit<8>(pl, q, k_pool, v_pool, out, lse, sel_idx, ws, hs);
  }
  return fail(GSA_ERR_UNSUPPORTED, "no kernel for g=%d", pl.g);
}

// ------------------------------------------------ decode without allocation
//
// gsa_decode_noalloc: gsa_decode for callers that cannot allocate device
// memory (code under stream capture, tight serving loops). Its workspace is
// this file's own device array, one copy per GPU, held until the process
// ends. Host code never uses the array's name as an address: the address of
// each device's copy comes from hipGetSymbolAddress with that device current.

constexpr size_t kScratchBytes = (size_t)16 << 20;   // 16 MiB per GPU
static __device__ __align__(256) char scratch[kScratchBytes];

namespace gsa {
namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch[kMaxScratchDevices];   // per device: the array's device address, once set up

__global__ __launch_bounds__(256) void zero_words_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The current device's copy of the scratch array; at its first use on a
// device the control words (the first kCtrlBytes) are cleared on `st`, with a
// fill kernel rather than a memset node.
gsa_status_t scratch_of_current_device(hipStream_t st, char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices) return fail(GSA_ERR_UNSUPPORTED, "device %d above %d", dev, kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(GSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    hipLaunchKernelGGL(zero_words_kernel, dim3(256), dim3(256), 0, st, reinterpret_cast<uint4*>(ptr),
                       kCtrlBytes / 16);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(GSA_ERR_HIP, "scratch clear launch: %s", hipGetErrorString(e));
    g_scratch[dev] = reinterpret_cast<char*>(ptr);
  }
  *out = g_scratch[dev];
  return GSA_OK;
}

}  // namespace
}  // namespace gsa

extern "C" gsa_status_t gsa_decode_noalloc(const gsa_decode_params* p, const void* q, const void* k_cache,
                                           const void* v_cache, float* out, float* lse, int32_t* sel_idx,
                                           void* stream) {
  clear_error();
  prof_begin_call();
  DecodePlan pl;
  gsa_status_t s = plan_decode(p, &pl);
  if (s != GSA_OK) return s;
  if ((s = check_ptr(q, "q")) != GSA_OK || (s = check_ptr(k_cache, "k_cache")) != GSA_OK ||
      (s = check_ptr(v_cache, "v_cache")) != GSA_OK || (s = check_ptr(out, "out")) != GSA_OK ||
      (s = check_ptr(lse, "lse", true)) != GSA_OK || (s = check_ptr(sel_idx, "sel_idx", true)) != GSA_OK)
    return s;
  if (pl.total > kScratchBytes)
    return fail(GSA_ERR_WORKSPACE, "the call needs %zu bytes of workspace, the library's scratch holds %zu",
                pl.total, kScratchBytes);
  if (ctrl_bytes(pl.units) > kCtrlBytes)
    return fail(GSA_ERR_UNSUPPORTED, "%d (batch, kv-head) units: at most %zu without a workspace", pl.units,
                kCtrlBytes / (sizeof(uint32_t) * kCtrlUnitWords));
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  char* ws = nullptr;
  if ((s = scratch_of_current_device(hs, &ws)) != GSA_OK) return s;
  return run_decode_plan(pl, q, k_cache, v_cache, out, lse, sel_idx, ws, hs);
}
