// GSA decode on gfx950 in one launch: gist scoring + online softmax over every
// gist, exact top-k chunk selection, gather of the unfolded chunks and the
// tail, and a log-sum-exp merge of the partial softmax states.
//
// Method: gist.science explainer "Forget, Then Recall", section 2 'Key
// Concepts' (routing by gist scores, top-k selection, selective unfolding,
// hybrid attention) and 'Hierarchical Extension (H-GSA)' for the two-level
// entry point (score the meta-gists, then the gists of the chosen groups,
// then unfold raw chunks).
//
// Work is cut into tasks per (batch, kv-head) unit and phase:
//   gist-like phase  a task streams a contiguous range of gist rows (K and V,
//                    each row read once), writes each gist's group score and
//                    one online-softmax partial (m, l, acc[D]) per query head;
//                    the unit's last task to finish runs the exact top-k over
//                    the phase's scores and raises the unit's ready flag;
//   unfold phase     a task waits for its unit's flag, then streams a share of
//                    the selected chunks' raw rows (each chunk one contiguous
//                    run; rows the tail owns are skipped) and of the tail; the
//                    unit's last task merges every partial into out and lse.
// Single-level decode runs [gist, unfold]; two-level decode runs [level-2
// gists, level-1 candidate gists, unfold].
//
// Tasks are numbered phase by phase and unit by unit, and a task only ever
// waits for tasks with lower numbers. The grid is persistent and no larger
// than the number of workgroups the chip holds at once (occupancy x CUs), so
// every workgroup is resident; workgroup w runs tasks w, w + P, w + 2P, ... in
// order. The lowest unfinished task is therefore always running with all its
// (lower) dependencies finished, so every wait ends. The wait is also bounded;
// on time-out the task poisons its partial with NaN instead of hanging.
//
// Memory-bound work stays on the VALU: 16 lanes cover one 256-byte row with
// one 16-byte load each, q.k uses v_dot2_f32_bf16, the 16-lane sum uses DPP,
// and the softmax weights stay fp32.
#include <hip/hip_runtime.h>

#include "gsa.h"
#include "gsa_device.hpp"
#include "gsa_plan.hpp"
#include "gsa_profile.hpp"

namespace gsa {
namespace {

using namespace dev;

constexpr int kThreads = 256;   // 4 waves per workgroup
constexpr int kWaves = kThreads / 64;
#ifndef GSA_ROWS_IN_FLIGHT
#define GSA_ROWS_IN_FLIGHT 2
#endif
constexpr int kU = GSA_ROWS_IN_FLIGHT;   // rows per lane group per batch (two batches in flight)
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

// Stream items [i0, i1) of one unit through the online softmax. row_of(i)
// gives the cache row of item i; with CAN_SKIP it may return -1 to skip the
// item. When score_out is set (LDS), the group score of item i goes to
// score_out[i - i0].
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
                                            float score_mul) {
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
        b.v[u] = load16_stream(Vb + off);
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
                           int32_t* __restrict__ dst, int32_t* __restrict__ dst2, TopkLds& L) {
  const int tid = threadIdx.x;
  const CohBuf sc(scores, (uint32_t)n * 4u);
  if (k <= 0) return;
  if (k >= n) {
    for (int i = tid; i < n; i += kThreads) {
      const int32_t id = map_id(im, unit, i);
      st_coh(dst + i, id);
      if (dst2) dst2[i] = id;
    }
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
      if (pick[q] && pos >= 0 && pos < k) {
        const int32_t id = map_id(im, unit, b0 + q * kThreads + tid);
        st_coh(dst + pos, id);
        if (dst2) dst2[pos] = id;
      }
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

// ------------------------------------------------------------ kernels ------

// Cache row of tail item i (position N - T + i) of the interleaved cache.
__device__ __forceinline__ int64_t tail_row(int64_t i, int64_t N, int32_t T, int64_t M, int32_t C) {
  const int64_t pos = N - T + i, MC = M * C;
  return pos < MC ? (pos / C) * (C + 1) + pos % C : M * (C + 1) + (pos - MC);
}

// A pass over gist-like rows of every unit: scores + attention partials, plus
// a share of the tail rows (attended, not scored). Selection of the pass's
// top-k: for k <= kFastSel each workgroup reduces its scores to its own top-k
// candidates and the unit's last workgroup merges them; for larger k every
// score goes out and the last workgroup runs a radix select. With out set the
// last workgroup also merges the unit's partials (the pass is the last one).
struct GistArgs {
  const void* q;
  const void* K;
  const void* V;
  int64_t unit_rows;      // rows per unit in K/V
  int64_t n_items;        // items per unit
  int64_t per_task;       // items per workgroup
  int32_t tasks;          // workgroups per unit
  RowMap rm;
  // tail rows, from the interleaved cache Kt/Vt
  const void* Kt;
  const void* Vt;
  int64_t tail_unit_rows;
  int64_t N, M;
  int32_t C, T, tail_per_task;
  // selection
  int32_t sel_k;
  IdMap im;
  float* scores;          // [units][score_stride] (k > kFastSel)
  int64_t score_stride;
  uint32_t* cand;         // [units][cand_stride] words: tasks * k keys (k <= kFastSel)
  int64_t cand_stride;
  int32_t* sel_ws;        // [units][sel_stride]
  int64_t sel_stride;
  int32_t* sel_out;       // [units][sel_k] or null
  // partial softmax states
  float* part;            // [units][NP][part_stride]
  int64_t part_stride;
  int32_t NP, part_base;
  float* out;             // set: the last workgroup merges into out / lse
  float* lse;
  uint32_t* cnt;          // unit u's counter at cnt[u * kCtrlUnitWords]
  float scale_log2;       // softmax logits in log2 units
  float score_mul;        // group score = sum_h(q_h . k) * score_mul
};

template <int D, int G>
struct GistLds {
  float scores[kTaskScores];   // this workgroup's scores
  uint32_t xs[2][64];          // wave 0's selection scratch
  union {
    PartLds<D, G> part;
    TopkLds topk;
  } u;
};

template <bool BF16, int D, int G>
__global__ __launch_bounds__(kThreads) void gist_kernel(GistArgs a) {
  using Gm = Geo<BF16, D>;
  __shared__ GistLds<D, G> lds;
  __shared__ uint32_t s_old;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int unit = blockIdx.x / a.tasks, split = blockIdx.x % a.tasks;
  uint4 qv[G];
  load_q<BF16, D, G>(a.q, unit, qv);
  State<BF16, G> st;
  init_state<BF16, G>(st);
  const size_t ub = (size_t)unit * (size_t)a.unit_rows * Gm::ROW_BYTES;
  const int64_t i0 = (int64_t)split * a.per_task;
  const int64_t i1 = i0 + a.per_task < a.n_items ? i0 + a.per_task : a.n_items;
  const RowMap rm = a.rm;
  stream_rows<BF16, D, G, false>(reinterpret_cast<const char*>(a.K) + ub,
                                 reinterpret_cast<const char*>(a.V) + ub, i0, i1,
                                 [&](int64_t i) { return map_row(rm, unit, i); }, qv, st,
                                 a.scale_log2, lds.scores, a.score_mul);
  // this workgroup's share of the tail
  const int64_t t0 = (int64_t)split * a.tail_per_task;
  const int64_t t1 = t0 + a.tail_per_task < a.T ? t0 + a.tail_per_task : a.T;
  if (t0 < t1) {
    const size_t tb = (size_t)unit * (size_t)a.tail_unit_rows * Gm::ROW_BYTES;
    const int64_t N = a.N, M = a.M;
    const int32_t C = a.C, T = a.T;
    stream_rows<BF16, D, G, false>(reinterpret_cast<const char*>(a.Kt) + tb,
                                   reinterpret_cast<const char*>(a.Vt) + tb, t0, t1,
                                   [&](int64_t i) { return tail_row(i, N, T, M, C); }, qv, st,
                                   a.scale_log2, nullptr, 0.f);
  }
  const int nw = (int)(i1 > i0 ? i1 - i0 : 0);
  float* part_u = a.part + (size_t)unit * a.NP * a.part_stride;
  write_partial<BF16, D, G>(st, part_u + (size_t)(a.part_base + split) * a.part_stride, lds.u.part, false);
  uint32_t* ctr = a.cnt + (size_t)unit * kCtrlUnitWords;

  if (a.sel_k > kFastSel) {
    // every score out (contiguous device-scope stores), radix select in the last workgroup
    float* so = a.scores + (size_t)unit * a.score_stride + i0;
    for (int i = tid; i < nw; i += kThreads) st_coh(so + i, lds.scores[i]);
    if (arrive_last(ctr, (uint32_t)a.tasks, &s_old)) {
      __syncthreads();   // LDS changes role: partial merge -> selection
      block_topk(a.scores + (size_t)unit * a.score_stride, (int)a.n_items, a.sel_k, a.im, unit,
                 a.sel_ws + (size_t)unit * a.sel_stride,
                 a.sel_out ? a.sel_out + (size_t)unit * a.sel_k : nullptr, lds.u.topk);
      if (a.out != nullptr)
        merge_unit<D, G>(part_u, a.NP, (uint32_t)a.part_stride, a.out + (size_t)unit * G * D,
                         a.lse ? a.lse + (size_t)unit * G : nullptr, kWaves);
    }
    return;
  }

  // k <= kFastSel: wave 0 alone finishes the workgroup (the other waves leave
  // once their partial stores have completed)
  done_stores();
  __syncthreads();   // scores in LDS; every wave's partial stores done
  if (w != 0) return;
  if (a.sel_k > 0) {
    // this workgroup's top-k candidates (key, id), in id order; unused slots
    // get key 0 (no item)
    const IdMap im = a.im;
    uint32_t rk, ri;
    wave_select(nw, a.sel_k,
                [&](int i, uint32_t& key, uint32_t& id) {
                  key = i < nw ? order_key(lds.scores[i]) : 0u;
                  id = i < nw ? (uint32_t)map_id(im, unit, (int32_t)(i0 + i)) : 0u;
                },
                lds.xs, rk, ri);
    if (lane < a.sel_k) {
      uint32_t* cb = a.cand + (size_t)unit * a.cand_stride + 2u * ((size_t)split * a.sel_k + lane);
      st_coh(reinterpret_cast<int32_t*>(cb), (int32_t)rk);
      st_coh(reinterpret_cast<int32_t*>(cb + 1), (int32_t)ri);
    }
  }
  // count this workgroup finished (wave 0's stores complete first)
  done_stores();
  uint32_t old = 0u;
  if (lane == 0) old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0);
  if (old != (uint32_t)a.tasks - 1u) return;
  if (lane == 0) ctrl_set(ctr, 0u);
  if (a.sel_k > 0) {
    // merge the candidates of every workgroup of the unit (split order = id order)
    const int n = a.tasks * a.sel_k;
    const CohBuf cb(a.cand + (size_t)unit * a.cand_stride, (uint32_t)n * 8u);
    uint32_t rk, ri;
    wave_select(n, a.sel_k,
                [&](int i, uint32_t& key, uint32_t& id) {   // past n the buffer returns 0
                  key = cb.u32(2u * (uint32_t)i);
                  id = cb.u32(2u * (uint32_t)i + 1u);
                },
                lds.xs, rk, ri);
    if (lane < a.sel_k) {
      st_coh(a.sel_ws + (size_t)unit * a.sel_stride + lane, (int32_t)ri);
      if (a.sel_out) a.sel_out[(size_t)unit * a.sel_k + lane] = (int32_t)ri;
    }
  }
  if (a.out != nullptr)
    merge_unit<D, G>(part_u, a.NP, (uint32_t)a.part_stride, a.out + (size_t)unit * G * D,
                     a.lse ? a.lse + (size_t)unit * G : nullptr, 1);
}

// Raw rows of the selected chunks (minus rows the tail owns); the unit's last
// workgroup merges every partial into out and lse.
struct UnfoldArgs {
  const void* q;
  const void* K;
  const void* V;
  int64_t unit_rows;
  const int32_t* sel;     // [units][sel_stride] chosen chunks (earlier launch)
  int64_t sel_stride;
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
};

template <int D, int G>
union UnfoldLds {
  struct {
    int32_t sel[kSelLds];
  } s;
  PartLds<D, G> part;
};

template <bool BF16, int D, int G>
__global__ __launch_bounds__(kThreads) void unfold_kernel(UnfoldArgs a) {
  using Gm = Geo<BF16, D>;
  __shared__ UnfoldLds<D, G> lds;
  __shared__ uint32_t s_old;
  const int tid = threadIdx.x;
  const int unit = blockIdx.x / a.tasks, split = blockIdx.x % a.tasks;
  const int32_t* us = a.sel + (size_t)unit * a.sel_stride;
  const bool in_lds = a.k <= kSelLds;
  if (in_lds)
    for (int i = tid; i < a.k; i += kThreads) lds.s.sel[i] = us[i];
  __syncthreads();
  uint4 qv[G];
  load_q<BF16, D, G>(a.q, unit, qv);
  State<BF16, G> st;
  init_state<BF16, G>(st);
  const size_t ub = (size_t)unit * (size_t)a.unit_rows * Gm::ROW_BYTES;
  const int64_t i0 = (int64_t)split * a.per_task;
  const int64_t i1 = i0 + a.per_task < a.n_items ? i0 + a.per_task : a.n_items;
  // 32-bit index math: items < 2^30
  const uint32_t C = (uint32_t)a.C;
  const int64_t M = a.M, tail0 = a.N - a.T;
  const int32_t* s_sel = lds.s.sel;
  auto row_of = [&](int64_t i64) -> int64_t {
    const uint32_t i = (uint32_t)i64;
    const uint32_t ci = i / C, j = i - ci * C;
    const int64_t m = in_lds ? s_sel[ci] : us[ci];
    if (m < 0 || m >= M) return -1;         // never taken for a valid selection
    if (m * C + j >= tail0) return -1;      // the tail attends this row
    return m * (C + 1) + j;
  };
  stream_rows<BF16, D, G, true>(reinterpret_cast<const char*>(a.K) + ub,
                                reinterpret_cast<const char*>(a.V) + ub, i0, i1, row_of, qv, st,
                                a.scale_log2, nullptr, 0.f);
  float* part_u = a.part + (size_t)unit * a.NP * a.part_stride;
  __syncthreads();   // LDS changes role: selected ids -> partial merge
  write_partial<BF16, D, G>(st, part_u + (size_t)(a.part_base + split) * a.part_stride, lds.part, false);
  if (arrive_last(a.cnt + (size_t)unit * kCtrlUnitWords, (uint32_t)a.tasks, &s_old))
    merge_unit<D, G>(part_u, a.NP, (uint32_t)a.part_stride, a.out + (size_t)unit * G * D,
                     a.lse ? a.lse + (size_t)unit * G : nullptr, kWaves);
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
  int32_t* wsel = reinterpret_cast<int32_t*>(ws + pl.off_sel);
  const int64_t ps = part_stride(G, D);
  GistArgs g{};
  g.q = q; g.K = K; g.V = V;
  g.unit_rows = pl.R; g.n_items = pl.M; g.per_task = pl.gists_per_split; g.tasks = pl.S;
  g.rm = RowMap{0, pl.C, nullptr, 0, 0, 0, 0};
  g.Kt = K; g.Vt = V; g.tail_unit_rows = pl.R;
  g.N = pl.N; g.M = pl.M; g.C = pl.C; g.T = pl.T; g.tail_per_task = pl.tail_per_split;
  g.sel_k = pl.k; g.im = IdMap{nullptr, 0, 0, 0, 0};
  g.scores = reinterpret_cast<float*>(ws + pl.off_scores); g.score_stride = pl.score_stride;
  g.cand = reinterpret_cast<uint32_t*>(ws + pl.off_cand); g.cand_stride = pl.cand_stride;
  g.sel_ws = wsel; g.sel_stride = pl.sel_stride; g.sel_out = sel_idx;
  g.part = part; g.part_stride = ps; g.NP = pl.NP; g.part_base = 0;
  g.out = pl.k > 0 ? nullptr : out; g.lse = pl.k > 0 ? nullptr : lse;
  g.cnt = ctrl_of(ws, pl.off_ctrl, 0);
  g.scale_log2 = pl.scale * kLog2e; g.score_mul = pl.scale / G;
  prof_begin_call();
  prof_mark(st);
  hipLaunchKernelGGL((gist_kernel<BF16, D, G>), dim3(pl.units * pl.S), dim3(kThreads), 0, st, g);
  prof_mark(st);
  if (pl.k > 0) {
    UnfoldArgs u{};
    u.q = q; u.K = K; u.V = V; u.unit_rows = pl.R;
    u.sel = wsel; u.sel_stride = pl.sel_stride; u.k = pl.k;
    u.C = pl.C; u.T = pl.T; u.M = pl.M; u.N = pl.N;
    u.n_items = pl.n_items; u.per_task = pl.items_per_split; u.tasks = pl.S2;
    u.part = part; u.part_stride = ps; u.NP = pl.NP; u.part_base = pl.S;
    u.out = out; u.lse = lse;
    u.cnt = ctrl_of(ws, pl.off_ctrl, 2);
    u.scale_log2 = pl.scale * kLog2e;
    hipLaunchKernelGGL((unfold_kernel<BF16, D, G>), dim3(pl.units * pl.S2), dim3(kThreads), 0, st, u);
    prof_mark(st);
  }
  return launch_status("gsa_decode launch");
}

template <bool BF16, int D, int G>
gsa_status_t run_hier(const HierPlan& hp, const void* q, const void* K, const void* V,
                      const void* K2, const void* V2, float* out, float* lse, int32_t* sel2,
                      int32_t* sel1, char* ws, hipStream_t st) {
  const DecodePlan& pl = hp.base;
  int32_t* wsel2 = reinterpret_cast<int32_t*>(ws + hp.off_sel2);
  int32_t* wsel1 = reinterpret_cast<int32_t*>(ws + hp.off_sel1);
  float* part = reinterpret_cast<float*>(ws + hp.off_part);
  const int64_t ps = part_stride(G, D);
  const int64_t orphan0 = hp.M2 * hp.G;
  // level 2: every meta-gist (dense rows of the level-2 array) and the tail,
  // top-k2 groups
  GistArgs g{};
  g.q = q; g.K = K2; g.V = V2;
  g.unit_rows = hp.M2; g.n_items = hp.M2; g.per_task = hp.l2_per_split; g.tasks = hp.S_l2;
  g.rm = RowMap{1, pl.C, nullptr, 0, 0, 0, 0};
  g.Kt = K; g.Vt = V; g.tail_unit_rows = pl.R;
  g.N = pl.N; g.M = pl.M; g.C = pl.C; g.T = pl.T; g.tail_per_task = hp.tail_per_split;
  g.sel_k = hp.k2; g.im = IdMap{nullptr, 0, 0, 0, 0};
  g.scores = reinterpret_cast<float*>(ws + hp.off_s2); g.score_stride = hp.s2_stride;
  g.cand = reinterpret_cast<uint32_t*>(ws + hp.off_cand2); g.cand_stride = hp.cand2_stride;
  g.sel_ws = wsel2; g.sel_stride = hp.sel2_stride; g.sel_out = sel2;
  g.part = part; g.part_stride = ps; g.NP = hp.NP; g.part_base = 0;
  g.out = nullptr; g.lse = nullptr;
  g.cnt = ctrl_of(ws, hp.off_ctrl, 0);
  g.scale_log2 = pl.scale * kLog2e; g.score_mul = pl.scale / G;
  prof_begin_call();
  prof_mark(st);
  hipLaunchKernelGGL((gist_kernel<BF16, D, G>), dim3(pl.units * hp.S_l2), dim3(kThreads), 0, st, g);
  prof_mark(st);
  // level 1: children of the chosen groups + the ungrouped gists, top-k1 chunks
  GistArgs c = g;
  c.K = K; c.V = V;
  c.unit_rows = pl.R; c.n_items = hp.n_cand; c.per_task = hp.cand_per_split; c.tasks = hp.S_c;
  c.rm = RowMap{2, pl.C, wsel2, hp.G, hp.k2, orphan0, hp.sel2_stride};
  c.T = 0; c.tail_per_task = 0;
  c.sel_k = pl.k; c.im = IdMap{wsel2, hp.G, hp.k2, orphan0, hp.sel2_stride};
  c.scores = reinterpret_cast<float*>(ws + hp.off_sc); c.score_stride = hp.sc_stride;
  c.cand = reinterpret_cast<uint32_t*>(ws + hp.off_cand1); c.cand_stride = hp.cand1_stride;
  c.sel_ws = wsel1; c.sel_stride = pl.sel_stride; c.sel_out = sel1;
  c.part_base = hp.S_l2;
  c.out = pl.k > 0 ? nullptr : out; c.lse = pl.k > 0 ? nullptr : lse;
  c.cnt = ctrl_of(ws, hp.off_ctrl, 1);
  hipLaunchKernelGGL((gist_kernel<BF16, D, G>), dim3(pl.units * hp.S_c), dim3(kThreads), 0, st, c);
  prof_mark(st);
  // unfold the chosen chunks, merge everything
  if (pl.k > 0) {
    UnfoldArgs u{};
    u.q = q; u.K = K; u.V = V; u.unit_rows = pl.R;
    u.sel = wsel1; u.sel_stride = pl.sel_stride; u.k = pl.k;
    u.C = pl.C; u.T = pl.T; u.M = pl.M; u.N = pl.N;
    u.n_items = pl.n_items; u.per_task = pl.items_per_split; u.tasks = pl.S2;
    u.part = part; u.part_stride = ps; u.NP = hp.NP; u.part_base = hp.S_l2 + hp.S_c;
    u.out = out; u.lse = lse;
    u.cnt = ctrl_of(ws, hp.off_ctrl, 2);
    u.scale_log2 = pl.scale * kLog2e;
    hipLaunchKernelGGL((unfold_kernel<BF16, D, G>), dim3(pl.units * pl.S2), dim3(kThreads), 0, st, u);
    prof_mark(st);
  }
  return launch_status("gsa_decode_hier launch");
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
  DecodePlan pl;
  gsa_status_t s = plan_decode(p, &pl);
  if (s != GSA_OK) return s;
  if ((s = check_ptr(q, "q")) != GSA_OK || (s = check_ptr(k_cache, "k_cache")) != GSA_OK ||
      (s = check_ptr(v_cache, "v_cache")) != GSA_OK || (s = check_ptr(out, "out")) != GSA_OK ||
      (s = check_ptr(lse, "lse", true)) != GSA_OK || (s = check_ptr(sel_idx, "sel_idx", true)) != GSA_OK)
    return s;
  if ((s = check_workspace(workspace, workspace_bytes, pl.total)) != GSA_OK) return s;
  return dispatch<DecodeRunner>(pl.dtype, pl.D, pl.g, pl, q, k_cache, v_cache, out, lse, sel_idx,
                                reinterpret_cast<char*>(workspace),
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
  return dispatch<HierRunner>(hp.base.dtype, hp.base.D, hp.base.g, hp, q, k_cache, v_cache, k_l2, v_l2,
                              out, lse, sel2, sel1, reinterpret_cast<char*>(workspace),
                              reinterpret_cast<hipStream_t>(stream));
}
