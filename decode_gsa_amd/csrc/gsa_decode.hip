// GSA decode on gfx950: gist scoring + online softmax over every gist,
// exact top-k chunk selection, gather of the unfolded chunks and the tail,
// and a log-sum-exp merge of the split partial states.
//
// Method: gist.science explainer "Forget, Then Recall", section 2 'Key
// Concepts' (routing by gist scores, top-k selection, selective unfolding,
// hybrid attention) and 'Hierarchical Extension (H-GSA)' for the two-level
// entry point. The work is split per (batch, kv-head) unit:
//
//   gist_pass   grid units x S   streams the unit's gist rows (K and V, each
//                                row read once), writes the group score of
//                                every gist and an online-softmax partial
//                                (m, l, acc[D]) per query head;
//   select      grid units       exact top-k of the group scores (bitwise
//                                search for the k-th key, then an ordered
//                                compaction: ties go to the smaller index);
//   unfold      grid units x S2  streams the raw rows of the selected chunks
//                                (each chunk is one contiguous run) and the
//                                tail, skipping rows the tail owns, and writes
//                                partials;
//   merge       grid units x g   combines the partials into out and lse.
//
// Memory-bound work stays on the VALU: 16 lanes cover one 256-byte row with
// one 16-byte load each, q.k uses v_dot2_f32_bf16, the 16-lane sum uses DPP,
// and the softmax weights stay fp32.
#include <hip/hip_runtime.h>

#include "gsa.h"
#include "gsa_device.hpp"
#include "gsa_plan.hpp"

namespace gsa {
namespace {

using namespace dev;

constexpr int kThreads = 256;   // 4 waves per streaming workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kU = 4;           // rows in flight per lane group per iteration
constexpr int kSelThreads = 1024;
constexpr int kSelLds = 16384;  // keys staged in LDS by the select kernel

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

// How item i of a pass maps to a cache row of the unit.
struct RowMap {
  int32_t kind;          // 0: gist i of the interleaved cache; 1: dense row i;
                         // 2: level-1 candidate i of a two-level call
  int32_t C;
  const int32_t* sel2;   // kind 2: chosen level-2 groups [units][k2]
  int32_t G, k2;
  int64_t orphan0;       // kind 2: first level-1 gist no group covers
};

__device__ __forceinline__ int64_t map_row(const RowMap& rm, int unit, int64_t i) {
  if (rm.kind == 0) return i * (rm.C + 1) + rm.C;
  if (rm.kind == 1) return i;
  const int64_t kg = (int64_t)rm.k2 * rm.G;
  int64_t m;
  if (i < kg) {
    const int64_t grp = rm.sel2[(int64_t)unit * rm.k2 + i / rm.G];
    if (grp < 0 || grp * rm.G >= rm.orphan0) return -1;   // never taken for a valid selection
    m = grp * rm.G + i % rm.G;
  } else {
    m = rm.orphan0 + (i - kg);
  }
  return m * (rm.C + 1) + rm.C;
}

// Stream items [i0, i1) of one unit through the online softmax. row_of(i)
// gives the cache row of item i or -1 to skip it. When score_out is set, the
// group score sum_h(q_h . k) * score_mul of item i goes to score_out[i - i0].
template <bool BF16, int D, int G, class RowOf>
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
  const int64_t per_iter = (int64_t)NS * kU;
  const int64_t n = i1 - i0;
  const int64_t iters = n > 0 ? (n + per_iter - 1) / per_iter : 0;
  const size_t lane_off = (size_t)lr * 16;

  for (int64_t it = 0; it < iters; ++it) {
    const int64_t base = i0 + it * per_iter;
    uint4 kr[kU], vr[kU];
    int64_t rows[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t item = base + u * NS + slot;
      const int64_t row = item < i1 ? row_of(item) : -1;
      rows[u] = row;
      if (row >= 0) {
        const size_t off = (size_t)row * Gm::ROW_BYTES + lane_off;
        kr[u] = load16(Kb + off);
        vr[u] = load16(Vb + off);
      } else {
        kr[u] = make_uint4(0u, 0u, 0u, 0u);
        vr[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    float s[kU][G];
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int h = 0; h < G; ++h) s[u][h] = group_sum<LPR>(dot_slice<BF16>(qv[h], kr[u]));
    if (score_out != nullptr) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (rows[u] >= 0 && lr == 0) {
          float t = 0.f;
#pragma unroll
          for (int h = 0; h < G; ++h) t += s[u][h];
          score_out[base + u * NS + slot - i0] = t * score_mul;
        }
      }
    }
    float vf[kU][VEC];
#pragma unroll
    for (int u = 0; u < kU; ++u) widen<BF16>(vr[u], vf[u]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = st.m[h];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        s[u][h] = rows[u] >= 0 ? s[u][h] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[u][h]);
      }
      const float a = fexp2(st.m[h] - mx);
      st.m[h] = mx;
      float l = st.l[h] * a;
#pragma unroll
      for (int e = 0; e < VEC; ++e) st.acc[h][e] *= a;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float p = fexp2(s[u][h] - mx);
        l += p;
#pragma unroll
        for (int e = 0; e < VEC; ++e) st.acc[h][e] = fmaf(p, vf[u][e], st.acc[h][e]);
      }
      st.l[h] = l;
    }
  }
}

// Merge the lane groups' states of the workgroup and write one partial
// (m, l, acc[D]) per head to `dst` ([G][D + 2] floats).
template <bool BF16, int D, int G>
__device__ __forceinline__ void write_partial(State<BF16, G>& st, float* __restrict__ dst) {
  using Gm = Geo<BF16, D>;
  constexpr int VEC = Gm::VEC, LPR = Gm::LPR;
  __shared__ float s_m[kWaves][G], s_l[kWaves][G];
  __shared__ float s_acc[kWaves][G][D];
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
      for (int e = 0; e < VEC; ++e) s_acc[w][h][lr * VEC + e] = acc[e];
      if (lane == 0) {
        s_m[w][h] = mw;
        s_l[w][h] = l;
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    float M = s_m[0][h];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, s_m[ww][h]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = fexp2(s_m[ww][h] - M);
      L = fmaf(s_l[ww][h], f, L);
      A = fmaf(s_acc[ww][h][d], f, A);
    }
    dst[h * (D + 2) + 2 + d] = A;
    if (d == 0) {
      dst[h * (D + 2)] = M;
      dst[h * (D + 2) + 1] = L;
    }
  }
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

// ---------------------------------------------------------------- kernels ---

// Scores and attends a contiguous range of gist-like items of one unit.
template <bool BF16, int D, int G>
__global__ __launch_bounds__(kThreads) void gist_pass_kernel(
    const void* __restrict__ q, const void* __restrict__ K, const void* __restrict__ V,
    int64_t unit_rows, int64_t n_items, int64_t per_split, int32_t S, RowMap rm,
    float* __restrict__ scores, int64_t score_stride, float* __restrict__ part, int32_t NP,
    int32_t part_base, float scale_log2, float score_mul) {
  using Gm = Geo<BF16, D>;
  const int unit = blockIdx.x / S;
  const int split = blockIdx.x % S;
  uint4 qv[G];
  load_q<BF16, D, G>(q, unit, qv);
  State<BF16, G> st;
  init_state<BF16, G>(st);
  const size_t ub = (size_t)unit * (size_t)unit_rows * Gm::ROW_BYTES;
  const char* Kb = reinterpret_cast<const char*>(K) + ub;
  const char* Vb = reinterpret_cast<const char*>(V) + ub;
  const int64_t i0 = (int64_t)split * per_split;
  const int64_t i1 = i0 + per_split < n_items ? i0 + per_split : n_items;
  float* so = scores ? scores + (size_t)unit * score_stride + i0 : nullptr;
  stream_rows<BF16, D, G>(Kb, Vb, i0, i1, [&](int64_t i) { return map_row(rm, unit, i); }, qv, st,
                          scale_log2, so, score_mul);
  write_partial<BF16, D, G>(st, part + ((size_t)unit * NP + part_base + split) * G * (D + 2));
}

// Raw rows of the selected chunks (minus rows the tail owns), then the tail.
template <bool BF16, int D, int G>
__global__ __launch_bounds__(kThreads) void unfold_kernel(
    const void* __restrict__ q, const void* __restrict__ K, const void* __restrict__ V,
    int64_t unit_rows, const int32_t* __restrict__ sel, int32_t k, int32_t C, int64_t M,
    int64_t N, int32_t T, int32_t n_items, int32_t per_split, int32_t S2,
    float* __restrict__ part, int32_t NP, int32_t part_base, float scale_log2) {
  using Gm = Geo<BF16, D>;
  __shared__ int32_t s_sel[1024];
  const int unit = blockIdx.x / S2;
  const int split = blockIdx.x % S2;
  const int32_t* us = sel + (size_t)unit * k;
  const bool sel_in_lds = k <= 1024;
  if (sel_in_lds)
    for (int i = threadIdx.x; i < k; i += kThreads) s_sel[i] = us[i];
  __syncthreads();
  uint4 qv[G];
  load_q<BF16, D, G>(q, unit, qv);
  State<BF16, G> st;
  init_state<BF16, G>(st);
  const size_t ub = (size_t)unit * (size_t)unit_rows * Gm::ROW_BYTES;
  const char* Kb = reinterpret_cast<const char*>(K) + ub;
  const char* Vb = reinterpret_cast<const char*>(V) + ub;
  const int64_t i0 = (int64_t)split * per_split;
  const int64_t i1 = i0 + per_split < n_items ? i0 + per_split : n_items;
  const int64_t kC = (int64_t)k * C;
  const int64_t tail0 = N - T;
  auto row_of = [&](int64_t i) -> int64_t {
    if (i < kC) {
      const int64_t m = sel_in_lds ? s_sel[i / C] : us[i / C];
      const int64_t j = i % C;
      if (m < 0 || m >= M) return -1;             // never taken for a valid selection
      if (m * C + j >= tail0) return -1;          // the tail attends this row
      return m * (C + 1) + j;
    }
    const int64_t p = tail0 + (i - kC);
    return p < M * C ? (p / C) * (C + 1) + p % C : M * (C + 1) + (p - M * C);
  };
  stream_rows<BF16, D, G>(Kb, Vb, i0, i1, row_of, qv, st, scale_log2, nullptr, 0.f);
  write_partial<BF16, D, G>(st, part + ((size_t)unit * NP + part_base + split) * G * (D + 2));
}

struct IdMap {
  const int32_t* sel2;  // nullptr: id = item index
  int32_t G, k2;
  int64_t orphan0;
};

__device__ __forceinline__ int32_t map_id(const IdMap& im, int unit, int32_t i) {
  if (im.sel2 == nullptr) return i;
  const int32_t kg = im.k2 * im.G;
  return i < kg ? im.sel2[(size_t)unit * im.k2 + i / im.G] * im.G + i % im.G
                : (int32_t)(im.orphan0 + (i - kg));
}

// Exact top-k of n scores per unit. The k-th largest order key T is found by
// a bitwise search over the 32 key bits (count(key >= candidate) >= k keeps
// the bit); then every key > T and the first (k - count(key > T)) keys == T in
// index order are written in ascending index order.
__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ scores,
                                                             int64_t stride, int32_t n, int32_t k,
                                                             IdMap im, int32_t* __restrict__ ws_sel,
                                                             int32_t* __restrict__ out_sel) {
  __shared__ uint32_t keys[kSelLds];
  __shared__ int red[3][kSelThreads / 64];
  const int unit = blockIdx.x;
  const int tid = threadIdx.x;
  if (k <= 0) return;
  const float* sc = scores + (size_t)unit * stride;
  int32_t* dst = ws_sel + (size_t)unit * k;
  int32_t* dst2 = out_sel ? out_sel + (size_t)unit * k : nullptr;
  if (k >= n) {  // everything is selected (k == n)
    for (int i = tid; i < n; i += kSelThreads) {
      const int32_t id = map_id(im, unit, i);
      dst[i] = id;
      if (dst2) dst2[i] = id;
    }
    return;
  }
  const bool in_lds = n <= kSelLds;
  if (in_lds)
    for (int i = tid; i < n; i += kSelThreads) keys[i] = order_key(sc[i]);
  __syncthreads();
  auto key_at = [&](int i) -> uint32_t { return in_lds ? keys[i] : order_key(sc[i]); };

  uint32_t T = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int c = 0;
    for (int i = tid; i < n; i += kSelThreads) c += key_at(i) >= cand ? 1 : 0;
    if (block_sum(c, red[bit & 1]) >= k) T = cand;
  }
  int cgt = 0;
  for (int i = tid; i < n; i += kSelThreads) cgt += key_at(i) > T ? 1 : 0;
  const int need = k - block_sum(cgt, red[2]);   // keys equal to T still to take (>= 1)

  const int E = (n + kSelThreads - 1) / kSelThreads;
  const int lo = tid * E < n ? tid * E : n;
  const int hi = lo + E < n ? lo + E : n;
  int gt = 0, eq = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = key_at(i);
    gt += key > T ? 1 : 0;
    eq += key == T ? 1 : 0;
  }
  const int eq_before = block_excl_scan(eq, red[0]);
  int take = need - eq_before;
  take = take < 0 ? 0 : (take > eq ? eq : take);
  int pos = block_excl_scan(gt + take, red[1]);
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = key_at(i);
    bool pick = key > T;
    if (!pick && key == T && take > 0) {
      pick = true;
      --take;
    }
    if (pick) {
      const int32_t id = map_id(im, unit, i);
      dst[pos] = id;
      if (dst2) dst2[pos] = id;
      ++pos;
    }
  }
}

// out[unit, h] = sum_p 2^(m_p - m*) acc_p / sum_p 2^(m_p - m*) l_p.
template <int D>
__global__ __launch_bounds__(D) void merge_kernel(const float* __restrict__ part, int32_t NP,
                                                  int32_t G, float* __restrict__ out,
                                                  float* __restrict__ lse) {
  const int uh = blockIdx.x;          // unit * G + h
  const int unit = uh / G, h = uh % G;
  const int d = threadIdx.x;
  const float* P = part + (size_t)unit * NP * G * (D + 2) + (size_t)h * (D + 2);
  const size_t ps = (size_t)G * (D + 2);
  float mx = kMinus;
  for (int p = 0; p < NP; ++p) mx = fmaxf(mx, P[p * ps]);
  float L = 0.f, A = 0.f;
  for (int p = 0; p < NP; ++p) {
    const float f = fexp2(P[p * ps] - mx);
    L = fmaf(P[p * ps + 1], f, L);
    A = fmaf(P[p * ps + 2 + d], f, A);
  }
  out[(size_t)uh * D + d] = A / L;
  if (lse != nullptr && d == 0) lse[uh] = (mx + log2f(L)) * kLn2;
}

// ------------------------------------------------------------------ host ---

gsa_status_t launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return GSA_OK;
}

template <bool BF16, int D, int G>
gsa_status_t run_decode(const DecodePlan& pl, const void* q, const void* K, const void* V,
                        float* out, float* lse, int32_t* sel_idx, char* ws, hipStream_t st) {
  float* scores = reinterpret_cast<float*>(ws + pl.off_scores);
  int32_t* wsel = reinterpret_cast<int32_t*>(ws + pl.off_sel);
  float* part = reinterpret_cast<float*>(ws + pl.off_part);
  const float sl2 = pl.scale * kLog2e;
  RowMap rm{0, pl.C, nullptr, 0, 0, 0};
  hipLaunchKernelGGL((gist_pass_kernel<BF16, D, G>), dim3(pl.units * pl.S), dim3(kThreads), 0, st,
                     q, K, V, pl.R, pl.M, pl.gists_per_split, pl.S, rm, scores, pl.score_stride,
                     part, pl.NP, 0, sl2, pl.scale / G);
  if (pl.k > 0)
    hipLaunchKernelGGL(select_kernel, dim3(pl.units), dim3(kSelThreads), 0, st, scores,
                       pl.score_stride, (int32_t)pl.M, pl.k, IdMap{nullptr, 0, 0, 0}, wsel, sel_idx);
  hipLaunchKernelGGL((unfold_kernel<BF16, D, G>), dim3(pl.units * pl.S2), dim3(kThreads), 0, st, q,
                     K, V, pl.R, wsel, pl.k, pl.C, pl.M, pl.N, pl.T, pl.n_items, pl.items_per_split,
                     pl.S2, part, pl.NP, pl.S, sl2);
  hipLaunchKernelGGL((merge_kernel<D>), dim3(pl.units * G), dim3(D), 0, st, part, pl.NP, G, out, lse);
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
  int32_t* wsel1 = reinterpret_cast<int32_t*>(ws + hp.off_sel1);
  float* part = reinterpret_cast<float*>(ws + hp.off_part);
  const float sl2 = pl.scale * kLog2e;
  const int64_t orphan0 = hp.M2 * hp.G;
  // level 2: every meta-gist (dense rows of the level-2 array)
  RowMap r2{1, pl.C, nullptr, 0, 0, 0};
  hipLaunchKernelGGL((gist_pass_kernel<BF16, D, G>), dim3(pl.units * hp.S_l2), dim3(kThreads), 0,
                     st, q, K2, V2, hp.M2, hp.M2, hp.l2_per_split, hp.S_l2, r2, s2, hp.s2_stride,
                     part, hp.NP, 0, sl2, pl.scale / G);
  if (hp.k2 > 0)
    hipLaunchKernelGGL(select_kernel, dim3(pl.units), dim3(kSelThreads), 0, st, s2, hp.s2_stride,
                       (int32_t)hp.M2, hp.k2, IdMap{nullptr, 0, 0, 0}, wsel2, sel2);
  // level 1: children of the chosen groups + ungrouped gists
  RowMap r1{2, pl.C, wsel2, hp.G, hp.k2, orphan0};
  hipLaunchKernelGGL((gist_pass_kernel<BF16, D, G>), dim3(pl.units * hp.S_c), dim3(kThreads), 0,
                     st, q, K, V, pl.R, (int64_t)hp.n_cand, (int64_t)hp.cand_per_split, hp.S_c, r1,
                     sc, hp.sc_stride, part, hp.NP, hp.S_l2, sl2, pl.scale / G);
  if (pl.k > 0)
    hipLaunchKernelGGL(select_kernel, dim3(pl.units), dim3(kSelThreads), 0, st, sc, hp.sc_stride,
                       hp.n_cand, pl.k, IdMap{wsel2, hp.G, hp.k2, orphan0}, wsel1, sel1);
  hipLaunchKernelGGL((unfold_kernel<BF16, D, G>), dim3(pl.units * pl.S2), dim3(kThreads), 0, st, q,
                     K, V, pl.R, wsel1, pl.k, pl.C, pl.M, pl.N, pl.T, pl.n_items, pl.items_per_split,
                     pl.S2, part, hp.NP, hp.S_l2 + hp.S_c, sl2);
  hipLaunchKernelGGL((merge_kernel<D>), dim3(pl.units * G), dim3(D), 0, st, part, hp.NP, G, out, lse);
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
