// Causal block-sparse GSA prefill on gfx950: bf16 MFMA (v_mfma_f32_16x16x32_bf16)
// with fp32 accumulation and an fp32 online softmax.
//
// Method: gist.science explainer "Forget, Then Recall", 'Training Procedure:
// Selective Finetuning' (each query attends to the top-k chunks chosen by its
// gist scores and to their raw tokens) with the causal gist order of section
// 2 'Key Concepts' (a gist follows its chunk, so query t may use gist m only
// once chunk m is complete: m < floor(t/C)); the slide deck's slides 7-10.
//
// One workgroup per (kv-head, block of 64 query positions); wave w owns
// queries 16w..16w+15 of the block with all g query heads of the kv-head, so
// every K/V tile staged in LDS serves 64*g query rows.
//
//   prefill_select  group score S[t][m] = (scale/g) * sum_h q_h(t) . k(gist m)
//                   for eligible gists, per query the exact top-k (ties to the
//                   smaller m) -> sel. The g heads of a query form one
//                   contraction of length g*D, so one MFMA chain gives the
//                   group score. Top-k is a streaming filter: a per-query LDS
//                   buffer of survivors (in gist order) is compacted to the
//                   exact top-k by a bit-serial radix select whenever it fills;
//                   afterwards only scores above the k-th best can enter.
//   prefill_attend  softmax attention over every eligible gist, the raw rows of
//                   the union of the block's selected chunks (a query sees a
//                   chunk only if it selected it) and the causal window
//                   [t-W+1, t]; a row in the window is attended once (by the
//                   window pass). S^T = K Q^T and O^T += V^T P^T so that both
//                   results keep one query row per lane; V^T comes from the
//                   row-major V tile through the transposing LDS read
//                   (ds_read_b64_tr_b16). P is split into bf16 hi + lo parts so
//                   that P.V keeps about 16 bits of the fp32 weights.
#include <hip/hip_runtime.h>

#include "gsa.h"
#include "gsa_device.hpp"
#include "gsa_plan.hpp"
#include "gsa_profile.hpp"

namespace gsa {
namespace {

using namespace dev;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short __attribute__((ext_vector_type(4))) __attribute__((address_space(3)))* lds_i16x4_ptr;

constexpr int kPThreads = 256;          // 4 waves
constexpr int kPWaves = 4;
constexpr int kQB = kQBlock;            // queries per workgroup (64)
static_assert(kQB == 16 * kPWaves, "one 16-query tile per wave");
constexpr int kD = 128;
constexpr int kRowBytes = kD * 2;       // bf16 row
constexpr int kKStride = 272;           // LDS row stride of K tiles: conflict-free 16 B operand reads
constexpr int kVStride = 288;           // LDS row stride of V tiles: conflict-free transposed reads
constexpr int kSelTile = 64;            // gists per selection tile
constexpr int kCap = 64;                // survivor buffer entries per query
constexpr int kAttTile = 32;            // rows per attention tile (the K of the P.V MFMA)
constexpr float kPLazy = 8.f;           // lazy running max, log2 units

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_b128(const char* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Four bf16 of a transposed LDS read (see the file header).
__device__ __forceinline__ i16x4 lds_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4_ptr)((__attribute__((address_space(3))) char*)p));
}

__device__ __forceinline__ bf16x8 cat8(const i16x4& lo, const i16x4& hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Cache row of raw position p of the interleaved cache.
__device__ __forceinline__ int32_t raw_row(int32_t p, int32_t C, int32_t M) {
  const int32_t MC = M * C;
  return p < MC ? (p / C) * (C + 1) + p % C : M * (C + 1) + (p - MC);
}

// Exclusive prefix and total over the four lanes {i, i+16, i+32, i+48} that
// share a query (jg = lane / 16 orders them).
__device__ __forceinline__ int excl4(int c, int jg, int* total) {
  const int x1 = __shfl_xor(c, 16);
  const int pair = c + x1;
  const int x2 = __shfl_xor(pair, 32);
  *total = pair + x2;
  return ((jg & 1) ? x1 : 0) + ((jg & 2) ? x2 : 0);
}
__device__ __forceinline__ int sum4(int c) {
  c += __shfl_xor(c, 16);
  return c + __shfl_xor(c, 32);
}
__device__ __forceinline__ float max4(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float fsum4(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup -> (kv-head, query block). Consecutive linear ids share a kv-head
// (its K/V rows); with 8 XCDs taking workgroups round-robin, the linear id
// groups each XCD's workgroups together so one XCD's L2 serves one kv-head.
__device__ __forceinline__ void wg_coords(int n_blocks, int Hkv, int* kvh, int* blk) {
  const int total = n_blocks * Hkv;
  int x = (int)blockIdx.x;
  if (total % 8 == 0) x = (x % 8) * (total / 8) + x / 8;
  *kvh = x / n_blocks;
  *blk = x % n_blocks;
}

// Query fragments (B operand of S^T = K Q^T): lane holds q_h[query][32ks + 8jg .. +7].
template <int G>
__device__ __forceinline__ void load_qfrag(const char* qbase, int64_t n_q, int64_t t_idx, bool valid,
                                           int jg, bf16x8 (&qf)[G][4]) {
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (valid) {
        const uint4 v = load16(qbase + (((int64_t)h * n_q + t_idx) * kD + 32 * ks + 8 * jg) * 2);
        qf[h][ks] = __builtin_bit_cast(bf16x8, v);
      } else {
        qf[h][ks] = __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
      }
    }
}

// ------------------------------------------------------------ selection ----

struct SelArgs {
  const void* q;          // [Hq][n_q][D] bf16
  const void* K;          // [Hkv][R][D] bf16
  int64_t R;
  int32_t M, C, k, Hkv, n_blocks, q_start, n_q;
  float score_mul;        // scale / g
  int32_t* sel_ws;        // [Hkv][n_q][k]
  int32_t* sel_out;       // [Hkv][n_q][k] or null
};

struct SelLds {
  char kt[2][kSelTile * kKStride];
  uint32_t bkey[kQB][kCap];
  uint32_t bid[kQB][kCap];
};

// Compact every query's survivor buffer of the wave to its exact top-k.
// Lanes (qi, jg) own entries [16jg, 16jg + 16) of query qloc's buffer (in
// gist order). Returns the new count; tau gets the k-th best key (0 if fewer
// than k entries: then every later eligible gist still enters).
__device__ __forceinline__ int compact_query(SelLds& L, int qloc, int jg, int cnt, int k, uint32_t* tau) {
  uint32_t kk[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) kk[e] = 16 * jg + e < cnt ? L.bkey[qloc][16 * jg + e] : 0u;
  uint32_t P = 0u;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = P | (1u << b);
    int n = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) n += kk[e] >= c ? 1 : 0;
    n = sum4(n);
    P = n >= k ? c : P;
  }
  int gt = 0, ce = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    gt += kk[e] > P ? 1 : 0;
    ce += (kk[e] == P && kk[e] != 0u) ? 1 : 0;
  }
  gt = sum4(gt);
  const int need = k - gt;
  int ce_tot;
  int eqb = excl4(ce, jg, &ce_tot);
  bool take[16];
  int ct = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const bool eq = kk[e] == P && kk[e] != 0u;
    take[e] = kk[e] > P || (eq && eqb < need);
    eqb += eq ? 1 : 0;
    ct += take[e] ? 1 : 0;
  }
  int tot;
  int pos = excl4(ct, jg, &tot);
  uint32_t ii[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) ii[e] = take[e] ? L.bid[qloc][16 * jg + e] : 0u;
  wave_lds_sync();
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    if (take[e]) {
      L.bkey[qloc][pos] = kk[e];
      L.bid[qloc][pos] = ii[e];
      ++pos;
    }
  }
  wave_lds_sync();
  *tau = tot >= k ? P : 0u;
  return tot;
}

// Stage gist rows [m0, m0 + kSelTile) of one kv-head into registers (zero rows
// past E); 4 x 16 B per thread, 16 consecutive threads per 256-byte row.
__device__ __forceinline__ void sel_load(const char* Kh, int m0, int E, int C, uint4 (&r)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int pair = (int)threadIdx.x + kPThreads * u;
    const int i = pair >> 4, ch = pair & 15;
    const int m = m0 + i;
    r[u] = m < E ? load16(Kh + ((int64_t)m * (C + 1) + C) * kRowBytes + ch * 16) : make_uint4(0u, 0u, 0u, 0u);
  }
}
__device__ __forceinline__ void sel_store(char* kt, const uint4 (&r)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int pair = (int)threadIdx.x + kPThreads * u;
    *reinterpret_cast<uint4*>(kt + (pair >> 4) * kKStride + (pair & 15) * 16) = r[u];
  }
}

template <int G>
__global__ __launch_bounds__(kPThreads) void prefill_select(SelArgs a) {
  __shared__ SelLds L;
  int kvh, blk;
  wg_coords(a.n_blocks, a.Hkv, &kvh, &blk);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int qi = lane & 15, jg = lane >> 4;
  const int qloc = 16 * w + qi;
  const int t_idx = blk * kQB + qloc;
  const bool valid = t_idx < a.n_q;
  const int t = a.q_start + t_idx;
  const int elig = valid ? min(a.M, t / a.C) : 0;
  const int t_last = a.q_start + min(a.n_q, (blk + 1) * kQB) - 1;
  const int E = min(a.M, t_last / a.C);     // gists any query of the block may use

  bf16x8 qf[G][4];
  load_qfrag<G>(reinterpret_cast<const char*>(a.q) + (int64_t)kvh * G * a.n_q * kRowBytes, a.n_q, t_idx,
                valid, jg, qf);
  const char* Kh = reinterpret_cast<const char*>(a.K) + (int64_t)kvh * a.R * kRowBytes;

  int cnt = 0;
  uint32_t tau = 0u;
  const int n_tiles = (E + kSelTile - 1) / kSelTile;
  uint4 stage[4];
  if (n_tiles > 0) {
    sel_load(Kh, 0, E, a.C, stage);
    sel_store(L.kt[0], stage);
  }
  __syncthreads();
  for (int it = 0; it < n_tiles; ++it) {
    if (it + 1 < n_tiles) sel_load(Kh, (it + 1) * kSelTile, E, a.C, stage);
    const char* kt = L.kt[it & 1];
#pragma unroll
    for (int s = 0; s < kSelTile / 16; ++s) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 kf = lds_b128(kt + (16 * s + qi) * kKStride + ks * 64 + jg * 16);
#pragma unroll
        for (int h = 0; h < G; ++h) acc = mfma(kf, qf[h][ks], acc);
      }
      // acc[r]: gist it*64 + 16s + 4jg + r against query qi (all heads summed)
      uint32_t key[4];
      bool sv[4];
      int c = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = it * kSelTile + 16 * s + 4 * jg + r;
        key[r] = m < elig ? order_key(acc[r] * a.score_mul) : 0u;
        sv[r] = key[r] > tau;
        c += sv[r] ? 1 : 0;
      }
      if (__ballot(c > 0) != 0ull) {
        int tot;
        int pos = cnt + excl4(c, jg, &tot);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (sv[r]) {
            L.bkey[qloc][pos] = key[r];
            L.bid[qloc][pos] = (uint32_t)(it * kSelTile + 16 * s + 4 * jg + r);
            ++pos;
          }
        }
        cnt += tot;
        wave_lds_sync();
        if (__ballot(cnt > kCap - 16) != 0ull) cnt = compact_query(L, qloc, jg, cnt, a.k, &tau);
      }
    }
    __syncthreads();   // every wave is done with the other buffer
    if (it + 1 < n_tiles) sel_store(L.kt[(it + 1) & 1], stage);
    __syncthreads();
  }
  cnt = compact_query(L, qloc, jg, cnt, a.k, &tau);
  if (valid) {
    const int64_t o = ((int64_t)kvh * a.n_q + t_idx) * a.k;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = 16 * jg + e;
      if (i < a.k) {
        const int32_t v = i < cnt ? (int32_t)L.bid[qloc][i] : -1;
        a.sel_ws[o + i] = v;
        if (a.sel_out) a.sel_out[o + i] = v;
      }
    }
  }
}

// ------------------------------------------------------------ attention ----

constexpr int kMaxChunkWords = kPrefillMaxGist / 32;   // bitmap of selectable chunks
constexpr int kMaxUnion = kQB * kPrefillMaxK;           // distinct chunks a block can select

struct AttArgs {
  const void* q;
  const void* K;
  const void* V;
  float* out;             // [Hq][n_q][D] fp32
  const int32_t* sel;     // [Hkv][n_q][k]
  int64_t R;
  int32_t M, C, k, W, Hkv, n_blocks, q_start, n_q;
  float scale_log2;
};

struct AttLds {
  char kt[2][kAttTile * kKStride];
  char vt[2][kAttTile * kVStride];
  uint32_t bitmap[kMaxChunkWords];
  uint32_t wpre[kMaxChunkWords];
  int32_t U[kMaxUnion];
  uint32_t qm[kMaxUnion][2];
  int scan[kPWaves];
  int nU;
};

// What a tile row is: a gist, a raw row of a selected chunk, a window row.
enum { kGist = 0, kChunk = 1, kWin = 2 };

struct Phase {
  int kind;
  int n;        // rows in the phase
  int lo;       // kWin: first position
};

__device__ __forceinline__ int phase_row(const Phase& ph, const AttLds& L, int i, int C, int M) {
  if (i >= ph.n) return -1;
  if (ph.kind == kGist) return i * (C + 1) + C;
  if (ph.kind == kChunk) {
    const int m = L.U[i / C];
    return m * (C + 1) + i % C;
  }
  return raw_row(ph.lo + i, C, M);
}

// Stage rows [i0, i0 + kAttTile) of a phase: K and V, 2 x 16 B each per thread.
__device__ __forceinline__ void att_load(const char* Kh, const char* Vh, const Phase& ph, const AttLds& L,
                                         int i0, int C, int M, uint4 (&rk)[2], uint4 (&rv)[2]) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int pair = (int)threadIdx.x + kPThreads * u;
    const int i = pair >> 4, ch = pair & 15;
    const int row = phase_row(ph, L, i0 + i, C, M);
    if (row >= 0) {
      rk[u] = load16(Kh + (int64_t)row * kRowBytes + ch * 16);
      rv[u] = load16(Vh + (int64_t)row * kRowBytes + ch * 16);
    } else {
      rk[u] = make_uint4(0u, 0u, 0u, 0u);
      rv[u] = rk[u];
    }
  }
}
__device__ __forceinline__ void att_store(char* kt, char* vt, const uint4 (&rk)[2], const uint4 (&rv)[2]) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int pair = (int)threadIdx.x + kPThreads * u;
    const int i = pair >> 4, ch = pair & 15;
    *reinterpret_cast<uint4*>(kt + i * kKStride + ch * 16) = rk[u];
    *reinterpret_cast<uint4*>(vt + i * kVStride + ch * 16) = rv[u];
  }
}

template <int G>
struct AttState {
  f32x4 o[G][8];      // O^T[16dt + 4jg + r][query qi] of head h
  float m[G], l[G];   // running max (log2 units) and this lane's share of the sum
};

// May query (t, qi) use row i of the phase?
__device__ __forceinline__ bool row_ok(const Phase& ph, const AttLds& L, int i, int qi, int t, int elig,
                                       int W, int C) {
  if (i >= ph.n) return false;
  if (ph.kind == kGist) return i < elig;
  if (ph.kind == kChunk) {
    const int u = i / C;
    if (!((L.qm[u][qi >> 5] >> (qi & 31)) & 1u)) return false;
    const int pos = L.U[u] * C + i % C;
    return pos < t - W + 1;                    // the window attends that row
  }
  const int pos = ph.lo + i;
  return pos >= t - W + 1 && pos <= t;
}

template <int G>
__device__ __forceinline__ void att_tile(const char* kt, const char* vt, const Phase& ph, const AttLds& L,
                                         int i0, int qloc, int t, int elig, bool valid, int W, int C,
                                         float c, const bf16x8 (&qf)[G][4], AttState<G>& st) {
  const int lane = threadIdx.x & 63, qi = lane & 15, jg = lane >> 4;
  f32x4 s[2][G];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int h = 0; h < G; ++h) s[sb][h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 kf = lds_b128(kt + (16 * sb + qi) * kKStride + ks * 64 + jg * 16);
#pragma unroll
      for (int h = 0; h < G; ++h) s[sb][h] = mfma(kf, qf[h][ks], s[sb][h]);
    }
  // s[sb][h][r]: row i0 + 16sb + 4jg + r against query qi, head h
  bool ok[2][4];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      ok[sb][r] = valid && row_ok(ph, L, i0 + 16 * sb + 4 * jg + r, qloc, t, elig, W, C);
  bf16x8 phi[G], plo[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sb = e >> 2, r = e & 3;
      x[e] = ok[sb][r] ? s[sb][h][r] * c : -INFINITY;
    }
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
    mx = max4(mx);
    const bool need = mx > st.m[h] + kPLazy;
    if (__ballot(need) != 0ull) {
      const float mn = need ? mx : st.m[h];
      const float al = fexp2(st.m[h] - mn);
      st.m[h] = mn;
      st.l[h] *= al;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) st.o[h][dt][r] *= al;
    }
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = fexp2(x[e] - st.m[h]);
      ps += p;
      const __bf16 hi = (__bf16)p;
      phi[h][e] = hi;
      plo[h][e] = (__bf16)(p - (float)hi);
    }
    st.l[h] += ps;
  }
  // O^T += V^T P^T: A operand = V^T rows of this tile, transposed out of LDS
  const int s16 = lane & 15;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const char* p1 = vt + (4 * jg + (s16 >> 2)) * kVStride + (16 * dt + 4 * (s16 & 3)) * 2;
    const char* p2 = p1 + 16 * kVStride;
    const bf16x8 vf = cat8(lds_tr(p1), lds_tr(p2));
#pragma unroll
    for (int h = 0; h < G; ++h) {
      st.o[h][dt] = mfma(vf, phi[h], st.o[h][dt]);
      st.o[h][dt] = mfma(vf, plo[h], st.o[h][dt]);
    }
  }
}

template <int G>
__device__ __forceinline__ void att_phase(const char* Kh, const char* Vh, const Phase& ph, AttLds& L,
                                          int qloc, int t, int elig, bool valid, int W, int C, int M, float c,
                                          const bf16x8 (&qf)[G][4], AttState<G>& st) {
  const int n_tiles = (ph.n + kAttTile - 1) / kAttTile;
  if (n_tiles == 0) return;
  uint4 rk[2], rv[2];
  att_load(Kh, Vh, ph, L, 0, C, M, rk, rv);
  att_store(L.kt[0], L.vt[0], rk, rv);
  __syncthreads();
  for (int it = 0; it < n_tiles; ++it) {
    if (it + 1 < n_tiles) att_load(Kh, Vh, ph, L, (it + 1) * kAttTile, C, M, rk, rv);
    att_tile<G>(L.kt[it & 1], L.vt[it & 1], ph, L, it * kAttTile, qloc, t, elig, valid, W, C, c, qf, st);
    __syncthreads();
    if (it + 1 < n_tiles) att_store(L.kt[(it + 1) & 1], L.vt[(it + 1) & 1], rk, rv);
    __syncthreads();
  }
}

template <int G>
__global__ __launch_bounds__(kPThreads) void prefill_attend(AttArgs a) {
  __shared__ AttLds L;
  int kvh, blk;
  wg_coords(a.n_blocks, a.Hkv, &kvh, &blk);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int qi = lane & 15, jg = lane >> 4;
  const int qloc = 16 * w + qi;
  const int t_idx = blk * kQB + qloc;
  const bool valid = t_idx < a.n_q;
  const int t = a.q_start + t_idx;
  const int elig = valid ? min(a.M, t / a.C) : 0;
  const int nq_blk = min(kQB, a.n_q - blk * kQB);
  const int t_first = a.q_start + blk * kQB;
  const int t_last = t_first + nq_blk - 1;
  const int E = min(a.M, t_last / a.C);

  // union of the block's selected chunks (ascending) and, per chunk, the
  // mask of the queries that selected it
  const int nwords = (E + 31) / 32;
  for (int i = tid; i < nwords; i += kPThreads) L.bitmap[i] = 0u;
  __syncthreads();
  const int32_t* sb = a.sel + ((int64_t)kvh * a.n_q + (int64_t)blk * kQB) * a.k;
  for (int pr = tid; pr < nq_blk * a.k; pr += kPThreads) {
    const int m = sb[pr];
    if (m >= 0 && m < E) atomicOr(&L.bitmap[m >> 5], 1u << (m & 31));
  }
  __syncthreads();
  {
    constexpr int kPer = kMaxChunkWords / kPThreads;
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int wd = tid * kPer + e;
      cnt += wd < nwords ? __popc(L.bitmap[wd]) : 0;
    }
    int run = block_excl_scan(cnt, L.scan);
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int wd = tid * kPer + e;
      if (wd < nwords) {
        L.wpre[wd] = (uint32_t)run;
        uint32_t bits = L.bitmap[wd];
        int r = run;
        while (bits) {
          const int b = __ffs(bits) - 1;
          L.U[r++] = wd * 32 + b;
          bits &= bits - 1u;
        }
        run = r;
      }
    }
    if (tid == kPThreads - 1) L.nU = run;
  }
  __syncthreads();
  const int nU = L.nU;
  for (int i = tid; i < nU; i += kPThreads) {
    L.qm[i][0] = 0u;
    L.qm[i][1] = 0u;
  }
  __syncthreads();
  for (int pr = tid; pr < nq_blk * a.k; pr += kPThreads) {
    const int m = sb[pr];
    if (m >= 0 && m < E) {
      const int u = (int)L.wpre[m >> 5] + __popc(L.bitmap[m >> 5] & ((1u << (m & 31)) - 1u));
      const int ql = pr / a.k;
      atomicOr(&L.qm[u][ql >> 5], 1u << (ql & 31));
    }
  }
  __syncthreads();

  bf16x8 qf[G][4];
  load_qfrag<G>(reinterpret_cast<const char*>(a.q) + (int64_t)kvh * G * a.n_q * kRowBytes, a.n_q, t_idx,
                valid, jg, qf);
  const char* Kh = reinterpret_cast<const char*>(a.K) + (int64_t)kvh * a.R * kRowBytes;
  const char* Vh = reinterpret_cast<const char*>(a.V) + (int64_t)kvh * a.R * kRowBytes;
  AttState<G> st;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = kMinus;
    st.l[h] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[h][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int lo = max(0, t_first - a.W + 1);
  const Phase phases[3] = {{kGist, E, 0}, {kChunk, nU * a.C, 0}, {kWin, t_last - lo + 1, lo}};
#pragma unroll 1
  for (int p = 0; p < 3; ++p)
    att_phase<G>(Kh, Vh, phases[p], L, qloc, t, elig, valid, a.W, a.C, a.M, a.scale_log2, qf, st);

  if (!valid) return;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float inv = 1.f / fsum4(st.l[h]);
    float* o = a.out + (((int64_t)kvh * G + h) * a.n_q + t_idx) * kD;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const float4 v = make_float4(st.o[h][dt][0] * inv, st.o[h][dt][1] * inv, st.o[h][dt][2] * inv,
                                   st.o[h][dt][3] * inv);
      *reinterpret_cast<float4*>(o + 16 * dt + 4 * jg) = v;
    }
  }
}

template <int G>
gsa_status_t run_prefill(const PrefillPlan& pl, const void* q, const void* K, const void* V, float* out,
                         int32_t* sel, char* ws, hipStream_t stream) {
  if (pl.n_q == 0) return GSA_OK;
  int32_t* wsel = reinterpret_cast<int32_t*>(ws);
  const int grid = pl.n_blocks * pl.Hkv;
  prof_begin_call();
  prof_mark(stream);
  if (pl.k > 0) {
    SelArgs s{};
    s.q = q; s.K = K; s.R = pl.R;
    s.M = (int32_t)pl.M; s.C = pl.C; s.k = pl.k; s.Hkv = pl.Hkv; s.n_blocks = pl.n_blocks;
    s.q_start = (int32_t)pl.q_start; s.n_q = (int32_t)pl.n_q;
    s.score_mul = pl.scale / G;
    s.sel_ws = wsel; s.sel_out = sel;
    hipLaunchKernelGGL((prefill_select<G>), dim3(grid), dim3(kPThreads), 0, stream, s);
    prof_mark(stream);
  }
  AttArgs t{};
  t.q = q; t.K = K; t.V = V; t.out = out; t.sel = wsel; t.R = pl.R;
  t.M = (int32_t)pl.M; t.C = pl.C; t.k = pl.k; t.W = pl.W; t.Hkv = pl.Hkv; t.n_blocks = pl.n_blocks;
  t.q_start = (int32_t)pl.q_start; t.n_q = (int32_t)pl.n_q;
  t.scale_log2 = pl.scale * kLog2e;
  hipLaunchKernelGGL((prefill_attend<G>), dim3(grid), dim3(kPThreads), 0, stream, t);
  prof_mark(stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GSA_ERR_HIP, "gsa_prefill_blocksparse launch: %s", hipGetErrorString(e));
  return GSA_OK;
}

}  // namespace
}  // namespace gsa

using namespace gsa;

extern "C" gsa_status_t gsa_prefill_workspace_size(const gsa_prefill_params* p, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(GSA_ERR_INVALID_ARG, "bytes is NULL");
  PrefillPlan pl;
  gsa_status_t s = plan_prefill(p, &pl);
  if (s != GSA_OK) return s;
  *bytes = pl.total;
  return GSA_OK;
}

extern "C" gsa_status_t gsa_prefill_blocksparse(const gsa_prefill_params* p, const void* q,
                                                const void* k_cache, const void* v_cache, float* out,
                                                int32_t* sel, void* workspace, size_t workspace_bytes,
                                                void* stream) {
  clear_error();
  PrefillPlan pl;
  gsa_status_t s = plan_prefill(p, &pl);
  if (s != GSA_OK) return s;
  if ((s = check_ptr(q, "q")) != GSA_OK || (s = check_ptr(k_cache, "k_cache")) != GSA_OK ||
      (s = check_ptr(v_cache, "v_cache")) != GSA_OK || (s = check_ptr(out, "out")) != GSA_OK ||
      (s = check_ptr(sel, "sel", true)) != GSA_OK)
    return s;
  if ((s = check_workspace(workspace, workspace_bytes, pl.total)) != GSA_OK) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  switch (pl.g) {
    case 1: return run_prefill<1>(pl, q, k_cache, v_cache, out, sel, ws, st);
    case 2: return run_prefill<2>(pl, q, k_cache, v_cache, out, sel, ws, st);
    case 4: return run_prefill<4>(pl, q, k_cache, v_cache, out, sel, ws, st);
  }
  return fail(GSA_ERR_UNSUPPORTED, "prefill: %d query heads per kv-head not in {1, 2, 4}", pl.g);
}
