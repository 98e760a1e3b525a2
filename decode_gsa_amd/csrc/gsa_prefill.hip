// Causal block-sparse GSA prefill on gfx950: bf16 MFMA (v_mfma_f32_16x16x32_bf16)
// with fp32 accumulation and an fp32 online softmax.
//
// Method: gist.science explainer "Forget, Then Recall", 'Training Procedure:
// Selective Finetuning' (each query attends to the top-k chunks chosen by its
// gist scores and to their raw tokens) with the causal gist order of section
// 2 'Key Concepts' (a gist follows its chunk, so query t may use gist m only
// once chunk m is complete: m < floor(t/C)); the slide deck's slides 7-10.
//
// One workgroup per (kv-head, block of 64 query positions); its waves own
// 16-query tiles of the block, so every K/V tile staged in LDS serves 64*g
// query rows.
//
//   prefill_select  group score S[t][m] = (scale/g) * sum_h q_h(t) . k(gist m)
//                   for eligible gists, per query the exact top-k (ties to the
//                   smaller m) -> sel. The sum over heads is taken on the
//                   query side (qbar = sum_h q_h, kept as bf16 hi + lo), so
//                   two MFMA chains give the group score. Top-k is a
//                   streaming filter: the four lanes that hold a query's
//                   scores keep candidate lists in LDS; a score enters when it
//                   beats the query's running bound tau; when a list fills,
//                   the workgroup prunes every list (a bisection finds a
//                   value with at least k entries at or above it) and the
//                   bound rises; the end is an exact radix selection.
//                   In a 32-gist tile a lane sees eight scores.
//   prefill_attend  softmax attention over every eligible gist, the raw rows of
//                   the union of the block's selected chunks (a query sees a
//                   chunk only if it selected it) and the causal window
//                   [t-W+1, t]; a row in the window is attended once (by the
//                   window pass). S^T = K Q^T and O^T += V^T P^T so that both
//                   results keep one query row per lane; V^T comes from the
//                   row-major V tile through the transposing LDS read
//                   (ds_read_b64_tr_b16). P is split into bf16 hi + lo parts so
//                   that P.V keeps about 16 bits of the fp32 weights (hi is p
//                   truncated to bf16, lo = p - hi rounded). With g = 4
//                   two waves share a query tile (two heads each), so each SIMD
//                   runs two waves.
//
// Gist tokens (gsa_gist_prefill): the gist of chunk m sees the chunk's C raw
// tokens and the gists before it (the gist causal mask, section 2 and slide
// 7), which is the attention of a raw query at position mC + C - 1 with k = 0
// and W = C. The attention kernel runs them as such, its queries C positions
// apart (AttArgs::q_stride).
//
// K/V tiles reach LDS by direct-to-LDS loads (global_load_lds_dwordx4) into a
// ring of tiles, several tiles in flight. Such a load writes lane i's 16 bytes
// at LDS base + 16 i, so the layout is made conflict-free by choosing which
// 16-byte chunk of the row each lane fetches: chunk c of tile row r sits in
// slot c ^ (r & 15) for K (16-byte operand reads, 16 rows at a time) and in
// slot c ^ 2(r & 7) for V (8-byte transposed reads of 8 rows).
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

constexpr int kQB = kQBlock;            // queries per workgroup (64)
constexpr int kD = 128;
constexpr int kRowBytes = kD * 2;       // bf16 row: 16 chunks of 16 bytes
constexpr float kPLazy = 8.f;           // lazy running max, log2 units

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_b128(const char* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x8 cat8(const i16x4& lo, const i16x4& hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// One direct-to-LDS load per lane: 16 bytes from src to lds_base + 16 * lane
// (lds_base is the same for the whole wave).
__device__ __forceinline__ void dma16(const char* src, char* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the memory fences of __syncthreads(). The fences
// would make every wave wait for all of its loads in flight, including the
// direct-to-LDS loads of later tiles; the hand-off of a tile is ordered instead
// by each wave's own vmcnt wait before the barrier. lgkmcnt(0) retires this
// wave's LDS reads of the tile whose buffer the next loads overwrite.
__device__ __forceinline__ void tile_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)p);
}


// A tile's K operand reads (eight 16-byte reads) and its V^T operands for
// all 8 column blocks of 16 (two transposed 8-byte reads per block: rows
// 0-15 and 16-31 of the tile, the second 4096 bytes further) in one asm block
// that also waits for them: the V reads' latency hides under the K reads'
// instead of following the score and softmax work, and the builtin form
// would make the compiler wait for every direct-to-LDS load in flight first.
__device__ __forceinline__ void lds_kv_tile(const uint32_t (&ka)[8], const uint32_t (&va)[8], uint4 (&r)[8],
                                            bf16x8 (&vf)[8]) {
  i16x4 a[8], b[8];
  __asm__ volatile(
      "ds_read_b128 %0, %24\n\t"
      "ds_read_b128 %1, %25\n\t"
      "ds_read_b128 %2, %26\n\t"
      "ds_read_b128 %3, %27\n\t"
      "ds_read_b128 %4, %28\n\t"
      "ds_read_b128 %5, %29\n\t"
      "ds_read_b128 %6, %30\n\t"
      "ds_read_b128 %7, %31\n\t"
      "ds_read_b64_tr_b16 %8, %32\n\t"
      "ds_read_b64_tr_b16 %9, %32 offset:4096\n\t"
      "ds_read_b64_tr_b16 %10, %33\n\t"
      "ds_read_b64_tr_b16 %11, %33 offset:4096\n\t"
      "ds_read_b64_tr_b16 %12, %34\n\t"
      "ds_read_b64_tr_b16 %13, %34 offset:4096\n\t"
      "ds_read_b64_tr_b16 %14, %35\n\t"
      "ds_read_b64_tr_b16 %15, %35 offset:4096\n\t"
      "ds_read_b64_tr_b16 %16, %36\n\t"
      "ds_read_b64_tr_b16 %17, %36 offset:4096\n\t"
      "ds_read_b64_tr_b16 %18, %37\n\t"
      "ds_read_b64_tr_b16 %19, %37 offset:4096\n\t"
      "ds_read_b64_tr_b16 %20, %38\n\t"
      "ds_read_b64_tr_b16 %21, %38 offset:4096\n\t"
      "ds_read_b64_tr_b16 %22, %39\n\t"
      "ds_read_b64_tr_b16 %23, %39 offset:4096\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
        "=&v"(a[0]), "=&v"(b[0]), "=&v"(a[1]), "=&v"(b[1]), "=&v"(a[2]), "=&v"(b[2]), "=&v"(a[3]),
        "=&v"(b[3]), "=&v"(a[4]), "=&v"(b[4]), "=&v"(a[5]), "=&v"(b[5]), "=&v"(a[6]), "=&v"(b[6]),
        "=&v"(a[7]), "=&v"(b[7])
      : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(ka[4]), "v"(ka[5]), "v"(ka[6]), "v"(ka[7]),
        "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7])
      : "memory");
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) vf[dt] = cat8(a[dt], b[dt]);
}

// Eight 16-byte LDS reads issued together in one asm block that also waits
// for them (the builtin reads would get a wait after every pair).
__device__ __forceinline__ void lds_read8x16(const uint32_t (&addr)[8], uint4 (&r)[8]) {
  __asm__ volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %12\n\t"
      "ds_read_b128 %5, %13\n\t"
      "ds_read_b128 %6, %14\n\t"
      "ds_read_b128 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]),
        "v"(addr[7])
      : "memory");
}

// LDS slot of chunk c of tile row r.
__device__ __forceinline__ int k_slot(int c, int r) { return c ^ (r & 15); }
__device__ __forceinline__ int v_slot(int c, int r) { return c ^ (2 * (r & 7)); }

// Cache row of raw position p of the interleaved cache.
__device__ __forceinline__ int32_t raw_row(int32_t p, int32_t C, int32_t M) {
  const int32_t MC = M * C;
  return p < MC ? (p / C) * (C + 1) + p % C : M * (C + 1) + (p - MC);
}

// Exclusive prefix and total over the four lanes {i, i+16, i+32, i+48} that
// share a query (jg = lane / 16 orders them).
__device__ __forceinline__ int xi16(int v) { return (int)lane_xor<16>((uint32_t)v); }
__device__ __forceinline__ int xi32(int v) { return (int)lane_xor<32>((uint32_t)v); }
__device__ __forceinline__ float xf16(float v) { return __uint_as_float(lane_xor<16>(__float_as_uint(v))); }
__device__ __forceinline__ float xf32(float v) { return __uint_as_float(lane_xor<32>(__float_as_uint(v))); }
__device__ __forceinline__ int excl4(int c, int jg, int* total) {
  const int x1 = xi16(c);
  const int pair = c + x1;
  const int x2 = xi32(pair);
  *total = pair + x2;
  return ((jg & 1) ? x1 : 0) + ((jg & 2) ? x2 : 0);
}
__device__ __forceinline__ int sum4(int c) {
  c += xi16(c);
  return c + xi32(c);
}
__device__ __forceinline__ float max4(float v) {
  v = fmaxf(v, xf16(v));
  return fmaxf(v, xf32(v));
}
__device__ __forceinline__ float min4(float v) {
  v = fminf(v, xf16(v));
  return fminf(v, xf32(v));
}
__device__ __forceinline__ float fsum4(float v) {
  v += xf16(v);
  return v + xf32(v);
}

// Maximum of the 8 scores of two accumulators, with v_max3 (the compiler's
// fmaxf adds NaN-quieting instructions; the scores are never NaN).
__device__ __forceinline__ float max8(const f32x4& a, const f32x4& b) {
  float m;
  __asm__("v_max3_f32 %0, %1, %2, %3\n\t"
          "v_max3_f32 %0, %0, %4, %5\n\t"
          "v_max3_f32 %0, %0, %6, %7\n\t"
          "v_max_f32 %0, %0, %8"
          : "=&v"(m)
          : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]));
  return m;
}

// This thread's wave in the workgroup, known to the compiler as wave-uniform.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup -> (kv-head, query block). Consecutive linear ids share a kv-head
// (its K/V rows); with 8 XCDs taking workgroups round-robin, the linear id
// groups each XCD's workgroups together so one XCD's L2 serves one kv-head.
// Blocks go out last first: under the causal order a later block sees more
// gists, so the longest workgroups start first and the short ones fill in
// behind them (a CU that ends a long block early takes a short one).
// A batch of sequences of different lengths (gsa_prefill_varlen): sequence
// b's (n_raw, n_gist, q_start, n_q) at seqs[4 b ..], its workgroups the
// consecutive range [b wgs, (b + 1) wgs) of the grid, its q / K / V / out /
// selection rows `*_bs` elements after sequence b - 1's.
struct SeqBatch {
  const int32_t* seqs;    // [B][4] device array, or null (one sequence)
  int32_t wgs;            // workgroups per sequence
  int32_t n_max, m_max;   // the call's largest n_raw, n_gist (the slabs hold N + M rows)
  int64_t q_bs, kv_bs, out_bs, sel_bs;
};

// The sequence of this workgroup: its lengths replace the call's and the
// returned offsets move the base pointers to its rows. False for a sequence
// whose lengths break the rules (it gets no work) and for a query block past
// its queries. *x becomes the workgroup's index inside its sequence.
__device__ __forceinline__ bool seq_of(const SeqBatch& sb, int C, int q_ld, int* x, int* M, int* q_start, int* n_q,
                                       int64_t* b_out) {
  if (sb.seqs == nullptr) {
    *b_out = 0;
    return true;
  }
  const int b = *x / sb.wgs;
  *x -= b * sb.wgs;
  const int4 v = *reinterpret_cast<const int4*>(sb.seqs + 4 * b);
  const int64_t n = v.x, m = v.y, qs = v.z, nq = v.w;
  const bool ok = n >= 1 && n <= sb.n_max && m >= 0 && m <= sb.m_max && m * C <= n && n <= m * C + C &&
                  qs >= 0 && nq >= 0 && nq <= q_ld && qs + nq <= n;
  *M = (int)m;
  *q_start = (int)qs;
  *n_q = (int)nq;
  *b_out = b;
  return ok;
}

__device__ __forceinline__ void wg_coords(int x, int n_blocks, int Hkv, int* kvh, int* blk) {
  const int total = n_blocks * Hkv;
  if (total % 8 == 0) x = (x % 8) * (total / 8) + x / 8;
  *kvh = x / n_blocks;
  *blk = n_blocks - 1 - x % n_blocks;
}

// Query fragments (B operand of S^T = K Q^T) of heads h0..h0+H-1: lane holds
// q_h[query][32ks + 8jg .. +7].
template <int H>
__device__ __forceinline__ void load_qfrag(const char* qbase, int64_t n_q, int64_t t_idx, bool valid,
                                           int h0, int jg, bf16x8 (&qf)[H][4]) {
#pragma unroll
  for (int h = 0; h < H; ++h)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (valid) {
        const uint4 v = load16(qbase + (((int64_t)(h0 + h) * n_q + t_idx) * kD + 32 * ks + 8 * jg) * 2);
        qf[h][ks] = __builtin_bit_cast(bf16x8, v);
      } else {
        qf[h][ks] = __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
      }
    }
  // Settle the fragments here: a first use inside the tile loop would make the
  // compiler wait for every load in flight (the tile loads too) in each tile.
#pragma unroll
  for (int h = 0; h < H; ++h)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) __asm__ volatile("" : "+v"(qf[h][ks]));
}

// ------------------------------------------------------------ selection ----

constexpr int kSelThreads = 256;        // 4 waves, one 16-query tile each
constexpr int kSelWaves = 4;
constexpr int kSelTile = 32;            // gists per tile
constexpr int kSelSub = kSelTile / 16;  // 16-gist subtiles per tile
constexpr int kSelNB = 3;               // tiles in the LDS ring
constexpr int kSelTileBytes = kSelTile * kRowBytes;
constexpr int kSelPer = kSelTile / 4 / kSelWaves;   // direct loads per wave per tile (4 rows each)
constexpr int kLaneCand = kSelTile / 4;             // scores one lane sees per tile
// Entries of a lane's candidate list: 24 for k <= 32 (two workgroups per
// compute unit), 32 for k up to 64.
template <int K> struct SelCap {
  static constexpr int CAP = K <= 32 ? 24 : 32;
};

struct SelArgs {
  const void* q;          // [Hq][n_q][D] bf16
  const void* K;          // [Hkv][R][D] bf16
  int64_t R;
  int32_t M, C, k, Hkv, n_blocks, q_start, n_q;
  float score_mul;        // scale / g
  int32_t* sel_ws;        // [Hkv][q_ld][k]
  int32_t* sel_out;       // [Hkv][q_ld][k] or null
  int32_t q_ld;           // query rows per head in q and sel (n_q of one sequence)
  SeqBatch sb;            // a batch of sequences, or none
};

// Each lane keeps a list of CAP candidate entries of its query: entry e of
// lane tid is ent[e][tid] = (score bits, gist id).
template <int CAP_>
struct SelLds {
  static constexpr int CAP = CAP_;
  static_assert(CAP % 8 == 0, "lists are read in groups of 8 entries");
  char ring[kSelNB][kSelTileBytes];
  uint2 ent[CAP][kSelThreads];
  uint32_t full[2][kSelWaves];   // per tile parity: a wave's lists need a compaction
};
static_assert(sizeof(SelLds<24>) <= 80 * 1024, "two workgroups per CU");

// Score of an order key (inverse of order_key on canonical values).
__device__ __forceinline__ float key_score(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// The candidates of a query are the entries of the four lists of the lanes
// (qi, jg = 0..3) that share it. Compactions rewrite the lists with a subset
// of them that still holds the query's top-k, dealt round-robin over the
// four lists (kept entry p goes to list p % 4, slot p / 4). The last slot of
// every list is a spare that takes the writes of dropped entries.
constexpr int keep_max(int cap) { return 4 * (cap - 1 - kLaneCand); }   // entries a compaction may keep
constexpr int kPruneSlack = 8;          // a prune stops once at most k + this many remain
static_assert(32 + kPruneSlack <= keep_max(SelCap<32>::CAP) && kPrefillMaxK + kPruneSlack <= keep_max(SelCap<kPrefillMaxK>::CAP),
              "a prune can always keep k + slack entries");

template <int NE, class SL>
__device__ __forceinline__ void sel_load(const SL& L, int tid, float (&v)[NE], uint32_t (&id)[NE]) {
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const uint2 x = L.ent[e][tid];
    v[e] = __uint_as_float(x.x);
    id[e] = x.y;
  }
}

// Rewrite the lists with the entries marked `take`; returns this lane's new
// list length and the query's kept count in *tot.
template <int NE, class SL>
__device__ __forceinline__ int sel_deal(SL& L, int w, int lane, const float (&v)[NE],
                                        const uint32_t (&id)[NE], const bool (&take)[NE], int* tot) {
  const int qi = lane & 15, jg = lane >> 4;
  int ct = 0;
#pragma unroll
  for (int e = 0; e < NE; ++e) ct += take[e] ? 1 : 0;
  int p = excl4(ct, jg, tot);
  wave_lds_sync();   // every lane has read its list
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int jt = take[e] ? (p & 3) : jg;
    const int slot = take[e] ? (p >> 2) : SL::CAP - 1;
    L.ent[slot][64 * w + qi + 16 * jt] = make_uint2(__float_as_uint(v[e]), id[e]);
    p += take[e] ? 1 : 0;
  }
  wave_lds_sync();
  return (*tot + 3 - jg) >> 2;
}

// Exact top-k: the k-th best order key P by a bit-serial radix select over
// the four lists; entries above P are kept and, of those equal to P, the ones
// with the smallest ids (ties go to the smaller gist index). *tau becomes the
// k-th best score, or -inf while the query has fewer than k candidates.
// NE: list entries that may be in use (wave-uniform).
constexpr int kIdBits = 18;             // gist ids below 2^18
static_assert(kPrefillMaxGist <= (1 << kIdBits), "gist ids fit the bisection");
template <int NE, class SL>
__device__ __forceinline__ int sel_exact_n(SL& L, int w, int lane, int pos, int k, float* tau) {
  float v[NE];
  uint32_t id[NE], key[NE];
  sel_load<NE>(L, 64 * w + lane, v, id);
#pragma unroll
  for (int e = 0; e < NE; ++e) key[e] = e < pos ? order_key(v[e]) : 0u;
  uint32_t P = 0u;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = P | (1u << b);
    int n = 0;
#pragma unroll
    for (int e = 0; e < NE; ++e) n += key[e] >= c ? 1 : 0;
    n = sum4(n);
    P = n >= k ? c : P;
  }
  int gt = 0, ce = 0;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    gt += key[e] > P ? 1 : 0;
    ce += (key[e] == P && key[e] != 0u) ? 1 : 0;
  }
  gt = sum4(gt);
  const int ce_tot = sum4(ce);
  const int need = k - gt;        // entries equal to P that are kept (>= 1 when P > 0)
  uint32_t I = 0xffffffffu;       // of those, the ones with id <= I
  if (__ballot(ce_tot > need) != 0ull) {
    // need-th smallest id among the entries equal to P (ids are distinct)
    uint32_t lo = 0u;
    for (int b = kIdBits - 1; b >= 0; --b) {
      const uint32_t trial = lo + (1u << b);
      int n = 0;
#pragma unroll
      for (int e = 0; e < NE; ++e) n += (key[e] == P && key[e] != 0u && id[e] < trial) ? 1 : 0;
      n = sum4(n);
      lo = n < need ? trial : lo;
    }
    if (ce_tot > need) I = lo;
  }
  bool take[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) take[e] = key[e] > P || (key[e] == P && key[e] != 0u && id[e] <= I);
  int tot;
  const int n = sel_deal<NE>(L, w, lane, v, id, take, &tot);
  *tau = tot >= k ? key_score(P) : -INFINITY;
  return n;
}

// Prune: a bisection of the query's score range finds lo with at least k
// entries >= lo, and the entries below lo are dropped (k entries beat each of
// them). lo becomes *tau: a later gist scoring <= lo has k earlier entries at
// least as good. The bisection stops once at most k + kPruneSlack entries are
// >= lo. Returns -1 (lists untouched) if some query would keep more than
// keep_max(CAP) entries (scores tied over a wide range); an exact compaction
// follows then.
template <int NE, class SL>
__device__ __forceinline__ int sel_prune_n(SL& L, int w, int lane, int pos, int k, float* tau) {
  float v[NE];
  uint32_t id[NE];
  sel_load<NE>(L, 64 * w + lane, v, id);
  float mx = -INFINITY, mn = INFINITY;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    if (e >= pos) v[e] = -INFINITY;     // unused slots count nowhere
    mx = e < pos ? fmaxf(mx, v[e]) : mx;
    mn = e < pos ? fminf(mn, v[e]) : mn;
  }
  mx = max4(mx);
  mn = min4(mn);
  const int total = sum4(pos);
  const bool full = total >= k;
  float lo = mn, hi = mx;
  int n_lo = total;
  for (int s = 0; s < 16; ++s) {
    if (__ballot(full && n_lo > k + kPruneSlack) == 0ull) break;
    const float mid = 0.5f * lo + 0.5f * hi;
    int n = 0;
#pragma unroll
    for (int e = 0; e < NE; ++e) n += v[e] >= mid ? 1 : 0;
    n = sum4(n);
    if (n >= k) {
      lo = mid;
      n_lo = n;
    } else {
      hi = mid;
    }
  }
  if (__ballot(n_lo > keep_max(SL::CAP)) != 0ull) return -1;
  bool take[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) take[e] = e < pos && (!full || v[e] >= lo);
  int tot;
  const int n = sel_deal<NE>(L, w, lane, v, id, take, &tot);
  if (full) *tau = lo;
  return n;
}

// Entries per list in use, rounded up to groups of 8 (wave-uniform).
template <int CAP>
__device__ __forceinline__ int list_groups(int pos) {
  if constexpr (CAP > 24)
    if (__ballot(pos > 24)) return 4;
  return __ballot(pos > 16) ? 3 : __ballot(pos > 8) ? 2 : 1;
}

template <class SL>
__device__ __forceinline__ int sel_exact(SL& L, int w, int lane, int pos, int k, float* tau) {
  static_assert(SL::CAP == 24 || SL::CAP == 32, "three or four groups");
  const int grp = list_groups<SL::CAP>(pos);
  if (grp == 1) return sel_exact_n<8>(L, w, lane, pos, k, tau);
  if (grp == 2) return sel_exact_n<16>(L, w, lane, pos, k, tau);
  if (SL::CAP == 24 || grp == 3) return sel_exact_n<24>(L, w, lane, pos, k, tau);
  return sel_exact_n<SL::CAP == 24 ? 24 : 32>(L, w, lane, pos, k, tau);
}

// Make room in the lists: prune, or compact exactly if a prune cannot.
template <class SL>
__device__ __forceinline__ int sel_compact(SL& L, int w, int lane, int pos, int k, float* tau) {
  int n;
  const int grp = list_groups<SL::CAP>(pos);
  if (grp == 1) n = sel_prune_n<8>(L, w, lane, pos, k, tau);
  else if (grp == 2) n = sel_prune_n<16>(L, w, lane, pos, k, tau);
  else if (SL::CAP == 24 || grp == 3) n = sel_prune_n<24>(L, w, lane, pos, k, tau);
  else n = sel_prune_n<SL::CAP == 24 ? 24 : 32>(L, w, lane, pos, k, tau);
  return n >= 0 ? n : sel_exact(L, w, lane, pos, k, tau);
}

// Direct loads of gist tile `it` (rows m = kSelTile it + r; rows past E read
// gist 0, whose scores the eligibility mask drops).
__device__ __forceinline__ void sel_issue(char* buf, const char* Kh, int it, int E, int C) {
  const int lane = threadIdx.x & 63, w = wave_id();
#pragma unroll
  for (int u = 0; u < kSelPer; ++u) {
    const int rb = 4 * (w + kSelWaves * u);
    const int r = rb + (lane >> 4);
    const int m = it * kSelTile + r;
    const int64_t row = m < E ? (int64_t)m * (C + 1) + C : C;
    dma16(Kh + row * kRowBytes + k_slot(lane & 15, r) * 16, buf + rb * kRowBytes);
  }
}

// The query summed over its group's heads, qbar = sum_h q_h (fp32, exact for
// bf16 heads of similar magnitude), as two bf16 parts hi + lo: the group
// score (scale/g) sum_h q_h . k = (scale/g) qbar . k then takes two MFMA
// chains instead of one per head, with qbar kept to about 16 bits (all of it
// for g = 1, where lo is zero).
template <int G>
__device__ __forceinline__ void load_qbar(const char* qbase, int64_t n_q, int64_t t_idx, bool valid, int jg,
                                          bf16x8 (&qh)[4], bf16x8 (&ql)[4]) {
  bf16x8 qf[G][4];
  load_qfrag<G>(qbase, n_q, t_idx, valid, 0, jg, qf);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float s = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) s += (float)qf[h][ks][e];
      const __bf16 hi = (__bf16)s;
      qh[ks][e] = hi;
      ql[ks][e] = (__bf16)(s - (float)hi);
    }
}

// Append the candidates of one 16-gist subtile (score[r]: gist m0 + r) that
// beat tau. Every score is written at the list's end, and the end advances
// past the ones that beat tau: no branch per score.
template <bool MASK, class SL>
__device__ __forceinline__ void sel_append(SL& L, int tid, const float (&score)[4], int m0, int elig,
                                           float tau, int* pos) {
  float v[4];
  bool ok[4];
  bool any = false;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    v[r] = MASK && m0 + r >= elig ? -INFINITY : score[r];
    ok[r] = v[r] > tau;
    any |= ok[r];
  }
  if (__ballot(any) == 0ull) return;
  int p = *pos;
  const uint32_t base = lds_addr(reinterpret_cast<const char*>(&L.ent[0][tid]));
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    // written as asm: the compiler would otherwise wait for every direct-to-
    // LDS load in flight (the K tiles ahead) before a list write
    const uint2 x = make_uint2(__float_as_uint(v[r]), (uint32_t)(m0 + r));
    __asm__ volatile("ds_write_b64 %0, %1" ::"v"(base + (uint32_t)p * (kSelThreads * 8)), "v"(x) : "memory");
    p += ok[r] ? 1 : 0;
  }
  *pos = p;
}

// KMAX: the largest k the launch takes (32: lists of 24 entries, two
// workgroups per compute unit; 64: lists of 32).
template <int G, int KMAX>
__global__ __launch_bounds__(kSelThreads, KMAX <= 32 ? 2 : 1) void prefill_select(SelArgs a) {
  __shared__ __attribute__((aligned(16))) SelLds<SelCap<KMAX>::CAP> L;
  constexpr int kCap = SelCap<KMAX>::CAP;
  int kvh, blk, wx = (int)blockIdx.x;
  int64_t sq;
  if (!seq_of(a.sb, a.C, a.q_ld, &wx, &a.M, &a.q_start, &a.n_q, &sq)) return;
  wg_coords(wx, a.n_blocks, a.Hkv, &kvh, &blk);
  if (blk * kQB >= a.n_q) return;   // past this sequence's queries (uniform)
  if (sq > 0) {
    a.q = reinterpret_cast<const char*>(a.q) + sq * a.sb.q_bs * 2;
    a.K = reinterpret_cast<const char*>(a.K) + sq * a.sb.kv_bs * 2;
    a.sel_ws += sq * a.sb.sel_bs;
    if (a.sel_out) a.sel_out += sq * a.sb.sel_bs;
  }
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int qi = lane & 15, jg = lane >> 4;
  const int qloc = 16 * w + qi;
  const int t_idx = blk * kQB + qloc;
  const bool valid = t_idx < a.n_q;
  const int t = a.q_start + t_idx;
  const int elig = valid ? min(a.M, t / a.C) : 0;
  const int t_last = a.q_start + min(a.n_q, (blk + 1) * kQB) - 1;
  const int E = min(a.M, t_last / a.C);     // gists any query of the block may use
  // gists every valid query of this wave may use (its first query's)
  const int e_lo = min(a.M, (a.q_start + blk * kQB + 16 * w) / a.C);

  bf16x8 qh[4], ql[4];
  load_qbar<G>(reinterpret_cast<const char*>(a.q) + (int64_t)kvh * G * a.q_ld * kRowBytes, a.q_ld, t_idx, valid,
               jg, qh, ql);
  const char* Kh = reinterpret_cast<const char*>(a.K) + (int64_t)kvh * a.R * kRowBytes;

  int pos = 0;
  float tau = valid ? -INFINITY : INFINITY;   // a query past n_q takes nothing
  const int n_tiles = (E + kSelTile - 1) / kSelTile;
  // this lane's operand offsets inside a tile: row 16s + qi, chunk 4ks + jg
  int koff[kSelSub][4];
#pragma unroll
  for (int s = 0; s < kSelSub; ++s)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) koff[s][ks] = (16 * s + qi) * kRowBytes + k_slot(4 * ks + jg, qi) * 16;

  for (int it = 0; it < kSelNB - 1 && it < n_tiles; ++it) sel_issue(L.ring[it], Kh, it, E, a.C);
  for (int it = 0; it < n_tiles; ++it) {
    // this wave's loads of tile `it` are done once at most (tiles issued
    // after it) x kSelPer loads are outstanding
    const int ahead = min(kSelNB - 2, n_tiles - 1 - it);
    if (ahead >= 2) wait_vm<2 * kSelPer>();
    else if (ahead == 1) wait_vm<kSelPer>();
    else wait_vm<0>();
    tile_barrier();    // every wave's loads of tile it landed; tile it-1's buffer is free
    if (it > 0) {
      // every wave compacts when one needs to: one wave alone would hold the
      // others at the next barrier
      const uint32_t* f = L.full[(it - 1) & 1];
      if (__builtin_amdgcn_readfirstlane(f[0] | f[1] | f[2] | f[3]) != 0u) {
        wave_lds_sync();
        pos = sel_compact(L, w, lane, pos, a.k, &tau);
      }
    }
    if (it + kSelNB - 1 < n_tiles) sel_issue(L.ring[(it + kSelNB - 1) % kSelNB], Kh, it + kSelNB - 1, E, a.C);
    const char* kt = L.ring[it % kSelNB];
    // per subtile two independent chains: qbar's hi and lo parts
    f32x4 acc[kSelSub][2];
#pragma unroll
    for (int s = 0; s < kSelSub; ++s) acc[s][0] = acc[s][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // every K operand read of the tile in one asm block: one LDS round trip,
    // not four (the compiler would wait after each pair)
    static_assert(kSelSub == 2, "eight operand reads per tile");
    bf16x8 kf[4][kSelSub];
    {
      const uint32_t kb = lds_addr(kt);
      uint32_t ad[8];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int sb = 0; sb < kSelSub; ++sb) ad[2 * ks + sb] = kb + koff[sb][ks];
      uint4 r[8];
      lds_read8x16(ad, r);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int s = 0; s < kSelSub; ++s) kf[ks][s] = __builtin_bit_cast(bf16x8, r[2 * ks + s]);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int s = 0; s < kSelSub; ++s) {
        acc[s][0] = mfma(kf[ks][s], qh[ks], acc[s][0]);
        if (G > 1) acc[s][1] = mfma(kf[ks][s], ql[ks], acc[s][1]);   // g = 1: lo is zero
      }
    }
    // score of gist kSelTile it + 16 s + 4 jg + r against query qi
    const int m0 = it * kSelTile + 4 * jg;
    const bool masked = (it + 1) * kSelTile > e_lo;
#pragma unroll
    for (int s = 0; s < kSelSub; ++s) {
      float sc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = (acc[s][0][r] + acc[s][1][r]) * a.score_mul;
      if (masked) sel_append<true>(L, tid, sc, m0 + 16 * s, elig, tau, &pos);
      else sel_append<false>(L, tid, sc, m0 + 16 * s, elig, tau, &pos);
    }
    const bool full = __ballot(pos > kCap - 1 - kLaneCand) != 0ull;
    if (lane == 0) L.full[it & 1][w] = full ? 1u : 0u;
  }
  wave_lds_sync();
  pos = sel_compact(L, w, lane, pos, a.k, &tau);
  pos = sel_exact(L, w, lane, pos, a.k, &tau);
  // the query's kept entries in ascending id order: each lane ranks its own
  // entries among all of the query's (at most k, dealt round-robin)
  const int tot = sum4(pos);
  uint32_t ids[KMAX];
#pragma unroll
  for (int p = 0; p < KMAX; ++p)
    ids[p] = p < tot ? L.ent[p >> 2][64 * w + qi + 16 * (p & 3)].y : 0xffffffffu;
  if (valid) {
    const int64_t o = ((int64_t)kvh * a.q_ld + t_idx) * a.k;
#pragma unroll
    for (int e = 0; e < (KMAX + 3) / 4; ++e) {
      if (e < pos) {
        const uint32_t mine = ids[4 * e + jg];
        int rank = 0;
#pragma unroll
        for (int p = 0; p < KMAX; ++p) rank += ids[p] < mine ? 1 : 0;
        a.sel_ws[o + rank] = (int32_t)mine;
        if (a.sel_out) a.sel_out[o + rank] = (int32_t)mine;
      }
      const int i = tot + 4 * e + jg;   // slots past the kept entries
      if (i < a.k) {
        a.sel_ws[o + i] = -1;
        if (a.sel_out) a.sel_out[o + i] = -1;
      }
    }
  }
}

// ------------------------------------------------------------ attention ----

constexpr int kMaxChunkWords = kPrefillMaxGist / 32;   // bitmap of selectable chunks
constexpr int kMaxUnion = kQB * kPrefillMaxK;           // distinct chunks a block can select
constexpr int kAttTile = 32;            // rows per ring tile (the K of the P.V MFMA)
constexpr int kAttSub = 32;             // rows per MFMA subtile
constexpr int kAttGroups = kAttTile / 4;                 // 4-row load groups of the K (or V) rows
constexpr int kAttNB = 4;               // tiles in the LDS ring
constexpr int kHalfTile = kAttTile * kRowBytes;          // K or V part of a tile (8 KB)

// Waves per 16-query tile and heads per wave.
template <int G> struct AttShape {
  static constexpr int WPQ = G == 4 ? 2 : 1;
  static constexpr int HPW = G / WPQ;
  static constexpr int NW = 4 * WPQ;          // waves per workgroup
  static constexpr int NT = 64 * NW;          // threads per workgroup
  static constexpr int PER = 2 * kAttGroups / NW;   // direct loads (4 rows each) per wave per tile
};

struct AttArgs {
  const void* q;
  const void* K;
  const void* V;
  float* out;             // [Hq][n_q][D] fp32
  const int32_t* sel;     // [Hkv][n_q][k]
  int64_t R;
  int32_t M, C, k, W, Hkv, n_blocks, q_start, n_q;
  int32_t q_stride;       // query i sits at position q_start + i * q_stride
  int32_t q_ld;           // query rows per head in q, out and sel
  SeqBatch sb;            // a batch of sequences, or none
  float scale_log2;
  // query heads per kv-head = kv_div * G: each kv-head's heads go to kv_div
  // workgroups of G heads each (head group v = kv-head v / kv_div)
  int32_t kv_div;
};

struct AttLds {
  char ring[kAttNB][2 * kHalfTile];   // [tile][K rows | V rows]
  uint32_t bitmap[kMaxChunkWords];
  int32_t U[kMaxUnion];
  uint32_t qm[kMaxUnion][2];
  int scan[8];
  int nU;
};

// What a tile row is: a gist, a raw row of a selected chunk, a window row.
enum { kGist = 0, kChunk = 1, kWin = 2 };

// Cache row of phase item i (a valid row for items past n: their scores are masked).
template <int KIND>
__device__ __forceinline__ int64_t phase_row(const AttLds& L, int i, int n, int lo, int C, int M) {
  if (i >= n) return 0;
  if (KIND == kGist) return (int64_t)i * (C + 1) + C;
  if (KIND == kChunk) return (int64_t)L.U[i / C] * (C + 1) + i % C;
  return raw_row(lo + i, C, M);
}

template <int NW, int KIND>
__device__ __forceinline__ void att_issue(char* buf, const char* Kh, const char* Vh, const AttLds& L,
                                          int i0, int n, int lo, int C, int M) {
  const int lane = threadIdx.x & 63, w = wave_id();
  if (KIND == kGist && i0 + kAttTile <= n) {
    // gist rows i0 + r sit (C+1) rows apart: a wave-uniform base for the
    // tile and a per-lane 32-bit offset
    const int64_t step = (int64_t)i0 * (C + 1) * kRowBytes;
    const char* kb = Kh + step;
    const char* vb = Vh + step;
#pragma unroll
    for (int u = 0; u < 2 * kAttGroups / NW; ++u) {
      const int j = w + NW * u;
      const int rb = 4 * (j % kAttGroups);
      const int r = rb + (lane >> 4);
      const uint32_t roff = (uint32_t)(r * (C + 1) + C) * kRowBytes;
      if (j < kAttGroups)
        dma16(kb + (roff + k_slot(lane & 15, r) * 16), buf + rb * kRowBytes);
      else
        dma16(vb + (roff + v_slot(lane & 15, r) * 16), buf + kHalfTile + rb * kRowBytes);
    }
    return;
  }
#pragma unroll
  for (int u = 0; u < 2 * kAttGroups / NW; ++u) {
    const int j = w + NW * u;                 // wave-uniform: K rows for j < kAttGroups, V rows after
    const int rb = 4 * (j % kAttGroups);
    const int r = rb + (lane >> 4);
    const int64_t row = phase_row<KIND>(L, i0 + r, n, lo, C, M);
    if (j < kAttGroups)
      dma16(Kh + row * kRowBytes + k_slot(lane & 15, r) * 16, buf + rb * kRowBytes);
    else
      dma16(Vh + row * kRowBytes + v_slot(lane & 15, r) * 16, buf + kHalfTile + rb * kRowBytes);
  }
}

template <int H>
struct AttState {
  f32x4 o[H][8];      // O^T[16dt + 4jg + r][query qi] of head h
  float m[H], l[H];   // running max (log2 units) and this lane's share of the sum
};

struct AttCtx {
  int qloc, t, elig, W, C, lo;
  bool valid;
  float c;            // scale * log2(e)
};

// May the lane's query use phase row i?
template <int KIND>
__device__ __forceinline__ bool row_ok(const AttLds& L, const AttCtx& x, int i, int n) {
  if (!x.valid || i >= n) return false;
  if (KIND == kGist) return i < x.elig;
  if (KIND == kChunk) {
    const int u = i / x.C;
    if (!((L.qm[u][x.qloc >> 5] >> (x.qloc & 31)) & 1u)) return false;
    return L.U[u] * x.C + i % x.C < x.t - x.W + 1;   // the window attends that row
  }
  const int pos = x.lo + i;
  return pos >= x.t - x.W + 1 && pos <= x.t;
}

template <int H, int KIND>
__device__ __forceinline__ void att_tile(const char* kt, const char* vt, const AttLds& L, const AttCtx& x,
                                         int i0, int n, bool masked, const bf16x8 (&qf)[H][4],
                                         AttState<H>& st) {
  const int lane = threadIdx.x & 63, qi = lane & 15, jg = lane >> 4;
  f32x4 s[2][H];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int h = 0; h < H; ++h) s[sb][h] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the tile's eight K operand reads and its V^T operand reads in one round
  // trip, then 2 H independent MFMA chains, interleaved so that no product
  // waits on the one just issued
  bf16x8 kf[4][2];
  bf16x8 vf[8];
  {
    uint32_t ad[8];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
        ad[2 * ks + sb] = lds_addr(kt) + (16 * sb + qi) * kRowBytes + k_slot(4 * ks + jg, qi) * 16;
    // V^T: lane (s16, jg) reads 4 columns of row 4 jg + s16 / 4
    const int s16 = lane & 15;
    const int R = 4 * jg + (s16 >> 2);
    const uint32_t vrow = lds_addr(vt) + R * kRowBytes + 8 * (s16 & 1);
    uint32_t va[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) va[dt] = vrow + v_slot(2 * dt + ((s16 & 3) >> 1), R) * 16;
    uint4 r[8];
    lds_kv_tile(ad, va, r, vf);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) kf[ks][sb] = __builtin_bit_cast(bf16x8, r[2 * ks + sb]);
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int h = 0; h < H; ++h) s[sb][h] = mfma(kf[ks][sb], qf[h][ks], s[sb][h]);
  // s[sb][h][r]: row i0 + 16sb + 4jg + r against the lane's query, head h
  if (masked) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = row_ok<KIND>(L, x, i0 + 16 * sb + 4 * jg + r, n);
#pragma unroll
        for (int h = 0; h < H; ++h) s[sb][h][r] = ok ? s[sb][h][r] : -INFINITY;
      }
  }
  bf16x8 phi[H], plo[H];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const float mx = max8(s[0][h], s[1][h]);
    const float cand = mx * x.c;
    if (__ballot(cand > st.m[h] + kPLazy) != 0ull) {
      // raise the row's max (the same on the row's four lanes) and rescale
      const float c4 = max4(cand);
      const float mn = c4 > st.m[h] + kPLazy ? c4 : st.m[h];
      const float al = fexp2(st.m[h] - mn);
      st.m[h] = mn;
      st.l[h] *= al;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) st.o[h][dt][r] *= al;
    }
    const float nm = -st.m[h];
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = fexp2(fmaf(s[e >> 2][h][e & 3], x.c, nm));
    float ps = p[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) ps += p[e];
    st.l[h] += ps;
    // p = hi + lo: hi is p truncated to bf16 (its top 16 bits), lo = p - hi
    // (exact in fp32, below 2^-7 p) rounded to bf16
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 hp;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const uint32_t b0 = __float_as_uint(p[e]), b1 = __float_as_uint(p[e + 1]);
      hp[e >> 1] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
      plo[h][e] = (__bf16)(p[e] - __uint_as_float(b0 & 0xffff0000u));
      plo[h][e + 1] = (__bf16)(p[e + 1] - __uint_as_float(b1 & 0xffff0000u));
    }
    phi[h] = __builtin_bit_cast(bf16x8, hp);
  }
  // O^T += V^T P^T (the V^T operand came transposed out of LDS above):
  // every hi product, then every lo product: 8 H independent accumulators
  // between the two products of one
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int h = 0; h < H; ++h) st.o[h][dt] = mfma(vf[dt], phi[h], st.o[h][dt]);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int h = 0; h < H; ++h) st.o[h][dt] = mfma(vf[dt], plo[h], st.o[h][dt]);
}

// One phase: rows [0, n) of kind KIND, kAttTile rows per tile, kAttNB tiles
// in the LDS ring. `all_ok` = items [0, all_ok) need no mask for any query.
template <int G, int KIND>
__device__ __forceinline__ void att_phase(AttLds& L, const char* Kh, const char* Vh, const AttCtx& x, int n,
                                          int all_ok, int M, const bf16x8 (&qf)[AttShape<G>::HPW][4],
                                          AttState<AttShape<G>::HPW>& st) {
  constexpr int NW = AttShape<G>::NW, PER = AttShape<G>::PER, H = AttShape<G>::HPW;
  const int nt = (n + kAttTile - 1) / kAttTile;
  if (nt == 0) return;
  __syncthreads();   // the ring is free (the previous phase's last tile was read)
  for (int t = 0; t < kAttNB - 1 && t < nt; ++t)
    att_issue<NW, KIND>(L.ring[t], Kh, Vh, L, t * kAttTile, n, x.lo, x.C, M);
  for (int t = 0; t < nt; ++t) {
    const int ahead = min(kAttNB - 2, nt - 1 - t);   // tiles issued after tile t
    static_assert(kAttNB <= 4, "at most two tiles ahead");
    if (ahead >= 2) wait_vm<2 * PER>();
    else if (ahead == 1) wait_vm<PER>();
    else wait_vm<0>();
    tile_barrier();    // every wave's loads of tile t landed; tile t-1's buffer is free
    if (t + kAttNB - 1 < nt)
      att_issue<NW, KIND>(L.ring[(t + kAttNB - 1) % kAttNB], Kh, Vh, L, (t + kAttNB - 1) * kAttTile, n, x.lo,
                          x.C, M);
    const char* buf = L.ring[t % kAttNB];
    static_assert(kAttTile == kAttSub, "one MFMA subtile per ring tile");
    const bool masked = KIND != kGist || (t + 1) * kAttTile > all_ok;
    att_tile<H, KIND>(buf, buf + kHalfTile, L, x, t * kAttTile, n, masked, qf, st);
  }
}

template <int G>
__global__ __launch_bounds__(AttShape<G>::NT) void prefill_attend(AttArgs a) {
  using S = AttShape<G>;
  constexpr int H = S::HPW, NT = S::NT;
  __shared__ __attribute__((aligned(16))) AttLds L;
  int hg, blk, wx = (int)blockIdx.x;
  int64_t sq;
  if (!seq_of(a.sb, a.C, a.q_ld, &wx, &a.M, &a.q_start, &a.n_q, &sq)) return;
  wg_coords(wx, a.n_blocks, a.Hkv * a.kv_div, &hg, &blk);
  if (blk * kQB >= a.n_q) return;   // past this sequence's queries (uniform)
  if (sq > 0) {
    a.q = reinterpret_cast<const char*>(a.q) + sq * a.sb.q_bs * 2;
    a.K = reinterpret_cast<const char*>(a.K) + sq * a.sb.kv_bs * 2;
    a.V = reinterpret_cast<const char*>(a.V) + sq * a.sb.kv_bs * 2;
    a.out += sq * a.sb.out_bs;
    a.sel += sq * a.sb.sel_bs;
  }
  const int kvh = hg / a.kv_div;        // the kv-head of head group hg (G query heads)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int qi = lane & 15, jg = lane >> 4;
  const int qt = w % 4;                 // 16-query tile of this wave
  const int h0 = (w / 4) * H;           // first head of this wave
  const int qloc = 16 * qt + qi;
  const int t_idx = blk * kQB + qloc;
  const bool valid = t_idx < a.n_q;
  const int t = a.q_start + t_idx * a.q_stride;
  const int nq_blk = min(kQB, a.n_q - blk * kQB);
  const int t_first = a.q_start + blk * kQB * a.q_stride;
  const int t_last = t_first + (nq_blk - 1) * a.q_stride;
  const int E = min(a.M, t_last / a.C);
  const int E0 = min(a.M, t_first / a.C);   // gists every query of the block may use

  // union of the block's selected chunks (ascending) and, per chunk, the
  // mask of the queries that selected it
  const int nwords = (E + 31) / 32;
  for (int i = tid; i < nwords; i += NT) L.bitmap[i] = 0u;
  __syncthreads();
  const int32_t* sb = a.sel + ((int64_t)kvh * a.q_ld + (int64_t)blk * kQB) * a.k;
  for (int pr = tid; pr < nq_blk * a.k; pr += NT) {
    const int m = sb[pr];
    if (m >= 0 && m < E) atomicOr(&L.bitmap[m >> 5], 1u << (m & 31));
  }
  __syncthreads();
  {
    constexpr int kPer = kMaxChunkWords / NT;
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
    if (tid == NT - 1) L.nU = run;
  }
  __syncthreads();
  const int nU = L.nU;
  for (int i = tid; i < nU; i += NT) {
    L.qm[i][0] = 0u;
    L.qm[i][1] = 0u;
  }
  __syncthreads();
  for (int pr = tid; pr < nq_blk * a.k; pr += NT) {
    const int m = sb[pr];
    if (m >= 0 && m < E) {
      // m's place in the ascending union (it is there): a binary search
      int lo = 0, hi = nU;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (L.U[mid] <= m) lo = mid;
        else hi = mid;
      }
      const int u = lo;
      const int ql = pr / a.k;
      atomicOr(&L.qm[u][ql >> 5], 1u << (ql & 31));
    }
  }
  __syncthreads();

  bf16x8 qf[H][4];
  load_qfrag<H>(reinterpret_cast<const char*>(a.q) + (int64_t)hg * G * a.q_ld * kRowBytes, a.q_ld, t_idx,
                valid, h0, jg, qf);
  const char* Kh = reinterpret_cast<const char*>(a.K) + (int64_t)kvh * a.R * kRowBytes;
  const char* Vh = reinterpret_cast<const char*>(a.V) + (int64_t)kvh * a.R * kRowBytes;
  AttState<H> st;
#pragma unroll
  for (int h = 0; h < H; ++h) {
    st.m[h] = kMinus;
    st.l[h] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[h][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  AttCtx x;
  x.qloc = qloc;
  x.t = t;
  x.elig = valid ? min(a.M, t / a.C) : 0;
  x.W = a.W;
  x.C = a.C;
  x.lo = max(0, t_first - a.W + 1);
  x.valid = valid;
  x.c = a.scale_log2;
  // rows every query of the block may use without a mask: the first E0 gists,
  // unless some query of the block is past n_q (then everything is masked)
  const int all_ok = nq_blk == kQB ? E0 : 0;
  att_phase<G, kGist>(L, Kh, Vh, x, E, all_ok, a.M, qf, st);
  att_phase<G, kChunk>(L, Kh, Vh, x, nU * a.C, 0, a.M, qf, st);
  att_phase<G, kWin>(L, Kh, Vh, x, t_last - x.lo + 1, 0, a.M, qf, st);

  if (!valid) return;
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const float inv = 1.f / fsum4(st.l[h]);
    float* o = a.out + (((int64_t)hg * G + h0 + h) * a.q_ld + t_idx) * kD;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const float4 v = make_float4(st.o[h][dt][0] * inv, st.o[h][dt][1] * inv, st.o[h][dt][2] * inv,
                                   st.o[h][dt][3] * inv);
      *reinterpret_cast<float4*>(o + 16 * dt + 4 * jg) = v;
    }
  }
}

// G query heads per kv-head; the attention launch takes them in groups of AG
// (g = 8: two workgroups of four heads per kv-head and query block, each
// reading the kv-head's tiles).
template <int G>
gsa_status_t run_prefill(const PrefillPlan& pl, const void* q, const void* K, const void* V, float* out,
                         int32_t* sel, char* ws, hipStream_t stream) {
  constexpr int AG = G == 8 ? 4 : G;
  prof_begin_call();
  if (pl.n_q == 0) return GSA_OK;
  int32_t* wsel = reinterpret_cast<int32_t*>(ws);
  const int grid = pl.n_blocks * pl.Hkv;   // per sequence
  // a batch of sequences: each one's rows lie these many elements apart
  SeqBatch sb{};
  sb.seqs = pl.seqs;
  sb.n_max = (int32_t)pl.N;
  sb.m_max = (int32_t)pl.M;
  sb.q_bs = (int64_t)pl.Hq * pl.n_q * kD;
  sb.kv_bs = (int64_t)pl.Hkv * pl.R * kD;
  sb.out_bs = (int64_t)pl.Hq * pl.n_q * kD;
  sb.sel_bs = (int64_t)pl.Hkv * pl.n_q * pl.k;
  if (pl.k > 0) {
    SelArgs s{};
    s.q = q; s.K = K; s.R = pl.R;
    s.M = (int32_t)pl.M; s.C = pl.C; s.k = pl.k; s.Hkv = pl.Hkv; s.n_blocks = pl.n_blocks;
    s.q_start = (int32_t)pl.q_start; s.n_q = (int32_t)pl.n_q;
    s.score_mul = pl.scale / G;
    s.sel_ws = wsel; s.sel_out = sel;
    s.q_ld = (int32_t)pl.n_q;
    s.sb = sb;
    s.sb.wgs = grid;
    if (pl.k <= 32)
      prof_launch((prefill_select<G, 32>), dim3(grid * pl.B), dim3(kSelThreads), 0, stream, s);
    else
      prof_launch((prefill_select<G, 64>), dim3(grid * pl.B), dim3(kSelThreads), 0, stream, s);
  }
  AttArgs t{};
  t.q = q; t.K = K; t.V = V; t.out = out; t.sel = wsel; t.R = pl.R;
  t.M = (int32_t)pl.M; t.C = pl.C; t.k = pl.k; t.W = pl.W; t.Hkv = pl.Hkv; t.n_blocks = pl.n_blocks;
  t.q_start = (int32_t)pl.q_start; t.n_q = (int32_t)pl.n_q; t.q_stride = pl.q_stride;
  t.scale_log2 = pl.scale * kLog2e;
  t.kv_div = G / AG;
  t.q_ld = (int32_t)pl.n_q;
  t.sb = sb;
  t.sb.wgs = grid * (G / AG);
  prof_launch((prefill_attend<AG>), dim3(grid * (G / AG) * pl.B), dim3(AttShape<AG>::NT), 0, stream, t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(GSA_ERR_HIP, "%s launch: %s", pl.q_stride == 1 ? "gsa_prefill_blocksparse" : "gsa_gist_prefill",
                hipGetErrorString(e));
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
  prof_begin_call();
  PrefillPlan pl;
  gsa_status_t s = plan_prefill(p, &pl);
  if (s != GSA_OK) return s;
  const bool none = pl.n_q == 0;   // no queries: q, out (and sel) may be NULL
  if ((s = check_ptr(q, "q", none)) != GSA_OK || (s = check_ptr(k_cache, "k_cache")) != GSA_OK ||
      (s = check_ptr(v_cache, "v_cache")) != GSA_OK || (s = check_ptr(out, "out", none)) != GSA_OK ||
      (s = check_ptr(sel, "sel", true)) != GSA_OK)
    return s;
  if ((s = check_workspace(workspace, workspace_bytes, pl.total)) != GSA_OK) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  switch (pl.g) {
    case 1: return run_prefill<1>(pl, q, k_cache, v_cache, out, sel, ws, st);
    case 2: return run_prefill<2>(pl, q, k_cache, v_cache, out, sel, ws, st);
    case 4: return run_prefill<4>(pl, q, k_cache, v_cache, out, sel, ws, st);
    case 8: return run_prefill<8>(pl, q, k_cache, v_cache, out, sel, ws, st);
  }
  return fail(GSA_ERR_UNSUPPORTED, "prefill: %d query heads per kv-head not in {1, 2, 4}", pl.g);
}

extern "C" gsa_status_t gsa_prefill_varlen_workspace_size(const gsa_prefill_varlen_params* p, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(GSA_ERR_INVALID_ARG, "bytes is NULL");
  PrefillPlan pl;
  gsa_status_t s = plan_prefill_varlen(p, &pl);
  if (s != GSA_OK) return s;
  *bytes = pl.total;
  return GSA_OK;
}

extern "C" gsa_status_t gsa_prefill_varlen(const gsa_prefill_varlen_params* p, const int32_t* seqs,
                                           const void* q, const void* k_cache, const void* v_cache, float* out,
                                           int32_t* sel, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  prof_begin_call();
  PrefillPlan pl;
  gsa_status_t s = plan_prefill_varlen(p, &pl);
  if (s != GSA_OK) return s;
  const bool none = pl.n_q == 0;   // no queries: q, out (and sel) may be NULL
  if ((s = check_ptr(seqs, "seqs")) != GSA_OK || (s = check_ptr(q, "q", none)) != GSA_OK ||
      (s = check_ptr(k_cache, "k_cache")) != GSA_OK || (s = check_ptr(v_cache, "v_cache")) != GSA_OK ||
      (s = check_ptr(out, "out", none)) != GSA_OK || (s = check_ptr(sel, "sel", true)) != GSA_OK)
    return s;
  if ((s = check_workspace(workspace, workspace_bytes, pl.total)) != GSA_OK) return s;
  pl.seqs = seqs;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  switch (pl.g) {
    case 1: return run_prefill<1>(pl, q, k_cache, v_cache, out, sel, ws, st);
    case 2: return run_prefill<2>(pl, q, k_cache, v_cache, out, sel, ws, st);
    case 4: return run_prefill<4>(pl, q, k_cache, v_cache, out, sel, ws, st);
    case 8: return run_prefill<8>(pl, q, k_cache, v_cache, out, sel, ws, st);
  }
  return fail(GSA_ERR_UNSUPPORTED, "prefill: %d query heads per kv-head not in {1, 2, 4, 8}", pl.g);
}

extern "C" gsa_status_t gsa_gist_prefill(const gsa_gist_params* p, const void* q, const void* k_cache,
                                         const void* v_cache, float* out, void* stream) {
  clear_error();
  prof_begin_call();
  PrefillPlan pl;
  gsa_status_t s = plan_gist(p, &pl);
  if (s != GSA_OK) return s;
  const bool none = pl.n_q == 0;   // no queries: q and out may be NULL
  if ((s = check_ptr(q, "q", none)) != GSA_OK || (s = check_ptr(k_cache, "k_cache")) != GSA_OK ||
      (s = check_ptr(v_cache, "v_cache")) != GSA_OK || (s = check_ptr(out, "out", none)) != GSA_OK)
    return s;
  // k = 0: no selection launch, no workspace
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  switch (pl.g) {
    case 1: return run_prefill<1>(pl, q, k_cache, v_cache, out, nullptr, nullptr, st);
    case 2: return run_prefill<2>(pl, q, k_cache, v_cache, out, nullptr, nullptr, st);
    case 4: return run_prefill<4>(pl, q, k_cache, v_cache, out, nullptr, nullptr, st);
    case 8: return run_prefill<8>(pl, q, k_cache, v_cache, out, nullptr, nullptr, st);
  }
  return fail(GSA_ERR_UNSUPPORTED, "gist prefill: %d query heads per kv-head not in {1, 2, 4}", pl.g);
}
