// Device helpers shared by the libgsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gsa {
namespace dev {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for -inf as the initial running maximum, so that
// exp2(m_old - m_new) never evaluates (-inf) - (-inf).
constexpr float kMinus = -1.0e30f;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over aligned groups of LPR lanes (LPR in {8, 16, 32}); every lane of
// the group ends with the total. Must be called with the whole wave active.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  v += __builtin_amdgcn_update_dpp(0.f, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0.f, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  if constexpr (LPR >= 8) v += __builtin_amdgcn_update_dpp(0.f, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  if constexpr (LPR >= 16) v += __builtin_amdgcn_update_dpp(0.f, v, 0x140, 0xF, 0xF, false); // row_mirror
  if constexpr (LPR >= 32) v += __shfl_xor(v, 16);
  return v;
}

// Hand-off of data between workgroups of one launch (scores, selections,
// partial softmax states). The chip has one L2 per XCD and they are not kept
// coherent with each other, so such data is written and read with
// device-scope accesses (agent-scope relaxed atomics, i.e. sc1 stores that
// write through the L2 and sc1 loads that do not hit a stale line). The
// producer waits for its stores to complete before it signals (done_stores),
// so no L2 write-back or invalidation is ever needed.
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's outstanding memory stores have completed.
__device__ __forceinline__ void done_stores() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Device-scope (sc1) loads through a buffer resource over [base, base + bytes);
// unlike atomic loads they are not serialised, so a batch of them is in
// flight together. Offsets are in 32-bit words; reads past the end return 0.
struct CohBuf {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ CohBuf(const void* base, uint32_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000)) {}
  __device__ __forceinline__ uint32_t u32(uint32_t word) const {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)(word * 4u), 0, 16 /* sc1 */);
  }
  // four consecutive words from a multiple of 4
  __device__ __forceinline__ uint4 u128(uint32_t word) const {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(word * 4u), 0, 16 /* sc1 */);
    return make_uint4(v.x, v.y, v.z, v.w);
  }
};

// 16-byte global load of raw bits.
__device__ __forceinline__ uint4 load16(const char* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// 16-byte load of data read once (nontemporal: streamed past the caches).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_stream(const char* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Elements held by one lane in a 16-byte slice.
template <bool BF16> struct Slice { static constexpr int N = BF16 ? 8 : 4; };

// Dot product of the lane's 16-byte slices of q and k, fp32 accumulation.
// bf16: v_dot2_f32_bf16 (products of bf16 values are exact in fp32).
template <bool BF16>
__device__ __forceinline__ float dot_slice(const uint4& q, const uint4& k) {
  if constexpr (BF16) {
    float d = 0.f;
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.x), __builtin_bit_cast(bf16x2, k.x), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.y), __builtin_bit_cast(bf16x2, k.y), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.z), __builtin_bit_cast(bf16x2, k.z), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.w), __builtin_bit_cast(bf16x2, k.w), d, false);
    return d;
  } else {
    float d = __uint_as_float(q.x) * __uint_as_float(k.x);
    d = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), d);
    d = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), d);
    d = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), d);
    return d;
  }
}

// Widen a 16-byte slice to fp32 (bf16 -> fp32 is exact: the bits move up).
template <bool BF16>
__device__ __forceinline__ void widen(const uint4& v, float (&o)[Slice<BF16>::N]) {
  if constexpr (BF16) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    o[0] = __uint_as_float(v.x);
    o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z);
    o[3] = __uint_as_float(v.w);
  }
}

// Order-preserving map of an fp32 score to uint32 (larger score -> larger
// key); -0 is folded onto +0 so that both compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Block-wide sum of an int; `buf` holds one int per wave and is written
// before the barrier, so two calls in a row must use different buffers.
__device__ __forceinline__ int block_sum(int v, int* buf) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) buf[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
  const int nw = (int)(blockDim.x >> 6);
  for (int w = 0; w < nw; ++w) t += buf[w];
  return t;
}

// Block-wide exclusive prefix sum in thread order; `buf` holds one int per wave.
__device__ __forceinline__ int block_excl_scan(int v, int* buf) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) buf[w] = x;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += buf[i];
  __syncthreads();
  return base + x - v;
}

// The value of lane (lane ^ J) of the wave. Within a 16-lane row the exchange
// uses DPP (quad permutes, row shifts, row rotate by 8); across rows the
// permlane swaps (VALU, no LDS round trip).
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (J == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  } else if constexpr (J == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  } else if constexpr (J == 4) {
    const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x104, 0xF, 0xF, false);   // row_shl:4, lane+4
    const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x114, 0xF, 0xF, false);   // row_shr:4, lane-4
    return (threadIdx.x & 4) ? dn : up;
  } else if constexpr (J == 8) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (J == 16) {
    // v_permlane16_swap of v with itself: [0] holds rows (0,0,2,2), [1] rows (1,1,3,3)
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  } else {
    static_assert(J == 32, "lane_xor: distance 1..32");
    // v_permlane32_swap of v with itself: [0] holds halves (0,0), [1] halves (1,1)
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}
template <int J>
__device__ __forceinline__ unsigned long long lane_xor(unsigned long long v) {
  return ((unsigned long long)lane_xor<J>((uint32_t)(v >> 32)) << 32) | lane_xor<J>((uint32_t)v);
}

}  // namespace dev
}  // namespace gsa
