// Cache append on gfx950: new tokens' K and V rows copied to their slots in
// the interleaved cache.
//
// Layout: gist.science explainer, section 2 'Interleaved Gist Tokens' (a gist
// token follows every C raw tokens; slide deck slide 7). Raw token p lives in
// row (p / C) * (C + 1) + p % C, the gist of chunk m in row m * (C + 1) + C,
// of every (sequence, kv-head) block of R rows.
//
// One launch; blockIdx.y picks one of up to four copies (raw K, raw V, gist K,
// gist V), each a [units, n, row] source scattered row by row. 16-byte loads
// and stores; a row of D = 64 or 128 elements is 8 to 32 of them.
#include <hip/hip_runtime.h>

#include "gsa_plan.hpp"
#include "gsa_profile.hpp"

namespace gsa {
namespace {

struct AppendJob {
  const uint4* src;     // [units][n][vpr]
  uint4* dst;           // [units][R][vpr]
  int64_t n;            // rows per unit
  int64_t first;        // first position (raw) or chunk (gist)
  int32_t gist;         // 1: gist rows
};

struct AppendArgs {
  AppendJob job[4];
  int64_t units, R;
  int32_t C, vpr;       // 16-byte vectors per row
};

__global__ __launch_bounds__(256) void cache_append(AppendArgs a) {
  const AppendJob j = a.job[blockIdx.y];
  const int64_t per_unit = j.n * a.vpr;
  const int64_t total = a.units * per_unit;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += step) {
    const int64_t u = i / per_unit;
    const int64_t rem = i - u * per_unit;
    const int64_t r = rem / a.vpr;
    const int32_t c = (int32_t)(rem - r * a.vpr);
    const int64_t x = j.first + r;
    const int64_t row = j.gist ? x * (a.C + 1) + a.C : (x / a.C) * (a.C + 1) + x % a.C;
    j.dst[(u * a.R + row) * a.vpr + c] = j.src[i];
  }
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const char* x = static_cast<const char*>(a);
  const char* y = static_cast<const char*>(b);
  return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

}  // namespace
}  // namespace gsa

using namespace gsa;

extern "C" gsa_status_t gsa_cache_append(const gsa_append_params* p, const void* k_raw, const void* v_raw,
                                         const void* k_gist, const void* v_gist, void* k_cache, void* v_cache,
                                         void* stream) {
  clear_error();
  prof_begin_call();
  AppendPlan pl;
  gsa_status_t s = plan_append(p, &pl);
  if (s != GSA_OK) return s;
  if (pl.raw_new == 0 && pl.gist_new == 0) return GSA_OK;
  if ((s = check_ptr(k_cache, "k_cache")) != GSA_OK || (s = check_ptr(v_cache, "v_cache")) != GSA_OK) return s;
  if (pl.raw_new > 0 && ((s = check_ptr(k_raw, "k_raw")) != GSA_OK || (s = check_ptr(v_raw, "v_raw")) != GSA_OK))
    return s;
  if (pl.gist_new > 0 &&
      ((s = check_ptr(k_gist, "k_gist")) != GSA_OK || (s = check_ptr(v_gist, "v_gist")) != GSA_OK))
    return s;
  const size_t cache_bytes = (size_t)pl.units * (size_t)pl.R * (size_t)pl.row_bytes;
  const size_t raw_bytes = (size_t)pl.units * (size_t)pl.raw_new * (size_t)pl.row_bytes;
  const size_t gist_bytes = (size_t)pl.units * (size_t)pl.gist_new * (size_t)pl.row_bytes;
  if (overlaps(k_cache, cache_bytes, v_cache, cache_bytes))
    return fail(GSA_ERR_INVALID_ARG, "k_cache and v_cache overlap");
  const void* srcs[4] = {k_raw, v_raw, k_gist, v_gist};
  const size_t sizes[4] = {raw_bytes, raw_bytes, gist_bytes, gist_bytes};
  for (int i = 0; i < 4; ++i)
    if (overlaps(srcs[i], sizes[i], k_cache, cache_bytes) || overlaps(srcs[i], sizes[i], v_cache, cache_bytes))
      return fail(GSA_ERR_INVALID_ARG, "a source overlaps a cache");

  AppendArgs a{};
  a.units = pl.units;
  a.R = pl.R;
  a.C = pl.C;
  a.vpr = pl.row_bytes / 16;
  int nj = 0;
  int64_t most = 0;
  auto add = [&](const void* src, void* dst, int64_t n, int64_t first, int gist) {
    if (n == 0) return;
    AppendJob& j = a.job[nj++];
    j.src = static_cast<const uint4*>(src);
    j.dst = static_cast<uint4*>(dst);
    j.n = n;
    j.first = first;
    j.gist = gist;
    if (n > most) most = n;
  };
  add(k_raw, k_cache, pl.raw_new, pl.N, 0);
  add(v_raw, v_cache, pl.raw_new, pl.N, 0);
  add(k_gist, k_cache, pl.gist_new, pl.M, 1);
  add(v_gist, v_cache, pl.gist_new, pl.M, 1);
  // enough workgroups for the largest copy, at most 4096 per copy (grid-stride beyond)
  const int64_t vecs = pl.units * most * a.vpr;
  const int64_t wgs = (vecs + 255) / 256;
  const unsigned gx = (unsigned)(wgs < 4096 ? wgs : 4096);
  prof_launch(cache_append, dim3(gx, nj), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GSA_ERR_HIP, "gsa_cache_append launch: %s", hipGetErrorString(e));
  return GSA_OK;
}
