// Split-K bookkeeping shared by the decode kernels (vector-ALU and MFMA) and their combine.
//
// TensorFold PR #1170 commit ce5b78d: decode attention is computed as partials that are merged
// afterwards.  The decomposition depends only on a stream's own key count n, never on the page size,
// the table or the other streams, so a stream's bytes are the same paged and contiguous, alone and
// in a batch:
//   tiles of 64 keys; tps = NWAVE * ceil(tiles / (NWAVE * MAX_SPLITS)) tiles a split (at most
//   MAX_SPLITS splits); split c holds tiles [c*tps, (c+1)*tps); wave w of the split's NWAVE-wave
//   workgroup takes the w-th contiguous part of them.
#pragma once

#include "internal.h"

#ifndef PAGED_DEC_MAX_SPLITS
#define PAGED_DEC_MAX_SPLITS 16  // splits a stream at most
#endif
#ifndef PAGED_DEC_NWAVE
#define PAGED_DEC_NWAVE 8        // waves a workgroup (a split is shared by its waves)
#endif

namespace paged {

constexpr int TILE = 64;
constexpr int NWAVE = PAGED_DEC_NWAVE;
constexpr int WGS = 64 * NWAVE;
constexpr int MAX_SPLITS = PAGED_DEC_MAX_SPLITS;

// Row types of the K/V regions.
enum : int { ET_F32 = 0, ET_BF16 = 1, ET_FP8 = 2 };

__host__ __device__ inline int dec_tiles(int n) { return (n + TILE - 1) / TILE; }
// Tiles a split: a multiple of the waves a workgroup, so that a stream never has more than MAX_SPLITS splits.
__host__ __device__ inline int dec_tps(int ntiles) {
  const int t = (ntiles + NWAVE * MAX_SPLITS - 1) / (NWAVE * MAX_SPLITS);
  return NWAVE * (t < 1 ? 1 : t);
}
__host__ __device__ inline int dec_splits(int n) {
  const int nt = dec_tiles(n);
  if (nt == 0) return 0;
  const int tps = dec_tps(nt);
  return (nt + tps - 1) / tps;
}

// Number of keys a stream attends to: its length (dense) or 4 x its selected blocks (sparse).
__device__ __forceinline__ int stream_keys(const DecArgs& a, int s) {
  const int v = a.lens[s];
  if (a.ids != nullptr) return 4 * min(max(v, 0), a.ids_stride);
  return min(max(v, 0), a.max_len);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load of streamed K/V data.  NT marks it nontemporal (rows read once, nothing to keep in
// cache); the hint changes where lines are kept, never a loaded value.
template <bool NT>
__device__ __forceinline__ uint4 ld_stream(const char* p) {
  u32x4_t v;
  if constexpr (NT) v = __builtin_nontemporal_load((const u32x4_t*)p);
  else v = *(const u32x4_t*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Whether a launch's K and V loads are nontemporal, by the number of workgroups (2^kvshift) over which
// the q heads of a KV head are spread; those workgroups read the same rows.  One workgroup a head:
// both nontemporal (4 x 40960: 112.5 us, against 128.1 with plain loads).  Two: V loads plain, so that
// the V lines stay in L2 for the other workgroup (2 x 40960 72.4-73.1 -> 68.9-70.0 us, 5 x 40960
// about 160 -> 154-156; plain K loads as well were slower, 76.9).  Four: both plain (sparse attention
// over 3 x 2048 keys 15.1 -> 13.1-13.3 us, 1 x 40960 55.9 -> 53.6; plain V only, 13.5-13.7).
__host__ __device__ inline bool dec_k_nontemporal(int kvshift) { return kvshift < 2; }
__host__ __device__ inline bool dec_v_nontemporal(int kvshift) { return kvshift < 1; }

// Orders this wave's LDS writes before its later LDS reads (no cross-wave sync).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace paged
