// Lane-level helpers of the MFMA kernels (prefill and decode): fragment types, reductions over a
// 16x16 accumulator's lane column, and the LDS transpose read with its bank-spreading slot map.
#pragma once

#include <hip/hip_runtime.h>

#include <utility>

namespace paged {

// f(std::integral_constant<int, I>) for I = 0 .. N-1, expanded at compile time: loop bodies whose
// index must be a constant (register arrays indexed by it) however large the body grows.
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// gfx950 permlane swaps: x keeps its lower 32 (16) lanes and takes y's, y gets the other halves.
__device__ __forceinline__ void mf_swap32(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
__device__ __forceinline__ void mf_swap16(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
// max / sum over the four lanes of a lane column (l, l^16, l^32, l^48); every lane gets the same bits.
__device__ __forceinline__ float col_max(float x) {
  float y = x;
  mf_swap32(x, y);
  x = fmaxf(x, y);
  y = x;
  mf_swap16(x, y);
  return fmaxf(x, y);
}
__device__ __forceinline__ float col_sum(float x) {
  float y = x;
  mf_swap32(x, y);
  x = x + y;
  y = x;
  mf_swap16(x, y);
  return x + y;
}

// ds_read_b64_tr_b16: 4 bf16 of one column from 4 rows (see the offsets built by the callers).
__device__ __forceinline__ bf16x4 lds_tr16(const char* lds_base, int byte_off) {
  const lds_s16x4* p = (const lds_s16x4*)((__attribute__((address_space(3))) const char*)lds_base + byte_off);
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
}

// LDS tiles hold rows of 512 bytes with the 16-byte chunks of a row permuted, so that the fragment
// reads hit distinct banks: K chunk c of row r sits at slot c ^ (r mod 16) (the 16 rows of a K
// fragment read), V chunk c at slot c ^ 2(r mod 8) (the 8 rows x 2 chunks of 32 lanes of a
// transpose read).
__device__ __forceinline__ int k_slot(int row, int c) { return c ^ (row & 15); }
__device__ __forceinline__ int v_slot(int row, int c) { return c ^ ((row & 7) << 1); }

// Byte offset, in a V tile of 512-byte rows swizzled by v_slot, of this lane's V^T half-fragment
// (dims block db = 8dh + dl, rows r0 .. of the first 16 rows of a 32-key step): the transpose read of
// rows r1 = 4u + c16/4 (+16 for the second half), dims 16db + 4(c16 mod 4).  Chunk (2db + j) of row
// r1 sits at slot (2db + j) ^ 2(r1 mod 8) = 2(db ^ x) + j with x = r1 mod 8 and j = (c16 mod 4)/2.
__device__ __forceinline__ int vt_offset(int u, int c16, int dl) {
  const int r0 = 4 * u + (c16 >> 2), x = r0 & 7, j = (c16 & 3) >> 1, hb = (c16 & 1) * 8;
  return r0 * 512 + (2 * (dl ^ x) + j) * 16 + hb;
}

}  // namespace paged
