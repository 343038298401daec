// Device-side row addressing shared by every kernel of libpagedattn.
//
// pg_at follows TensorFold PR #1169 "What this changes": without a table a row
// sits where the earlier contiguous formula puts it; with one, at the base of the
// page containing the position plus the row's offset within that page.  One uniform branch on the
// table pointer is the only difference between the two forms.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace paged {

// Page table as the kernels see it (byte units).
struct PgDev {
  const int32_t* table;  // [n_streams][stride] or nullptr
  int32_t stride;        // entries per stream row
  int32_t ptok;          // positions a page (cap when there is no table)
  int64_t page_bytes;    // bytes a page (stream stride when there is no table)
};

// The page that holds position p of stream s: its table entry, or s itself when there is no table.
__device__ __forceinline__ int32_t pg_page(const PgDev& pg, int s, int p) {
  if (pg.table != nullptr) return pg.table[(int64_t)s * pg.stride + (uint32_t)p / (uint32_t)pg.ptok];
  return s;
}

// The word a lookup of pg_page reads: the table entry of position p of stream s, or `dummy` (any
// readable word, its value then unused) when there is no table, so that the load can be issued
// with no branch around it.
__device__ __forceinline__ const int32_t* pg_entry(const PgDev& pg, int s, int p, const int32_t* dummy) {
  return pg.table != nullptr ? pg.table + ((int64_t)s * pg.stride + (uint32_t)p / (uint32_t)pg.ptok) : dummy;
}

// Byte offset of row (h, p) inside `page`, for a region whose page part is [H][ptok][row_bytes].
__device__ __forceinline__ int64_t pg_offset(const PgDev& pg, int32_t page, int h, int p, int row_bytes) {
  const int within = pg.table != nullptr ? (int)((uint32_t)p % (uint32_t)pg.ptok) : p;
  return (int64_t)page * pg.page_bytes + ((int64_t)h * pg.ptok + within) * (int64_t)row_bytes;
}

// Byte offset of row (s, h, p): base of the page containing position p, plus the row's offset in it.
__device__ __forceinline__ int64_t pg_at(const PgDev& pg, int s, int h, int p, int row_bytes) {
  return pg_offset(pg, pg_page(pg, s, p), h, p, row_bytes);
}

// Byte offset of the pooled row of block b (positions 4b..4b+3) in a region whose
// page part is [ptok/4][row_bytes]: the block's page, row (4b mod ptok)/4 inside it.
__device__ __forceinline__ int64_t pool_at(const PgDev& pg, int s, int b, int row_bytes) {
  const int p = 4 * b;
  int64_t page;
  int within;
  if (pg.table != nullptr) {
    const uint32_t lp = (uint32_t)p / (uint32_t)pg.ptok;
    within = p - (int)lp * pg.ptok;
    page = pg.table[(int64_t)s * pg.stride + lp];
  } else {
    page = s;
    within = p;
  }
  return page * pg.page_bytes + (int64_t)(within >> 2) * row_bytes;
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

constexpr float NEG_INF = -__builtin_inff();

}  // namespace paged
