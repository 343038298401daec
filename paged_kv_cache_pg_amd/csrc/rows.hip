// Row stores and gathers through the page table, and the addressing test hook.
//
// TensorFold PR #1169 "What this changes": fn_attn_prep stores keys, values and
// indexer keys through pg_at, and prompt-cache saves and restores copy page runs
// in the contiguous layout so kept states move between the two forms.
#include "internal.h"

namespace paged {

namespace {

// item = (row, 16-byte chunk), chunk fastest so consecutive lanes touch consecutive bytes.
__global__ __launch_bounds__(256) void rows_kernel(RowsArgs a) {
  const int s = blockIdx.y;
  const int p0 = min(max(a.begin[s], 0), a.max_len);
  const int p1 = min(max(a.end[s], 0), a.max_len);
  if (p1 <= p0) return;
  const int cpr = a.row_bytes / 16;
  const int64_t rows = (int64_t)(p1 - p0) * a.n_heads;
  const int64_t items = rows * cpr;
  for (int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x; it < items; it += (int64_t)gridDim.x * 256) {
    const int64_t r = it / cpr;
    const int ch = (int)(it - r * cpr);
    const int h = (int)(r / (p1 - p0));
    const int p = p0 + (int)(r - (int64_t)h * (p1 - p0));
    char* pg_row = a.region + pg_at(a.pg, s, h, p, a.row_bytes) + 16 * ch;
    char* lin_row = a.lin + (int64_t)s * a.ss + (int64_t)h * a.sh + (int64_t)p * a.sp + 16 * ch;
    if (a.gather) *(uint4*)lin_row = *(const uint4*)pg_row;
    else *(uint4*)pg_row = *(const uint4*)lin_row;
  }
}

__global__ __launch_bounds__(256) void row_offsets_kernel(OffArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= a.n) return;
  const int s = a.streams[i], h = a.heads[i], p = a.positions[i];
  int64_t r = -1;
  if (s >= 0 && s < a.n_streams && p >= 0 && p < a.max_pos && h >= 0) {
    // page_bytes carries the page's element count here, row_width elements: offsets in elements.
    r = pg_at(a.pg, s, h, p, a.row_width);
  }
  a.out[i] = r;
}

}  // namespace

hipError_t launch_rows(const RowsArgs& a, hipStream_t st) {
  if (a.n_streams <= 0 || a.max_len <= 0) return hipSuccess;
  const int64_t items = (int64_t)a.max_len * a.n_heads * (a.row_bytes / 16);
  int gx = (int)((items + 255) / 256);
  if (gx > 8192) gx = 8192;
  if (gx < 1) gx = 1;
  hipLaunchKernelGGL(rows_kernel, dim3(gx, a.n_streams), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_row_offsets(const OffArgs& a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(row_offsets_kernel, dim3((a.n + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace paged
