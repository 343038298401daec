// Row stores and gathers through the page table, and the addressing test hook.
//
// TensorFold PR #1169 "What this changes": fn_attn_prep writes keys, values and
// indexer keys at pg_at addresses, and saving or restoring a prompt cache moves runs
// of pages to and from the contiguous layout, so a kept state passes between the forms.
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

// One step's rows in, through the table, and the pooled row of every block of four the step
// completes.  Per stream: item = (token, 16-byte chunk of its K, V or indexer-key row), then
// item = (completed block, 8 dims).  A completed block's rows at positions before the step come
// from the arena (stored by earlier steps), the others from the step's input, so no item waits
// for another; the pooled value is the same float64 sum, in row order, that pool_kernel forms.
template <bool BF16>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int ES = BF16 ? 2 : 4;
  const int s = blockIdx.y;
  const int p0 = min(max(a.pos0[s], 0), a.max_len);
  const int nn = max(0, min(a.n, a.max_len - p0));
  if (nn == 0) return;
  const int cpr = a.row_bytes / 16, icpr = a.ik_row_bytes / 16;
  const int per_tok = 2 * a.hkv * cpr + icpr;
  const int64_t items_a = (int64_t)nn * per_tok;
  const int b_lo = p0 / 4, b_hi = a.ik_row_bytes ? (p0 + nn) / 4 : b_lo;  // blocks whose last row is new
  const int cpb = a.idx_dim / 8;
  const int64_t items = items_a + (int64_t)(b_hi - b_lo) * cpb;
  for (int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x; it < items; it += (int64_t)gridDim.x * 256) {
    if (it < items_a) {
      const int t = (int)(it / per_tok);
      const int r = (int)(it - (int64_t)t * per_tok);
      const int p = p0 + t;
      const int64_t tok = (int64_t)s * a.n + t;
      if (r < 2 * a.hkv * cpr) {
        const int v = r >= a.hkv * cpr;
        const int rr = r - v * a.hkv * cpr;
        const int h = rr / cpr, c = rr - h * cpr;
        const char* src = (v ? a.v_new : a.k_new) + (tok * a.hkv + h) * a.row_bytes + 16 * c;
        char* dst = (v ? a.vb : a.kb) + pg_at(a.pg, s, h, p, a.row_bytes) + 16 * c;
        *(uint4*)dst = *(const uint4*)src;
      } else {
        const int c = r - 2 * a.hkv * cpr;
        const char* src = a.ik_new + tok * a.ik_row_bytes + 16 * c;
        char* dst = a.ikb + pg_at(a.pg, s, 0, p, a.ik_row_bytes) + 16 * c;
        *(uint4*)dst = *(const uint4*)src;
      }
    } else {
      const int64_t j = it - items_a;
      const int b = b_lo + (int)(j / cpb);
      const int c8 = (int)(j - (int64_t)(b - b_lo) * cpb);
      float x[4][8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = 4 * b + r;
        const char* row = p >= p0 ? a.ik_new + ((int64_t)s * a.n + (p - p0)) * a.ik_row_bytes
                                  : a.ikb + pg_at(a.pg, s, 0, p, a.ik_row_bytes);
        const char* src = row + c8 * 8 * ES;
        if constexpr (BF16) {
          const uint4 u = *(const uint4*)src;
          x[r][0] = bf16lo(u.x); x[r][1] = bf16hi(u.x); x[r][2] = bf16lo(u.y); x[r][3] = bf16hi(u.y);
          x[r][4] = bf16lo(u.z); x[r][5] = bf16hi(u.z); x[r][6] = bf16lo(u.w); x[r][7] = bf16hi(u.w);
        } else {
          const float4 u = *(const float4*)src, w = *(const float4*)(src + 16);
          x[r][0] = u.x; x[r][1] = u.y; x[r][2] = u.z; x[r][3] = u.w;
          x[r][4] = w.x; x[r][5] = w.y; x[r][6] = w.z; x[r][7] = w.w;
        }
      }
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        double acc = (double)x[0][e] + (double)x[1][e];
        acc = acc + (double)x[2][e];
        acc = acc + (double)x[3][e];
        y[e] = (float)(acc * 0.25);
      }
      float4* dst = (float4*)(a.pooled + pool_at(a.pg, s, b, a.idx_dim * 4) + c8 * 32);
      dst[0] = make_float4(y[0], y[1], y[2], y[3]);
      dst[1] = make_float4(y[4], y[5], y[6], y[7]);
    }
  }
}

// e4m3 code of y (OCP E4M3 from its definition: bias 7, 3 mantissa bits, subnormal step 2^-9):
// the nearest code, ties to the even code, magnitudes past the largest finite value (448) held
// at 448, the sign bit kept.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float m = fminf(fabsf(y), 448.f);
  uint32_t mag;
  if (m < 0.015625f) {
    // below the smallest normal 2^-6 the codes step by 2^-9; 8 steps reach code 0x08 = 2^-6
    mag = (uint32_t)__builtin_rintf(m * 512.f);
  } else {
    // keep 3 of float32's 23 mantissa bits, round half to even (a carry moves into the exponent),
    // then move the exponent bias from 127 to 7
    const uint32_t b = __float_as_uint(m);
    mag = ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - (120u << 3);
  }
  return sign | mag;
}

// e4m3 store of a step's K and V rows (PR #1170 commit 5c09685: the fp8 store takes a row's codes and
// fp32 scale through the page table).  A bf16 row x becomes scale = amax / 448 and codes
// e4m3(x / scale) (amax = max |x|; float32 quotients, correctly rounded); a row of zeros gets scale 0
// and zero codes.  Item = (token, K or V, head) row; 16 lanes a row, 16 dims (one 16-byte code chunk)
// a lane.
__global__ __launch_bounds__(256) void append8_kernel(AppendArgs a) {
  const int s = blockIdx.y;
  const int p0 = min(max(a.pos0[s], 0), a.max_len);
  const int nn = max(0, min(a.n, a.max_len - p0));
  if (nn == 0) return;
  const int64_t rows = (int64_t)nn * 2 * a.hkv;
  const int l = threadIdx.x & 15;
  for (int64_t r0 = (int64_t)blockIdx.x * 16; r0 < rows; r0 += (int64_t)gridDim.x * 16) {
    const int64_t r = r0 + (threadIdx.x >> 4);  // the same for the 16 lanes of a row
    if (r < rows) {
      const int t = (int)(r / (2 * a.hkv));
      const int rem = (int)(r - (int64_t)t * 2 * a.hkv);
      const int v = rem >= a.hkv;
      const int h = rem - v * a.hkv;
      const int p = p0 + t;
      const char* src = (v ? a.v_new : a.k_new) + (((int64_t)s * a.n + t) * a.hkv + h) * (HD * 2) + 32 * l;
      const uint4 u0 = *(const uint4*)src, u1 = *(const uint4*)(src + 16);
      const uint32_t wv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
      float x[16];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        x[2 * k] = bf16lo(wv[k]);
        x[2 * k + 1] = bf16hi(wv[k]);
      }
      float amax = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(x[k]));
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
      const float scale = amax / 448.f;
      uint32_t cw[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) w |= (amax > 0.f ? e4m3_code(x[4 * k + e] / scale) : 0u) << (8 * e);
        cw[k] = w;
      }
      *(uint4*)((v ? a.vb : a.kb) + pg_at(a.pg, s, h, p, HD) + 16 * l) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
      if (l == 0) *(float*)((v ? a.vsb : a.ksb) + pg_at(a.pg, s, h, p, 4)) = scale;
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int n_streams, hipStream_t st) {
  if (n_streams <= 0 || a.n <= 0 || a.max_len <= 0) return hipSuccess;
  const int cpr = a.row_bytes / 16, icpr = a.ik_row_bytes / 16;
  const int64_t items = (int64_t)a.n * (2 * a.hkv * cpr + icpr) + (int64_t)((a.n + 3) / 4 + 1) * (a.idx_dim / 8);
  int gx = (int)((items + 255) / 256);
  if (gx > 4096) gx = 4096;
  if (gx < 1) gx = 1;
  if (a.fp8) {
    const int64_t rows = (int64_t)a.n * 2 * a.hkv;
    int g8 = (int)((rows + 15) / 16);
    if (g8 > 4096) g8 = 4096;
    hipLaunchKernelGGL(append8_kernel, dim3(g8, n_streams), dim3(256), 0, st, a);
  } else if (a.bf16) hipLaunchKernelGGL(append_kernel<true>, dim3(gx, n_streams), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(append_kernel<false>, dim3(gx, n_streams), dim3(256), 0, st, a);
  return hipGetLastError();
}

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
