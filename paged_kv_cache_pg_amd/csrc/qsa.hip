// Block pooling, block scores and top-k block selection over a paged cache.
//
// TensorFold PR #1169 "What this changes": a page of n positions holds the
// indexer keys of its n positions and the pooled rows of their n/4 blocks;
// fn_qsa_pool reads and writes through pg_at once per block of four, and
// fn_qsa_scores reads the pooled rows through pg_at.  The selection itself is
// not described on the pages; it keeps the k highest scores with the lower
// block id first among equal scores and returns the ids ascending.
#include "internal.h"

namespace paged {

namespace {

// ---------------------------------------------------------------------------
// Pooling: item = (block, 8-dim chunk); a block's four rows share one lookup.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
  constexpr int ES = BF16 ? 2 : 4;
  const int s = blockIdx.y;
  const int cpb = a.idx_dim / 8;  // chunks a block
  const int b0 = min(max(a.begin[s], 0), a.max_blocks);
  const int b1 = min(max(a.end[s], 0), a.max_blocks);
  if (b1 <= b0) return;
  const int64_t items = (int64_t)(b1 - b0) * cpb;
  const int rowb = a.idx_dim * ES;
  for (int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x; it < items; it += (int64_t)gridDim.x * 256) {
    const int b = b0 + (int)(it / cpb);
    const int ch = (int)(it - (int64_t)(b - b0) * cpb);
    const char* src = a.ik + pg_at(a.pg, s, 0, 4 * b, rowb) + ch * 8 * ES;
    float x[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (BF16) {
        const uint4 v = *(const uint4*)(src + (int64_t)r * rowb);
        x[r][0] = bf16lo(v.x); x[r][1] = bf16hi(v.x); x[r][2] = bf16lo(v.y); x[r][3] = bf16hi(v.y);
        x[r][4] = bf16lo(v.z); x[r][5] = bf16hi(v.z); x[r][6] = bf16lo(v.w); x[r][7] = bf16hi(v.w);
      } else {
        const float4 u = *(const float4*)(src + (int64_t)r * rowb);
        const float4 v = *(const float4*)(src + (int64_t)r * rowb + 16);
        x[r][0] = u.x; x[r][1] = u.y; x[r][2] = u.z; x[r][3] = u.w;
        x[r][4] = v.x; x[r][5] = v.y; x[r][6] = v.z; x[r][7] = v.w;
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
    float4* dst = (float4*)(a.pooled + pool_at(a.pg, s, b, a.idx_dim * 4) + ch * 32);
    dst[0] = make_float4(y[0], y[1], y[2], y[3]);
    dst[1] = make_float4(y[4], y[5], y[6], y[7]);
  }
}

// ---------------------------------------------------------------------------
// Indexer queries widened to float64 once per stream (workspace).
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void qi_widen_kernel(TopkArgs a) {
  const int s = blockIdx.x;
  const int m = a.n_idx_heads * a.idx_dim;
  for (int i = threadIdx.x; i < m; i += 256) {
    double v;
    if constexpr (BF16) {
      const uint16_t u = ((const uint16_t*)a.qi)[(int64_t)s * m + i];
      v = (double)__uint_as_float((uint32_t)u << 16);
    } else {
      v = (double)((const float*)a.qi)[(int64_t)s * m + i];
    }
    a.qi64[(int64_t)s * m + i] = v;
  }
}

// ---------------------------------------------------------------------------
// Scores: one thread a block, one float64 accumulator, head-major then
// dimension order (each product of a bf16/fp32 query and a fp32 pooled value
// is exact in float64, so fused and unfused forms agree).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void scores_kernel(TopkArgs a) {
  const int s = blockIdx.y;
  const int nb = min(max(a.lens[s], 0), a.max_blocks * 4) >> 2;
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (blockIdx.x * 256 >= nb) return;
  const double* qs = a.qi64 + (int64_t)s * a.n_idx_heads * a.idx_dim;
  if (b >= nb) return;
  const float* row = (const float*)(a.pooled + pool_at(a.pg, s, b, a.idx_dim * 4));
  double acc = 0.0;
  for (int h = 0; h < a.n_idx_heads; ++h) {
    const double* qh = qs + h * a.idx_dim;
    for (int d = 0; d < a.idx_dim; d += 4) {
      const float4 p = *(const float4*)(row + d);
      acc = __fma_rn(qh[d + 0], (double)p.x, acc);
      acc = __fma_rn(qh[d + 1], (double)p.y, acc);
      acc = __fma_rn(qh[d + 2], (double)p.z, acc);
      acc = __fma_rn(qh[d + 3], (double)p.w, acc);
    }
  }
  a.scores[(int64_t)s * a.max_blocks + b] = acc;
}

// ---------------------------------------------------------------------------
// Top-k: one workgroup a stream.  Radix select of the k-th largest key over
// order-preserving 64-bit keys (8 passes of 8 bits), then selection in id order.
// ---------------------------------------------------------------------------
constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_COPIES = 4;  // histogram copies a wave, picked by lane & 3, to spread same-bin atomics

__device__ __forceinline__ uint64_t order_key(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  if (x == 0.0) u = 0;  // -0.0 == +0.0
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Exclusive scan over the workgroup; returns the prefix, writes the total.
__device__ __forceinline__ int wg_exclusive_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_tmp[w] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int i = 0; i < TK_WAVES; ++i) {
      const int t = s_tmp[i];
      s_tmp[i] = acc;
      acc += t;
    }
    s_tmp[TK_WAVES] = acc;
  }
  __syncthreads();
  const int r = s_tmp[w] + x - v;
  *total = s_tmp[TK_WAVES];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t s_hist[TK_WAVES][TK_COPIES][256];
  __shared__ uint32_t s_tot[256];
  __shared__ int s_tmp[TK_WAVES + 1];
  __shared__ uint64_t s_prefix;
  __shared__ int s_krem;

  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nb = min(max(a.lens[s], 0), a.max_blocks * 4) >> 2;
  const int k = a.k;
  int32_t* ids = a.out_ids + (int64_t)s * k;
  const double* sc = a.scores + (int64_t)s * a.max_blocks;

  if (nb <= k) {
    for (int i = tid; i < k; i += TK_THREADS) ids[i] = i < nb ? i : -1;
    if (tid == 0) a.out_count[s] = nb;
    return;
  }

  const int ipt = (nb + TK_THREADS - 1) / TK_THREADS;  // items a thread, contiguous ids
  const int i0 = tid * ipt;
  const int i1 = min(i0 + ipt, nb);

  uint64_t prefix = 0, pmask = 0;
  int krem = k;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    for (int i = tid; i < TK_WAVES * TK_COPIES * 256; i += TK_THREADS) (&s_hist[0][0][0])[i] = 0;
    __syncthreads();
    for (int i = i0; i < i1; ++i) {
      const uint64_t key = order_key(sc[i]);
      if ((key & pmask) == prefix) atomicAdd(&s_hist[w][lane & (TK_COPIES - 1)][(key >> shift) & 0xff], 1u);
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t t = 0;
      for (int ww = 0; ww < TK_WAVES; ++ww)
        for (int cc = 0; cc < TK_COPIES; ++cc) t += s_hist[ww][cc][tid];
      s_tot[tid] = t;
    }
    __syncthreads();
    if (tid == 0) {
      int above = 0, dsel = 0;
      for (int dgt = 255; dgt >= 0; --dgt) {
        const int c = (int)s_tot[dgt];
        if (above + c >= krem) { dsel = dgt; break; }
        above += c;
      }
      s_krem = krem - above;
      s_prefix = prefix | ((uint64_t)dsel << shift);
    }
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
    pmask |= (uint64_t)0xff << shift;
    __syncthreads();
  }
  // prefix is the k-th largest key; krem of the keys equal to it are taken, lowest ids first.
  int n_gt = 0, n_eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint64_t key = order_key(sc[i]);
    n_gt += key > prefix;
    n_eq += key == prefix;
  }
  int tot;
  int eq_before = wg_exclusive_scan(n_eq, s_tmp, &tot);
  int sel_cnt = 0;
  {
    int e = eq_before;
    for (int i = i0; i < i1; ++i) {
      const uint64_t key = order_key(sc[i]);
      if (key > prefix) ++sel_cnt;
      else if (key == prefix) { if (e < krem) ++sel_cnt; ++e; }
    }
  }
  int out_before = wg_exclusive_scan(sel_cnt, s_tmp, &tot);
  {
    int e = eq_before, o = out_before;
    for (int i = i0; i < i1; ++i) {
      const uint64_t key = order_key(sc[i]);
      bool take = false;
      if (key > prefix) take = true;
      else if (key == prefix) { take = e < krem; ++e; }
      if (take && o < k) ids[o++] = i;
    }
  }
  if (tid == 0) a.out_count[s] = k;
  (void)n_gt;
}

}  // namespace

hipError_t launch_pool(const PoolArgs& a, bool bf16, hipStream_t st) {
  if (a.n_streams <= 0 || a.max_blocks <= 0) return hipSuccess;
  const int64_t items = (int64_t)a.max_blocks * (a.idx_dim / 8);
  int gx = (int)((items + 255) / 256);
  if (gx > 4096) gx = 4096;
  if (gx < 1) gx = 1;
  dim3 grid(gx, a.n_streams);
  if (bf16) hipLaunchKernelGGL(pool_kernel<true>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(pool_kernel<false>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

size_t topk_workspace_bytes(int n_streams, int max_blocks, int k, int scores_external) {
  (void)k;
  // qi in float64 (up to 2048 values a stream) + scores unless the caller keeps them
  size_t b = (size_t)n_streams * 2048 * sizeof(double);
  if (!scores_external) b += (size_t)n_streams * (size_t)max_blocks * sizeof(double);
  return b;
}

hipError_t launch_scores_topk(const TopkArgs& a, bool qi_bf16, int n_streams, hipStream_t st) {
  if (n_streams <= 0) return hipSuccess;
  if (qi_bf16) hipLaunchKernelGGL(qi_widen_kernel<true>, dim3(n_streams), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(qi_widen_kernel<false>, dim3(n_streams), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.max_blocks > 0) {
    dim3 grid((a.max_blocks + 255) / 256, n_streams);
    hipLaunchKernelGGL(scores_kernel, grid, dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(topk_kernel, dim3(n_streams), dim3(TK_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace paged
