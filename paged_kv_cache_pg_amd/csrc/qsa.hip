// Block pooling, block scores and top-k block selection over a paged cache.
//
// TensorFold PR #1169 "What this changes": besides keys and values, each page of
// n positions stores their indexer keys and one pooled row for each n/4 block;
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

// Cross-lane steps with DPP (row shifts, row broadcasts, quad and half-row permutations): the value
// moves between lanes inside the vector unit, with no LDS round trip as a shuffle takes.  Called with
// every lane of the wave active.  A lane whose source is outside its row, or whose row is masked off,
// takes `old`.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, CTRL, ROWS, 0xf, false);
}
constexpr int DPP_QUAD_XOR1 = 0xb1;  // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4e;  // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // row_half_mirror: lane i of each 8 takes lane 7 - i
constexpr int DPP_SHR1 = 0x111, DPP_SHR2 = 0x112, DPP_SHR4 = 0x114, DPP_SHR8 = 0x118;  // row_shr:n
constexpr int DPP_BCAST15 = 0x142, DPP_BCAST31 = 0x143;  // row_bcast:15 / :31

// A float64 moved by a DPP pattern whose sources are all inside the row (quad and half-row ones).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = dpp_u32<CTRL, 0xf>((uint32_t)u, 0u), hi = dpp_u32<CTRL, 0xf>((uint32_t)(u >> 32), 0u);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// ---------------------------------------------------------------------------
// Scores.  In exact arithmetic sum_h sum_d qI[h][d] p[d] = sum_d q[d] p[d] with q[d] = sum_h qI[h][d],
// so the workgroup first sums the indexer queries over the heads (float64, head by head) into LDS.
// A block is then scored by 8 lanes: lane j of the block takes the 4-dim chunks c = j, j+8, j+16, ...
// of its pooled row (so the 8 lanes of a block read 128 contiguous bytes a load), adds each product
// p[d] * q[d] (rounded to float64, not fused) to its float64 sum in increasing dim order, and the 8
// lane sums meet in a fixed butterfly, ((g0+g1)+(g2+g3))+((g4+g5)+(g6+g7)) (float64 addition
// commutes, so every lane of the block ends with the same value).  This is the order of the oracle's
// definition, so scores are bit for bit the oracle's.
// A wave scores 8 blocks a round and R rounds (2 for 128-wide rows), all of whose row loads are issued
// before the first sum; a workgroup is 4 waves.  The stream's length and the table entries of a
// lane's blocks are requested together, then the rows; the queries are summed while the rows are in
// flight.
// ---------------------------------------------------------------------------
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int SC_THREADS = 256;
constexpr int SC_LPB = 8;                      // lanes a block
constexpr int SC_MAXD = 1024;                  // dims at most

// The first workgroup of each stream clears the stream's coarse top-k histogram (the
// histogram kernel, launched next on the same stream, adds into it).
__device__ __forceinline__ void zero_hist(const TopkArgs& a, int s) {
  uint4* h = (uint4*)(a.hist + (int64_t)s * 4096);
  for (int i = threadIdx.x; i < 4096 / 4; i += SC_THREADS) h[i] = make_uint4(0u, 0u, 0u, 0u);
}

// q[d] = sum over heads of the stream's indexer queries, float64, head by head, for d < idx_dim.
template <bool QBF16>
__device__ __forceinline__ void sum_queries(const TopkArgs& a, int s, double* s_q) {
#pragma clang fp contract(off)
  const int m = a.n_idx_heads * a.idx_dim;
  for (int d = threadIdx.x; d < a.idx_dim; d += SC_THREADS) {
    double q = 0.0;
    for (int h = 0; h < a.n_idx_heads; ++h) {
      const int64_t i = (int64_t)s * m + h * a.idx_dim + d;
      const double v = QBF16 ? (double)__uint_as_float((uint32_t)((const uint16_t*)a.qi)[i] << 16)
                             : (double)((const float*)a.qi)[i];
      q = q + v;
    }
    s_q[d] = q;
  }
}

// NCH: 4-dim chunks a lane at most (idx_dim <= 32 NCH); R: rounds of 8 blocks a wave.
template <bool QBF16, int NCH, int R>
__global__ __launch_bounds__(SC_THREADS) void scores_kernel(TopkArgs a) {
  // the products are rounded before they are added (no fused multiply-add): float32 queries summed over
  // heads can carry more than 29 bits, and then a product is not exact in float64
#pragma clang fp contract(off)
  __shared__ __attribute__((aligned(16))) double s_q[SC_MAXD];
  const int s = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = lane & (SC_LPB - 1), slot = lane >> 3;
  constexpr int BPW = 8 * R;                          // blocks a wave
  const int b_wg = blockIdx.x * (SC_THREADS / 64) * BPW;
  const int b_wave = b_wg + w * BPW;
  if (blockIdx.x == 0) zero_hist(a, s);
  // The stream's length and the table entries of this lane's blocks are requested together (every
  // block below max_blocks has an entry; an entry is used as an address only below the length).
  const bool paged = a.pg.table != nullptr;
  int32_t entry[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int b = min(b_wave + 8 * r + slot, a.max_blocks - 1);
    entry[r] = paged ? a.pg.table[(int64_t)s * a.pg.stride + (uint32_t)(4 * b) / (uint32_t)a.pg.ptok] : 0;
  }
  const int nb = min(max(a.lens[s], 0), a.max_blocks * 4) >> 2;
  if (b_wg >= nb) return;                             // the whole workgroup is past the blocks
  const int nch = (a.idx_dim + 3) >> 2;               // 4-dim chunks a row
  const int rowb = a.idx_dim * 4;
  // Row loads of every round (blocks past nb, and chunks past the row, re-read chunk 0 of block
  // 0 of the stream, which exists).
  auto row_base = [&](int b, int32_t e) -> int64_t {
    const int p = 4 * b;
    const int within = paged ? p - (int)((uint32_t)p / (uint32_t)a.pg.ptok) * a.pg.ptok : p;
    const int64_t page = paged ? (int64_t)e : (int64_t)s;
    return page * a.pg.page_bytes + (int64_t)(within >> 2) * rowb;
  };
  const char* first = a.pooled + pool_at(a.pg, s, 0, rowb);
  u32x4 v[R][NCH];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int b = b_wave + 8 * r + slot;
    const char* base = a.pooled + row_base(b < nb ? b : 0, entry[r]);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = j + SC_LPB * i;
      const char* src = (b < nb && c < nch) ? base + c * 16 : first;
      v[r][i] = *(const u32x4*)src;
    }
  }
  // the queries summed over heads into LDS while the rows are in flight
  sum_queries<QBF16>(a, s, s_q);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = j + SC_LPB * i;
      if (c < nch) {
        const double2 q01 = *(const double2*)(s_q + 4 * c);
        const double2 q23 = *(const double2*)(s_q + 4 * c + 2);
        const float p[4] = {__uint_as_float(v[r][i].x), __uint_as_float(v[r][i].y), __uint_as_float(v[r][i].z),
                            __uint_as_float(v[r][i].w)};
        const double q[4] = {q01.x, q01.y, q23.x, q23.y};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * c + e < a.idx_dim) acc = acc + (double)p[e] * q[e];
      }
    }
    // the butterfly: after the quad steps every lane of a quad holds its quad's sum, so the half-row
    // mirror adds the other quad's
    acc = acc + dpp_f64<DPP_QUAD_XOR1>(acc);
    acc = acc + dpp_f64<DPP_QUAD_XOR2>(acc);
    acc = acc + dpp_f64<DPP_HALF_MIRROR>(acc);
    const int b = b_wave + 8 * r + slot;
    if (j == 0 && b < nb) a.scores[(int64_t)s * a.max_blocks + b] = acc;
  }
}

// ---------------------------------------------------------------------------
// Top-k (the block order a score sorts by: score descending, then id ascending;
// -0.0 == +0.0), after the scores kernel:
//  1. Coarse histogram (hist_kernel, a workgroup per 1024 scores): 4096 bins of
//     the top 12 bits of the float32 order key of each score (sign, exponent, 3
//     mantissa bits).  Rounding to float32 is monotone, so every score in a
//     higher bin is larger than every score in a lower one.  The scores kernel
//     zeroes the histogram; this kernel adds each workgroup's LDS histogram to it.
//     Bin T, where the count from the top reaches k, holds the k-th block.
//  2. Selection (select_kernel, a workgroup per 1024 blocks): each workgroup
//     finds T from the histogram itself and writes, for its blocks, a taken bit
//     per block (bin above T), its taken count, and its bin-T candidates (exact
//     64-bit key, id) with their count.
//  3. Finish (topk_kernel, a workgroup per stream): krem = k minus the taken
//     count; the candidates are gathered into LDS, a 256-bin histogram of their
//     keys above the smallest finds the sub-bin holding the krem-th, candidates
//     above it are selected and the sub-bin's members ranked exactly (members
//     ahead of each in the sort order); selected candidates are marked in an LDS
//     bitmap.  The ids come out in id order: a thread per 64-block chunk or's
//     the chunk's taken and selected words, and a scan of the chunks' counts
//     gives each chunk's first output place.
// Streams of more than TK_SBITS blocks take the single-workgroup list path: one
// sweep lists the ids above bin T and bin T's candidates in LDS, each candidate
// is ranked exactly, and each listed id's place is the number of listed ids below
// it.  With more than TK_CMAX candidates (heavy ties) or, on the list path,
// k > TK_AMAX, a radix refinement on the exact 64-bit keys of bin T finds the
// threshold instead (ties at it go to the lowest ids), and a count sweep, a
// 16-entry scan of the waves' counts and a write sweep compact the ids in order
// (wave w holds ids [64 J w, 64 J (w+1))).
// ---------------------------------------------------------------------------
constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_BINS = 4096;       // coarse bins
constexpr int TK_CMAX = 4096;       // candidates ranked in LDS
constexpr int TK_AMAX = 8192;       // k at most for the list path
constexpr int TK_BATCH = 16;        // score chunks a thread reads at once
#ifndef PAGED_HK_ITEMS
#define PAGED_HK_ITEMS 1024
#endif
constexpr int HK_ITEMS = PAGED_HK_ITEMS;  // scores a histogram workgroup
constexpr int SEL_ITEMS = 1024;     // blocks a selection workgroup
constexpr int SEL_THREADS = 1024;  // a thread a block (256: scores + top-k 0.5-1 us slower)
constexpr int TK_SBITS = 1 << 18;   // blocks a stream whose selected candidates are marked in LDS
constexpr int TK_CPT = TK_SBITS / 64 / 1024;  // 64-block chunks a thread at most in the id output (4)
constexpr int HK_THREADS = 1024;   // a thread a score; the bins cleared and flushed 4 a thread (256: 2 us slower)

__device__ __forceinline__ uint64_t order_key(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  if (x == 0.0) u = 0;  // -0.0 == +0.0
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}
__device__ __forceinline__ uint32_t coarse_bin(double x) {
  const float f = (float)x;
  uint32_t u = __float_as_uint(f);
  if (f == 0.f) u = 0;
  u = (u >> 31) ? ~u : (u | 0x80000000u);
  return u >> 20;
}

// Increments an LDS counter once for each active lane; a wave whose active lanes all
// hit one counter adds their count with one atomic (all-equal scores would otherwise
// serialise 64 same-address atomics an instruction).
__device__ __forceinline__ void lds_count(uint32_t* hist, uint32_t bin) {
  const uint64_t act = __ballot(1);
  const uint32_t b0 = __builtin_amdgcn_readfirstlane(bin);
  const uint64_t same = __ballot(bin == b0);
  if (same == act) {
    if ((threadIdx.x & 63) == (uint32_t)__builtin_ctzll(act)) atomicAdd(&hist[b0], (uint32_t)__popcll(act));
  } else {
    atomicAdd(&hist[bin], 1u);
  }
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inclusive prefix sum over the wave's 64 lanes in lane order (sums within rows of 16 by row shifts,
// then the last lane of row 0 added to row 1 and of row 2 to row 3, then lane 31 to rows 2 and 3).
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
  x += dpp_u32<DPP_SHR1, 0xf>(x, 0u);
  x += dpp_u32<DPP_SHR2, 0xf>(x, 0u);
  x += dpp_u32<DPP_SHR4, 0xf>(x, 0u);
  x += dpp_u32<DPP_SHR8, 0xf>(x, 0u);
  x += dpp_u32<DPP_BCAST15, 0xa>(x, 0u);
  x += dpp_u32<DPP_BCAST31, 0xc>(x, 0u);
  return x;
}

// Minimum and maximum of a 64-bit value over the wave, in lane 63 (the same steps as the sum; min and
// max do not depend on the order in which values meet).
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x, uint64_t old) {
  const uint32_t lo = dpp_u32<CTRL, ROWS>((uint32_t)x, (uint32_t)old);
  const uint32_t hi = dpp_u32<CTRL, ROWS>((uint32_t)(x >> 32), (uint32_t)(old >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ void wave_minmax_u64(uint64_t& mn, uint64_t& mx) {
#define MINMAX_STEP(C, R)                         \
  {                                               \
    const uint64_t a = dpp_u64<C, R>(mn, ~0ull);  \
    const uint64_t b = dpp_u64<C, R>(mx, 0ull);   \
    mn = a < mn ? a : mn;                         \
    mx = b > mx ? b : mx;                         \
  }
  MINMAX_STEP(DPP_SHR1, 0xf)
  MINMAX_STEP(DPP_SHR2, 0xf)
  MINMAX_STEP(DPP_SHR4, 0xf)
  MINMAX_STEP(DPP_SHR8, 0xf)
  MINMAX_STEP(DPP_BCAST15, 0xa)
  MINMAX_STEP(DPP_BCAST31, 0xc)
#undef MINMAX_STEP
}

// Exclusive scan of one 32-bit value a thread over the workgroup, in thread order; every thread gets
// the total.  s_tmp holds TK_WAVES + 1 words.
__device__ __forceinline__ uint32_t wg_scan32(uint32_t v, uint32_t* s_tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t x = wave_incl_sum(v);
  if (lane == 63) s_tmp[w] = x;
  __syncthreads();
  if (threadIdx.x < 64) {
    const uint32_t t = lane < TK_WAVES ? s_tmp[lane] : 0u;
    const uint32_t z = wave_incl_sum(t);
    if (lane < TK_WAVES) s_tmp[lane] = z - t;
    if (lane == TK_WAVES - 1) s_tmp[TK_WAVES] = z;
  }
  __syncthreads();
  const uint32_t r = s_tmp[w] + x - v;
  *total = s_tmp[TK_WAVES];
  __syncthreads();
  return r;
}

// Exclusive scan of one 64-bit value a thread, in thread order; every thread gets the total.
__device__ __forceinline__ uint64_t wg_scan64(uint64_t v, uint64_t* s_tmp, uint64_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint64_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_tmp[w] = x;
  __syncthreads();
  if (threadIdx.x < 64) {
    const uint64_t t = threadIdx.x < TK_WAVES ? s_tmp[threadIdx.x] : 0;
    uint64_t z = t;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint64_t y = __shfl_up(z, off);
      if (lane >= off) z += y;
    }
    if (threadIdx.x < TK_WAVES) s_tmp[threadIdx.x] = z - t;
    if (threadIdx.x == TK_WAVES - 1) s_tmp[TK_WAVES] = z;
  }
  __syncthreads();
  const uint64_t r = s_tmp[w] + x - v;
  *total = s_tmp[TK_WAVES];
  __syncthreads();
  return r;
}

__device__ __forceinline__ int stream_blocks(const TopkArgs& a, int s) {
  return min(max(a.lens[s], 0), a.max_blocks * 4) >> 2;
}

// Step 1: each workgroup histograms HK_ITEMS scores of one stream in LDS and adds the
// non-zero bins to the stream's histogram (zeroed by the scores kernel).
__global__ __launch_bounds__(HK_THREADS) void hist_kernel(TopkArgs a) {
  __shared__ uint32_t s_h[TK_BINS];
  const int s = blockIdx.y;
  const int nb = stream_blocks(a, s);
  const int i0 = blockIdx.x * HK_ITEMS;
  if (nb <= a.k || i0 >= nb) return;  // nothing to select, or past the stream's blocks
  for (int i = threadIdx.x; i < TK_BINS; i += HK_THREADS) s_h[i] = 0;
  const double* sc = a.scores + (int64_t)s * a.max_blocks;
  double x[HK_ITEMS / HK_THREADS];
#pragma unroll
  for (int r = 0; r < HK_ITEMS / HK_THREADS; ++r) {
    const int i = i0 + r * HK_THREADS + threadIdx.x;
    x[r] = i < nb ? sc[i] : 0.0;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < HK_ITEMS / HK_THREADS; ++r) {
    const int i = i0 + r * HK_THREADS + threadIdx.x;
    if (i < nb) lds_count(s_h, coarse_bin(x[r]));
  }
  __syncthreads();
  uint32_t* gh = a.hist + (int64_t)s * TK_BINS;
  for (int b = threadIdx.x; b < TK_BINS; b += HK_THREADS) {
    const uint32_t c = s_h[b];
    if (c) atomicAdd(&gh[b], c);
  }
}

// Step 2a: selection spread over the stream.  Workgroup b of stream s owns blocks [1024 b, 1024 b + 1024):
// it finds bin T and krem from the histogram itself, then writes the taken bits of its blocks (bin > T),
// its count of them, and its bin-T (key, id) pairs with their count.  No counter is shared between
// workgroups; inside one, a wave adds its ballot counts with one LDS atomic.
__global__ __launch_bounds__(SEL_THREADS) void select_kernel(TopkArgs a) {
  __shared__ uint64_t s_tmp[SEL_THREADS / 64 + 1];
  __shared__ uint32_t s_T, s_nt, s_nc;
  const int s = blockIdx.y, b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nb = stream_blocks(a, s);
  const int k = a.k;
  const int i0 = b * SEL_ITEMS;
  if (nb <= k || i0 >= nb) return;  // nothing to select, or past the stream's blocks
  if (tid == 0) {
    s_nt = 0;
    s_nc = 0;
  }
  // the bin of the k-th block: thread t owns bins 4095 - BPT t .. 4096 - BPT (t + 1) (descending)
  {
    constexpr int BPT = TK_BINS / SEL_THREADS;
    const uint32_t* gh = a.hist + (int64_t)s * TK_BINS;
    const int top = TK_BINS - 1 - BPT * tid;
    uint32_t c[BPT];
    uint64_t loc = 0;
#pragma unroll
    for (int r = 0; r < BPT; ++r) {
      c[r] = gh[top - r];
      loc += c[r];
    }
    // exclusive scan over the workgroup, in thread (= descending bin) order (counts below 2^28)
    const uint64_t x = wave_incl_sum((uint32_t)loc);
    if (lane == 63) s_tmp[w] = x;
    __syncthreads();
    uint64_t before = x - loc;
    for (int v = 0; v < w; ++v) before += s_tmp[v];
    if (before < (uint64_t)k && before + loc >= (uint64_t)k) {
#pragma unroll
      for (int r = 0; r < BPT; ++r) {
        if (before + c[r] >= (uint64_t)k) {
          s_T = (uint32_t)(top - r);
          break;
        }
        before += c[r];
      }
    }
    __syncthreads();
  }
  const uint32_t T = s_T;
  const double* sc = a.scores + (int64_t)s * a.max_blocks;
  double x[SEL_ITEMS / SEL_THREADS];
#pragma unroll
  for (int r = 0; r < SEL_ITEMS / SEL_THREADS; ++r) {
    const int i = i0 + r * SEL_THREADS + tid;
    x[r] = i < nb ? sc[i] : (double)NEG_INF;
  }
  uint64_t* keys = a.sel_key + ((int64_t)s * a.nsel + b) * SEL_ITEMS;
  int32_t* cids = a.sel_id + ((int64_t)s * a.nsel + b) * SEL_ITEMS;
  uint32_t* bits = a.sel_bits + (int64_t)s * a.nsel * (SEL_ITEMS / 32);
#pragma unroll
  for (int r = 0; r < SEL_ITEMS / SEL_THREADS; ++r) {
    const int i = i0 + r * SEL_THREADS + tid;
    const uint32_t cb = coarse_bin(x[r]);
    const bool taken = i < nb && cb > T, cand = i < nb && cb == T;
    const uint64_t tm = __ballot(taken), cm = __ballot(cand);
    // the 64 blocks of this wave and round are 64 consecutive ids: two words of taken bits
    if (lane == 0) {
      const int word = (i - lane) >> 5;
      bits[word] = (uint32_t)tm;
      bits[word + 1] = (uint32_t)(tm >> 32);
    }
    uint32_t cbase = 0;
    if (lane == 0) {
      atomicAdd(&s_nt, (uint32_t)__popcll(tm));
      if (cm) cbase = atomicAdd(&s_nc, (uint32_t)__popcll(cm));
    }
    cbase = (uint32_t)__builtin_amdgcn_readlane((int)cbase, 0);
    if (cand) {
      const uint32_t slot = cbase + lanes_below(cm);
      keys[slot] = order_key(x[r]);
      cids[slot] = i;
    }
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t* cnt = a.sel_cnt + ((int64_t)s * a.nsel + b) * 2;
    cnt[0] = s_nt;
    cnt[1] = s_nc;
  }
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(TopkArgs a) {
  __shared__ __attribute__((aligned(16))) int32_t s_aid[TK_AMAX];  // ids taken (unordered until the final ranking)
  __shared__ uint64_t s_ckey[TK_CMAX]; // candidates of bin T: exact keys and ids
  __shared__ int32_t s_cid[TK_CMAX];
  __shared__ uint32_t s_dig[256];
  __shared__ uint64_t s_tmp[TK_WAVES + 1];
  __shared__ uint64_t s_red[2][TK_WAVES];
  __shared__ uint32_t s_wg[TK_WAVES], s_we[TK_WAVES];
  __shared__ uint32_t s_T, s_na, s_nc;
  __shared__ int s_krem, s_done;
  __shared__ uint64_t s_prefix;
  __shared__ uint64_t s_sbit[TK_SBITS / 64];   // selected bin-T blocks, a bit a block
  __shared__ uint32_t s_coff[TK_SBITS / SEL_ITEMS + 1];  // per selection workgroup: first candidate
  __shared__ uint32_t s_h2[256];
  __shared__ int32_t s_l2id[TK_CMAX];
  __shared__ uint64_t s_kmin, s_kmax;
  __shared__ uint32_t s_n2;
  __shared__ int s_over;

  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nb = stream_blocks(a, s);
  const int k = a.k;
  int32_t* ids = a.out_ids + (int64_t)s * k;
  const double* sc = a.scores + (int64_t)s * a.max_blocks;

  if (nb <= k) {
    for (int i = tid; i < k; i += TK_THREADS) ids[i] = i < nb ? i : -1;
    if (tid == 0) a.out_count[s] = nb;
    return;
  }
  const int J = (nb + TK_THREADS - 1) / TK_THREADS;  // chunks a wave
  // item (w, j, lane) has id (w * J + j) * 64 + lane: a wave's ids are consecutive.  f(j, i, x) for every
  // item of this thread in chunk (= id) order, TK_BATCH chunks' reads in flight at a time; items past
  // the stream's blocks read as -inf and carry i >= nb.
  auto item_id = [&](int j) { return (w * J + j) * 64 + lane; };
  auto for_items = [&](auto&& f) {
    for (int j8 = 0; j8 < J; j8 += TK_BATCH) {
      double t[TK_BATCH];
#pragma unroll
      for (int u = 0; u < TK_BATCH; ++u) {
        const int i = item_id(j8 + u);
        t[u] = (j8 + u < J && i < nb) ? sc[i] : (double)NEG_INF;
      }
#pragma unroll
      for (int u = 0; u < TK_BATCH; ++u)
        if (j8 + u < J) f(j8 + u, item_id(j8 + u), t[u]);
    }
  };

  // ---- fast path: the selection workgroups' counts, taken bits and bin-T candidates ----
  // Every load that depends on nothing computed here is issued first, so their latencies overlap.
  const int nw = (nb + SEL_ITEMS - 1) / SEL_ITEMS;  // selection workgroups of this stream (<= 256)
  if (nb <= TK_SBITS) {
    const int nchunk = (nb + 63) / 64;
    // candidates, speculatively: thread t holds slot t % P of selection workgroup t / P (slots past
    // the workgroup's count are ignored)
    const int P = TK_THREADS / nw;
    const int cb = tid / P, cj = tid - cb * P;
    uint64_t ck = 0;
    int32_t ci = 0;
    if (cb < nw) {
      const int64_t src = ((int64_t)s * a.nsel + cb) * SEL_ITEMS + cj;
      ck = a.sel_key[src];
      ci = a.sel_id[src];
    }
    // taken bits: thread t holds the words of chunks (64 blocks) t*CPT .. t*CPT + CPT-1, in id order
    const uint64_t* bits = (const uint64_t*)(a.sel_bits + (int64_t)s * a.nsel * (SEL_ITEMS / 32));
    const int cpt = (nchunk + TK_THREADS - 1) / TK_THREADS;  // <= TK_CPT
    uint64_t tw[TK_CPT];
#pragma unroll
    for (int j = 0; j < TK_CPT; ++j) {
      const int ch = tid * cpt + j;
      tw[j] = (j < cpt && ch < nchunk) ? bits[ch] : 0ull;
    }
    // counts: wave 0, lane l holds selection workgroups 4l .. 4l + 3 (taken, candidates)
    if (w == 0) {
      const uint32_t* cnt = a.sel_cnt + (int64_t)s * a.nsel * 2;
      uint32_t nt[4], nc[4], st = 0, sc = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int b = 4 * lane + r;
        const uint2 v = b < nw ? *(const uint2*)(cnt + 2 * b) : make_uint2(0u, 0u);
        nt[r] = v.x;
        nc[r] = v.y;
        st += v.x;
        sc += v.y;
      }
      const uint32_t it = wave_incl_sum(st), ic = wave_incl_sum(sc);
      uint32_t pt = it - st, pc = ic - sc;
      bool over = false;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int b = 4 * lane + r;
        if (b < nw) {
          s_coff[b] = pc;
          over |= nc[r] > (uint32_t)P;
        }
        pt += nt[r];
        pc += nc[r];
      }
      over = __ballot(over) != 0;
      if (lane == 63) {
        s_coff[nw] = pc;  // = every candidate
        s_na = pt;        // = every taken block
        s_nc = pc;
        s_over = over;
        s_kmin = ~0ull;
        s_kmax = 0;
        s_n2 = 0;
      }
    } else if (w == 1) {
      for (int q = lane; q < 256; q += 64) s_h2[q] = 0;
    }
    for (int q = tid; q < nchunk; q += TK_THREADS) s_sbit[q] = 0;
    __syncthreads();
    const int NC = (int)s_nc;
    if (NC <= TK_CMAX) {
      const int krem = k - (int)s_na;  // 1 <= krem <= NC: bin T holds the k-th block
      // the candidates into one list (in selection workgroup order), with their smallest and largest key
      uint64_t kmn = ~0ull, kmx = 0;
      if (cb < nw) {
        const uint32_t o = s_coff[cb];
        if (cj < (int)(s_coff[cb + 1] - o)) {
          s_ckey[o + cj] = ck;
          s_cid[o + cj] = ci;
          kmn = ck;
          kmx = ck;
        }
      }
      if (s_over) {  // a selection workgroup holds more than P candidates: the rest one by one
        for (int f = tid; f < NC; f += TK_THREADS) {
          int lo = 0, hi = nw - 1;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_coff[mid] <= (uint32_t)f) lo = mid;
            else hi = mid - 1;
          }
          const int j = f - (int)s_coff[lo];
          if (j >= P) {
            const int64_t src = ((int64_t)s * a.nsel + lo) * SEL_ITEMS + j;
            const uint64_t key = a.sel_key[src];
            s_ckey[f] = key;
            s_cid[f] = a.sel_id[src];
            kmn = key < kmn ? key : kmn;
            kmx = key > kmx ? key : kmx;
          }
        }
      }
      wave_minmax_u64(kmn, kmx);
      if (lane == 63 && kmx != 0) {
        atomicMin((unsigned long long*)&s_kmin, (unsigned long long)kmn);
        atomicMax((unsigned long long*)&s_kmax, (unsigned long long)kmx);
      }
      __syncthreads();
      // a 256-bin histogram of the candidates' keys above the smallest one, at the resolution that
      // spreads them over the bins; sub-bin T2 holds the krem-th
      const uint64_t kmin = s_kmin, span = s_kmax - kmin;
      const int shift = span < 256 ? 0 : 56 - __builtin_clzll(span);  // (span >> shift) <= 255
      for (int f = tid; f < NC; f += TK_THREADS) lds_count(s_h2, (uint32_t)((s_ckey[f] - kmin) >> shift));
      __syncthreads();
      if (w == 0) {
        // lane l owns sub-bins 255-4l .. 252-4l (descending)
        uint32_t c4[4], loc = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          c4[r] = s_h2[255 - 4 * lane - r];
          loc += c4[r];
        }
        const uint32_t incl = wave_incl_sum(loc);
        uint32_t above = incl - loc;
        if (above < (uint32_t)krem && incl >= (uint32_t)krem) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (above + c4[r] >= (uint32_t)krem) {
              s_T = (uint32_t)(255 - 4 * lane - r);
              s_krem = krem - (int)above;
              break;
            }
            above += c4[r];
          }
        }
      }
      __syncthreads();
      // candidates above sub-bin T2 are selected; those in it are listed for an exact ranking
      const uint32_t T2 = s_T;
      const int k2 = s_krem;
      uint64_t* s_k2 = (uint64_t*)s_aid;  // keys of the sub-bin T2 list (s_aid is free on this path)
      auto select = [&](int32_t id) { atomicOr((unsigned long long*)&s_sbit[id >> 6], 1ull << (id & 63)); };
      for (int f = tid; f < NC; f += TK_THREADS) {
        const uint64_t key = s_ckey[f];
        const uint32_t sub = (uint32_t)((key - kmin) >> shift);
        if (sub > T2) {
          select(s_cid[f]);
        } else if (sub == T2) {
          const uint32_t slot = atomicAdd(&s_n2, 1u);
          s_k2[slot] = key;
          s_l2id[slot] = s_cid[f];
        }
      }
      __syncthreads();
      // exact ranks inside sub-bin T2, four lanes a member (each counts a quarter of the others)
      const int n2 = (int)s_n2;
      for (int c0 = 0; c0 < n2; c0 += TK_THREADS / 4) {
        const int c = c0 + (tid >> 2), q = tid & 3;
        int r = 0;
        uint64_t kc = 0;
        int32_t ic = 0;
        if (c < n2) {
          kc = s_k2[c];
          ic = s_l2id[c];
          const int o0 = (n2 * q) >> 2, o1 = (n2 * (q + 1)) >> 2;
          for (int o = o0; o < o1; ++o) {
            const uint64_t ko = s_k2[o];
            const int32_t io = s_l2id[o];
            r += (int)((ko > kc) | ((ko == kc) & (io < ic)));
          }
        }
        r += (int)dpp_u32<DPP_QUAD_XOR1, 0xf>((uint32_t)r, 0u);
        r += (int)dpp_u32<DPP_QUAD_XOR2, 0xf>((uint32_t)r, 0u);
        if (c < n2 && q == 0 && r < k2) select(ic);
      }
      __syncthreads();
      // the ids in id order: thread t's chunks (taken word or'ed with selected word), their counts
      // scanned over the workgroup in thread (= id) order, then each thread writes its chunks' ids
      uint64_t mk[TK_CPT];
      uint32_t mine = 0;
#pragma unroll
      for (int j = 0; j < TK_CPT; ++j) {
        const int ch = tid * cpt + j;
        mk[j] = (j < cpt && ch < nchunk) ? (tw[j] | s_sbit[ch]) : 0ull;
        mine += (uint32_t)__popcll(mk[j]);
      }
      uint32_t total;
      uint32_t pos = wg_scan32(mine, (uint32_t*)s_tmp, &total);
#pragma unroll
      for (int j = 0; j < TK_CPT; ++j) {
        uint64_t m = mk[j];
        const int id0 = (tid * cpt + j) * 64;
        while (m != 0) {
          const int bit = __builtin_ctzll(m);
          if (pos < (uint32_t)k) ids[pos] = id0 + bit;
          ++pos;
          m &= m - 1;
        }
      }
      if (tid == 0) a.out_count[s] = k;
      return;
    }
    __syncthreads();
    if (tid == 0) {
      s_na = 0;
      s_nc = 0;
    }
  }

  // ---- 2. the bin of the k-th block, from the coarse histogram ----
  if (tid == 0) {
    s_na = 0;
    s_nc = 0;
  }
  {
    // thread t owns bins 4095-4t .. 4092-4t (descending)
    const uint32_t* gh = a.hist + (int64_t)s * TK_BINS;
    const int top = TK_BINS - 1 - 4 * tid;
    uint32_t c4[4];
    uint64_t loc = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      c4[r] = gh[top - r];
      loc += c4[r];
    }
    uint64_t tot;
    uint64_t before = wg_scan64(loc, s_tmp, &tot);
    if (before < (uint64_t)k && before + loc >= (uint64_t)k) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (before + c4[r] >= (uint64_t)k) {
          s_T = (uint32_t)(top - r);
          s_krem = k - (int)before;
          break;
        }
        before += c4[r];
      }
    }
    __syncthreads();
  }
  const uint32_t T = s_T;
  int krem = s_krem;

  // ---- one sweep: ids above bin T are taken; bin T's scores become candidates ----
  const bool lists_fit = k <= TK_AMAX;
  for_items([&](int, int i, double x) {
    const uint32_t cb = coarse_bin(x);
    if (i < nb && cb >= T) {
      if (cb > T) {
        const uint32_t slot = atomicAdd(&s_na, 1u);
        if (slot < TK_AMAX) s_aid[slot] = i;
      } else {
        const uint32_t slot = atomicAdd(&s_nc, 1u);
        if (slot < TK_CMAX) {
          s_ckey[slot] = order_key(x);
          s_cid[slot] = i;
        }
      }
    }
  });
  __syncthreads();
  const int nc = (int)s_nc;

  if (lists_fit && nc <= TK_CMAX) {
    // Exact rank of each candidate: the number of candidates ahead of it in the sort order,
    // counted by its own thread over broadcast LDS reads; the krem of rank < krem are taken.
    for (int c = tid; c < nc; c += TK_THREADS) {
      const uint64_t kc = s_ckey[c];
      const int32_t ic = s_cid[c];
      int r = 0;
#pragma unroll 8
      for (int o = 0; o < nc; ++o) {
        const uint64_t ko = s_ckey[o];
        const int32_t io = s_cid[o];
        r += (int)((ko > kc) | ((ko == kc) & (io < ic)));
      }
      if (r < krem) s_aid[atomicAdd(&s_na, 1u)] = ic;
    }
    __syncthreads();
    // the k taken ids, ascending: an id's place is the number of taken ids below it
    for (int e = tid; e < k; e += TK_THREADS) {
      const int32_t ie = s_aid[e];
      int r = 0;
#pragma unroll 8
      for (int o = 0; o < k; ++o) r += (int)(s_aid[o] < ie);
      ids[r] = ie;
    }
    if (tid == 0) a.out_count[s] = k;
    return;
  }

  // ---- fallback (more than TK_CMAX candidates or k > TK_AMAX): radix refinement inside bin T ----
  // Skip the bits all candidates share, then 8-bit digits until the chosen digit holds exactly the
  // keys still needed or all bits are fixed; ties at the threshold go to the lowest ids.
  uint64_t prefix = 0, mask = 0;
  {
    uint64_t kmin = ~0ull, kmax = 0;
    for_items([&](int, int i, double x) {
      if (i < nb && coarse_bin(x) == T) {
        const uint64_t ok = order_key(x);
        kmin = ok < kmin ? ok : kmin;
        kmax = ok > kmax ? ok : kmax;
      }
    });
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint64_t a0 = __shfl_xor(kmin, off), a1 = __shfl_xor(kmax, off);
      kmin = a0 < kmin ? a0 : kmin;
      kmax = a1 > kmax ? a1 : kmax;
    }
    if (lane == 0) {
      s_red[0][w] = kmin;
      s_red[1][w] = kmax;
    }
    __syncthreads();
    kmin = ~0ull;
    kmax = 0;
    for (int i = 0; i < TK_WAVES; ++i) {
      kmin = s_red[0][i] < kmin ? s_red[0][i] : kmin;
      kmax = s_red[1][i] > kmax ? s_red[1][i] : kmax;
    }
    if (kmin == kmax) {
      prefix = kmin;
      mask = ~0ull;  // every candidate ties: the lowest krem ids are taken
    } else {
      int hb = 63 - __builtin_clzll(kmin ^ kmax);  // highest bit where candidates differ
      mask = hb == 63 ? 0ull : ~((2ull << hb) - 1);
      prefix = kmin & mask;
      while (true) {
        const int lo = hb >= 7 ? hb - 7 : 0;
        const int nd = hb - lo + 1;
        const uint64_t dmask = ((1ull << nd) - 1) << lo;
        __syncthreads();
        for (int i = tid; i < 256; i += TK_THREADS) s_dig[i] = 0;
        __syncthreads();
        for_items([&](int, int i, double x) {
          if (i < nb && coarse_bin(x) == T) {
            const uint64_t ok = order_key(x);
            if ((ok & mask) == prefix) lds_count(s_dig, (uint32_t)((ok & dmask) >> lo));
          }
        });
        __syncthreads();
        if (tid < 64) {
          // wave 0 finds the digit where the count from the top reaches krem: lane l owns digits
          // 255-4l .. 252-4l (descending); digits past 2^nd are empty
          uint32_t c4[4], loc = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int d = 255 - 4 * lane - r;
            c4[r] = d < (1 << nd) ? s_dig[d] : 0u;
            loc += c4[r];
          }
          uint32_t incl = loc;
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
          }
          uint32_t above = incl - loc;
          if (above < (uint32_t)krem && incl >= (uint32_t)krem) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if (above + c4[r] >= (uint32_t)krem) {
                const int dsel = 255 - 4 * lane - r;
                const int kr = krem - (int)above;
                s_krem = kr;
                s_prefix = prefix | ((uint64_t)dsel << lo);
                s_done = ((int)c4[r] == kr) || lo == 0;
                break;
              }
              above += c4[r];
            }
          }
        }
        __syncthreads();
        krem = s_krem;
        prefix = s_prefix;
        mask |= dmask;
        if (s_done) break;
        hb = lo - 1;
      }
    }
  }
  // gt: taken for certain; eq: tied at the threshold (the first krem of them by id are taken)
  auto classify = [&](int i, double x, bool& gt, bool& eq) {
    const uint32_t cb = coarse_bin(x);
    const uint64_t om = order_key(x) & mask;
    gt = (i < nb) & ((cb > T) | ((cb == T) & (om > prefix)));
    eq = (i < nb) & (cb == T) & (om == prefix);
  };
  // compaction in id order: a count sweep, a 16-entry scan of the waves' counts, a write sweep
  {
    uint32_t ng = 0, ne = 0;
    for_items([&](int, int i, double x) {
      bool gt, eq;
      classify(i, x, gt, eq);
      ng += (uint32_t)__popcll(__ballot(gt));
      ne += (uint32_t)__popcll(__ballot(eq));
    });
    if (lane == 0) {
      s_wg[w] = ng;
      s_we[w] = ne;
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t g = lane < TK_WAVES ? s_wg[lane] : 0u, e = lane < TK_WAVES ? s_we[lane] : 0u;
      uint32_t gi = g, ei = e;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(gi, off), z = __shfl_up(ei, off);
        if (lane >= off) {
          gi += y;
          ei += z;
        }
      }
      if (lane < TK_WAVES) {
        s_wg[lane] = gi - g;
        s_we[lane] = ei - e;
      }
    }
    __syncthreads();
    uint32_t run_g = s_wg[w], run_e = s_we[w];
    for_items([&](int, int i, double x) {
      bool gt, eq;
      classify(i, x, gt, eq);
      const uint64_t mg = __ballot(gt), me = __ballot(eq);
      const uint32_t eb = run_e + lanes_below(me);
      const uint32_t pos = run_g + lanes_below(mg) + min(eb, (uint32_t)krem);
      if ((gt || (eq && eb < (uint32_t)krem)) && pos < (uint32_t)k) ids[pos] = i;
      run_g += (uint32_t)__popcll(mg);
      run_e += (uint32_t)__popcll(me);
    });
  }
  if (tid == 0) a.out_count[s] = k;
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

int topk_nsel(int max_blocks) { return (max_blocks + SEL_ITEMS - 1) / SEL_ITEMS; }

// Workspace: coarse histograms [S][4096] u32 | selection counts [S][nsel][2] u32 | taken bits
// [S][nsel][32] u32 | candidate keys [S][nsel][1024] u64 | candidate ids [S][nsel][1024] i32 | scores
// [S][max_blocks] f64 (when the caller keeps none).  Every part starts 8-byte aligned.
size_t topk_workspace_bytes(int n_streams, int max_blocks, int k, int scores_external) {
  (void)k;
  const size_t S = (size_t)n_streams, nsel = (size_t)topk_nsel(max_blocks);
  size_t b = S * TK_BINS * sizeof(uint32_t);
  b += S * nsel * 2 * sizeof(uint32_t);
  b += S * nsel * (SEL_ITEMS / 32) * sizeof(uint32_t);
  b += S * nsel * SEL_ITEMS * sizeof(uint64_t);
  b += S * nsel * SEL_ITEMS * sizeof(int32_t);
  if (!scores_external) b += S * (size_t)max_blocks * sizeof(double);
  return b;
}

template <bool QBF16, int NCH, int R>
void launch_scores_t(const TopkArgs& a, int n_streams, hipStream_t st) {
  constexpr int per_wg = (SC_THREADS / 64) * 8 * R;
  dim3 grid((a.max_blocks + per_wg - 1) / per_wg, n_streams);
  hipLaunchKernelGGL((scores_kernel<QBF16, NCH, R>), grid, dim3(SC_THREADS), 0, st, a);
}

template <bool QBF16>
void launch_scores(const TopkArgs& a, int n_streams, hipStream_t st) {
  const int nch = (a.idx_dim + 3) / 4;  // 4-dim chunks a row; a lane takes ceil(nch / 8)
  if (nch <= 8) launch_scores_t<QBF16, 1, 4>(a, n_streams, st);
  else if (nch <= 16) launch_scores_t<QBF16, 2, 2>(a, n_streams, st);
  else if (nch <= 32) launch_scores_t<QBF16, 4, 2>(a, n_streams, st);
  else if (nch <= 64) launch_scores_t<QBF16, 8, 1>(a, n_streams, st);
  else if (nch <= 128) launch_scores_t<QBF16, 16, 1>(a, n_streams, st);
  else launch_scores_t<QBF16, 32, 1>(a, n_streams, st);
}

hipError_t launch_scores_topk(const TopkArgs& a, bool qi_bf16, int n_streams, hipStream_t st) {
  if (n_streams <= 0) return hipSuccess;
  hipError_t e;
  if (a.max_blocks > 0) {
    if (qi_bf16) launch_scores<true>(a, n_streams, st);
    else launch_scores<false>(a, n_streams, st);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.max_blocks > 0) {
    dim3 grid((a.max_blocks + HK_ITEMS - 1) / HK_ITEMS, n_streams);
    hipLaunchKernelGGL(hist_kernel, grid, dim3(HK_THREADS), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.max_blocks > 0) {
    hipLaunchKernelGGL(select_kernel, dim3(a.nsel, n_streams), dim3(SEL_THREADS), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(topk_kernel, dim3(n_streams), dim3(TK_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace paged
