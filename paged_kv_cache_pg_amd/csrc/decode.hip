// Dense and sparse decode attention over a paged KV cache (split partials + combine).
//
// TensorFold PR #1169 "What this changes": fn_attn_chunks gets its key and value
// tiles via pg_at, resolving each key's row a single time per tile and keeping the
// result (key_at) in shared memory next to key_ids.  PR #1170 commit ce5b78d: the contiguous path branches
// once instead of testing the table for every key.  Here the only table test is
// inside pg_at, taken once per key per tile while key_at is staged in LDS.
//
// Work decomposition (fixed by the stream's own key count n only, so a stream's
// bytes never depend on the page size, the table or the other streams):
//   tiles of 64 keys; tps = 8 * ceil(tiles / 128) tiles a split (at most 16
//   splits); split c holds tiles [c*tps, (c+1)*tps); wave w of the split's
//   8-wave workgroup takes the w-th contiguous eighth of them.
// A wave processes one tile in three phases:
//   QK:   16 lanes a key, 4 keys a step; each lane holds 16 dims of q for the G
//         query heads of the KV group and reduces its partial dots across its
//         16-lane row with permlane swaps and DPP; scores go to LDS.
//   soft: online softmax over the tile (running max m and sum l a head).
//   PV:   32 lanes a key, 4 keys a step; each lane accumulates G x 8 outputs.
// The 16 K steps and 16 V steps of a tile form one sequence of loads; a ring keeps
// the next steps in flight across the softmax and across tile boundaries, so the
// memory pipe never drains between phases or tiles.
// Waves merge in order inside the workgroup, splits merge in order in the
// combine kernel.  No atomics anywhere.
//
// Element types: float32 and bf16 rows, with q of the same type.  (e4m3 rows take the
// MFMA decode, decode_mfma.hip.)
#include "split.h"

namespace paged {

namespace {

// 1 KiB of zero bytes (a float32 row): the row a masked key reads (its zero V adds 0 to the PV sums,
// and its score is replaced by -inf), and the word read in place of a block id or a table entry when
// there are none (its value then adds nothing).  Never written.
__device__ __attribute__((aligned(16))) char zero_row_d[1024];
typedef const char __attribute__((address_space(1)))* gptr_t;

// Tuning knobs (compile-time; the defaults are the measured best on MI355X).
#ifndef PAGED_DEC_RING
#define PAGED_DEC_RING 4         // 4-key steps of bf16 K/V buffered a lane (float32 rows: 2)
#endif

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <int ET> struct Rows {
  static_assert(ET == ET_F32 || ET == ET_BF16, "float32 or bf16 rows");
  static constexpr int ROWB = ET == ET_F32 ? HD * 4 : HD * 2;  // K/V (and q) row bytes
  static constexpr int QROWB = ROWB;
  static constexpr int NCQ = ROWB / 256;  // 16-byte K chunks a lane in QK (16 lanes a key)
  static constexpr int NQC = QROWB / 256; // 16-byte q chunks a lane and head
};

template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Exchange halves: x keeps its lower 32 lanes and takes y's lower 32 lanes into its upper half; y gets the
// two upper halves (gfx950 permlane swaps).  x + y then reduces x over lane pairs (l, l^32) in the lower
// half and y in the upper half.
__device__ __forceinline__ void swap32(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
// The same between rows (16 lanes) 0 and 1 and between rows 2 and 3.
__device__ __forceinline__ void swap16(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}

// A key's dot products are spread over 16 lanes: lane q of a quad in each of the 4 rows (quad = key).
// Recursive halving across rows (swaps) then a butterfly inside the quad leaves, in every lane of row r,
// the complete dots of heads  2r, 2r+1 (G = 8),  r (G = 4),  r/2 (G = 2),  0 (G = 1).
template <int G>
struct QkReduce {
  static constexpr int NR = G >= 8 ? 2 : 1;  // values a lane keeps
  __device__ static __forceinline__ void run(float (&a)[G], float (&res)[NR]) {
    if constexpr (G == 8) {
#pragma unroll
      for (int k = 0; k < 4; ++k) swap32(a[k], a[k + 4]);
      float b[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) b[k] = a[k] + a[k + 4];   // rows 0,1: head k; rows 2,3: head k+4
      swap16(b[0], b[2]);
      swap16(b[1], b[3]);
      res[0] = b[0] + b[2];                                   // rows 0..3: heads 0, 2, 4, 6
      res[1] = b[1] + b[3];                                   // rows 0..3: heads 1, 3, 5, 7
    } else if constexpr (G == 4) {
      swap32(a[0], a[2]);
      swap32(a[1], a[3]);
      float b0 = a[0] + a[2], b1 = a[1] + a[3];               // rows 0,1: heads 0,1; rows 2,3: heads 2,3
      swap16(b0, b1);
      res[0] = b0 + b1;                                       // rows 0..3: heads 0..3
    } else if constexpr (G == 2) {
      swap32(a[0], a[1]);
      float b0 = a[0] + a[1], b1 = b0;                        // rows 0,1: head 0; rows 2,3: head 1
      swap16(b0, b1);
      res[0] = b0 + b1;
    } else {
      float y = a[0];
      swap32(a[0], y);
      float b0 = a[0] + y, b1 = b0;
      swap16(b0, b1);
      res[0] = b0 + b1;
    }
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      res[k] += dppf<0xB1>(res[k]);  // quad_perm(1,0,3,2)
      res[k] += dppf<0x4E>(res[k]);  // quad_perm(2,3,0,1)
    }
  }
  // head of value k held by a lane of row r
  __device__ static __forceinline__ int head(int r, int k) {
    if constexpr (G == 8) return 2 * r + k;
    else if constexpr (G == 4) return r;
    else if constexpr (G == 2) return r >> 1;
    else return 0;
  }
  // rows that write (one copy of each head)
  __device__ static __forceinline__ bool writer_row(int r) {
    if constexpr (G >= 4) return true;
    else if constexpr (G == 2) return (r & 1) == 0;
    else return r == 0;
  }
};

// Over the 8 lanes l ^ {G, 2G, 4G} (the 8 partial sums of one head; with G < 8 each group of 8G lanes
// holds a full copy).
template <int G>
__device__ __forceinline__ float head_max8(float v) {
#pragma unroll
  for (int off = G; off < 8 * G; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

template <int G>
__device__ __forceinline__ float head_sum8(float v) {
#pragma unroll
  for (int off = G; off < 8 * G; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

// Partial dot product of a lane's q chunks with its K chunks (16 lanes a key).
//   f32:  4 chunks of 4 dims;  bf16: 2 chunks of 8 dims.
template <int ET>
__device__ __forceinline__ float qk_dot(const uint4 (&q)[Rows<ET>::NQC], const uint4 (&k)[Rows<ET>::NCQ]) {
  float acc = 0.f;
#pragma unroll
  for (int cc = 0; cc < Rows<ET>::NCQ; ++cc) {
    if constexpr (ET == ET_BF16) {
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[cc].x), __builtin_bit_cast(bf16x2_t, k[cc].x), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[cc].y), __builtin_bit_cast(bf16x2_t, k[cc].y), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[cc].z), __builtin_bit_cast(bf16x2_t, k[cc].z), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[cc].w), __builtin_bit_cast(bf16x2_t, k[cc].w), acc, false);
    } else {
      acc = fmaf(__uint_as_float(q[cc].x), __uint_as_float(k[cc].x), acc);
      acc = fmaf(__uint_as_float(q[cc].y), __uint_as_float(k[cc].y), acc);
      acc = fmaf(__uint_as_float(q[cc].z), __uint_as_float(k[cc].z), acc);
      acc = fmaf(__uint_as_float(q[cc].w), __uint_as_float(k[cc].w), acc);
    }
  }
  return acc;
}

// The 8 values a lane takes of one V row in PV (32 lanes a key; dims 8*j32 .. 8*j32+7 for bf16,
// dims 4*j32 + {0..3, 128..131} for float32).  v holds the lane's chunks of the row in load order.
template <int ET>
__device__ __forceinline__ void pv_unpack(const uint4& v0, const uint4& v1, float* f) {
  if constexpr (ET == ET_BF16) {
    f[0] = bf16lo(v0.x); f[1] = bf16hi(v0.x); f[2] = bf16lo(v0.y); f[3] = bf16hi(v0.y);
    f[4] = bf16lo(v0.z); f[5] = bf16hi(v0.z); f[6] = bf16lo(v0.w); f[7] = bf16hi(v0.w);
  } else {
    f[0] = __uint_as_float(v0.x); f[1] = __uint_as_float(v0.y); f[2] = __uint_as_float(v0.z); f[3] = __uint_as_float(v0.w);
    f[4] = __uint_as_float(v1.x); f[5] = __uint_as_float(v1.y); f[6] = __uint_as_float(v1.z); f[7] = __uint_as_float(v1.w);
  }
}

// One 4-key step of loads, the same register footprint for both kinds: a K step (QK, 16 lanes a
// key) fills x[0 .. NCQ-1]; a V step (PV, 32 lanes a key, two half steps of 2 keys) fills half step j's
// part of x (chunks NCP*j .. NCP*j+NCP-1).
template <int ET>
struct StepBuf {
  uint4 x[Rows<ET>::NCQ];
};

template <int ET, int G, int RING, bool NTK, bool NTV>
__global__ __launch_bounds__(WGS, 1) void decode_split_kernel(DecArgs a) {
  using RT = Rows<ET>;
  constexpr int ROWB = RT::ROWB;     // bytes a K/V row
  constexpr int QROWB = RT::QROWB;   // bytes a q row
  constexpr int NCQ = RT::NCQ;       // 16-byte K chunks a lane in QK
  constexpr int NQC = RT::NQC;       // 16-byte q chunks a lane and head
  constexpr int NCP = ROWB / 512;    // V chunks a lane in PV
  constexpr int NO = 8;              // outputs a lane a head
  constexpr int NSTEP = TILE / 4;    // 4-key steps a tile and phase
  constexpr int SPT = 2 * NSTEP;     // load steps a tile: NSTEP of K, then NSTEP of V
  constexpr int DEPTH = RING - 1;    // steps of K/V in flight ahead of the one computed
  static_assert(SPT % RING == 0, "ring slots must be compile-time");
  using Buf = StepBuf<ET>;

  // key_at kept as the K and V row pointers themselves (the zero row for a masked key), so a load adds
  // only its byte offset: no select, no base, no sign test a load
  __shared__ gptr_t s_kp[NWAVE][4][TILE];
  __shared__ gptr_t s_vp[NWAVE][4][TILE];
  __shared__ float s_sc[NWAVE][TILE * G];
  __shared__ float s_alpha[NWAVE][G];
  __shared__ float s_o[NWAVE][G][HD];
  __shared__ float s_m[NWAVE][G];
  __shared__ float s_l[NWAVE][G];

  // g: the group of G q heads g*G .. g*G+G-1; gk: their KV head (a KV head's q heads may be spread
  // over 2^kvshift groups)
  // blockIdx.y = j * Hkv + gk: the 2^kvshift workgroups of a KV head are Hkv * ns_max ids apart, so
  // with the round-robin placement of workgroups on XCDs (linear id mod 8) they share one XCD's L2
  // whenever Hkv * ns_max is a multiple of 8
  const int s = a.s0 + (int)blockIdx.z, c = blockIdx.x;
  const int gk = (int)blockIdx.y % a.hkv;
  const int g = (gk << a.kvshift) | ((int)blockIdx.y / a.hkv);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = stream_keys(a, s);
  const int nt = dec_tiles(n);
  if (nt == 0) return;
  const int tps = dec_tps(nt);
  const int ns = (nt + tps - 1) / tps;
  if (c >= ns) return;
  const int qt = tps / NWAVE;
  const int t_begin = c * tps + w * qt;
  const int T = max(0, min(t_begin + qt, nt) - t_begin);  // tiles of this wave

  // QK: the key of a step is the quad index inside the row; the lane's dims chunk is jj (chunks jj and jj+16).
  const int grp = (lane & 15) >> 2, row = lane >> 4;
  const int jj = row * 4 + (lane & 3);
  const int j32 = lane & 31, half = lane >> 5;
  const int max_blocks = a.max_len >> 2;

  // q rows of this (stream, KV head)
  const char* qrow = (const char*)a.q + ((int64_t)s * a.hq + (int64_t)g * G) * QROWB;
  // The zero row (its address taken once, kept in scalar registers): the row a masked key reads, and
  // the word read in place of a block id or a table entry when there are none.
  gptr_t zg = (gptr_t)zero_row_d;
  asm volatile("" : "+s"(zg));
  const char* zrow = (const char*)zg;

  // Key ids: key (tile tt, lane) is position i = (t_begin + tt) * 64 + lane (dense) or 4 * ids[i / 4] + i % 4
  // (sparse); -1 when masked.  The id and table loads are issued early and finished later so that their
  // latency hides behind the steps in flight; every index is clamped so each load reads valid memory.
  // Both are issued whether or not there is an id list or a table (reading a word of the zero row
  // instead, which then enters the result as + 0, so that no path can drop the load): a load under a
  // branch leaves the compiler unsure how many loads follow it, and its wait for that load becomes a
  // wait for every load in flight.
  auto load_id = [&](int tt) -> int {
    const int i = (t_begin + tt) * TILE + lane;
    const int32_t* p = a.ids != nullptr ? a.ids + ((int64_t)s * a.ids_stride + ((i < n && tt < T) ? (i >> 2) : 0))
                                        : (const int32_t*)zrow;
    return *p;  // the zero word when there are no ids
  };
  auto load_page = [&](int pos) -> int32_t {
    const int32_t e = *pg_entry(a.pg, s, pos >= 0 ? pos : 0, (const int32_t*)zrow);
    return e + (a.pg.table != nullptr ? 0 : s);  // e: the zero word when there is no table
  };
  auto key_pos = [&](int tt, int id) -> int {
    const int i = (t_begin + tt) * TILE + lane;
    if (i >= n || tt >= T) return -1;
    if (a.ids == nullptr) return i + id;  // id: the zero word
    return (id >= 0 && id < max_blocks) ? 4 * id + (i & 3) : -1;
  };

  // Loads of global step gs = SPT * tt + i: i < NSTEP is K step i of tile tt, else V step i - NSTEP.
  // Every load is issued (masked keys, and every key of a tile past the wave's last, read the zero row
  // instead) so none sits under a branch.
  auto load_step = [&](int tt, int i, Buf& b) {
    if (i < NSTEP) {
      const char* kp = (const char*)s_kp[w][tt & 3][4 * i + grp];
#pragma unroll
      for (int cc = 0; cc < NCQ; ++cc) b.x[cc] = ld_stream<NTK>(kp + 256 * cc + 16 * jj);
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const char* vp = (const char*)s_vp[w][tt & 3][4 * (i - NSTEP) + 2 * j + half];
#pragma unroll
        for (int cc = 0; cc < NCP; ++cc) b.x[NCP * j + cc] = ld_stream<NTV>(vp + 512 * cc + 16 * j32);
      }
    }
  };

  // q rows of the G query heads of KV head g: the lane's 16 dims, chunks at 256*cc + 16*jj (the dims
  // its K chunks hold).
  uint4 qr[G][NQC];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int cc = 0; cc < NQC; ++cc) qr[h][cc] = *(const uint4*)(qrow + h * QROWB + 256 * cc + 16 * jj);

  float m_run = NEG_INF, l_run = 0.f;  // for head lane % G
  float o[G][NO];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < NO; ++e) o[h][e] = 0.f;

  if (T > 0) {
    {
      const int pos0 = key_pos(0, load_id(0));
      const int32_t page0 = load_page(pos0);
      const int64_t off0 = pg_offset(a.pg, page0, gk, pos0 >= 0 ? pos0 : 0, ROWB);
      s_kp[w][0][lane] = pos0 >= 0 ? (gptr_t)(a.kb + off0) : zg;
      s_vp[w][0][lane] = pos0 >= 0 ? (gptr_t)(a.vb + off0) : zg;
    }
    int id_next = load_id(1);
    wave_lds_sync();
    Buf buf[RING];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) load_step(0, d, buf[d]);

    for (int t = 0; t < T; ++t) {
      // key_ids -> key_at for tile t+1: one table lookup a key, written four steps later and first
      // needed DEPTH steps before tile t+1 starts
      const int pos1 = key_pos(t + 1, id_next);
      const int32_t page1 = load_page(pos1);
      id_next = load_id(t + 2);

#pragma unroll
      for (int i = 0; i < SPT; ++i) {
        if (i == 4) {
          const int64_t off1 = pg_offset(a.pg, page1, gk, pos1 >= 0 ? pos1 : 0, ROWB);
          s_kp[w][(t + 1) & 3][lane] = pos1 >= 0 ? (gptr_t)(a.kb + off1) : zg;
          s_vp[w][(t + 1) & 3][lane] = pos1 >= 0 ? (gptr_t)(a.vb + off1) : zg;
          wave_lds_sync();
        }
        if (i == NSTEP) {
          // Online softmax over tile t.  Lane l takes head hh = l % G and the 8 keys 8k + m (k = 0..7,
          // in order) of m = (l / G) % 8; a head's 8 partial sums meet in a 3-level butterfly.  The
          // tree is the same for every G (with G < 8 the lanes past 8G repeat the first 8G), so a
          // head's bytes do not depend on how many heads share the wave.
          wave_lds_sync();
          float* sc = s_sc[w];
          const int hh = lane % G, m8 = (lane / G) & 7;
          float ev[8];
          float tmax = NEG_INF;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            ev[k] = sc[(8 * k + m8) * G + hh];
            tmax = fmaxf(tmax, ev[k]);
          }
          tmax = head_max8<G>(tmax);
          const float m_new = fmaxf(m_run, tmax);
          float tsum = 0.f;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float p = (ev[k] == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(ev[k] - m_new);
            if (lane < 8 * G) sc[(8 * k + m8) * G + hh] = p;
            tsum += p;
          }
          tsum = head_sum8<G>(tsum);
          const float alpha = (m_run == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
          l_run = l_run * alpha + tsum;
          m_run = m_new;
          if (lane < G) s_alpha[w][lane] = alpha;
          wave_lds_sync();
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float al = s_alpha[w][h];
#pragma unroll
            for (int e = 0; e < NO; ++e) o[h][e] *= al;
          }
        }
        // prefetch global step SPT*t + i + DEPTH (possibly in the next tile)
        {
          const int ii = i + DEPTH;
          if (ii < SPT) load_step(t, ii, buf[ii % RING]);
          else load_step(t + 1, ii - SPT, buf[ii % RING]);
        }
        const Buf& cur = buf[i % RING];
        if (i < NSTEP) {
          float acc[G];
#pragma unroll
          for (int h = 0; h < G; ++h) acc[h] = qk_dot<ET>(qr[h], cur.x);
          using R = QkReduce<G>;
          float res[R::NR];
          R::run(acc, res);
          const int kk = 4 * i + grp;
          if ((lane & 3) == 0 && R::writer_row(row)) {
            const bool valid = s_kp[w][t & 3][kk] != zg;
#pragma unroll
            for (int k = 0; k < R::NR; ++k)
              s_sc[w][kk * G + R::head(row, k)] = valid ? res[k] * a.zscale : NEG_INF;
          }
        } else {
          const float* pp = s_sc[w];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int kk = 4 * (i - NSTEP) + 2 * j + half;
            float vf[NO];
            pv_unpack<ET>(cur.x[NCP * j], cur.x[NCP * j + NCP - 1], vf);
#pragma unroll
            for (int h = 0; h < G; ++h) {
              const float p = pp[kk * G + h];
#pragma unroll
              for (int e = 0; e < NO; ++e) o[h][e] = fmaf(p, vf[e], o[h][e]);
            }
          }
        }
      }
      // every lane is done reading this tile's probabilities before the next tile's scores land
      wave_lds_sync();
    }
  }

  // Even and odd keys were accumulated by the two half waves: add them.
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < NO; ++e) o[h][e] += __shfl_xor(o[h][e], 32);

  if (half == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < NO; ++e) {
        // f32: dims 4*j32 + {0..3} and 128 + 4*j32 + {0..3}; bf16: dims 8*j32 + e
        const int d = ET == ET_F32 ? (e < 4 ? 4 * j32 + e : 128 + 4 * j32 + e - 4) : 8 * j32 + e;
        s_o[w][h][d] = o[h][e];
      }
  }
  if (lane < G) {
    s_m[w][lane] = m_run;
    s_l[w][lane] = l_run;
  }
  __syncthreads();

  // Merge the waves in order; a thread owns output dimension d of head h for (h, d) = idx / HD, idx % HD.
#pragma unroll
  for (int idx = threadIdx.x; idx < G * HD; idx += WGS) {
    const int h = idx / HD, d = idx % HD;
    float M = NEG_INF;
#pragma unroll
    for (int ww = 0; ww < NWAVE; ++ww) M = fmaxf(M, s_m[ww][h]);
    float O = 0.f, L = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWAVE; ++ww) {
      const float mw = s_m[ww][h];
      const float sc = (mw == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      O += sc * s_o[ww][h][d];
      L += sc * s_l[ww][h];
    }
    const int64_t row = ((int64_t)s * a.hq + (int64_t)g * G + h) * a.ns_max + c;
    a.part_o[row * HD + d] = O;
    if (d == 0) {
      a.part_ml[row * 2] = M;
      a.part_ml[row * 2 + 1] = L;
    }
  }
}

// Merge a (stream, head)'s split partials in split order; thread d owns dimension d.
static_assert(MAX_SPLITS <= 64, "the combine kernel keeps one split a lane");

__device__ __forceinline__ float lane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// A stream's output rows are its nq window queries x hq heads (one query in plain decode).  Every wave
// derives the splits' weights itself (lane c holds split c's (m, l); the reference max and the
// running sum walk the lanes in split order through scalar reads), so no wave waits on another.
__global__ __launch_bounds__(256) void decode_combine_kernel(DecArgs a) {
  const int h = blockIdx.x, s = blockIdx.y, d = threadIdx.x;
  const int64_t rows = (int64_t)a.hq * a.nq;
  const int64_t row0 = ((int64_t)s * rows + h) * a.ns_max;
  // Every load is issued before any result is needed: the split count (from the stream's length),
  // the splits' (m, l) and this thread's output dimension of every split slot (slots past ns_max
  // read the last slot; slots past the stream's split count are never used).
  const int n = stream_keys(a, s);
  float po[MAX_SPLITS];
#pragma unroll
  for (int c = 0; c < MAX_SPLITS; ++c) po[c] = a.part_o[(row0 + min(c, a.ns_max - 1)) * HD + d];
  const int lc = threadIdx.x & 63;
  const int64_t mrow = row0 + min(lc, a.ns_max - 1);
  float mc = a.part_ml[mrow * 2], lv = a.part_ml[mrow * 2 + 1];
  const int ns = dec_splits(n);
  float* outp = a.out + ((int64_t)s * rows + h) * HD;
  if (ns == 0) {
    outp[d] = 0.f;
    return;
  }
  if (lc >= ns) {
    mc = NEG_INF;
    lv = 0.f;
  }
  float M = NEG_INF;
#pragma unroll
  for (int cc = 0; cc < MAX_SPLITS; ++cc) M = fmaxf(M, lane_f(mc, cc));
  const float sc = (mc == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(mc - M);
  // The partials were loaded before (m, l), so they have landed by now; taking them here keeps the
  // compiler from moving each load under its split's test below (one memory round trip a split).
#pragma unroll
  for (int c = 0; c < MAX_SPLITS; ++c) asm volatile("" : "+v"(po[c]));
  // L and O in split order
  const float term = sc * lv;
  float L = 0.f, O = 0.f;
#pragma unroll
  for (int c = 0; c < MAX_SPLITS; ++c)
    if (c < ns) {
      L += lane_f(term, c);
      O += lane_f(sc, c) * po[c];
    }
  outp[d] = (L > 0.f) ? O / L : 0.f;
}

// Ring depth: bf16 rows keep three steps in flight a wave.  One step was slower wherever CUs sat idle
// (1 to 3 streams of 40960 keys) and no faster when all were busy; seven was slower for workgroups
// of 2 and 4 heads and spills with 8.  float32 rows, twice the registers a step, keep one.  The
// depth changes only when loads are issued, never the arithmetic, so results do not depend on it.
// Launches the split kernel over streams a.s0 .. a.s0 + n - 1.
template <int ET, int G>
hipError_t launch_split_t(const DecArgs& a, int n, hipStream_t st) {
  dim3 grid(a.ns_max, a.hkv << a.kvshift, n);
  constexpr int R = ET == ET_BF16 ? PAGED_DEC_RING : 2;
  if (dec_v_nontemporal(a.kvshift))
    hipLaunchKernelGGL((decode_split_kernel<ET, G, R, true, true>), grid, dim3(WGS), 0, st, a);
  else if (dec_k_nontemporal(a.kvshift))
    hipLaunchKernelGGL((decode_split_kernel<ET, G, R, true, false>), grid, dim3(WGS), 0, st, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<ET, G, R, false, false>), grid, dim3(WGS), 0, st, a);
  return hipGetLastError();
}

// A KV head's q heads may be spread over up to 2^PAGED_DEC_HSPLIT workgroups, which read the same
// K/V rows (the later reads mostly from L2) with fewer registers each: more waves keep loads in
// flight where the grid alone would leave CUs idle.  That is the case for short key lists (at most
// two tiles a wave), and for batches whose grid is so small that doubling it still fits the CUs in
// one round (one 8-wave workgroup a CU): 1 or 2 streams at 40960 keys.  A head's arithmetic does
// not depend on the heads that share its workgroup, so neither does its output.  float32 rows hold
// twice the q registers of bf16 rows, so a float32 workgroup takes at most 4 heads (8 would spill):
// a group of 8 always runs as two workgroups of 4.
#ifndef PAGED_DEC_HSPLIT
#define PAGED_DEC_HSPLIT 2
#endif

// CUs of the current device (asked once a device).
int device_cus() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev >= 64) {
    int n = 0;
    return hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? n : 0;
  }
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) cus[dev] = n;
  }
  return cus[dev];
}

// The split kernel over streams a.s0 .. a.s0 + n - 1, with the head split chosen for them.
template <int ET>
hipError_t launch_split_g(const DecArgs& a0, int G, int n, bool short_keys, hipStream_t st) {
  constexpr int GMAX = ET == ET_F32 ? 4 : 8;  // heads a workgroup at most
  DecArgs a = a0;
  a.kvshift = 0;
  if (short_keys) {
    while (a.kvshift < PAGED_DEC_HSPLIT && (G >> a.kvshift) > 1) ++a.kvshift;
  } else {
    const long wgs = (long)a.ns_max * a.hkv * n, cus = device_cus();
    while (a.kvshift < PAGED_DEC_HSPLIT && (G >> a.kvshift) > 1 && (wgs << (a.kvshift + 1)) <= cus) ++a.kvshift;
  }
  while ((G >> a.kvshift) > GMAX) ++a.kvshift;
  switch (G >> a.kvshift) {
    case 1: return launch_split_t<ET, 1>(a, n, st);
    case 2: return launch_split_t<ET, 2>(a, n, st);
    case 4: return launch_split_t<ET, 4>(a, n, st);
    case 8: if constexpr (GMAX >= 8) return launch_split_t<ET, 8>(a, n, st); break;
  }
  return hipErrorInvalidValue;
}

// A batch whose grid takes more than one round of workgroups (one a CU) and ends in a partial round
// runs as two split launches: the streams of the whole rounds, then the rest, whose smaller grid
// the head split above can spread over all CUs.  A rest of one stream takes one more with it (5
// streams at 40960 keys: 3 + 2, 9: 7 + 2), as one stream alone keeps too few bytes in flight.
// Every stream's output is the same either way; one combine merges them all.
template <int ET>
hipError_t launch_g(const DecArgs& a, int G, int n_streams, hipStream_t st) {
  const int max_keys = a.ids != nullptr ? 4 * a.ids_stride : a.max_len;
  const bool short_keys = dec_tps(dec_tiles(max_keys)) <= 2 * NWAVE;
  const long w = (long)a.ns_max * a.hkv, cus = device_cus();  // workgroups a stream, unsplit
  int first = n_streams;
  if (!short_keys && w > 0 && w <= cus) {
    const int per_round = (int)(cus / w);
    if (n_streams > per_round && n_streams % per_round != 0) first = n_streams - n_streams % per_round;
    if (n_streams - first == 1 && per_round >= 2) first -= 1;
  }
  hipError_t e = launch_split_g<ET>(a, G, first, short_keys, st);
  if (e == hipSuccess && first < n_streams) {
    DecArgs b = a;
    b.s0 = a.s0 + first;
    e = launch_split_g<ET>(b, G, n_streams - first, short_keys, st);
  }
  if (e != hipSuccess) return e;
  return launch_decode_combine(a, n_streams, st);
}

}  // namespace

// Split slots a (stream, query, head) needs in the workspace.
int dec_splits_max(int max_keys) {
  const int nt = dec_tiles(max_keys);
  const int a = (nt + NWAVE - 1) / NWAVE;
  return a < MAX_SPLITS ? a : MAX_SPLITS;
}

hipError_t launch_decode_combine(const DecArgs& a, int n_streams, hipStream_t st) {
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.hq * a.nq, n_streams), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecArgs& a, int elem, int G, int n_streams, hipStream_t st) {
  if (n_streams <= 0) return hipSuccess;
  switch (elem) {
    case ET_F32: return launch_g<ET_F32>(a, G, n_streams, st);
    case ET_BF16: return launch_g<ET_BF16>(a, G, n_streams, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace paged
