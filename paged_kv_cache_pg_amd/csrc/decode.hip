// Dense and sparse decode attention over a paged KV cache (split partials + combine).
//
// TensorFold PR #1169 "What this changes": fn_attn_chunks reads its key and value
// tiles through pg_at, looking a key's row up once per tile (key_at in shared
// memory, beside key_ids).  PR #1170 commit ce5b78d: the contiguous path branches
// once instead of testing the table for every key.  Here the only table test is
// inside pg_at, taken once per key per tile while key_at is staged in LDS.
//
// Work decomposition (fixed by the stream's own key count n only, so a stream's
// bytes never depend on the page size, the table or the other streams):
//   tiles of 64 keys; tps = 4 * ceil(tiles / 160) tiles a split; split c holds
//   tiles [c*tps, (c+1)*tps); wave w of the split's workgroup takes the w-th
//   contiguous quarter of them.
// A wave processes one tile in three phases:
//   QK:   16 lanes a key, 4 keys a step; each lane holds 16 dims of q for the G
//         query heads of the KV group and reduces its partial dots across its
//         16-lane row with DPP; scores go to LDS.
//   soft: online softmax over the tile (running max m and sum l a head).
//   PV:   32 lanes a key, 2 keys a step; each lane accumulates G x 8 outputs.
// Waves merge in order inside the workgroup, splits merge in order in the
// combine kernel.  No atomics anywhere.
#include "internal.h"

namespace paged {

namespace {

constexpr int TILE = 64;
constexpr int NWAVE = 4;
constexpr int WGS = 64 * NWAVE;

__host__ __device__ inline int dec_tiles(int n) { return (n + TILE - 1) / TILE; }
__host__ __device__ inline int dec_tps(int ntiles) {
  const int t = (ntiles + 159) / 160;
  return NWAVE * (t < 1 ? 1 : t);
}
__host__ __device__ inline int dec_splits(int n) {
  const int nt = dec_tiles(n);
  if (nt == 0) return 0;
  const int tps = dec_tps(nt);
  return (nt + tps - 1) / tps;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over a 16-lane DPP row; every lane of the row ends with the same bits.
__device__ __forceinline__ float row16_sum(float x) {
  x += dppf<0xB1>(x);   // quad_perm(1,0,3,2): partner lane ^ 1
  x += dppf<0x4E>(x);   // quad_perm(2,3,0,1): partner lane ^ 2
  x += dppf<0x141>(x);  // row_half_mirror: quad q <-> quad 1-q inside each half row
  x += dppf<0x140>(x);  // row_mirror: half row 0 <-> half row 1
  return x;
}

template <int G>
__device__ __forceinline__ float head_max(float v) {
#pragma unroll
  for (int off = G; off < 64; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

template <int G>
__device__ __forceinline__ float head_sum(float v) {
#pragma unroll
  for (int off = G; off < 64; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

// Orders this wave's LDS writes before its later LDS reads (no cross-wave sync).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <bool BF16>
__device__ __forceinline__ float dot16(const uint4& q, const uint4& k, float acc) {
  if constexpr (BF16) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.x), __builtin_bit_cast(bf16x2_t, k.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.y), __builtin_bit_cast(bf16x2_t, k.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.z), __builtin_bit_cast(bf16x2_t, k.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w), __builtin_bit_cast(bf16x2_t, k.w), acc, false);
  } else {
    acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
    acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
    acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
    acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  }
  return acc;
}

template <bool BF16>
__device__ __forceinline__ void unpack16(const uint4& v, float* f) {
  if constexpr (BF16) {
    f[0] = bf16lo(v.x); f[1] = bf16hi(v.x); f[2] = bf16lo(v.y); f[3] = bf16hi(v.y);
    f[4] = bf16lo(v.z); f[5] = bf16hi(v.z); f[6] = bf16lo(v.w); f[7] = bf16hi(v.w);
  } else {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
}

// Number of keys a stream attends to: its length (dense) or 4 x its selected blocks (sparse).
__device__ __forceinline__ int stream_keys(const DecArgs& a, int s) {
  const int v = a.lens[s];
  if (a.ids != nullptr) return 4 * min(max(v, 0), a.ids_stride);
  return min(max(v, 0), a.max_len);
}

template <bool BF16, int G>
__global__ __launch_bounds__(WGS, 2) void decode_split_kernel(DecArgs a) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int ROWB = HD * ES;    // bytes a row
  constexpr int NCQ = ROWB / 256;  // 16-byte chunks a lane in QK (16 lanes a key)
  constexpr int NCP = ROWB / 512;  // 16-byte chunks a lane in PV (32 lanes a key)
  constexpr int EPC = 16 / ES;     // elements a chunk
  constexpr int NO = NCP * EPC;    // outputs a lane a head (8)

  __shared__ int64_t s_keyat[NWAVE][TILE];
  __shared__ float s_sc[NWAVE][TILE * G];
  __shared__ float s_alpha[NWAVE][G];
  __shared__ float s_o[NWAVE][G][HD];
  __shared__ float s_m[NWAVE][G];
  __shared__ float s_l[NWAVE][G];

  const int s = blockIdx.z, g = blockIdx.y, c = blockIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = stream_keys(a, s);
  const int nt = dec_tiles(n);
  if (nt == 0) return;
  const int tps = dec_tps(nt);
  const int ns = (nt + tps - 1) / tps;
  if (c >= ns) return;
  const int qt = tps / NWAVE;
  const int t_begin = c * tps + w * qt;
  const int t_end = min(t_begin + qt, nt);

  const int j16 = lane & 15, grp = lane >> 4;
  const int j32 = lane & 31, half = lane >> 5;
  const int max_blocks = a.max_len >> 2;

  // q rows of the G query heads of KV head g: 16 dims a lane (chunks at 256*cc + 16*j16).
  uint4 qr[G][NCQ];
  {
    const char* qb = (const char*)a.q + ((int64_t)s * a.hq + (int64_t)g * G) * ROWB;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int cc = 0; cc < NCQ; ++cc) qr[h][cc] = *(const uint4*)(qb + h * ROWB + 256 * cc + 16 * j16);
  }

  float m_run = NEG_INF, l_run = 0.f;  // for head lane % G
  float o[G][NO];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < NO; ++e) o[h][e] = 0.f;

  for (int t = t_begin; t < t_end; ++t) {
    // key_ids -> key_at: one table lookup a key a tile.
    {
      const int i = t * TILE + lane;
      int pos = -1;
      if (i < n) {
        if (a.ids != nullptr) {
          const int b = a.ids[(int64_t)s * a.ids_stride + (i >> 2)];
          if (b >= 0 && b < max_blocks) pos = 4 * b + (i & 3);
        } else {
          pos = i;
        }
      }
      s_keyat[w][lane] = pos >= 0 ? pg_at(a.pg, s, g, pos, ROWB) : (int64_t)-1;
    }
    wave_lds_sync();

    // QK: 4 keys a step.
#pragma unroll 4
    for (int st = 0; st < TILE / 4; ++st) {
      const int kk = st * 4 + grp;
      const int64_t off = s_keyat[w][kk];
      uint4 kr[NCQ];
      if (off >= 0) {
        const char* kp = a.kb + off + 16 * j16;
#pragma unroll
        for (int cc = 0; cc < NCQ; ++cc) kr[cc] = *(const uint4*)(kp + 256 * cc);
      } else {
#pragma unroll
        for (int cc = 0; cc < NCQ; ++cc) kr[cc] = make_uint4(0u, 0u, 0u, 0u);
      }
      float acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float x = 0.f;
#pragma unroll
        for (int cc = 0; cc < NCQ; ++cc) x = dot16<BF16>(qr[h][cc], kr[cc], x);
        acc[h] = row16_sum(x);
      }
      float v = acc[0];
#pragma unroll
      for (int h = 1; h < G; ++h) v = (j16 == h) ? acc[h] : v;
      if (j16 < G) s_sc[w][kk * G + j16] = (off >= 0) ? v * a.zscale : NEG_INF;
    }
    wave_lds_sync();

    // Online softmax over the tile: lane handles flat entries i*64 + lane (head lane % G).
    float ev[G];
    float tmax = NEG_INF;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      ev[i] = s_sc[w][i * 64 + lane];
      tmax = fmaxf(tmax, ev[i]);
    }
    tmax = head_max<G>(tmax);
    const float m_new = fmaxf(m_run, tmax);
    float tsum = 0.f;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float p = (ev[i] == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(ev[i] - m_new);
      s_sc[w][i * 64 + lane] = p;
      tsum += p;
    }
    tsum = head_sum<G>(tsum);
    const float alpha = (m_run == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run = l_run * alpha + tsum;
    m_run = m_new;
    if (lane < G) s_alpha[w][lane] = alpha;
    wave_lds_sync();

    // PV: 2 keys a step.
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float al = s_alpha[w][h];
#pragma unroll
      for (int e = 0; e < NO; ++e) o[h][e] *= al;
    }
#pragma unroll 4
    for (int st = 0; st < TILE / 2; ++st) {
      const int kk = st * 2 + half;
      const int64_t off = s_keyat[w][kk];
      float vf[NO];
      if (off >= 0) {
        const char* vp = a.vb + off + 16 * j32;
#pragma unroll
        for (int cc = 0; cc < NCP; ++cc) unpack16<BF16>(*(const uint4*)(vp + 512 * cc), vf + cc * EPC);
      } else {
#pragma unroll
        for (int e = 0; e < NO; ++e) vf[e] = 0.f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = s_sc[w][kk * G + h];
#pragma unroll
        for (int e = 0; e < NO; ++e) o[h][e] = fmaf(p, vf[e], o[h][e]);
      }
    }
    wave_lds_sync();
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
      for (int cc = 0; cc < NCP; ++cc) {
        const int e0 = (512 * cc + 16 * j32) / ES;
#pragma unroll
        for (int e = 0; e < EPC; ++e) s_o[w][h][e0 + e] = o[h][cc * EPC + e];
      }
  }
  if (lane < G) {
    s_m[w][lane] = m_run;
    s_l[w][lane] = l_run;
  }
  __syncthreads();

  // Merge the four waves in order; thread d owns output dimension d.
  const int d = threadIdx.x;
#pragma unroll
  for (int h = 0; h < G; ++h) {
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

__global__ __launch_bounds__(256) void decode_combine_kernel(DecArgs a) {
  const int h = blockIdx.x, s = blockIdx.y, d = threadIdx.x;
  const int n = stream_keys(a, s);
  const int ns = dec_splits(n);
  float* outp = a.out + ((int64_t)s * a.hq + h) * HD;
  const int64_t row0 = ((int64_t)s * a.hq + h) * a.ns_max;
  float M = NEG_INF;
  for (int c = 0; c < ns; ++c) M = fmaxf(M, a.part_ml[(row0 + c) * 2]);
  float O = 0.f, L = 0.f;
  for (int c = 0; c < ns; ++c) {
    const float mc = a.part_ml[(row0 + c) * 2];
    const float sc = (mc == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(mc - M);
    O += sc * a.part_o[(row0 + c) * HD + d];
    L += sc * a.part_ml[(row0 + c) * 2 + 1];
  }
  outp[d] = (L > 0.f) ? O / L : 0.f;
}

template <bool BF16, int G>
hipError_t launch_t(const DecArgs& a, int n_streams, hipStream_t st) {
  dim3 grid(a.ns_max, a.hkv, n_streams);
  hipLaunchKernelGGL((decode_split_kernel<BF16, G>), grid, dim3(WGS), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.hq, n_streams), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int dec_splits_max(int max_keys) {
  const int nt = dec_tiles(max_keys);
  const int a = (nt + NWAVE - 1) / NWAVE;
  return a < 40 ? a : 40;
}

hipError_t launch_decode(const DecArgs& a, bool bf16, int G, int n_streams, hipStream_t st) {
  if (n_streams <= 0) return hipSuccess;
  if (bf16) {
    switch (G) {
      case 1: return launch_t<true, 1>(a, n_streams, st);
      case 2: return launch_t<true, 2>(a, n_streams, st);
      case 4: return launch_t<true, 4>(a, n_streams, st);
      case 8: return launch_t<true, 8>(a, n_streams, st);
    }
  } else {
    switch (G) {
      case 1: return launch_t<false, 1>(a, n_streams, st);
      case 2: return launch_t<false, 2>(a, n_streams, st);
      case 4: return launch_t<false, 4>(a, n_streams, st);
      case 8: return launch_t<false, 8>(a, n_streams, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace paged
