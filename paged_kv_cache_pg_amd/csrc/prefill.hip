// Chunked causal prefill over a paged KV cache on MFMA (bf16 in, fp32 accumulate).
//
// TensorFold PR #1170 (maintainer reply): prompt batches that read paged caches take a
// "page-run path" while flat ones use tensor-core attention; the page-run path had lost
// prompt speed until tensor-core attention came back.  Here one MFMA kernel serves both
// forms: the only difference is pg_at, taken once per key per tile while the tile's key
// offsets are staged in LDS.
//
// A workgroup owns 128 (query, head) rows -- 128/G queries x the G query heads of one KV
// head -- so every K/V tile is read once for all G heads.  Each of its 4 waves owns 32 rows.
// Per 64-key tile:
//   S^T = K Q^T   (MFMA 16x16x32 bf16: A = K rows from LDS, B = Q^T kept in registers).
//                 A lane's accumulators hold 4 keys of one row, so a row's statistics live
//                 in the 4 lanes {c, c+16, c+32, c+48} and never leave a lane column.
//   softmax       fp32 online max/sum in the log2 domain; causal mask key <= query position.
//                 A row's reference max is moved (and O rescaled) only when a tile's max
//                 passes it by more than 8, so most tiles skip the rescale.
//   O^T += V^T P^T  (MFMA; A = V^T via LDS transpose reads, B = P^T straight from the S^T
//                 accumulators, with P split into bf16 hi + lo so P keeps ~16 bits).
// K/V tiles are double-buffered in LDS; the next tile's rows are loaded into registers
// while the current one is computed.  Workgroups of one KV head are spread round-robin so
// that consecutive workgroups (one per XCD) share KV heads two XCDs apiece.
#include "internal.h"

namespace paged {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int PF_ROWS = 128;        // (query, head) rows a workgroup
constexpr int PF_WAVES = 4;         // 32 rows a wave
constexpr int PF_THREADS = 64 * PF_WAVES;
constexpr int PF_KT = 64;           // keys a tile
constexpr int ROWB = HD * 2;        // bytes a bf16 key / value row
constexpr int K_STRIDE = ROWB + 16; // K rows in LDS: 16 rows of a fragment read land 4 banks apart
constexpr int V_STRIDE = ROWB + 32; // V rows in LDS: the 4 rows of a transpose read land 8 banks apart
constexpr int CH = ROWB / 16;       // 16-byte chunks a row (32)
constexpr int LD_PER_THREAD = PF_KT * CH / PF_THREADS;  // 8 chunks of K and of V a thread a tile
constexpr float RESCALE_SLACK = 8.f;  // log2 units a row's running max may lag behind before O is rescaled

__device__ __forceinline__ void swap32(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
// max / sum over the four lanes of a lane column (l, l^16, l^32, l^48); every lane gets the same bits.
__device__ __forceinline__ float col_max(float x) {
  float y = x;
  swap32(x, y);
  x = fmaxf(x, y);
  y = x;
  swap16(x, y);
  return fmaxf(x, y);
}
__device__ __forceinline__ float col_sum(float x) {
  float y = x;
  swap32(x, y);
  x = x + y;
  y = x;
  swap16(x, y);
  return x + y;
}

__device__ __forceinline__ bf16x4 lds_tr16(const char* lds_base, int byte_off) {
  const lds_s16x4* p = (const lds_s16x4*)((__attribute__((address_space(3))) const char*)lds_base + byte_off);
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
}

template <int G>
__global__ __launch_bounds__(PF_THREADS, 1) void prefill_kernel(PreArgs a) {
  constexpr int QB = PF_ROWS / G;  // queries a workgroup
  __shared__ __attribute__((aligned(16))) char s_k[2][PF_KT * K_STRIDE];
  __shared__ __attribute__((aligned(16))) char s_v[2][PF_KT * V_STRIDE];
  __shared__ int64_t s_keyat[2][PF_KT];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, u = l >> 4, c16 = l & 15;
  const int nblk = (a.n_q + QB - 1) / QB;
  const int g = blockIdx.x % a.hkv;
  const int qblk = nblk - 1 - (int)(blockIdx.x / a.hkv);  // most work first
  const int q_begin = qblk * QB;
  const int kv_len = a.q_pos0 + a.n_q;
  const int q_last = min(a.n_q, q_begin + QB) - 1;          // last query of the block (chunk index)
  const int kmax = a.causal ? a.q_pos0 + q_last + 1 : kv_len;
  const int nt = (kmax + PF_KT - 1) / PF_KT;

  // rows of this lane: r = 32w + 16rb + c16 -> query qi = r / G, head h = r % G
  int prow[2];
  bool vrow[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = 32 * w + 16 * rb + c16;
    const int qi = q_begin + r / G;
    vrow[rb] = qi < a.n_q;
    prow[rb] = a.q_pos0 + qi;
  }

  // Q^T fragments (B operand): lane holds Q[row 16rb + c16][32ds + 8u .. +7]
  bf16x8 qf[2][8];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = 32 * w + 16 * rb + c16;
    const int qi = q_begin + r / G, h = r % G;
    const char* qp = (const char*)a.q + (((int64_t)qi * a.hq + (int64_t)g * G + h) * HD) * 2;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (vrow[rb]) v = *(const uint4*)(qp + (32 * ds + 8 * u) * 2);
      qf[rb][ds] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // key_at of a tile: thread < 64 looks up one key
  auto stage_keyat = [&](int tt) {
    if (tid < PF_KT) {
      const int key = tt * PF_KT + tid;
      s_keyat[tt & 1][tid] = key < kmax ? pg_at(a.pg, 0, g, key, ROWB) : (int64_t)-1;
    }
  };
  uint4 kreg[LD_PER_THREAD], vreg[LD_PER_THREAD];
  auto load_tile = [&](int tt) {
#pragma unroll
    for (int i = 0; i < LD_PER_THREAD; ++i) {
      const int idx = i * PF_THREADS + tid;
      const int key = idx / CH, ch = idx % CH;
      const int64_t off = s_keyat[tt & 1][key];
      if (off >= 0) {
        kreg[i] = *(const uint4*)(a.kb + off + ch * 16);
        vreg[i] = *(const uint4*)(a.vb + off + ch * 16);
      } else {
        kreg[i] = make_uint4(0u, 0u, 0u, 0u);
        vreg[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LD_PER_THREAD; ++i) {
      const int idx = i * PF_THREADS + tid;
      const int key = idx / CH, ch = idx % CH;
      *(uint4*)(s_k[buf] + key * K_STRIDE + ch * 16) = kreg[i];
      *(uint4*)(s_v[buf] + key * V_STRIDE + ch * 16) = vreg[i];
    }
  };

  f32x4 oacc[16][2];
#pragma unroll
  for (int db = 0; db < 16; ++db)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) oacc[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {NEG_INF, NEG_INF}, l_run[2] = {0.f, 0.f};

  // prologue: tile 0 into LDS, tile 1 into registers
  stage_keyat(0);
  __syncthreads();
  load_tile(0);
  store_tile(0);
  if (nt > 1) stage_keyat(1);
  __syncthreads();
  if (nt > 1) load_tile(1);

  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    const char* kbuf = s_k[buf];
    const char* vbuf = s_v[buf];
    const int k0 = t * PF_KT;

    // ---- S^T = K Q^T for this tile ----
    f32x4 sacc[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) sacc[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) {
        const bf16x8 kf = *(const bf16x8*)(kbuf + (16 * kb + c16) * K_STRIDE + (32 * ds + 8 * u) * 2);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          sacc[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rb][ds], sacc[kb][rb], 0, 0, 0);
      }
    }

    // ---- online softmax (rows live in lane columns) ----
    bf16x8 phi[2][2], plo[2][2];  // [32-key step][rb]
    float alpha_rb[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int lim = a.causal ? min(prow[rb] + 1, kv_len) : kv_len;
      float z[4][4];
      float mx = NEG_INF;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + 16 * kb + 4 * u + i;
          z[kb][i] = key < lim ? sacc[kb][rb][i] * a.zscale : NEG_INF;
          mx = fmaxf(mx, z[kb][i]);
        }
      mx = col_max(mx);
      // The reference max moves only when the tile's max passes it by more than RESCALE_SLACK
      // (so P <= 2^RESCALE_SLACK): most tiles leave O untouched.
      const bool move = m_run[rb] == NEG_INF || mx > m_run[rb] + RESCALE_SLACK;
      const float m_new = move ? fmaxf(m_run[rb], mx) : m_run[rb];
      const float alpha = !move ? 1.f : (m_run[rb] == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
      alpha_rb[rb] = alpha;
      float rs = 0.f;
      float p[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kb][i] = (z[kb][i] == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(z[kb][i] - m_new);
          rs += p[kb][i];
        }
      rs = col_sum(rs);
      l_run[rb] = l_run[rb] * alpha + rs;
      m_run[rb] = m_new;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = p[2 * s2 + (e >> 2)][e & 3];
          const __bf16 hi = (__bf16)pv;
          phi[s2][rb][e] = hi;
          plo[s2][rb][e] = (__bf16)(pv - (float)hi);
        }
    }

    // rescale O only when some row of the wave moved its reference max (multiplying by 1 is exact)
    if (__builtin_amdgcn_read_exec() &&
        __ballot(alpha_rb[0] != 1.f || alpha_rb[1] != 1.f) != 0) {
#pragma unroll
      for (int db = 0; db < 16; ++db)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) oacc[db][rb] *= alpha_rb[rb];
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int db = 0; db < 16; ++db) {
        // source lane c16 points at key 32s2 + 4u + c16/4 (+16 for the second half), dims 16db + 4(c16%4)
        const int d_off = (16 * db + 4 * (c16 & 3)) * 2;
        const int r1 = 32 * s2 + 4 * u + (c16 >> 2);
        const bf16x4 v1 = lds_tr16(vbuf, r1 * V_STRIDE + d_off);
        const bf16x4 v2 = lds_tr16(vbuf, (r1 + 16) * V_STRIDE + d_off);
        const bf16x8 vf = {v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          oacc[db][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, phi[s2][rb], oacc[db][rb], 0, 0, 0);
          oacc[db][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, plo[s2][rb], oacc[db][rb], 0, 0, 0);
        }
      }
    }

    // ---- next tile: registers -> the other LDS buffer, then prefetch the one after ----
    if (t + 1 < nt) {
      store_tile(buf ^ 1);
      if (t + 2 < nt) stage_keyat(t + 2);
    }
    __syncthreads();
    if (t + 2 < nt) load_tile(t + 2);
  }

  // ---- normalise and write: lane holds O^T[16db + 4u + i][row 16rb + c16] ----
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    if (!vrow[rb]) continue;
    const int r = 32 * w + 16 * rb + c16;
    const int qi = q_begin + r / G, h = r % G;
    float* op = a.out + ((int64_t)qi * a.hq + (int64_t)g * G + h) * HD;
    const float inv = 1.f / l_run[rb];
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      const f32x4 o = oacc[db][rb];
      *(float4*)(op + 16 * db + 4 * u) = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PreArgs& a, int G, hipStream_t st) {
  if (a.n_q <= 0) return hipSuccess;
  const int qb = PF_ROWS / G;
  const int nblk = (a.n_q + qb - 1) / qb;
  dim3 grid(nblk * a.hkv);
  switch (G) {
    case 1: hipLaunchKernelGGL(prefill_kernel<1>, grid, dim3(PF_THREADS), 0, st, a); break;
    case 2: hipLaunchKernelGGL(prefill_kernel<2>, grid, dim3(PF_THREADS), 0, st, a); break;
    case 4: hipLaunchKernelGGL(prefill_kernel<4>, grid, dim3(PF_THREADS), 0, st, a); break;
    case 8: hipLaunchKernelGGL(prefill_kernel<8>, grid, dim3(PF_THREADS), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace paged
