// Chunked causal prefill over a paged KV cache on MFMA (bf16 in, fp32 accumulate).
//
// TensorFold PR #1170 (maintainer reply): prompt batches that read paged caches take a
// page-run path while flat ones use tensor-core attention; the page-run path had lost
// prompt speed until tensor-core attention came back.  Here one MFMA kernel serves both
// forms: the only difference is pg_at, taken once per key per tile while the tile's key
// offsets are staged in LDS.
//
// A workgroup owns 128 (query, head) rows -- 128/G queries x the G query heads of one KV
// head -- so every K/V tile is read once for all G heads.  Each of its 8 waves owns 16 rows, so
// two waves share a SIMD and one's softmax runs while the other's MFMAs do (four waves of 32
// rows need 420 registers a wave, one wave a SIMD, and each wave then waits on its own chain of
// QK MFMAs -> softmax -> PV MFMAs).  Per 64-key tile:
//   S^T = K Q^T   (MFMA 16x16x32 bf16: A = K rows from LDS, B = Q^T kept in registers).
//                 A lane's accumulators hold 4 keys of one row, so a row's statistics live
//                 in the 4 lanes {c, c+16, c+32, c+48} and never leave a lane column.
//   softmax       fp32 online max/sum in the log2 domain; causal mask key <= query position,
//                 applied only on tiles that cross the diagonal (a tile every row sees whole
//                 takes no mask and no -inf tests).
//                 A row's reference max is moved (and O rescaled) only when a tile's max
//                 passes it by more than 8, so most tiles skip the rescale.
//   O^T += V^T P^T  (MFMA; A = V^T via LDS transpose reads, B = P^T straight from the S^T
//                 accumulators, with P split into bf16 hi + lo so P keeps ~16 bits).
// One barrier a tile: K and V live in two LDS buffers each; the loads of tile t+1 go from
// global memory straight into LDS (no registers), issued at the start of iteration t into the
// buffers tile t-1 left, and are waited for at its end.  The four buffers are separate LDS
// objects and the tile loop is unrolled by two, so that every access names its buffer: with one
// array indexed by tile parity the compiler could not tell a tile's loads from its reads and
// waited for the next tile's loads before the first K read.  Workgroups of one KV head are spread
// round-robin so that consecutive workgroups (one per XCD) share KV heads two XCDs apiece.
#include "internal.h"
#include "mfma.h"

namespace paged {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#ifndef PAGED_PF_RB
#define PAGED_PF_RB 1               // 16-row blocks a wave (1: eight waves of 16 rows; 2: four of 32)
#endif
#ifndef PAGED_PF_QK_AHEAD
#define PAGED_PF_QK_AHEAD 4         // K fragment reads ahead of their MFMAs
#endif
#ifndef PAGED_PF_PV_AHEAD
#define PAGED_PF_PV_AHEAD 8         // V^T fragment reads (pairs) ahead of their MFMAs
#endif
#ifndef PAGED_PF_ROWS
#define PAGED_PF_ROWS 128           // (query, head) rows a workgroup
#endif
#ifndef PAGED_PF_KT
#define PAGED_PF_KT 64              // keys a tile (a multiple of 32)
#endif
#ifndef PAGED_PF_WG_PER_CU
#define PAGED_PF_WG_PER_CU 1        // workgroups a CU the register budget is set for
#endif
constexpr int RB = PAGED_PF_RB;
constexpr int PF_ROWS = PAGED_PF_ROWS;
constexpr int PF_WAVES = PF_ROWS / (16 * RB);
constexpr int PF_THREADS = 64 * PF_WAVES;
constexpr int PF_KT = PAGED_PF_KT;
constexpr int KB = PF_KT / 16;      // 16-key blocks of S^T a tile
constexpr int NS2 = PF_KT / 32;     // 32-key PV steps a tile
constexpr int ROWB = HD * 2;        // bytes a bf16 key / value row
constexpr int CH = ROWB / 16;       // 16-byte chunks a row (32)
constexpr int TILEB = PF_KT * ROWB; // bytes a K or V tile in LDS (rows unpadded, chunks swizzled)
constexpr int LD_PER_WAVE = PF_KT * CH / PF_THREADS;  // 1 KB global->LDS loads a wave a tile
static_assert(PF_KT % 32 == 0 && PF_KT * CH % PF_THREADS == 0, "tile shape");
constexpr float RESCALE_SLACK = 8.f;  // log2 units a row's running max may lag behind before O is rescaled

template <int G>
__global__ __launch_bounds__(PF_THREADS, PAGED_PF_WG_PER_CU) void prefill_kernel(PreArgs a) {
  constexpr int QB = PF_ROWS / G;  // queries a workgroup
  // two K and two V buffers, four separate LDS objects: the compiler can then tell the buffer a
  // tile's loads land in from the one the tile reads, and does not wait for the former before
  // reading the latter
  __shared__ __attribute__((aligned(16))) char s_k0[TILEB];
  __shared__ __attribute__((aligned(16))) char s_k1[TILEB];
  __shared__ __attribute__((aligned(16))) char s_v0[TILEB];
  __shared__ __attribute__((aligned(16))) char s_v1[TILEB];
  // key_at of a tile kept as the K and V row pointers themselves (the first q row for a key past the
  // keys, valid and finite memory), so a load adds only its chunk offset
  typedef const char __attribute__((address_space(1)))* gptr;
  __shared__ gptr s_kp[2][PF_KT];
  __shared__ gptr s_vp[2][PF_KT];

  // w is read from the first lane so that the compiler knows it is the same across the wave (wave-uniform
  // LDS addresses, such as the destinations of the global->LDS loads, then stay in scalar registers)
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, u = l >> 4, c16 = l & 15;
  const int nblk = (a.n_q + QB - 1) / QB;
  const int g = blockIdx.x % a.hkv;
  const int qblk = nblk - 1 - (int)(blockIdx.x / a.hkv);  // most work first
  const int q_begin = qblk * QB;
  const int kv_len = a.q_pos0 + a.n_q;
  const int q_last = min(a.n_q, q_begin + QB) - 1;          // last query of the block (chunk index)
  const int kmax = a.causal ? a.q_pos0 + q_last + 1 : kv_len;
  const int nt = (kmax + PF_KT - 1) / PF_KT;

  // rows of this lane: r = 16 RB w + 16rb + c16 -> query qi = r / G, head h = r % G
  int lim[RB];
  bool vrow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = 16 * RB * w + 16 * rb + c16;
    const int qi = q_begin + r / G;
    vrow[rb] = qi < a.n_q;
    lim[rb] = a.causal ? min(a.q_pos0 + qi + 1, kv_len) : kv_len;  // keys < lim are seen
  }

  // Q^T fragments (B operand): lane holds Q[row 16rb + c16][32ds + 8u .. +7]
  bf16x8 qf[RB][8];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = 16 * RB * w + 16 * rb + c16;
    const int qi = q_begin + r / G, h = r % G;
    const char* qp = (const char*)a.q + (((int64_t)qi * a.hq + (int64_t)g * G + h) * HD) * 2;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (vrow[rb]) v = *(const uint4*)(qp + (32 * ds + 8 * u) * 2);
      qf[rb][ds] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // key_at of a tile: thread < 64 looks up one key (slot tt mod 2).  The table entry is read one
  // iteration before its offset is written, so no wave waits on a table read inside the loop.
  auto key_page = [&](int tt) -> int32_t {
    const int key = tt * PF_KT + tid;
    return (tid < PF_KT && tt < nt && key < kmax) ? pg_page(a.pg, 0, key) : 0;
  };
  auto stage_keyat = [&](int tt, int32_t page) {
    if (tid < PF_KT && tt < nt) {
      const int key = tt * PF_KT + tid;
      const int64_t off = pg_offset(a.pg, page, g, key < kmax ? key : 0, ROWB);
      s_kp[tt & 1][tid] = key < kmax ? (gptr)(a.kb + off) : (gptr)a.q;
      s_vp[tt & 1][tid] = key < kmax ? (gptr)(a.vb + off) : (gptr)a.q;
    }
  };
  // One tile's K and V rows, global -> LDS directly (no registers): load i of wave w fills LDS
  // slots (8w + i) * 64 + lane, i.e. rows 2(8w + i) and 2(8w + i) + 1 of each buffer, each lane
  // fetching the chunk that belongs in its slot (the slot maps are involutions).  Keys past kmax
  // read the first q row instead (their key_at): masked keys then meet a zero weight.
  auto load_tile = [&](int tt, char* kbuf, char* vbuf) {
#pragma unroll
    for (int i = 0; i < LD_PER_WAVE; ++i) {
      const int slot = (LD_PER_WAVE * w + i) * 64 + l;
      const int row = slot / CH, pos = slot % CH;
      const char* ks = (const char*)s_kp[tt & 1][row] + k_slot(row, pos) * 16;
      const char* vs = (const char*)s_vp[tt & 1][row] + v_slot(row, pos) * 16;
      __builtin_amdgcn_global_load_lds((const void*)ks,
                                       (__attribute__((address_space(3))) void*)(kbuf + (LD_PER_WAVE * w + i) * 1024),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)vs,
                                       (__attribute__((address_space(3))) void*)(vbuf + (LD_PER_WAVE * w + i) * 1024),
                                       16, 0, 0);
    }
  };
  // Swizzled LDS read offsets, the same for every tile: K fragment (kb, ds) of this lane is row
  // 16kb + c16, chunk 4ds + u -> koff[ds] + 8192 kb.  V^T half-fragment (s2, db, second half h)
  // is row r1 = 32s2 + 4u + c16/4 + 16h, dims 16db + 4(c16%4): its slot is (2db + j) ^ 2x with
  // j = (c16%4)/2 and x = r1 mod 8 = (4u + c16/4) mod 8, i.e. 2(db ^ x) + j, so with db = 8dh + dl
  // the offset is voff[dl] + 256 dh + 16384 s2 + 8192 h.
  int koff[8], voff[8];
#pragma unroll
  for (int ds = 0; ds < 8; ++ds) koff[ds] = c16 * ROWB + k_slot(c16, 4 * ds + u) * 16;
#pragma unroll
  for (int dl = 0; dl < 8; ++dl) voff[dl] = vt_offset(u, c16, dl);

  // S^T of one tile: sacc[kb][rb] holds keys 16kb + 4u + i of rows 16rb + c16, summed over ds
  // in order.  Steps run ds-major so that the 8 accumulators take turns (a dependent MFMA is
  // 8 issues behind its predecessor); the K fragment of step (ds, kb) is read QK_AHEAD steps
  // before its two MFMAs.
  auto qk = [&](const char* kbuf, f32x4 (&sacc)[KB][RB]) {
    constexpr int QK_AHEAD = PAGED_PF_QK_AHEAD;
    auto kfrag = [&](int st) {
      const int ds = st / KB, kb = st % KB;
      return *(const bf16x8*)(kbuf + koff[ds] + 16 * ROWB * kb);
    };
    bf16x8 ring[QK_AHEAD];
#pragma unroll
    for (int st = 0; st < QK_AHEAD; ++st) ring[st] = kfrag(st);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sacc[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 8 * KB; ++st) {
      const bf16x8 kf = ring[st % QK_AHEAD];
      if (st + QK_AHEAD < 8 * KB) ring[st % QK_AHEAD] = kfrag(st + QK_AHEAD);
      const int ds = st / KB, kb = st % KB;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        sacc[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rb][ds], sacc[kb][rb], 0, 0, 0);
    }
    // keep one fragment read a step: reads QK_AHEAD steps ahead, two MFMAs a step
    __builtin_amdgcn_sched_group_barrier(0x100, QK_AHEAD, 0);
#pragma unroll
    for (int st = 0; st < 8 * KB - QK_AHEAD; ++st) {
      __builtin_amdgcn_sched_group_barrier(0x008, RB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, RB * QK_AHEAD, 0);
  };

  f32x4 oacc[16][RB];
#pragma unroll
  for (int db = 0; db < 16; ++db)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) oacc[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = NEG_INF;
    l_run[rb] = 0.f;
  }

  // ---- prologue: K(0), V(0) into LDS ----
  stage_keyat(0, key_page(0));
  stage_keyat(1, key_page(1));
  int32_t page_next = key_page(2);
  __syncthreads();
  load_tile(0, s_k0, s_v0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Tile t reads kcur / vcur and loads tile t+1 into knext / vnext (the buffers tile t-1 left).
  auto tile = [&](int t, const char* kcur, const char* vcur, char* knext, char* vnext) {
    const int k0 = t * PF_KT;
    // K(t+1), V(t+1) land during this tile and are waited for at its end
    if (t + 1 < nt) load_tile(t + 1, knext, vnext);
    stage_keyat(t + 2, page_next);
    page_next = key_page(t + 3);

    f32x4 s_cur[KB][RB];
    qk(kcur, s_cur);

    bf16x8 phi[NS2][RB], plo[NS2][RB];  // [32-key step][rb]
    float alpha_rb[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      // A tile every row of the block sees whole (below the diagonal) takes no mask; on the others a
      // masked key's score becomes -inf in place, and exp2(-inf - m) = 0 gives it weight 0, so both
      // kinds of tile share one max and one exponential loop.
      const bool full = __all(k0 + PF_KT <= lim[rb]);
      float z[KB][4];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) z[kb][i] = s_cur[kb][rb][i] * a.zscale;
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = k0 + 16 * kb + 4 * u + i;
            z[kb][i] = key < lim[rb] ? z[kb][i] : NEG_INF;
          }
      }
      float mx = NEG_INF;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, z[kb][i]);
      mx = col_max(mx);
      // The reference max moves only when the tile's max passes it by more than RESCALE_SLACK
      // (so P <= 2^RESCALE_SLACK): most tiles leave O untouched.
      const bool move = m_run[rb] == NEG_INF || mx > m_run[rb] + RESCALE_SLACK;
      const float m_new = move ? fmaxf(m_run[rb], mx) : m_run[rb];
      const float alpha = !move ? 1.f : (m_run[rb] == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
      alpha_rb[rb] = alpha;
      // a row that has seen no key yet keeps m_new = -inf with every score -inf: subtract 0 instead
      const float m_sub = m_new == NEG_INF ? 0.f : m_new;
      float rs = 0.f;
      float p[KB][4];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kb][i] = __builtin_amdgcn_exp2f(z[kb][i] - m_sub);
          rs += p[kb][i];
        }
      rs = col_sum(rs);
      l_run[rb] = l_run[rb] * alpha + rs;
      m_run[rb] = m_new;
      // P^T fragment of 32-key step s2: element e is key 32s2 + 16(e/4) + 4u + e%4
#pragma unroll
      for (int s2 = 0; s2 < NS2; ++s2)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const f32x2 pv = {p[2 * s2 + (e >> 2)][e & 3], p[2 * s2 + (e >> 2)][(e & 3) + 1]};
          const bf16x2 hi = __builtin_convertvector(pv, bf16x2);
          const f32x2 rest = pv - __builtin_convertvector(hi, f32x2);
          const bf16x2 lo = __builtin_convertvector(rest, bf16x2);
          phi[s2][rb][e] = hi[0];
          phi[s2][rb][e + 1] = hi[1];
          plo[s2][rb][e] = lo[0];
          plo[s2][rb][e + 1] = lo[1];
        }
    }

    // rescale O only when some row of the wave moved its reference max (multiplying by 1 is exact)
    bool any_move = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) any_move = any_move || alpha_rb[rb] != 1.f;
    if (__ballot(any_move) != 0) {
#pragma unroll
      for (int db = 0; db < 16; ++db)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) oacc[db][rb] *= alpha_rb[rb];
    }

    // ---- O^T += V(t)^T P(t)^T ----
    // Step (s2, db pair): two V^T fragments (four transpose reads), then 8 MFMAs: the hi parts of
    // both dims blocks and both row blocks, then the lo parts, so an accumulator's lo MFMA is 4
    // issues behind its hi MFMA (each accumulator still adds hi then lo, s2 = 0 then 1).
    // Fragments are read PV_AHEAD steps ahead.
    {
      constexpr int PV_AHEAD = PAGED_PF_PV_AHEAD;
      const char* vbuf = vcur;
      auto vfrag = [&](int s2, int db) {
        const int o = voff[db & 7] + 256 * (db >> 3) + 32 * ROWB * s2;
        const bf16x4 v1 = lds_tr16(vbuf, o);
        const bf16x4 v2 = lds_tr16(vbuf, o + 16 * ROWB);
        return bf16x8{v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
      };
      bf16x8 ring[PV_AHEAD][2];
#pragma unroll
      for (int st = 0; st < PV_AHEAD; ++st)
#pragma unroll
        for (int e = 0; e < 2; ++e) ring[st][e] = vfrag(st >> 3, 2 * (st & 7) + e);
#pragma unroll
      for (int st = 0; st < 8 * NS2; ++st) {
        const int s2 = st >> 3, db0 = 2 * (st & 7);
        bf16x8 vf[2] = {ring[st % PV_AHEAD][0], ring[st % PV_AHEAD][1]};
        if (st + PV_AHEAD < 8 * NS2) {
          const int sn = st + PV_AHEAD;
#pragma unroll
          for (int e = 0; e < 2; ++e) ring[st % PV_AHEAD][e] = vfrag(sn >> 3, 2 * (sn & 7) + e);
        }
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            oacc[db0 + e][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[e], phi[s2][rb], oacc[db0 + e][rb], 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            oacc[db0 + e][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[e], plo[s2][rb], oacc[db0 + e][rb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * PV_AHEAD, 0);
#pragma unroll
      for (int st = 0; st < 8 * NS2 - PV_AHEAD; ++st) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * RB, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * RB * PV_AHEAD, 0);
    }

    // ---- K(t+1) and V(t+1) have landed; every wave is done with K(t) and V(t) ----
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // two tiles an iteration, so that each buffer is a fixed LDS object in each call
  for (int t = 0; t < nt; t += 2) {
    tile(t, s_k0, s_v0, s_k1, s_v1);
    if (t + 1 < nt) tile(t + 1, s_k1, s_v1, s_k0, s_v0);
  }

  // ---- normalise and write: lane holds O^T[16db + 4u + i][row 16rb + c16] ----
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (!vrow[rb]) continue;
    const int r = 16 * RB * w + 16 * rb + c16;
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
