// Decode attention on the matrix cores, for bf16 rows and e4m3 rows (bf16 queries), and for a
// window of several queries a stream.
//
// TensorFold PR #1169 "What this changes": fn_attn_chunks gets its key and value tiles via pg_at,
// resolving each key's row a single time per tile (key_at kept next to key_ids); PR #1170 commit ce5b78d: attention
// partials merged afterwards; commit 5c09685: e4m3 rows with a float32 scale a row through the
// table.  The name fn_attn_chunks_ahead (PR #1169) is taken as the windowed form: W query tokens at
// the end of the cache, query w at position n - W + w seeing keys 0 .. n - W + w.
//
// The split decomposition is the vector-ALU decode's (split.h), so partials merge in the same
// combine kernel.  Per wave and 64-key tile, with the q rows of one KV head -- the W queries x G
// query heads, at most 16 -- as the 16 columns of the MFMA tiles:
//   S^T = K Q^T    MFMA 16x16x32 bf16; A = K fragments loaded from HBM straight into registers
//                  (16 keys x 64 contiguous bytes a load; e4m3 codes widened to bf16 exactly,
//                  which permutes the dims of a 32-dim step; q is loaded in the same order).
//   softmax        a row lives in the lane column {c, c+16, c+32, c+48}; online max/sum in the
//                  log2 domain, the reference max moved only when a tile passes it by more than 8.
//                  e4m3: the score takes the key's K scale, the PV weight p * v_scale (the sum p).
//   O^T += V^T P^T MFMA; B = P^T straight from the S^T accumulators (split into bf16 hi + lo),
//                  A = V^T by transpose reads of a 32-key half tile staged in the wave's LDS (bf16;
//                  e4m3 codes widened on the way in).
// Every K and V byte streams through a ring of R 16-byte loads a lane that runs across phases and
// tiles, so the memory pipe never drains.
#include "mfma.h"
#include "split.h"

namespace paged {

namespace {

#ifndef PAGED_DECM_RING
#define PAGED_DECM_RING 8        // 16-byte loads in flight a lane
#endif

// A K fragment load takes 64 bytes of each of 16 rows; the other half of each 128-byte line is read
// by the next load, and K loads are ordinary cached loads (marked nontemporal when the halves were four
// loads apart, the lines left before their second half was read and K was fetched from HBM twice; with
// the halves back to back, nontemporal K measured no faster for e4m3 and slower for the bf16 window).
// V loads read whole lines: streamed (ld_stream, nontemporal unless several workgroups of a KV head
// read the same rows).
__device__ __forceinline__ uint4 ld_k(const char* p) { return *(const uint4*)p; }

constexpr int HALF = 32;                 // keys a PV half tile
constexpr int VROWB = 2 * HD;            // a staged V row (bf16) in LDS
constexpr int VBUF = HALF * VROWB;       // V staging a wave (16 KiB); the wave's partial O after the loop
constexpr float RESCALE_SLACK = 8.f;     // log2 units a row's reference max may lag behind

static_assert(VBUF >= 16 * HD * 4, "a wave's partial O must fit in its staging buffer");

// The row a masked key reads in place of its own (and the word read in place of a block id or a table
// entry when there are none): zero bytes, whose e4m3 codes are zeros, so a masked key's V row adds
// 0 x 0 to the PV product with no select, whatever the arena holds.  Never written.
__device__ __attribute__((aligned(16))) char zero_row[2 * HD];

// 8 e4m3 codes (two dwords) widened to 8 bf16, exactly.
__device__ __forceinline__ bf16x8 widen8(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <int ET, int G, int W, int R, bool NT>
__global__ __launch_bounds__(WGS, 1) void decode_mfma_kernel(DecArgs a) {
  constexpr bool FP8 = ET == ET_FP8;
  constexpr int NK = FP8 ? 16 : 32;      // K loads a tile (4 key blocks x 4 or 8 steps)
  constexpr int NVH = FP8 ? 8 : 16;      // V loads a half tile
  constexpr int NS = NK + 2 * NVH;       // loads a tile
  constexpr int ROWB = FP8 ? HD : 2 * HD;
  constexpr int ROWS = G * W;
  static_assert(ROWS <= 16, "the window's query rows must fit one MFMA column block");
  static_assert(NS % R == 0 && R < NS - 8, "ring slots must be compile-time and the tile long enough");

  // key_at of a tile kept as the K and V row pointers themselves (the zero row for a masked key), so a
  // load adds only its byte offset: no select, no base, no sign test a load
  typedef const char __attribute__((address_space(1)))* gptr;
  __shared__ gptr s_kp[NWAVE][2][TILE];
  __shared__ gptr s_vp[NWAVE][2][TILE];
  __shared__ __attribute__((aligned(16))) float s_ks[FP8 ? NWAVE : 1][2][TILE];
  __shared__ __attribute__((aligned(16))) float s_vs[FP8 ? NWAVE : 1][2][TILE];
  __shared__ __attribute__((aligned(16))) char s_v[NWAVE][VBUF];
  __shared__ float s_m[NWAVE][16];
  __shared__ float s_l[NWAVE][16];

  // g: the group of G q heads g*G .. g*G+G-1; gk: their KV head (a KV head's q heads may be spread
  // over 2^kvshift groups; each q row is its own MFMA column, so the split changes no arithmetic)
  // blockIdx.y = j * Hkv + gk: the 2^kvshift workgroups of a KV head are Hkv * ns_max ids apart, so
  // with the round-robin placement of workgroups on XCDs (linear id mod 8) they share one XCD's L2
  // whenever Hkv * ns_max is a multiple of 8
  const int s = blockIdx.z, c = blockIdx.x;
  const int gk = (int)blockIdx.y % a.hkv;
  const int g = (gk << a.kvshift) | ((int)blockIdx.y / a.hkv);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, u = l >> 4, c16 = l & 15;
  const int n = stream_keys(a, s);
  const int nt = dec_tiles(n);
  if (nt == 0) return;
  const int tps = dec_tps(nt);
  const int ns = (nt + tps - 1) / tps;
  if (c >= ns) return;
  const int qt = tps / NWAVE;
  const int t_begin = c * tps + w * qt;
  const int T = max(0, min(t_begin + qt, nt) - t_begin);  // tiles of this wave
  const int max_blocks = a.max_len >> 2;

  // This lane's q row (its MFMA column): window query wq, head hh of the group.  Dense keys below lim
  // are visible to it; block lists (one query) see every listed key.
  const int wq = c16 / G, hh = c16 % G;
  const bool vrow = c16 < ROWS;
  const int lim = a.ids == nullptr ? n - (W - 1 - wq) : n;

  // Key ids: key (tile tt, lane) is position i = (t_begin + tt) * 64 + lane (dense) or 4 * ids[i / 4] + i % 4
  // (sparse); -1 when masked.  Every index is clamped so each load reads valid memory.
  // The loads take no branch around them (one under a branch makes the compiler drain every load
  // in flight before the next use of any of them): with no ids or no table they read a word of the
  // zero row, and the value read always enters the result (as + 0), so no path can drop the load.
  // The zero row's address is taken once, kept in scalar registers.
  const char __attribute__((address_space(1)))* zg = (const char __attribute__((address_space(1)))*)zero_row;
  asm volatile("" : "+s"(zg));
  const char* zrow = (const char*)zg;
  auto load_id = [&](int tt) -> int {
    const int i = (t_begin + tt) * TILE + l;
    const int* p = a.ids != nullptr ? a.ids + ((int64_t)s * a.ids_stride + ((i < n && tt < T) ? (i >> 2) : 0))
                                    : (const int*)zrow;
    return *p;
  };
  auto load_entry = [&](int pos) -> int32_t { return *pg_entry(a.pg, s, pos >= 0 ? pos : 0, (const int32_t*)zrow); };
  auto entry_page = [&](int32_t e) -> int32_t { return e + (a.pg.table != nullptr ? 0 : s); };
  auto key_pos = [&](int tt, int id) -> int {
    const int i = (t_begin + tt) * TILE + l;
    if (i >= n || tt >= T) return -1;
    if (a.ids == nullptr) return i + id;  // id: the zero word
    return (id >= 0 && id < max_blocks) ? 4 * id + (i & 3) : -1;
  };

  // Q^T fragments (B operand): lane holds row c16's dims 32ds + 8u .. +7 (bf16 K), or for e4m3 K, step
  // ds = 2t + h, dims 64t + 16u + 8h .. +7 (the dims the widened codes of a 16-byte load hold).
  bf16x8 qf[8];
  {
    const char* qp = (const char*)a.q + (((int64_t)s * W + wq) * a.hq + (int64_t)g * G + hh) * (2 * HD);
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      const int off = FP8 ? 128 * (ds >> 1) + 32 * u + 16 * (ds & 1) : 64 * ds + 16 * u;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (vrow) v = *(const uint4*)(qp + off);
      qf[ds] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Load slot i of a tile: i < NK is K block kb = (i / 2) % 4, step st = 2 (i / 8) + i % 2 (16 keys x 64
  // bytes), so that slots i and i + 1 read the two halves of the same 128-byte lines (e4m3 step 63.0-63.4
  // -> 61.7-62.2 us against blocks in the inner place); each block still takes its steps in increasing
  // order.  Then the two halves' V loads, each 2 (bf16) or 4 (e4m3) rows of 512 / 256 contiguous bytes.
  // (The key_at of a tile past the wave's last holds the zero row for every key.)
  auto load_slot = [&](int tt, int i, uint4& x) {
    int key;
    int boff;
    if (i < NK) {
      key = 16 * ((i >> 1) & 3) + c16;
      boff = 64 * (((i >> 3) << 1) | (i & 1)) + 16 * u;
    } else {
      const int j = (i - NK) % NVH, hf = (i - NK) / NVH;
      key = FP8 ? HALF * hf + 4 * j + (l >> 4) : HALF * hf + 2 * j + (l >> 5);
      boff = FP8 ? 16 * (l & 15) : 16 * (l & 31);
    }
    const gptr p = (i < NK ? s_kp : s_vp)[w][tt & 1][key] + boff;
    x = i < NK ? ld_k((const char*)p) : ld_stream<NT>((const char*)p);
  };

  f32x4 oacc[16];
#pragma unroll
  for (int db = 0; db < 16; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = NEG_INF, l_run = 0.f;

  // e4m3: the scales of a key, read through its page (the lookup its row takes); a masked key reads the
  // region's first scale and gets V scale 0.
  auto scale_off = [&](int32_t page, int pos) -> int64_t { return pos >= 0 ? pg_offset(a.pg, page, gk, pos, 4) : 0; };

  // Bit k of the ballot of a tile: key k of the tile has a row (key_at >= 0).
  uint64_t kv_cur = 0;

  if (T > 0) {
    {
      const int pos0 = key_pos(0, load_id(0));
      const int32_t page0 = entry_page(load_entry(pos0));
      kv_cur = __ballot(pos0 >= 0);
      {
        const int64_t off = pg_offset(a.pg, page0, gk, pos0 >= 0 ? pos0 : 0, ROWB);
        s_kp[w][0][l] = pos0 >= 0 ? (gptr)(a.kb + off) : zg;
        s_vp[w][0][l] = pos0 >= 0 ? (gptr)(a.vb + off) : zg;
      }
      if constexpr (FP8) {
        const int64_t so = scale_off(page0, pos0);
        const float ks = *(const float*)(a.ksb + so), vs = *(const float*)(a.vsb + so);
        s_ks[w][0][l] = ks;
        s_vs[w][0][l] = pos0 >= 0 ? vs : 0.f;
      }
    }
    int id_next = load_id(1);
    wave_lds_sync();
    uint4 rx[R];
#pragma unroll
    for (int d = 0; d < R; ++d) load_slot(0, d, rx[d]);

    // key_ids -> key_at for tile t+1: the table entry is read at the top of tile t, the row offsets
    // written at slot IKA (the entry has long landed, so waiting for it drains no load in flight) and
    // first read at slot NS - R, by the prefetch of tile t+1's first slot
    constexpr int IKA = NS - R - 4;
    static_assert(IKA >= 4, "the table entry needs a few slots to land");
    for (int t = 0; t < T; ++t) {
      const int pos1 = key_pos(t + 1, id_next);
      const int32_t e1 = load_entry(pos1);
      const uint64_t kv_next = __ballot(pos1 >= 0);
      id_next = load_id(t + 2);
      float ks1 = 0.f, vs1 = 0.f;

      f32x4 sacc[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      bf16x8 phi[2], plo[2];

      static_for<NS>([&](auto I) {
        constexpr int i = decltype(I)::value;
        if constexpr (i == IKA) {
          const int32_t page1 = entry_page(e1);
          {
            const int64_t off = pg_offset(a.pg, page1, gk, pos1 >= 0 ? pos1 : 0, ROWB);
            s_kp[w][(t + 1) & 1][l] = pos1 >= 0 ? (gptr)(a.kb + off) : zg;
            s_vp[w][(t + 1) & 1][l] = pos1 >= 0 ? (gptr)(a.vb + off) : zg;
          }
          if constexpr (FP8) {
            const int64_t so = scale_off(page1, pos1);
            ks1 = *(const float*)(a.ksb + so);
            vs1 = *(const float*)(a.vsb + so);
          }
          wave_lds_sync();
        }
        const uint4 x = rx[i % R];
        // prefetch slot i + R (possibly of the next tile)
        if constexpr (i + R < NS) load_slot(t, i + R, rx[i % R]);
        else load_slot(t + 1, i + R - NS, rx[i % R]);

        if constexpr (i < NK) {
          // ---- S^T += K Q^T: key block kb, one (bf16) or two (e4m3) 32-dim steps ----
          constexpr int kb = (i >> 1) & 3, st = ((i >> 3) << 1) | (i & 1);
          if constexpr (FP8) {
            sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8(x.x, x.y), qf[2 * st], sacc[kb], 0, 0, 0);
            sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8(x.z, x.w), qf[2 * st + 1], sacc[kb], 0, 0, 0);
          } else {
            sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x), qf[st], sacc[kb], 0, 0, 0);
          }
        }

        if constexpr (i == NK - 1) {
          // ---- online softmax over tile t: lane holds keys 16kb + 4u + e of its row ----
          const int kbase = (t_begin + t) * TILE;
          const uint64_t kvl = kv_cur >> (4 * u);  // bit 16kb + e: the lane's key 16kb + 4u + e has a row
          float z[4][4];
          float mx = NEG_INF;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            float ksc[4] = {1.f, 1.f, 1.f, 1.f};
            if constexpr (FP8) {
              const float4 k4 = *(const float4*)&s_ks[w][t & 1][16 * kb + 4 * u];
              ksc[0] = k4.x; ksc[1] = k4.y; ksc[2] = k4.z; ksc[3] = k4.w;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // a key counts when it has a row and, for a window's query, is not past the query
              bool valid = vrow & (((kvl >> (16 * kb + e)) & 1) != 0);
              if constexpr (W > 1) valid = valid & (kbase + 16 * kb + 4 * u + e < lim);
              z[kb][e] = valid ? sacc[kb][e] * (a.zscale * ksc[e]) : NEG_INF;
              mx = fmaxf(mx, z[kb][e]);
            }
          }
          mx = col_max(mx);
          const bool move = m_run == NEG_INF || mx > m_run + RESCALE_SLACK;
          const float m_new = move ? fmaxf(m_run, mx) : m_run;
          const float alpha = !move ? 1.f : (m_run == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
          float rs = 0.f;
          float p[4][4];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            float vsc[4] = {1.f, 1.f, 1.f, 1.f};
            if constexpr (FP8) {
              const float4 v4 = *(const float4*)&s_vs[w][t & 1][16 * kb + 4 * u];
              vsc[0] = v4.x; vsc[1] = v4.y; vsc[2] = v4.z; vsc[3] = v4.w;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float pe = (z[kb][e] == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(z[kb][e] - m_new);
              rs += pe;
              p[kb][e] = FP8 ? pe * vsc[e] : pe;
            }
          }
          rs = col_sum(rs);
          l_run = l_run * alpha + rs;
          m_run = m_new;
          // P^T fragment of half hf: element e is key 32hf + 16(e/4) + 4u + e%4, split into bf16 hi + lo
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const f32x2 pv = {p[2 * hf + (e >> 2)][e & 3], p[2 * hf + (e >> 2)][(e & 3) + 1]};
              const bf16x2 hi = __builtin_convertvector(pv, bf16x2);
              const f32x2 rest = pv - __builtin_convertvector(hi, f32x2);
              const bf16x2 lo = __builtin_convertvector(rest, bf16x2);
              phi[hf][e] = hi[0];
              phi[hf][e + 1] = hi[1];
              plo[hf][e] = lo[0];
              plo[hf][e + 1] = lo[1];
            }
          // rescale O only when some row of the wave moved its reference max (multiplying by 1 is exact)
          if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
            for (int db = 0; db < 16; ++db) oacc[db] *= alpha;
          }
        }

        if constexpr (FP8) {
          // tile t+1's scales, stored once their loads have long landed (read from tile t+1 on)
          if constexpr (i == NS - 1) {
            s_ks[w][(t + 1) & 1][l] = ks1;
            s_vs[w][(t + 1) & 1][l] = pos1 >= 0 ? vs1 : 0.f;
          }
        }

        if constexpr (i >= NK) {
          // ---- stage V rows of the half tile in LDS as bf16 (chunks swizzled by v_slot) ----
          constexpr int j = (i - NK) % NVH, hf = (i - NK) / NVH;
          char* vbuf = s_v[w];
          if constexpr (FP8) {
            // a masked key's row is the zero row: zero codes
            const int row = 4 * j + (l >> 4), cc = l & 15;
            *(bf16x8*)(vbuf + row * VROWB + v_slot(row, 2 * cc) * 16) = widen8(x.x, x.y);
            *(bf16x8*)(vbuf + row * VROWB + v_slot(row, 2 * cc + 1) * 16) = widen8(x.z, x.w);
          } else {
            const int row = 2 * j + (l >> 5), cc = l & 31;
            *(uint4*)(vbuf + row * VROWB + v_slot(row, cc) * 16) = x;
          }
          if constexpr (j == NVH - 1) {
            // ---- O^T += V^T P^T over the half tile: 16 dims blocks, hi then lo ----
            wave_lds_sync();
            auto vfrag = [&](int db) {
              const int o = vt_offset(u, c16, db & 7) + 256 * (db >> 3);
              const bf16x4 v1 = lds_tr16(vbuf, o);
              const bf16x4 v2 = lds_tr16(vbuf, o + 16 * VROWB);
              return bf16x8{v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
            };
            bf16x8 vr[2];
            vr[0] = vfrag(0);
            vr[1] = vfrag(1);
#pragma unroll
            for (int db = 0; db < 16; ++db) {
              const bf16x8 vf = vr[db & 1];
              if (db + 2 < 16) vr[db & 1] = vfrag(db + 2);
              oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, phi[hf], oacc[db], 0, 0, 0);
              oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, plo[hf], oacc[db], 0, 0, 0);
            }
            // every lane is done reading the half tile before the next one is written
            wave_lds_sync();
          }
        }
      });
      kv_cur = kv_next;
    }
  }

  // ---- merge the waves in order: each wave's O^T (rows x dims) goes through its staging buffer ----
  float* so = (float*)s_v[w];
#pragma unroll
  for (int db = 0; db < 16; ++db)
    *(float4*)(so + c16 * HD + 16 * db + 4 * u) = make_float4(oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]);
  if (u == 0) {
    s_m[w][c16] = m_run;
    s_l[w][c16] = l_run;
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < ROWS * HD; idx += WGS) {
    const int r = idx / HD, d = idx % HD;
    float M = NEG_INF;
#pragma unroll
    for (int ww = 0; ww < NWAVE; ++ww) M = fmaxf(M, s_m[ww][r]);
    float O = 0.f, L = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWAVE; ++ww) {
      const float mw = s_m[ww][r];
      const float sc = (mw == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      O += sc * ((const float*)s_v[ww])[r * HD + d];
      L += sc * s_l[ww][r];
    }
    const int64_t row = (((int64_t)s * W + r / G) * a.hq + (int64_t)g * G + r % G) * a.ns_max + c;
    a.part_o[row * HD + d] = O;
    if (d == 0) {
      a.part_ml[row * 2] = M;
      a.part_ml[row * 2 + 1] = L;
    }
  }
}

template <int ET, int G, int W>
hipError_t launch_w(const DecArgs& a, int n_streams, hipStream_t st) {
  dim3 grid(a.ns_max, a.hkv << a.kvshift, n_streams);
  if (dec_v_nontemporal(a.kvshift))
    hipLaunchKernelGGL((decode_mfma_kernel<ET, G, W, PAGED_DECM_RING, true>), grid, dim3(WGS), 0, st, a);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<ET, G, W, PAGED_DECM_RING, false>), grid, dim3(WGS), 0, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_combine(a, n_streams, st);
}

// Windows of 2 to 4 queries, as long as window x group fits the 16 columns; one query only over e4m3
// rows (one query over bf16 rows takes the vector-ALU decode).
template <int ET, int G>
hipError_t launch_g(const DecArgs& a, int n_streams, hipStream_t st) {
  switch (a.nq) {
    case 1: if constexpr (ET == ET_FP8) return launch_w<ET, G, 1>(a, n_streams, st); break;
    case 2: return launch_w<ET, G, 2>(a, n_streams, st);
    case 3: if constexpr (3 * G <= 16) return launch_w<ET, G, 3>(a, n_streams, st); break;
    case 4: if constexpr (4 * G <= 16) return launch_w<ET, G, 4>(a, n_streams, st); break;
  }
  return hipErrorInvalidValue;
}

// Short key lists (at most two tiles a wave): a KV head's q heads spread over up to
// 2^PAGED_DECM_HSPLIT workgroups, as in the vector-ALU decode (more waves with loads in flight).
#ifndef PAGED_DECM_HSPLIT
#define PAGED_DECM_HSPLIT 2
#endif
template <int ET>
hipError_t launch_e(const DecArgs& a0, int G, int n_streams, hipStream_t st) {
  DecArgs a = a0;
  const int max_keys = a.ids != nullptr ? 4 * a.ids_stride : a.max_len;
  a.kvshift = 0;
  if (dec_tps(dec_tiles(max_keys)) <= 2 * NWAVE) {
    while (a.kvshift < PAGED_DECM_HSPLIT && (G >> a.kvshift) > 1) ++a.kvshift;
  }
  switch (G >> a.kvshift) {
    case 1: return launch_g<ET, 1>(a, n_streams, st);
    case 2: return launch_g<ET, 2>(a, n_streams, st);
    case 4: return launch_g<ET, 4>(a, n_streams, st);
    case 8: return launch_g<ET, 8>(a, n_streams, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_mfma(const DecArgs& a, int elem, int G, int n_streams, hipStream_t st) {
  if (n_streams <= 0) return hipSuccess;
  if (elem == ET_BF16) return launch_e<ET_BF16>(a, G, n_streams, st);
  if (elem == ET_FP8) return launch_e<ET_FP8>(a, G, n_streams, st);
  return hipErrorInvalidValue;
}

}  // namespace paged
