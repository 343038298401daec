// C-ABI entry points of libpagedattn: argument checks, workspace carving, launches.
// Every refusal happens before anything is enqueued; the library allocates
// nothing, keeps no state and never synchronises.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "paged_attn.h"
#include "internal.h"

using namespace paged;

namespace {

constexpr int64_t MAX_POS = (int64_t)1 << 30;

inline bool al(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline int esize(int32_t dt) { return dt == PAGED_FP8_E4M3 ? 1 : dt == PAGED_BF16 ? 2 : 4; }
// types of q, indexer keys, pooled and copied rows
inline bool dtype_ok(int32_t dt) { return dt == PAGED_F32 || dt == PAGED_BF16; }
// types of K/V regions
inline bool kv_dtype_ok(int32_t dt) { return dtype_ok(dt) || dt == PAGED_FP8_E4M3; }

// Page-table checks shared by every call.  need4: page_pos must hold whole blocks of four.
int check_pg(const paged_pg* pg, int32_t dtype, int64_t max_len, bool need4) {
  if (pg == nullptr) return PAGED_EINVAL;
  if (pg->reserved != 0) return PAGED_EINVAL;
  if (pg->page_pos < 1 || pg->page_elems < 1) return PAGED_EINVAL;
  if (need4 && (pg->page_pos % 4) != 0) return PAGED_EINVAL;
  if ((pg->page_elems * esize(dtype)) % 16 != 0) return PAGED_EINVAL;
  if (pg->table != nullptr) {
    if (!al(pg->table, 4) || pg->table_stride < 1) return PAGED_EINVAL;
    if ((int64_t)pg->table_stride * pg->page_pos < max_len) return PAGED_EINVAL;  // the run has fewer pages than max_len needs
  } else {
    if ((int64_t)pg->page_pos < max_len) return PAGED_EINVAL;  // cap rows a head must cover max_len
  }
  return PAGED_OK;
}

int check_kv(const paged_kv* kv, const paged_pg* pg) {
  if (kv == nullptr) return PAGED_EINVAL;
  if (kv->reserved != 0 || !kv_dtype_ok(kv->dtype)) return PAGED_EINVAL;
  if (kv->n_kv_heads < 1) return PAGED_EINVAL;
  if (kv->k == nullptr || kv->v == nullptr || !al(kv->k, 16) || !al(kv->v, 16)) return PAGED_EINVAL;
  if (kv->dtype == PAGED_FP8_E4M3 &&
      (kv->k_scale == nullptr || kv->v_scale == nullptr || !al(kv->k_scale, 4) || !al(kv->v_scale, 4)))
    return PAGED_EINVAL;
  if (kv->head_dim != HD) return PAGED_EUNSUPPORTED;
  if (pg != nullptr && pg->page_elems < (int64_t)kv->n_kv_heads * pg->page_pos * kv->head_dim) return PAGED_EINVAL;
  return PAGED_OK;
}

PgDev to_dev(const paged_pg* pg, int32_t dtype) {
  PgDev d;
  d.table = pg->table;
  d.stride = pg->table_stride;
  d.ptok = pg->page_pos;
  d.page_bytes = pg->page_elems * esize(dtype);
  return d;
}

int group_ok(int32_t hq, int32_t hkv) {
  if (hq < 1 || hkv < 1 || hq % hkv != 0) return PAGED_EINVAL;
  const int G = hq / hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PAGED_EUNSUPPORTED;
  return PAGED_OK;
}

// Workspace: the split partials' o, then their (m, l).
size_t dec_ws(int32_t n_streams, int32_t n_q_heads, int64_t max_keys) {
  if (n_streams <= 0 || n_q_heads <= 0 || max_keys < 0) return 0;
  int ns = dec_splits_max((int)max_keys);
  if (ns < 1) ns = 1;
  const size_t rows = (size_t)n_streams * (size_t)n_q_heads * (size_t)ns;
  return rows * HD * sizeof(float) + rows * 2 * sizeof(float);
}

int hip_status(hipError_t e) { return e == hipSuccess ? PAGED_OK : PAGED_EHIP; }

// Decode, sparse decode (ids != NULL) and the windowed decode (nq > 1 queries a stream): checks the
// request and fills `a` except its workspace pointers; *need = the workspace bytes it takes.  With
// n_streams == 0 there is nothing to launch (PAGED_OK, *need = 0).
int decode_prepare(const void* q, int32_t q_dtype, int32_t n_q_heads, int32_t nq, const paged_kv* kv,
                   const paged_pg* pg, const int32_t* lens, const int32_t* ids, int32_t k, int32_t n_streams,
                   int32_t max_len, float scale, float* out, DecArgs* a, size_t* need) {
  *need = 0;
  if (n_streams < 0 || max_len < 0 || max_len > MAX_POS || nq < 1) return PAGED_EINVAL;
  int r = check_kv(kv, pg);
  if (r) return r;
  r = check_pg(pg, kv->dtype, max_len, ids != nullptr);
  if (r) return r;
  r = group_ok(n_q_heads, kv->n_kv_heads);
  if (r) return r;
  // windows: 1 .. 4 queries, window x group <= 16, on bf16 or e4m3 rows
  if (nq > 1 && (nq > 4 || nq * (n_q_heads / kv->n_kv_heads) > 16 || kv->dtype == PAGED_F32))
    return PAGED_EUNSUPPORTED;
  // q has the rows' type; e4m3 rows take bf16 queries
  const int32_t q_want = kv->dtype == PAGED_FP8_E4M3 ? PAGED_BF16 : kv->dtype;
  if (q_dtype != q_want) return dtype_ok(q_dtype) ? PAGED_EUNSUPPORTED : PAGED_EINVAL;
  if (!isfinite(scale)) return PAGED_EINVAL;
  if (n_streams == 0) return PAGED_OK;
  if (q == nullptr || !al(q, 16) || out == nullptr || !al(out, 16)) return PAGED_EINVAL;
  if (lens == nullptr || !al(lens, 4)) return PAGED_EINVAL;
  int64_t max_keys = max_len;
  if (ids != nullptr) {
    if (k < 1 || !al(ids, 4) || (int64_t)k * 4 > MAX_POS) return PAGED_EINVAL;
    max_keys = (int64_t)4 * k;
  }
  *need = dec_ws(n_streams, n_q_heads * nq, max_keys);

  a->q = q;
  a->kb = (const char*)kv->k;
  a->vb = (const char*)kv->v;
  const bool fp8 = kv->dtype == PAGED_FP8_E4M3;
  a->ksb = fp8 ? (const char*)kv->k_scale : nullptr;
  a->vsb = fp8 ? (const char*)kv->v_scale : nullptr;
  a->pg = to_dev(pg, kv->dtype);
  a->lens = lens;
  a->ids = ids;
  a->ids_stride = ids ? k : 0;
  a->max_len = max_len;
  a->hq = n_q_heads;
  a->hkv = kv->n_kv_heads;
  a->nq = nq;
  a->kvshift = 0;
  a->s0 = 0;
  a->zscale = (float)((double)scale * 1.4426950408889634);
  const int ns = dec_splits_max((int)max_keys);
  a->ns_max = ns < 1 ? 1 : ns;
  a->part_o = nullptr;
  a->part_ml = nullptr;
  a->out = out;
  return PAGED_OK;
}

// Carves the split partials out of `ws` (16-byte aligned, at least the prepared need) and launches.
int decode_launch(DecArgs& a, int32_t q_dtype_rows, void* ws, int32_t n_streams, hipStream_t stream) {
  const size_t rows = (size_t)n_streams * a.hq * a.nq * a.ns_max;
  a.part_o = (float*)ws;
  a.part_ml = (float*)((char*)a.part_o + rows * HD * sizeof(float));
  const bool fp8 = q_dtype_rows == PAGED_FP8_E4M3;
  const int elem = fp8 ? 2 : q_dtype_rows == PAGED_BF16 ? 1 : 0;
  const int G = a.hq / a.hkv;
  // Windows and e4m3 rows take the MFMA decode (e4m3 decode is bound by the vector units there); one
  // query over bf16 or float32 rows takes the vector-ALU decode.
  if (a.nq > 1 || fp8) return hip_status(launch_decode_mfma(a, elem, G, n_streams, stream));
  return hip_status(launch_decode(a, elem, G, n_streams, stream));
}

int decode_common(const void* q, int32_t q_dtype, int32_t n_q_heads, int32_t nq, const paged_kv* kv,
                  const paged_pg* pg, const int32_t* lens, const int32_t* ids, int32_t k, int32_t n_streams,
                  int32_t max_len, float scale, float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  DecArgs a;
  size_t need = 0;
  const int r = decode_prepare(q, q_dtype, n_q_heads, nq, kv, pg, lens, ids, k, n_streams, max_len, scale, out, &a,
                               &need);
  if (r || n_streams == 0) return r;
  if (ws_bytes < need || (need > 0 && (ws == nullptr || !al(ws, 16)))) return PAGED_EWORKSPACE;
  return decode_launch(a, kv->dtype, ws, n_streams, stream);
}

int rows_common(int gather, void* lin, int64_t ss, int64_t sh, int64_t sp, void* region, int32_t n_heads,
                int32_t row_elems, int32_t dtype, const paged_pg* pg, const int32_t* pos_begin,
                const int32_t* pos_end, int32_t n_streams, int32_t max_len, hipStream_t stream) {
  if (!dtype_ok(dtype)) return PAGED_EINVAL;
  if (n_streams < 0 || max_len < 0 || max_len > MAX_POS || n_heads < 1 || row_elems < 1) return PAGED_EINVAL;
  int r = check_pg(pg, dtype, max_len, false);
  if (r) return r;
  const int es = esize(dtype);
  if (((int64_t)row_elems * es) % 16 != 0) return PAGED_EINVAL;
  if (pg->page_elems < (int64_t)n_heads * pg->page_pos * row_elems) return PAGED_EINVAL;
  if (n_streams == 0) return PAGED_OK;
  if (lin == nullptr || region == nullptr || !al(lin, 16) || !al(region, 16)) return PAGED_EINVAL;
  if (pos_begin == nullptr || pos_end == nullptr || !al(pos_begin, 4) || !al(pos_end, 4)) return PAGED_EINVAL;
  if (((ss * es) % 16) || ((sh * es) % 16) || ((sp * es) % 16)) return PAGED_EINVAL;
  RowsArgs a;
  a.lin = (char*)lin;
  a.ss = ss * es;
  a.sh = sh * es;
  a.sp = sp * es;
  a.region = (char*)region;
  a.pg = to_dev(pg, dtype);
  a.begin = pos_begin;
  a.end = pos_end;
  a.n_heads = n_heads;
  a.row_bytes = row_elems * es;
  a.max_len = max_len;
  a.n_streams = n_streams;
  a.gather = gather;
  return hip_status(launch_rows(a, stream));
}

// ---- scratch of the allocation-free decode -------------------------------------------------
// One array a GPU, in the library's own device memory (it lives as long as the process), for callers
// that cannot allocate.  Host code never passes `scratch` itself to a kernel or a copy: on the host
// that name stands for a host-side shadow, not the device array.  Its device address is looked up
// once a device, with that device current, and kept in scratch_dev.
static __device__ __align__(256) char scratch[PAGED_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::atomic<void*> scratch_dev[MAX_DEVICES];
std::mutex scratch_mu;

// The current device's copy of `scratch` (looked up on the first call on that device).
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return PAGED_EHIP;
  void* p = scratch_dev[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(scratch_mu);
    p = scratch_dev[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PAGED_EHIP;
      scratch_dev[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PAGED_OK;
}

}  // namespace

extern "C" {

size_t paged_attn_decode_workspace(int32_t n_streams, int32_t n_q_heads, int32_t max_len) {
  return dec_ws(n_streams, n_q_heads, max_len);
}

int paged_attn_decode(const void* q, int32_t q_dtype, int32_t n_q_heads, const paged_kv* kv, const paged_pg* pg,
                      const int32_t* seq_lens, int32_t n_streams, int32_t max_len, float scale, float* out,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_common(q, q_dtype, n_q_heads, 1, kv, pg, seq_lens, nullptr, 0, n_streams, max_len, scale, out,
                       workspace, workspace_bytes, stream);
}

int paged_attn_decode_noalloc(const void* q, int32_t q_dtype, int32_t n_q_heads, const paged_kv* kv,
                              const paged_pg* pg, const int32_t* seq_lens, int32_t n_streams, int32_t max_len,
                              float scale, float* out, hipStream_t stream) {
  DecArgs a;
  size_t need = 0;
  int r = decode_prepare(q, q_dtype, n_q_heads, 1, kv, pg, seq_lens, nullptr, 0, n_streams, max_len, scale, out, &a,
                         &need);
  if (r || n_streams == 0) return r;
  if (need > (size_t)PAGED_NOALLOC_SCRATCH_BYTES) return PAGED_ESCRATCH;
  void* ws = nullptr;
  r = scratch_of_current_device(&ws);
  if (r) return r;
  return decode_launch(a, kv->dtype, ws, n_streams, stream);
}

size_t paged_attn_decode_window_workspace(int32_t n_streams, int32_t n_q_heads, int32_t n_window, int32_t max_len) {
  if (n_window < 1) return 0;
  return dec_ws(n_streams, n_q_heads * n_window, max_len);
}

int paged_attn_decode_window(const void* q, int32_t q_dtype, int32_t n_q_heads, int32_t n_window, const paged_kv* kv,
                             const paged_pg* pg, const int32_t* seq_lens, int32_t n_streams, int32_t max_len,
                             float scale, float* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_common(q, q_dtype, n_q_heads, n_window, kv, pg, seq_lens, nullptr, 0, n_streams, max_len, scale,
                       out, workspace, workspace_bytes, stream);
}

size_t paged_sparse_attn_workspace(int32_t n_streams, int32_t n_q_heads, int32_t k) {
  if (k < 1) return 0;
  return dec_ws(n_streams, n_q_heads, (int64_t)4 * k);
}

int paged_sparse_attn(const void* q, int32_t q_dtype, int32_t n_q_heads, const paged_kv* kv, const paged_pg* pg,
                      const int32_t* block_ids, const int32_t* n_selected, int32_t k, int32_t n_streams,
                      int32_t max_len, float scale, float* out, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  if (block_ids == nullptr || k < 1) return PAGED_EINVAL;
  return decode_common(q, q_dtype, n_q_heads, 1, kv, pg, n_selected, block_ids, k, n_streams, max_len, scale, out,
                       workspace, workspace_bytes, stream);
}

size_t paged_attn_prefill_workspace(int32_t n_q, int32_t n_q_heads, int32_t kv_len) {
  (void)n_q;
  (void)n_q_heads;
  (void)kv_len;
  return 0;
}

int paged_attn_prefill(const void* q, int32_t q_dtype, int32_t n_q, int32_t q_pos0, int32_t n_q_heads,
                       const paged_kv* kv, const paged_pg* pg, int32_t causal, float scale, float* out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (n_q < 0 || q_pos0 < 0 || (int64_t)q_pos0 + n_q > MAX_POS) return PAGED_EINVAL;
  int r = check_kv(kv, pg);
  if (r) return r;
  r = check_pg(pg, kv->dtype, (int64_t)q_pos0 + n_q, false);
  if (r) return r;
  r = group_ok(n_q_heads, kv->n_kv_heads);
  if (r) return r;
  if (q_dtype != PAGED_BF16 || kv->dtype != PAGED_BF16) return dtype_ok(q_dtype) ? PAGED_EUNSUPPORTED : PAGED_EINVAL;
  if (!isfinite(scale)) return PAGED_EINVAL;
  if (n_q == 0) return PAGED_OK;
  if (q == nullptr || !al(q, 16) || out == nullptr || !al(out, 16)) return PAGED_EINVAL;
  PreArgs a;
  a.q = q;
  a.kb = (const char*)kv->k;
  a.vb = (const char*)kv->v;
  a.pg = to_dev(pg, kv->dtype);
  a.n_q = n_q;
  a.q_pos0 = q_pos0;
  a.hq = n_q_heads;
  a.hkv = kv->n_kv_heads;
  a.causal = causal != 0;
  a.zscale = (float)((double)scale * 1.4426950408889634);
  a.out = out;
  return hip_status(launch_prefill(a, n_q_heads / kv->n_kv_heads, stream));
}

int paged_pool_blocks(const void* ik, void* pooled, int32_t idx_dim, int32_t arena_dtype, const paged_pg* pg,
                      const int32_t* block_begin, const int32_t* block_end, int32_t n_streams, int32_t max_len,
                      hipStream_t stream) {
  if (!dtype_ok(arena_dtype)) return PAGED_EINVAL;
  if (n_streams < 0 || max_len < 0 || max_len > MAX_POS) return PAGED_EINVAL;
  if (idx_dim < 8 || idx_dim > 1024 || idx_dim % 8 != 0) return PAGED_EINVAL;
  int r = check_pg(pg, arena_dtype, max_len, true);
  if (r) return r;
  if (pg->page_elems * esize(arena_dtype) <
      (int64_t)pg->page_pos * idx_dim * esize(arena_dtype) + (int64_t)(pg->page_pos / 4) * idx_dim * 4)
    return PAGED_EINVAL;
  if (n_streams == 0) return PAGED_OK;
  if (ik == nullptr || pooled == nullptr || !al(ik, 16) || !al(pooled, 16)) return PAGED_EINVAL;
  if (block_begin == nullptr || block_end == nullptr || !al(block_begin, 4) || !al(block_end, 4)) return PAGED_EINVAL;
  PoolArgs a;
  a.ik = (const char*)ik;
  a.pooled = (char*)pooled;
  a.pg = to_dev(pg, arena_dtype);
  a.begin = block_begin;
  a.end = block_end;
  a.idx_dim = idx_dim;
  a.max_blocks = max_len / 4;
  a.n_streams = n_streams;
  return hip_status(launch_pool(a, arena_dtype == PAGED_BF16, stream));
}

size_t paged_topk_workspace(int32_t n_streams, int32_t max_len, int32_t k) {
  if (n_streams <= 0 || max_len < 0) return 0;
  return topk_workspace_bytes(n_streams, max_len / 4, k, 0);
}

int paged_block_scores_topk(const void* qi, int32_t qi_dtype, int32_t n_idx_heads, int32_t idx_dim,
                            const void* pooled, int32_t arena_dtype, const paged_pg* pg, const int32_t* seq_lens,
                            int32_t n_streams,
                            int32_t max_len, int32_t k, int32_t* out_ids, int32_t* out_count, double* out_scores,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!dtype_ok(qi_dtype) || !dtype_ok(arena_dtype)) return PAGED_EINVAL;
  if (n_streams < 0 || max_len < 0 || max_len > MAX_POS || k < 1) return PAGED_EINVAL;
  if (n_idx_heads < 1 || idx_dim < 4 || idx_dim > 1024 || idx_dim % 4 != 0 || (int64_t)n_idx_heads * idx_dim > 2048)
    return PAGED_EINVAL;
  int r = check_pg(pg, arena_dtype, max_len, true);
  if (r) return r;
  if (n_streams == 0) return PAGED_OK;
  if (qi == nullptr || !al(qi, 16) || pooled == nullptr || !al(pooled, 16)) return PAGED_EINVAL;
  if (seq_lens == nullptr || !al(seq_lens, 4) || out_ids == nullptr || !al(out_ids, 4) || out_count == nullptr ||
      !al(out_count, 4))
    return PAGED_EINVAL;
  if (out_scores != nullptr && !al(out_scores, 8)) return PAGED_EINVAL;
  const int max_blocks = max_len / 4;
  const size_t need = topk_workspace_bytes(n_streams, max_blocks, k, out_scores != nullptr);
  if (workspace_bytes < need || workspace == nullptr || !al(workspace, 16)) return PAGED_EWORKSPACE;
  TopkArgs a;
  a.qi = qi;
  a.pooled = (const char*)pooled;
  a.pg = to_dev(pg, arena_dtype);
  a.lens = seq_lens;
  a.n_idx_heads = n_idx_heads;
  a.idx_dim = idx_dim;
  a.max_blocks = max_blocks;
  a.k = k;
  {
    // workspace layout: see topk_workspace_bytes
    const size_t S = (size_t)n_streams;
    const int nsel = topk_nsel(max_blocks);
    char* p = (char*)workspace;
    a.hist = (uint32_t*)p;
    p += S * 4096 * sizeof(uint32_t);
    a.sel_cnt = (uint32_t*)p;
    p += S * nsel * 2 * sizeof(uint32_t);
    a.sel_bits = (uint32_t*)p;
    p += S * nsel * 32 * sizeof(uint32_t);
    a.sel_key = (uint64_t*)p;
    p += S * nsel * 1024 * sizeof(uint64_t);
    a.sel_id = (int32_t*)p;
    p += S * nsel * 1024 * sizeof(int32_t);
    a.nsel = nsel;
    a.scores = out_scores ? out_scores : (double*)p;
  }
  a.out_ids = out_ids;
  a.out_count = out_count;
  return hip_status(launch_scores_topk(a, qi_dtype == PAGED_BF16, n_streams, stream));
}

int paged_rows_store(const void* src, int64_t stride_s, int64_t stride_h, int64_t stride_p, void* region,
                     int32_t n_heads, int32_t row_elems, int32_t dtype, const paged_pg* pg, const int32_t* pos_begin,
                     const int32_t* pos_end, int32_t n_streams, int32_t max_len, hipStream_t stream) {
  return rows_common(0, (void*)src, stride_s, stride_h, stride_p, region, n_heads, row_elems, dtype, pg, pos_begin,
                     pos_end, n_streams, max_len, stream);
}

int paged_rows_gather(void* dst, int64_t stride_s, int64_t stride_h, int64_t stride_p, const void* region,
                      int32_t n_heads, int32_t row_elems, int32_t dtype, const paged_pg* pg, const int32_t* pos_begin,
                      const int32_t* pos_end, int32_t n_streams, int32_t max_len, hipStream_t stream) {
  return rows_common(1, dst, stride_s, stride_h, stride_p, (void*)region, n_heads, row_elems, dtype, pg, pos_begin,
                     pos_end, n_streams, max_len, stream);
}

int paged_kv_append(const void* k_new, const void* v_new, const void* ik_new, int32_t n_new, const paged_kv* kv,
                    void* ik, void* pooled, int32_t idx_dim, const paged_pg* pg, const int32_t* pos0,
                    int32_t n_streams, int32_t max_len, hipStream_t stream) {
  if (n_new < 0 || n_streams < 0 || max_len < 0 || max_len > MAX_POS) return PAGED_EINVAL;
  int r = check_kv(kv, pg);
  if (r) return r;
  const bool has_ik = ik_new != nullptr;
  const bool fp8 = kv->dtype == PAGED_FP8_E4M3;
  if (fp8 && has_ik) return PAGED_EUNSUPPORTED;  // indexer keys are not kept in e4m3 arenas
  r = check_pg(pg, kv->dtype, max_len, has_ik);
  if (r) return r;
  const int es = esize(kv->dtype);
  const int64_t kv_bytes = (int64_t)kv->n_kv_heads * pg->page_pos * kv->head_dim * es;
  if (has_ik) {
    if (idx_dim < 8 || idx_dim > 1024 || idx_dim % 8 != 0) return PAGED_EINVAL;
    if (ik == nullptr || pooled == nullptr || !al(ik, 16) || !al(pooled, 16) || !al(ik_new, 16)) return PAGED_EINVAL;
    if (pg->page_elems * es < 2 * kv_bytes + (int64_t)pg->page_pos * idx_dim * es + (int64_t)(pg->page_pos / 4) * idx_dim * 4)
      return PAGED_EINVAL;
  }
  if (n_streams == 0 || n_new == 0) return PAGED_OK;
  if (k_new == nullptr || v_new == nullptr || !al(k_new, 16) || !al(v_new, 16)) return PAGED_EINVAL;
  if (pos0 == nullptr || !al(pos0, 4)) return PAGED_EINVAL;
  AppendArgs a;
  a.k_new = (const char*)k_new;
  a.v_new = (const char*)v_new;
  a.ik_new = (const char*)ik_new;
  a.kb = (char*)kv->k;
  a.vb = (char*)kv->v;
  a.ikb = (char*)ik;
  a.pooled = (char*)pooled;
  a.ksb = fp8 ? (char*)kv->k_scale : nullptr;
  a.vsb = fp8 ? (char*)kv->v_scale : nullptr;
  a.pg = to_dev(pg, kv->dtype);
  a.pos0 = pos0;
  a.n = n_new;
  a.hkv = kv->n_kv_heads;
  a.row_bytes = kv->head_dim * es;
  a.ik_row_bytes = has_ik ? idx_dim * es : 0;
  a.idx_dim = has_ik ? idx_dim : 8;
  a.max_len = max_len;
  a.bf16 = kv->dtype == PAGED_BF16;
  a.fp8 = fp8;
  return hip_status(launch_append(a, n_streams, stream));
}

int paged_row_offsets(const paged_pg* pg, int32_t n_streams, int32_t row_width, const int32_t* streams,
                      const int32_t* heads, const int32_t* positions, int64_t* out, int32_t n, hipStream_t stream) {
  if (pg == nullptr || pg->reserved != 0 || pg->page_pos < 1 || pg->page_elems < 1) return PAGED_EINVAL;
  if (n < 0 || n_streams < 0 || row_width < 1) return PAGED_EINVAL;
  if (pg->table != nullptr && (!al(pg->table, 4) || pg->table_stride < 1)) return PAGED_EINVAL;
  if (n == 0) return PAGED_OK;
  if (streams == nullptr || heads == nullptr || positions == nullptr || out == nullptr || !al(out, 8))
    return PAGED_EINVAL;
  OffArgs a;
  a.pg.table = pg->table;
  a.pg.stride = pg->table_stride;
  a.pg.ptok = pg->page_pos;
  a.pg.page_bytes = pg->page_elems;  // element units for this hook
  a.n_streams = n_streams;
  a.row_width = row_width;
  const int64_t ext = pg->table ? (int64_t)pg->table_stride * pg->page_pos : (int64_t)pg->page_pos;
  a.max_pos = (int32_t)(ext > MAX_POS ? MAX_POS : ext);
  a.streams = streams;
  a.heads = heads;
  a.positions = positions;
  a.out = out;
  a.n = n;
  return hip_status(launch_row_offsets(a, stream));
}

const char* paged_strerror(int status) {
  switch (status) {
    case PAGED_OK: return "ok";
    case PAGED_EINVAL: return "invalid argument";
    case PAGED_EUNSUPPORTED: return "unsupported by this library";
    case PAGED_EWORKSPACE: return "workspace missing or too small";
    case PAGED_EHIP: return "HIP launch failed";
    case PAGED_EFULL: return "no free page or run (the request waits)";
    case PAGED_ESCRATCH: return "request needs more than the allocation-free decode's scratch";
    default: return "unknown status";
  }
}

}  // extern "C"
