/*
 * paged_attn.h -- C ABI of libpagedattn.so: attention over a KV cache read
 * through an int page table, on one AMD MI355X (gfx950).
 *
 * Sources (page titles and sections):
 *   [P1] TensorFold PR #1169 "Flash Next attention caches readable through a
 *        page table", sections "What this changes" and "Receipt".
 *   [P2] TensorFold PR #1170 "Flash Next CUDA: the streams beside the first
 *        take KV pages from the core pool": description, commit messages
 *        3f5b87d (Seg/kv_row), ce5b78d (attention partials branch once),
 *        1ac2075 (pool runs), 51f8354 (mapRun refuses a short run) and the
 *        maintainer replies (drain before free; page-run prompt path).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Page table (the pages' Pg argument, [P1 "What this changes"]): three values
 * describe paging, the int table itself and how many elements and positions a
 * page holds.  The row of
 * (stream s, head h, position p) in a region whose page part is
 * [H][page_pos][W] starts at element
 *     table[s * table_stride + p / page_pos] * page_elems + (h * page_pos + p % page_pos) * W
 * and, with no table (table == NULL), at the old contiguous expression
 *     s * page_elems + (h * cap + p) * W       with page_pos = cap,
 * i.e. each stream reserves cap rows per head ([P2 commit 3f5b87d]).  page_elems
 * counts elements of the arena's K/V type; a float32 pooled row in a bf16
 * arena uses two slots per value.
 *
 * Region bases: each cache pointer addresses the share of page 0 that belongs to
 * its layer ([P1 "What this changes"]); k, v, ik and pooled are such pointers into one arena.
 *
 * Ownership ([P2 maintainer replies: drain before anything is freed, fills on
 * the engine stream]): the caller allocates and owns every buffer (inputs,
 * arena, table, lengths, outputs, workspace).  The library allocates nothing,
 * frees nothing, keeps no global state (one exception: the scratch array of
 * paged_attn_decode_noalloc, below), reads no environment variable and never
 * synchronises: all work is enqueued on `stream`.  Inputs are only read.
 * The caller must not free, reuse or re-table pages until `stream` has drained.
 * Structs are passed by host pointer and read only during the call.
 *
 * Errors: a negative status is returned before anything is enqueued when an
 * argument is refused (the pages refuse what they cannot serve: a page size
 * that does not divide by 4 [P2 "What this changes"], a run with fewer pages
 * than its parts need [P2 commit 51f8354]).  PAGED_EHIP reports a failed launch.  Table
 * entries are not range-checked on the device: an entry outside the arena is
 * undefined behaviour.  Lengths, block ranges and block ids are clamped or
 * ignored on the device as stated per call, so that no table entry past the
 * validated extent is ever read.
 *
 * Numerics: every sum keeps one fixed order that depends only on a stream's
 * own length (never on the page size, the table or the other streams), so the
 * paged result is byte-equal to the contiguous one for every page size made of
 * whole rows ([P1 "What this changes": paging alters where rows are read, never
 * the order of a sum]), and a stream in a batch equals the same stream alone.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  PAGED_FP8_E4M3 rows are 256 e4m3 codes (OCP E4M3: 1 sign, 4 exponent bits with
   bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN, largest finite 448) that stand for
   code x scale with one float32 scale a row ([P2 commit 5c09685]: each row's fp8 codes and its
   float32 scale are reached via the page holding the row).  Only the K/V regions of an attention layer take this type. */
typedef enum { PAGED_F32 = 0, PAGED_BF16 = 1, PAGED_FP8_E4M3 = 2 } paged_dtype;

/* Status codes. */
enum {
  PAGED_OK = 0,
  PAGED_EINVAL = -1,       /* an argument is out of range, NULL or misaligned  */
  PAGED_EUNSUPPORTED = -2, /* a valid request this library does not serve      */
  PAGED_EWORKSPACE = -3,   /* workspace missing or smaller than required        */
  PAGED_EHIP = -4,         /* a HIP launch failed                               */
  PAGED_EFULL = -5,        /* no free page or run: the request waits (page pool) */
  PAGED_ESCRATCH = -6      /* the request needs more scratch than paged_attn_decode_noalloc holds */
};

/* The pages' Pg argument ([P1 "What this changes"]). */
typedef struct {
  const int32_t *table;  /* device [n_streams][table_stride] arena page ids, or NULL (contiguous) */
  int32_t table_stride;  /* entries per stream row; table_stride * page_pos >= max_len            */
  int32_t page_pos;      /* positions a page; = cap (rows a head) when table == NULL              */
  int64_t page_elems;    /* elements (of the arena's K/V type) a page; the stream stride when
                            table == NULL; page_elems * element size must be a multiple of 16   */
  int64_t reserved;      /* must be 0 (a poisoned struct is refused)                            */
} paged_pg;

/* Key and value regions of one attention layer ([P2 commit 3f5b87d]:
   [key, value][head][position][row] inside a page).
   PAGED_FP8_E4M3 ([P2 commit 5c09685]; page_elems then counts bytes, as the pages size an fp8 page in
   bytes): k and v hold the codes, [Hkv][page_pos][256] bytes a page, and k_scale / v_scale the
   rows' float32 scales, [Hkv][page_pos] a page, addressed like rows of 4 bytes:
     scale of (s, h, p) at byte  table[s * table_stride + p / page_pos] * page_elems + (h * page_pos + p % page_pos) * 4
   from k_scale (v_scale).  The scale fields are read only when dtype == PAGED_FP8_E4M3. */
typedef struct {
  const void *k;         /* device, 16-byte aligned: the K region of page 0, [Hkv][page_pos][D] a page */
  const void *v;         /* device, 16-byte aligned: the V region of page 0, same shape              */
  int32_t dtype;         /* paged_dtype of K and V                                                     */
  int32_t n_kv_heads;    /* Hkv >= 1                                                                   */
  int32_t head_dim;      /* D; the library serves D = 256                                              */
  int32_t reserved;      /* must be 0                                                                  */
  const void *k_scale;   /* PAGED_FP8_E4M3: device, 4-byte aligned, K scale region of page 0           */
  const void *v_scale;   /* PAGED_FP8_E4M3: device, 4-byte aligned, V scale region of page 0           */
} paged_kv;

/* ------------------------------------------------------------------------ */
/* Dense decode ([P1 "What this changes": fn_attn_chunks gets its key and value
 * tiles via pg_at, resolving each key's row a single time per tile and keeping
 * key_at in shared memory next to key_ids;
 * P2 commit ce5b78d: attention partials]).
 *
 * For every stream s and query head h: out[s][h] = softmax(scale * K q) V over
 * the L_s cached positions 0..L_s-1 of KV head h / (Hq / Hkv).
 *   q        device [n_streams][n_q_heads][256], q_dtype == kv->dtype (PAGED_BF16 for PAGED_FP8_E4M3
 *            rows), 16-byte aligned
 *   seq_lens device [n_streams] int32; values are clamped to [0, max_len]
 *   max_len  host bound on every length; table_stride * page_pos >= max_len
 *            (page_pos >= max_len when table == NULL)
 *   out      device [n_streams][n_q_heads][256] float32; a stream of length 0 gets zeros
 *   workspace device, >= paged_attn_decode_workspace(n_streams, n_q_heads, max_len) bytes,
 *            16-byte aligned: split partials, contents undefined after the call.  Calls that
 *            share a workspace must not overlap in time (one stream, or ordered).
 * Serves n_q_heads / n_kv_heads in {1, 2, 4, 8}, head_dim 256, F32, BF16 or FP8_E4M3 rows.  With
 * e4m3 rows a key's score is scale * k_scale * (q . codes) and its value row v_scale * codes; the
 * scales must be finite.
 */
int paged_attn_decode(const void *q, int32_t q_dtype, int32_t n_q_heads,
                      const paged_kv *kv, const paged_pg *pg,
                      const int32_t *seq_lens, int32_t n_streams, int32_t max_len,
                      float scale, float *out,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);
size_t paged_attn_decode_workspace(int32_t n_streams, int32_t n_q_heads, int32_t max_len);

/* ------------------------------------------------------------------------ */
/* Dense decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Arguments, results and refusals are those of
 * paged_attn_decode, and the output is bit for bit the same; the split partials
 * go to a scratch array of PAGED_NOALLOC_SCRATCH_BYTES (16,908,288 bytes: the
 * partials of 1024 (stream, q head) rows at the most splits a stream takes, so
 * 32 streams x 32 q heads fit at any length) that the library keeps in each
 * GPU's memory for the life of the process.  No allocation is made by this call.
 *   - PAGED_ESCRATCH when paged_attn_decode_workspace(n_streams, n_q_heads,
 *     max_len) exceeds that size.
 *   - The first call on a device, with that device current, looks up the device
 *     address of that GPU's array (no stream work, no allocation); `stream` must
 *     belong to the current device.
 *   - Every call on one GPU shares that GPU's array: calls that overlap in time on
 *     one GPU (two streams, or two threads) race on it and must be ordered by the
 *     caller.  Its contents are undefined between calls; nothing in it has to
 *     start at zero.
 */
#define PAGED_NOALLOC_SCRATCH_BYTES (1024u * 16u * (256u + 2u) * 4u)
int paged_attn_decode_noalloc(const void *q, int32_t q_dtype, int32_t n_q_heads,
                              const paged_kv *kv, const paged_pg *pg,
                              const int32_t *seq_lens, int32_t n_streams, int32_t max_len,
                              float scale, float *out, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Windowed decode ([P1 "What this changes" names fn_attn_chunks_ahead beside
 * fn_attn_chunks; the reading taken: the form that verifies drafted tokens,
 * a window of queries at the end of each stream's cache, read through pg_at
 * like decode).
 *
 * Query w (0 <= w < n_window) of stream s stands at position L_s - n_window + w
 * (L_s = seq_lens[s] clamped to [0, max_len]; the window's rows are already
 * stored) and attends, per head, to keys 0 .. L_s - n_window + w; a query
 * with no key gets a zero row.  n_window = 1 is paged_attn_decode.
 *   q        device [n_streams][n_window][n_q_heads][256] bf16, 16-byte aligned
 *   out      device [n_streams][n_window][n_q_heads][256] float32
 *   workspace >= paged_attn_decode_window_workspace(n_streams, n_q_heads, n_window, max_len)
 *            bytes, as for decode
 * Serves BF16 and FP8_E4M3 rows, n_window 1 .. 4 with n_window * (n_q_heads / n_kv_heads) <= 16
 * (PAGED_EUNSUPPORTED otherwise).
 */
int paged_attn_decode_window(const void *q, int32_t q_dtype, int32_t n_q_heads, int32_t n_window,
                             const paged_kv *kv, const paged_pg *pg,
                             const int32_t *seq_lens, int32_t n_streams, int32_t max_len,
                             float scale, float *out,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);
size_t paged_attn_decode_window_workspace(int32_t n_streams, int32_t n_q_heads, int32_t n_window,
                                          int32_t max_len);

/* ------------------------------------------------------------------------ */
/* Chunked causal prefill for one stream ([P2 maintainer reply: paged or mixed
 * prompts read from paged caches go down the page-run path and flat ones use
 * tensor-core attention;
 * here one MFMA kernel serves both through pg_at]).
 *
 * Queries at absolute positions q_pos0 .. q_pos0+n_q-1 attend, per head, to the
 * cached keys 0 .. p (causal != 0) or 0 .. q_pos0+n_q-1 (causal == 0); the
 * chunk's own rows must already be stored.  The stream's table row is
 * pg->table[0 .. table_stride-1] (pass the row's address for stream s).
 *   q    device [n_q][n_q_heads][256] bf16 (q_dtype == PAGED_BF16 == kv->dtype)
 *   out  device [n_q][n_q_heads][256] float32
 *   table_stride * page_pos >= q_pos0 + n_q
 *   workspace: >= paged_attn_prefill_workspace(n_q, n_q_heads, q_pos0 + n_q) bytes (may be 0)
 * Serves bf16, head_dim 256, n_q_heads / n_kv_heads in {1, 2, 4, 8}.
 */
int paged_attn_prefill(const void *q, int32_t q_dtype, int32_t n_q, int32_t q_pos0,
                       int32_t n_q_heads, const paged_kv *kv, const paged_pg *pg,
                       int32_t causal, float scale, float *out,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);
size_t paged_attn_prefill_workspace(int32_t n_q, int32_t n_q_heads, int32_t kv_len);

/* ------------------------------------------------------------------------ */
/* Block pooling ([P1 "What this changes": fn_qsa_pool reads and writes through
 * pg_at once per block of four; a page holds the pooled rows of its n/4 blocks]).
 *
 * For each stream s and block b in [block_begin[s], block_end[s]) (clamped to
 * [0, max_len / 4)): pooled row b = float32(((IK[4b] + IK[4b+1]) + IK[4b+2]) + IK[4b+3]) / 4)
 * with the sum in float64.  IK rows are [page_pos][idx_dim] a page (one row a
 * position), pooled rows [page_pos/4][idx_dim] float32 a page, both read and
 * written through the table.
 *   ik      device, region base of page 0, arena_dtype elements, 16-byte aligned
 *   pooled  device, region base of page 0, float32, 16-byte aligned
 *   idx_dim multiple of 8, 8 .. 1024; page_pos a multiple of 4
 */
int paged_pool_blocks(const void *ik, void *pooled, int32_t idx_dim, int32_t arena_dtype,
                      const paged_pg *pg, const int32_t *block_begin, const int32_t *block_end,
                      int32_t n_streams, int32_t max_len, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Block scores and top-k selection ([P1 "What this changes": fn_qsa_scores reads
 * pooled rows through pg_at; four-head QSA scores]).
 *
 * score[s][b] = sum over indexer heads h and dimensions d of qi[s][h][d] * pooled[s][b][d] in
 * float64, in this order: q[d] = sum over h of qi[s][h][d], head by head; each product
 * pooled[s][b][d] * q[d] rounded to float64; the products added in 8 groups (group j: the
 * 4-dim chunks c = j, j+8, j+16, ..., dims 4c .. 4c+3, in increasing dim order) whose sums meet
 * as ((g0 + g1) + (g2 + g3)) + ((g4 + g5) + (g6 + g7)); for the
 * nb_s = min(seq_lens[s], max_len) / 4 complete blocks.  Then the k blocks with
 * the highest score (lower id first among equal scores; -0.0 == +0.0) are
 * written ascending to out_ids[s][0 .. n-1] with n = min(k, nb_s); the rest of
 * the row is filled with -1 and out_count[s] = n.
 *   qi         device [n_streams][n_idx_heads][idx_dim], qi_dtype; idx_dim a multiple of 4, at
 *              most 1024, n_idx_heads x idx_dim at most 2048
 *   pooled     device, pooled region base (float32 rows, see paged_pool_blocks);
 *              arena_dtype is the arena's K/V type, which gives page_elems its byte size
 *   out_scores optional device [n_streams][max_len/4] float64 (NULL: kept in workspace); entries
 *              past a stream's floor(L/4) blocks are not written
 *   workspace  >= paged_topk_workspace(n_streams, max_len, k) bytes, 16-byte aligned: per-stream
 *              coarse score histograms (4096 uint32), per 1024 blocks the selection counts,
 *              taken bits and candidate (key, id) pairs (12 KiB + 136 bytes) and, without
 *              out_scores, the scores; contents undefined after the call.  Calls sharing a
 *              workspace must not overlap.
 * Scores are NaN-free for finite inputs; NaN scores are undefined behaviour.
 */
int paged_block_scores_topk(const void *qi, int32_t qi_dtype, int32_t n_idx_heads, int32_t idx_dim,
                            const void *pooled, int32_t arena_dtype, const paged_pg *pg,
                            const int32_t *seq_lens, int32_t n_streams, int32_t max_len, int32_t k,
                            int32_t *out_ids, int32_t *out_count, double *out_scores,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);
size_t paged_topk_workspace(int32_t n_streams, int32_t max_len, int32_t k);

/* ------------------------------------------------------------------------ */
/* Sparse attention over selected blocks ([P1 "Receipt": dense and sparse
 * attention rows equal contiguous]).
 *
 * Like paged_attn_decode, over the positions 4b .. 4b+3 of the blocks
 * block_ids[s][0 .. n_selected[s]-1], in list order.  With ascending ids and
 * every block of a stream selected the result is byte-equal to dense decode.
 * Ids outside [0, max_len/4) are skipped; n_selected is clamped to [0, k].
 *   block_ids  device [n_streams][k] int32
 *   n_selected device [n_streams] int32
 *   workspace  >= paged_sparse_attn_workspace(n_streams, n_q_heads, k) bytes (as for decode)
 */
int paged_sparse_attn(const void *q, int32_t q_dtype, int32_t n_q_heads,
                      const paged_kv *kv, const paged_pg *pg,
                      const int32_t *block_ids, const int32_t *n_selected, int32_t k,
                      int32_t n_streams, int32_t max_len, float scale, float *out,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);
size_t paged_sparse_attn_workspace(int32_t n_streams, int32_t n_q_heads, int32_t k);

/* ------------------------------------------------------------------------ */
/* Row stores and gathers ([P1 "What this changes": fn_attn_prep writes keys,
 * values and indexer keys at pg_at addresses; a saved or restored prompt cache
 * moves runs of pages to and from the contiguous layout]).
 *
 * paged_rows_store copies rows (s, h, p) for p in [pos_begin[s], pos_end[s])
 * (clamped to [0, max_len)) and h < n_heads from a strided source into a
 * region whose page part is [n_heads][page_pos][row_elems]; paged_rows_gather
 * copies the other way.  Strides are in elements; the source (destination)
 * row of (s, h, p) starts at s*stride_s + h*stride_h + p*stride_p.
 * row_elems * element size must be a multiple of 16; strides and base
 * pointers must keep every row 16-byte aligned.
 */
int paged_rows_store(const void *src, int64_t stride_s, int64_t stride_h, int64_t stride_p,
                     void *region, int32_t n_heads, int32_t row_elems, int32_t dtype,
                     const paged_pg *pg, const int32_t *pos_begin, const int32_t *pos_end,
                     int32_t n_streams, int32_t max_len, hipStream_t stream);
int paged_rows_gather(void *dst, int64_t stride_s, int64_t stride_h, int64_t stride_p,
                      const void *region, int32_t n_heads, int32_t row_elems, int32_t dtype,
                      const paged_pg *pg, const int32_t *pos_begin, const int32_t *pos_end,
                      int32_t n_streams, int32_t max_len, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Append a step's rows ([P1 "What this changes": fn_attn_prep stores keys, values and
 * indexer keys through pg_at; the pool kernel reads and writes through pg_at once per
 * block of four]).
 *
 * For each stream s the n_new new tokens sit at positions pos0[s] .. pos0[s]+n_new-1
 * (positions at or past max_len are dropped; pos0 is clamped to [0, max_len]).  Their K
 * and V rows (all heads) and indexer-key rows are stored through the table, and every
 * block of four whose last position is among the new ones gets its pooled row
 * float32(((IK[4b] + IK[4b+1]) + IK[4b+2]) + IK[4b+3]) / 4) (float64 sum), the value
 * paged_pool_blocks writes: rows before pos0[s] are read from the arena (stored by
 * earlier steps), the new ones from ik_new.  One launch.
 *   k_new, v_new device [n_streams][n_new][n_kv_heads][head_dim], kv->dtype (bf16 for e4m3 arenas),
 *                16-byte aligned
 *   ik_new       device [n_streams][n_new][idx_dim] of kv->dtype, or NULL (no indexer keys:
 *                ik, pooled and idx_dim are ignored)
 *   kv           K and V region bases; ik, pooled: region bases as for paged_pool_blocks
 *   pos0         device [n_streams] int32
 * page_pos must divide by 4 when ik_new is given.  The caller must not run two
 * appends that write the same rows concurrently.
 *
 * e4m3 arenas (kv->dtype == PAGED_FP8_E4M3, [P2 commit 5c09685]: the fp8 store takes a row's
 * codes and fp32 scale through the table): k_new and v_new are bf16 and every (token, head) row x
 * is stored as scale = amax / 448 (amax = max |x|) in the scale regions and codes e4m3(x / scale)
 * in the code regions, both quotients float32 and correctly rounded, e4m3() the nearest code with
 * ties to the even code, magnitudes beyond 448 held at 448 and the sign bit kept; a row of zeros
 * stores scale 0 and zero codes.  Inputs must be finite.  ik_new must be NULL
 * (PAGED_EUNSUPPORTED otherwise): indexer keys are not kept in e4m3 arenas.
 */
int paged_kv_append(const void *k_new, const void *v_new, const void *ik_new, int32_t n_new,
                    const paged_kv *kv, void *ik, void *pooled, int32_t idx_dim, const paged_pg *pg,
                    const int32_t *pos0, int32_t n_streams, int32_t max_len, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Test hook: the row addressing itself, on the device.  [P1 "What this changes"]:
 * pg_at gives, without a table, the earlier contiguous offset of a row and, with
 * one, the base of the page holding the position plus the row's offset inside that
 * page.  out[i] = that element offset of row (streams[i], heads[i], positions[i])
 * in a region whose page part is [H][page_pos][row_width], from the same device
 * function every kernel above uses; it lets a test compare the library's
 * addressing with an independent one bit for bit.  Entries whose stream or
 * position is negative or past the table's extent get -1.  Refusals as for every
 * call (PAGED_EINVAL for a NULL pg, non-zero reserved, page_pos or page_elems
 * below 1, a misaligned table, NULL arrays or a misaligned out).
 */
int paged_row_offsets(const paged_pg *pg, int32_t n_streams, int32_t row_width,
                      const int32_t *streams, const int32_t *heads, const int32_t *positions,
                      int64_t *out, int32_t n, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Host page pool ([P2 commit 1ac2075]: single KV pages come off a free stack
 * that starts at the low end of the arena; findRun / claimRun / releaseRun take
 * k adjacent free pages at the high end; when fragmentation leaves no such run
 * the request has to wait.  [P2 description]: pages and runs are returned only
 * after the engine's stream has drained -- the caller's duty; nothing here
 * touches the GPU).
 *
 * The pool lives in host memory the caller owns and passes to every call:
 * paged_pool_state_bytes(n_pages) bytes, 8-byte aligned, set up by
 * paged_pool_init.  Calls on one state must not run concurrently.
 *   init         all n_pages free; the stack hands out page 0 first, then 1, 2, ...
 *   alloc        n pages off the free stack into pages[0..n-1] (in the order taken);
 *                PAGED_EFULL (nothing taken) when fewer than n are free
 *   free         pages handed out by alloc go back onto the stack in list order (the
 *                last listed is handed out next); PAGED_EINVAL, with nothing changed,
 *                for a page not handed out by alloc or listed twice
 *   claim_run    the highest k consecutive free pages (*first = the lowest of them),
 *                taken off the free stack; PAGED_EFULL when no such run exists
 *   release_run  a claimed run's pages go back onto the stack, its lowest page on top;
 *                PAGED_EINVAL, with nothing changed, unless (first, k) is a run exactly
 *                as claim_run handed it out and not yet released (part of a run, or
 *                two adjacent runs as one, is refused)
 *   free_count   pages on the free stack (negative status for a bad state)
 */
size_t  paged_pool_state_bytes(int32_t n_pages);
int     paged_pool_init(void *state, size_t state_size, int32_t n_pages);
int     paged_pool_alloc(void *state, int32_t n, int32_t *pages);
int     paged_pool_free(void *state, const int32_t *pages, int32_t n);
int     paged_pool_claim_run(void *state, int32_t k, int32_t *first);
int     paged_pool_release_run(void *state, int32_t first, int32_t k);
int32_t paged_pool_free_count(const void *state);

/* Text for a status code, so that a binding can raise an error that names the
 * refusal (the pages' calls report why they refuse a page table: [P1 "Gotchas"],
 * [P2 "What this changes"]).  Returns a pointer to static storage the caller must
 * not free; an unknown code gives "unknown status". */
const char *paged_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
