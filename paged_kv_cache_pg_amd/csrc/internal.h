// Launchers shared between the C-ABI host code (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace paged {

constexpr int HD = 256;  // head dimension served by the attention kernels

// ---- decode / sparse (decode.hip) -----------------------------------------
struct DecArgs {
  const void* q;          // [S][Hq][HD]
  const char* kb;         // K region base
  const char* vb;         // V region base
  const char* ksb;        // e4m3 rows: K scale region base ([H][ptok] float32 a page)
  const char* vsb;        // e4m3 rows: V scale region base
  PgDev pg;
  const int32_t* lens;    // dense: lengths [S]; sparse: selected block counts [S]
  const int32_t* ids;     // sparse: block ids [S][ids_stride]; dense: nullptr
  int32_t ids_stride;     // k
  int32_t max_len;        // bound on lengths and on block positions
  int32_t hq;
  int32_t hkv;
  int32_t nq;             // queries a stream (1, or the window of the windowed decode)
  int32_t kvshift;        // vector-ALU decode: workgroups a KV head = 2^kvshift, each G / 2^kvshift q heads
  int32_t s0;             // vector-ALU decode: the launch's first stream (stream = s0 + blockIdx.z)
  float zscale;           // softmax scale * log2(e)
  int32_t ns_max;         // split slots a (stream, query, head) in the workspace
  float* part_o;          // [S][nq][Hq][ns_max][HD]
  float* part_ml;         // [S][nq][Hq][ns_max][2]
  float* out;             // [S][nq][Hq][HD]
};

int dec_splits_max(int max_keys);
// elem: 0 float32, 1 bf16, 2 e4m3 codes with a float32 scale a row (q bf16)
hipError_t launch_decode(const DecArgs& a, int elem, int G, int n_streams, hipStream_t st);
// The MFMA decode (bf16 or e4m3 rows, q bf16): nq window queries x G heads <= 16 rows a KV head.
hipError_t launch_decode_mfma(const DecArgs& a, int elem, int G, int n_streams, hipStream_t st);
hipError_t launch_decode_combine(const DecArgs& a, int n_streams, hipStream_t st);

// ---- prefill (prefill.hip) ------------------------------------------------
struct PreArgs {
  const void* q;          // [n_q][Hq][HD] bf16
  const char* kb;
  const char* vb;
  PgDev pg;               // one stream: table row 0
  int32_t n_q;
  int32_t q_pos0;
  int32_t hq;
  int32_t hkv;
  int32_t causal;
  float zscale;
  float* out;             // [n_q][Hq][HD] float32
};
hipError_t launch_prefill(const PreArgs& a, int G, hipStream_t st);

// ---- pooling, scores, top-k (qsa.hip) ---------------------------------------
struct PoolArgs {
  const char* ik;
  char* pooled;
  PgDev pg;               // page_bytes of the arena
  const int32_t* begin;
  const int32_t* end;
  int32_t idx_dim;
  int32_t max_blocks;
  int32_t n_streams;
};
hipError_t launch_pool(const PoolArgs& a, bool bf16, hipStream_t st);

struct TopkArgs {
  const void* qi;         // [S][Hi][DI]
  const char* pooled;
  PgDev pg;
  const int32_t* lens;
  int32_t n_idx_heads;
  int32_t idx_dim;
  int32_t max_blocks;     // max_len / 4
  int32_t k;
  double* scores;         // [S][max_blocks]
  uint32_t* hist;         // workspace [S][4096]: coarse score histograms
  uint32_t* sel_cnt;      // workspace [S][nsel][2]: a selection workgroup's taken and candidate counts
  uint32_t* sel_bits;     // workspace [S][nsel * 32]: taken bits, a bit a block
  uint64_t* sel_key;      // workspace [S][nsel][1024]: a selection workgroup's bin-T keys
  int32_t* sel_id;        // workspace [S][nsel][1024]: and their ids
  int32_t nsel;           // selection workgroups a stream: ceil(max_blocks / 1024)
  int32_t* out_ids;       // [S][k]
  int32_t* out_count;     // [S]
};
size_t topk_workspace_bytes(int n_streams, int max_blocks, int k, int scores_external);
int topk_nsel(int max_blocks);
hipError_t launch_scores_topk(const TopkArgs& a, bool qi_bf16, int n_streams, hipStream_t st);

// ---- row stores / gathers and the addressing hook (rows.hip) ----------------
struct RowsArgs {
  char* lin;              // strided side (source of a store, destination of a gather)
  int64_t ss, sh, sp;     // strides in bytes
  char* region;           // paged side
  PgDev pg;
  const int32_t* begin;
  const int32_t* end;
  int32_t n_heads;
  int32_t row_bytes;
  int32_t max_len;
  int32_t n_streams;
  int32_t gather;         // 0: lin -> region, 1: region -> lin
};
hipError_t launch_rows(const RowsArgs& a, hipStream_t st);

struct AppendArgs {
  const char* k_new;      // [S][n][Hkv][row] token-major step rows
  const char* v_new;
  const char* ik_new;     // [S][n][DI] or nullptr (no indexer keys)
  char* kb;               // region bases (page 0)
  char* vb;
  char* ikb;
  char* pooled;
  char* ksb;              // e4m3 arenas: K and V scale region bases
  char* vsb;
  PgDev pg;               // page_bytes of the arena
  const int32_t* pos0;    // [S] position of each stream's first new token
  int32_t n;              // new tokens a stream
  int32_t hkv;
  int32_t row_bytes;      // K / V row
  int32_t ik_row_bytes;   // indexer-key row (0: none)
  int32_t idx_dim;
  int32_t max_len;
  int32_t bf16;           // arena element type: bf16 (else float32) ...
  int32_t fp8;            // ... or e4m3 codes with a float32 scale a row (bf16 step rows, no indexer keys)
};
hipError_t launch_append(const AppendArgs& a, int n_streams, hipStream_t st);

struct OffArgs {
  PgDev pg;               // page_bytes holds page_elems (element units) for this hook
  int32_t n_streams;
  int32_t row_width;
  int32_t max_pos;
  const int32_t* streams;
  const int32_t* heads;
  const int32_t* positions;
  int64_t* out;
  int32_t n;
};
hipError_t launch_row_offsets(const OffArgs& a, hipStream_t st);

}  // namespace paged
