// Host page pool for a KV arena: hands out pages for the page tables and runs of consecutive
// pages, in the caller's memory (no allocation, no global state).
//
// TensorFold PR #1170, commit 1ac2075 (a pool lane keeps its recurrent state in a run of pool
// pages): single KV pages come off a free stack from the low end of the arena; findRun /
// claimRun / releaseRun take k adjacent free pages from the high end; with no such run free, the
// request waits.  Description of PR #1170: pages and runs are returned only after the engine's
// stream has drained (the caller's duty: nothing here touches the GPU).
//
// State (host memory the caller owns, paged_pool_state_bytes(n) bytes):
//   header | below[n] int32 | above[n] int32 | kind[n] uint8
// The free pages form a stack kept as a doubly linked list: below[p] / above[p] are the free pages
// under and over p (-1 at the ends), header.top the page handed out next.  Taking a run's pages out
// of the middle of the stack then costs k steps and keeps the order of the rest.
// kind: 0 free, 1 handed out as a page, 2 part of a run (3 marks a page while a free list is checked).
#include <stdint.h>
#include <string.h>

#include "paged_attn.h"

namespace {

constexpr uint32_t POOL_MAGIC = 0x4c504751u;  // "QGPL"

struct PoolHeader {
  uint32_t magic;
  int32_t n_pages;
  int32_t n_free;
  int32_t top;     // free page on top of the stack, -1 when none
  int32_t bottom;  // free page at the bottom of the stack, -1 when none
  int32_t reserved;
};

// A claimed run's lowest page is KIND_RUN and keeps the run's length in its stack link (below[],
// unused while the page is off the stack); its other pages are KIND_RUN_BODY.
enum : uint8_t { KIND_FREE = 0, KIND_PAGE = 1, KIND_RUN = 2, KIND_MARK = 3, KIND_RUN_BODY = 4 };

size_t state_bytes(int64_t n) {
  const size_t b = sizeof(PoolHeader) + (size_t)n * 2 * sizeof(int32_t) + (size_t)n;
  return (b + 7) & ~(size_t)7;
}

struct View {
  PoolHeader* h;
  int32_t* below;
  int32_t* above;
  uint8_t* kind;
};

bool view_of(void* state, View* v) {
  if (state == nullptr || ((uintptr_t)state & 7) != 0) return false;
  PoolHeader* h = (PoolHeader*)state;
  if (h->magic != POOL_MAGIC || h->n_pages < 1 || h->n_free < 0 || h->n_free > h->n_pages) return false;
  v->h = h;
  v->below = (int32_t*)(h + 1);
  v->above = v->below + h->n_pages;
  v->kind = (uint8_t*)(v->above + h->n_pages);
  return true;
}

void push(View& v, int32_t p) {
  v.below[p] = v.h->top;
  v.above[p] = -1;
  if (v.h->top >= 0) v.above[v.h->top] = p;
  else v.h->bottom = p;
  v.h->top = p;
  v.kind[p] = KIND_FREE;
  ++v.h->n_free;
}

void unlink(View& v, int32_t p) {
  const int32_t b = v.below[p], a = v.above[p];
  if (b >= 0) v.above[b] = a;
  else v.h->bottom = a;
  if (a >= 0) v.below[a] = b;
  else v.h->top = b;
  --v.h->n_free;
}

}  // namespace

extern "C" {

size_t paged_pool_state_bytes(int32_t n_pages) {
  if (n_pages < 1) return 0;
  return state_bytes(n_pages);
}

int paged_pool_init(void* state, size_t state_size, int32_t n_pages) {
  if (state == nullptr || ((uintptr_t)state & 7) != 0 || n_pages < 1) return PAGED_EINVAL;
  if (state_size < state_bytes(n_pages)) return PAGED_EWORKSPACE;
  PoolHeader* h = (PoolHeader*)state;
  h->magic = POOL_MAGIC;
  h->n_pages = n_pages;
  h->n_free = n_pages;
  h->reserved = 0;
  View v;
  view_of(state, &v);
  // page 0 on top: pages come off the stack from the bottom of the arena up
  for (int32_t p = 0; p < n_pages; ++p) {
    v.below[p] = p + 1 < n_pages ? p + 1 : -1;
    v.above[p] = p - 1;
  }
  h->top = 0;
  h->bottom = n_pages - 1;
  memset(v.kind, KIND_FREE, (size_t)n_pages);
  return PAGED_OK;
}

int32_t paged_pool_free_count(const void* state) {
  View v;
  if (!view_of((void*)state, &v)) return PAGED_EINVAL;
  return v.h->n_free;
}

int paged_pool_alloc(void* state, int32_t n, int32_t* pages) {
  View v;
  if (!view_of(state, &v) || n < 0 || (n > 0 && pages == nullptr)) return PAGED_EINVAL;
  if (n > v.h->n_free) return PAGED_EFULL;  // nothing is taken: the request waits
  for (int32_t i = 0; i < n; ++i) {
    const int32_t p = v.h->top;
    unlink(v, p);
    v.kind[p] = KIND_PAGE;
    pages[i] = p;
  }
  return PAGED_OK;
}

int paged_pool_free(void* state, const int32_t* pages, int32_t n) {
  View v;
  if (!view_of(state, &v) || n < 0 || (n > 0 && pages == nullptr)) return PAGED_EINVAL;
  // every page must be one handed out as a page, each at most once; nothing changes otherwise
  int32_t i = 0;
  for (; i < n; ++i) {
    const int32_t p = pages[i];
    if (p < 0 || p >= v.h->n_pages || v.kind[p] != KIND_PAGE) break;
    v.kind[p] = KIND_MARK;  // a page listed twice meets its mark
  }
  if (i < n) {
    for (int32_t j = 0; j < i; ++j) v.kind[pages[j]] = KIND_PAGE;
    return PAGED_EINVAL;
  }
  for (i = 0; i < n; ++i) push(v, pages[i]);
  return PAGED_OK;
}

int paged_pool_claim_run(void* state, int32_t k, int32_t* first) {
  View v;
  if (!view_of(state, &v) || k < 1 || k > v.h->n_pages || first == nullptr) return PAGED_EINVAL;
  // the highest k consecutive free pages
  int32_t found = -1, len = 0;
  for (int32_t p = v.h->n_pages - 1; p >= 0; --p) {
    len = v.kind[p] == KIND_FREE ? len + 1 : 0;
    if (len == k) {
      found = p;
      break;
    }
  }
  if (found < 0) return PAGED_EFULL;  // too fragmented for the run: the request waits
  // out of the free stack, the order of the rest kept
  for (int32_t p = found; p < found + k; ++p) {
    unlink(v, p);
    v.kind[p] = p == found ? KIND_RUN : KIND_RUN_BODY;
  }
  v.below[found] = k;
  *first = found;
  return PAGED_OK;
}

int paged_pool_release_run(void* state, int32_t first, int32_t k) {
  View v;
  if (!view_of(state, &v) || k < 1 || first < 0 || (int64_t)first + k > v.h->n_pages) return PAGED_EINVAL;
  // only a run exactly as claim_run handed it out: not part of one, not two together
  if (v.kind[first] != KIND_RUN || v.below[first] != k) return PAGED_EINVAL;
  for (int32_t p = first + 1; p < first + k; ++p)
    if (v.kind[p] != KIND_RUN_BODY) return PAGED_EINVAL;
  // pushed from the top page down, so the run's lowest page comes off the stack first
  for (int32_t p = first + k - 1; p >= first; --p) push(v, p);
  return PAGED_OK;
}

}  // extern "C"
