// Chunked causal prefill over a paged cache (MFMA): not built yet.
#include "internal.h"

namespace paged {

hipError_t launch_prefill(const PreArgs& a, int G, hipStream_t st) {
  (void)a;
  (void)G;
  (void)st;
  return hipErrorNotSupported;
}

}  // namespace paged
