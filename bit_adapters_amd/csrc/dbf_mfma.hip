// MFMA path of the double-binary layer (T large): not built yet.
#include "dbf_internal.h"

namespace dbf {

size_t mfma_ws_bytes(int64_t /*N*/, int64_t /*M*/, int64_t R, int n_terms,
                     int64_t T) {
  return static_cast<size_t>(n_terms) * static_cast<size_t>(T) *
         static_cast<size_t>(ws_rstride(R)) * 4u;
}

hipError_t launch_mfma(const TermPtrs&, int64_t, int64_t, int64_t, const void*,
                       int, int64_t, int64_t, void*, int, int64_t, int, void*,
                       hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace dbf
