// Frame-chunked MFMA path (placeholder until its kernels land).
#include "gdn_internal.h"

namespace gdn {

const char* chunked_unsupported_reason(const Problem&) { return "not implemented in this build"; }
size_t chunked_workspace(const Problem&, int) { return 0; }
hipError_t chunked_launch(const Problem&, int, const Tensors&, void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace gdn
