// nha_bwd.hip -- backward kernels of the NHA layer operator (gfx950).
#include "nha_common.h"
#include "nha_internal.h"

namespace nha {

size_t bwd_ws_bytes(const Shape& s) { return fwd_ws_layout(s).total; }

int bwd_stages(const Shape&, const char**, int) { return 0; }

hipError_t launch_bwd(const Shape&, const RopeTheta&, const BwdPtrs&, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace nha
