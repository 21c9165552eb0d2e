// attn_bwd.hip -- attention backward for gfx950 (placeholder until the
// kernels land: reports the problem as unsupported).
#include "attn_internal.h"
#include "launch.h"

namespace attn {

attn_status launch_bwd(const attn_plan *, const void *, const void *, const void *, const void *,
                       const float *, const void *, float *, float *, float *, hipStream_t) {
  return ATTN_E_UNSUPPORTED;
}

}  // namespace attn
