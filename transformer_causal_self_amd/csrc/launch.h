// launch.h -- host launchers of the gfx950 kernels, called by the C-ABI entry
// points in plan.cpp after argument checks.
#pragma once

#include <hip/hip_runtime_api.h>

#include "attn_internal.h"

namespace attn {

attn_status launch_rope(const attn_plan *p, const void *q, int64_t qs, const void *k, int64_t ks,
                        const void *v, int64_t vs, void *q_out, void *k_out, void *v_out,
                        hipStream_t stream);

attn_status launch_rope_fp8(const attn_plan *p, const void *q, int64_t qs, const void *k,
                            int64_t ks, const void *v, int64_t vs, const float *scales,
                            void *q_out, void *k_out, void *v_out, hipStream_t stream);

attn_status launch_rope_bwd(const attn_plan *p, const void *q, int64_t qs, const void *k,
                            int64_t ks, const float *dq_in, const float *dk_in, const float *dv_in,
                            float *dq, float *dk, float *dv, hipStream_t stream);

attn_status launch_fwd(const attn_plan *p, const void *q, const void *k, const void *v, void *o,
                       float *lse, hipStream_t stream);

// delta: device scratch of Hs x Ns floats (D of every attention head and slot)
attn_status launch_bwd(const attn_plan *p, const void *q, const void *k, const void *v,
                       const void *o, const float *lse, const void *d_o, float *dq, float *dk,
                       float *dv, float *delta, hipStream_t stream);

// The argument checks of attn_bwd (plan, dtype, binding, pointers, alignment);
// ATTN_OK also for an empty problem, where nothing is launched.
attn_status check_bwd_args(const attn_plan *p, const void *q, const void *k, const void *v,
                           const void *o, const float *lse, const void *d_o, float *dq,
                           float *dk, float *dv);

}  // namespace attn
