// C-ABI layer of the backward: argument checks and dispatch. See include/hyena.h
// for the contract.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hyena.h"
#include "backward.hpp"
#include "plan.hpp"

namespace {

size_t backward_ws(hyena_plan_t plan, int64_t B, bool per_sample) {
    if (!plan || B < 1) return 0;
    // circular plans: the LDS path only (transform length L/2 for rows of L samples)
    if (plan->path == HYENA_PATH_LDS)
        return hy::bwd_ws_bytes(B, plan->D, int64_t(1) << plan->logT, plan->order, plan->circular);
    if (plan->path == HYENA_PATH_FOURSTEP && !plan->circular)
        return hy::fs_bwd_ws_bytes(plan->logT, B, plan->D, plan->order, per_sample);
    return 0;
}

hyena_status_t backward_impl(hyena_plan_t plan, int64_t B, const void* u_proj, const float* short_w, const void* spec,
                             const float* bias, const void* dy, void* du_proj, float* dshort_w, float* dh, float* dbias,
                             void* workspace, size_t workspace_bytes, hipStream_t stream, bool per_sample) {
    using hy::aligned16;
    if (!plan || B < 1 || !u_proj || !short_w || !spec || !bias || !dy || !du_proj || !dshort_w || !dh || !dbias)
        return HYENA_ERR_INVALID_ARG;
    if (!aligned16(u_proj) || !aligned16(short_w) || !aligned16(spec) || !aligned16(bias) || !aligned16(dy) ||
        !aligned16(du_proj) || !aligned16(dshort_w) || !aligned16(dh) || !aligned16(dbias))
        return HYENA_ERR_INVALID_ARG;
    if (B > (int64_t(1) << 24) || B * plan->D > (int64_t(1) << 26)) return HYENA_ERR_INVALID_ARG;
    const bool fs = plan->path == HYENA_PATH_FOURSTEP;
    if (!(plan->path == HYENA_PATH_LDS || fs) || (fs && plan->circular)) return HYENA_ERR_UNSUPPORTED;
    if ((int64_t)B * 8 * ((plan->D + 7) / 8) > 0x7fffffff) return HYENA_ERR_INVALID_ARG;
    // per sample, dh alone is 4*B*(N-1)*D*L bytes; the bound keeps every grid below 2^32 work-items
    if (per_sample && B * (plan->order - 1) * plan->D * plan->L > (int64_t(1) << 35)) return HYENA_ERR_INVALID_ARG;
    if (!workspace || !aligned16(workspace) || workspace_bytes < backward_ws(plan, B, per_sample))
        return HYENA_ERR_WORKSPACE;
    if (hy::check_device(plan) != HYENA_OK) return HYENA_ERR_DEVICE;
    // sample b reads spectrum b when every sample has its own filters
    const int64_t sbs = per_sample ? (int64_t)(plan->order - 1) * plan->D * (int64_t(1) << plan->logT) : 0;
    if (fs) {
        hy::FsBwdArgs a{u_proj, short_w, (const float2*)spec, bias, dy, du_proj, dshort_w, dh, dbias, workspace,
                        plan->fs, (int)B, (int)plan->D, plan->order, plan->dtype == HYENA_BF16, sbs, per_sample};
        return hy::launch_fs_backward(plan->logT, a, stream) == hipSuccess ? HYENA_OK : HYENA_ERR_DEVICE;
    }
    hy::LdsBwdArgs a{u_proj,   short_w,   (const float2*)spec, bias,      dy,         du_proj,
                     dshort_w, dh,        dbias,               (float2*)workspace, plan->tw, plan->wpair,
                     (int)B,   (int)plan->D, plan->order,       plan->dtype == HYENA_BF16, sbs, per_sample,
                     plan->circular};
    return hy::launch_lds_backward(plan->logT, a, stream) == hipSuccess ? HYENA_OK : HYENA_ERR_DEVICE;
}

}  // namespace

extern "C" {

size_t hyena_backward_workspace_bytes(hyena_plan_t plan, int64_t B) { return backward_ws(plan, B, false); }

size_t hyena_backward_per_sample_workspace_bytes(hyena_plan_t plan, int64_t B) { return backward_ws(plan, B, true); }

hyena_status_t hyena_backward(hyena_plan_t plan, int64_t B, const void* u_proj, const float* short_w,
                              const void* spec, const float* bias, const void* dy, void* du_proj, float* dshort_w,
                              float* dh, float* dbias, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return backward_impl(plan, B, u_proj, short_w, spec, bias, dy, du_proj, dshort_w, dh, dbias, workspace,
                         workspace_bytes, stream, false);
}

hyena_status_t hyena_backward_per_sample(hyena_plan_t plan, int64_t B, const void* u_proj, const float* short_w,
                                         const void* spec, const float* bias, const void* dy, void* du_proj,
                                         float* dshort_w, float* dh, float* dbias, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
    return backward_impl(plan, B, u_proj, short_w, spec, bias, dy, du_proj, dshort_w, dh, dbias, workspace,
                         workspace_bytes, stream, true);
}

}  // extern "C"
