// C-ABI layer of libhyena: plans, argument checks, twiddle tables, dispatch.
// See include/hyena.h for the contract of every entry point.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <new>
#include <vector>

#include "../../include/hyena.h"
#include "fft_core.hpp"
#include "kernels.hpp"
#include "plan.hpp"
#include "tables.hpp"

using hy::aligned16;
using hy::append_stockham;
using hy::check_device;
using hy::wfwd;

namespace {

constexpr int64_t kMaxLog = 20;
constexpr size_t kChunkTargetBytes = 128u << 20;  // in-flight four-step intermediates per sequential chunk
constexpr int64_t kMaxChunkRows = 65536;
// Order-2 four-step forwards run as pipelined launches (one launch per chunk of
// rows plus two) when the workspace holds three tile slots of at least
// min(rows, kPipeMinRows) rows; chunks are capped at kPipeRows rows (measured
// on MI355X at L = 65536: 128-row chunks were fastest; chunks of 32 rows or
// fewer leave the launches too small to fill the GPU).
constexpr int64_t kPipeRows = 128;
constexpr int64_t kPipeMinRows = 32;

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2_64(int64_t x) {
    int l = 0;
    while ((int64_t(1) << l) < x) ++l;
    return l;
}

// Workspace bytes one (b, d) row needs in flight: its transposed tile on the
// four-step path; its window spectra, plus the gated output of a step above order
// 2, on the partitioned path.
size_t ws_per_row(const hyena_plan_t plan) {
    const size_t T = (size_t)1 << plan->logT;
    if (plan->path == HYENA_PATH_PARTITIONED) return T * sizeof(float2) + (plan->order > 2 ? T * sizeof(float) : 0);
    return T * sizeof(float2);
}

int64_t chunk_rows(const hyena_plan_t plan, int64_t rows, size_t ws_bytes) {
    const size_t per_row = ws_per_row(plan);
    int64_t n = (int64_t)(ws_bytes / per_row);
    if (n > rows) n = rows;
    if (n > kMaxChunkRows) n = kMaxChunkRows;  // keeps every grid dimension far below 2^31
    return n;
}

// Rows per chunk of a pipelined four-step forward with this workspace, or 0 when
// the forward runs as sequential chunks instead.
int64_t pipe_rows(const hyena_plan_t plan, int64_t rows, size_t ws_bytes) {
    if (plan->path != HYENA_PATH_FOURSTEP || plan->order != 2 || !hy::fs_pipe_supported(plan->logT)) return 0;
    const size_t slots = (size_t)(2 * plan->order - 1);
    int64_t R = (int64_t)(ws_bytes / (slots * ws_per_row(plan)));
    if (R > kPipeRows) R = kPipeRows;
    if (R > rows) R = rows;
    const int64_t need = rows < kPipeMinRows ? rows : kPipeMinRows;
    return R >= need ? R : 0;
}

}  // namespace

extern "C" {

const char* hyena_status_string(hyena_status_t s) {
    switch (s) {
        case HYENA_OK: return "ok";
        case HYENA_ERR_INVALID_ARG: return "invalid argument";
        case HYENA_ERR_UNSUPPORTED: return "unsupported size or option";
        case HYENA_ERR_WORKSPACE: return "workspace missing or too small";
        case HYENA_ERR_DEVICE: return "HIP device error";
        default: return "unknown status";
    }
}

hyena_status_t hyena_plan_create_ex(hyena_plan_t* out, int64_t L, int64_t D, int order, hyena_dtype_t dtype,
                                    hyena_path_t path, uint32_t flags) {
    if (!out) return HYENA_ERR_INVALID_ARG;
    if (flags & ~(uint32_t)HYENA_FLAG_CIRCULAR) return HYENA_ERR_INVALID_ARG;
    const bool circ = (flags & HYENA_FLAG_CIRCULAR) != 0;
    if (D < 1 || L < 1 || order < 2) return HYENA_ERR_INVALID_ARG;
    if (dtype != HYENA_F32 && dtype != HYENA_BF16) return HYENA_ERR_INVALID_ARG;
    if (path != HYENA_PATH_AUTO && path != HYENA_PATH_LDS && path != HYENA_PATH_FOURSTEP &&
        path != HYENA_PATH_PARTITIONED)
        return HYENA_ERR_INVALID_ARG;
    if (!is_pow2(L) || L < 16 || L > (int64_t(1) << kMaxLog) || order > 8) return HYENA_ERR_UNSUPPORTED;
    if (D > (int64_t(1) << 24)) return HYENA_ERR_UNSUPPORTED;
    const int logL = ilog2_64(L);
    // a zero-padded plan transforms 2L real samples as L complex values; a circular
    // plan transforms its L samples as L/2 complex values
    const int logT = circ ? logL - 1 : logL;
    const int64_t T = int64_t(1) << logT;
    if (logT < hy::kLdsMinLog) return HYENA_ERR_UNSUPPORTED;
    hyena_path_t p = path;
    if (p == HYENA_PATH_AUTO) {
        if (logT <= hy::kLdsMaxLog) p = HYENA_PATH_LDS;
        else p = HYENA_PATH_FOURSTEP;
    }
    if (p == HYENA_PATH_LDS && logT > hy::kLdsMaxLog) return HYENA_ERR_UNSUPPORTED;
    if (p == HYENA_PATH_FOURSTEP && logT < hy::kFsMinLog) return HYENA_ERR_UNSUPPORTED;
    if (p == HYENA_PATH_PARTITIONED && (circ || logT < hy::kPartMinLog || logT > hy::kPartMaxLog))
        return HYENA_ERR_UNSUPPORTED;

    // host tables (fp64 -> fp32)
    std::vector<float2> tab;
    size_t o_tw = 0, o_wpair = 0, o_tw1 = 0, o_tw2 = 0, o_lo = 0, o_hi = 0, o_pa = 0, o_pb = 0;
    int log1 = 0, log2 = 0;
    if (p == HYENA_PATH_LDS || p == HYENA_PATH_PARTITIONED) {
        // the partitioned path transforms 2Q-sample windows: the LDS tables for length Q
        const int lt = p == HYENA_PATH_LDS ? logT : hy::kPartLogQ;
        const int64_t Tl = int64_t(1) << lt;
        o_tw = append_stockham(tab, lt);
        o_wpair = tab.size();
        for (int64_t k = 0; k <= Tl / 2; ++k) tab.push_back(wfwd(k, 2 * Tl));
    } else {
        hy::fs_split(logT, &log1, &log2);
        const int64_t L1 = int64_t(1) << log1, L2 = int64_t(1) << log2;
        o_tw1 = append_stockham(tab, log1);
        o_tw2 = append_stockham(tab, log2);
        // the four-step twiddle W_L^(k1*m2) with k1 = t + T1*e is the product of
        // W_L^(t*m2) and W_L^(T1*e*m2): two small tables, both read with m2 fastest
        const int64_t T1 = L1 / 16;
        o_lo = tab.size();
        for (int64_t t = 0; t < T1; ++t)
            for (int64_t m2 = 0; m2 < L2; ++m2) tab.push_back(wfwd(t * m2, T));
        o_hi = tab.size();
        for (int64_t e = 0; e < 16; ++e)
            for (int64_t m2 = 0; m2 < L2; ++m2) tab.push_back(wfwd(T1 * e * m2, T));
        o_pa = tab.size();
        for (int64_t k1 = 0; k1 < L1; ++k1) tab.push_back(wfwd(k1, 2 * T));
        o_pb = tab.size();
        for (int64_t k2 = 0; k2 < L2; ++k2) tab.push_back(wfwd(L1 * k2, 2 * T));
    }

    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return HYENA_ERR_DEVICE;
    float2* dtab = nullptr;
    if (hipMalloc((void**)&dtab, tab.size() * sizeof(float2)) != hipSuccess) return HYENA_ERR_DEVICE;
    if (hipMemcpy(dtab, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(dtab);
        return HYENA_ERR_DEVICE;
    }
    hyena_plan_s* plan = new (std::nothrow) hyena_plan_s();
    if (!plan) {
        (void)hipFree(dtab);
        return HYENA_ERR_DEVICE;
    }
    plan->L = L;
    plan->D = D;
    plan->order = order;
    plan->logL = logL;
    plan->logT = logT;
    plan->circular = circ;
    plan->dtype = dtype;
    plan->path = p;
    plan->device = dev;
    plan->dtab = dtab;
    if (p == HYENA_PATH_LDS || p == HYENA_PATH_PARTITIONED) {
        plan->tw = dtab + o_tw;
        plan->wpair = dtab + o_wpair;
    } else {
        plan->log1 = log1;
        plan->log2 = log2;
        plan->fs.tw1 = dtab + o_tw1;
        plan->fs.tw2 = dtab + o_tw2;
        plan->fs.tbase = dtab + o_lo;
        plan->fs.tstep = dtab + o_hi;
        plan->fs.pa = dtab + o_pa;
        plan->fs.pb = dtab + o_pb;
    }
    *out = plan;
    return HYENA_OK;
}

hyena_status_t hyena_plan_create_path(hyena_plan_t* out, int64_t L, int64_t D, int order, hyena_dtype_t dtype,
                                      hyena_path_t path) {
    return hyena_plan_create_ex(out, L, D, order, dtype, path, 0);
}

hyena_status_t hyena_plan_create(hyena_plan_t* out, int64_t L, int64_t D, int order, hyena_dtype_t dtype) {
    return hyena_plan_create_path(out, L, D, order, dtype, HYENA_PATH_AUTO);
}

hyena_status_t hyena_plan_destroy(hyena_plan_t plan) {
    if (!plan) return HYENA_OK;
    hyena_status_t st = HYENA_OK;
    if (plan->dtab && hipFree(plan->dtab) != hipSuccess) st = HYENA_ERR_DEVICE;
    if (plan->op && plan->op_free) plan->op_free(plan->op);
    delete plan;
    return st;
}

hyena_path_t hyena_plan_path(hyena_plan_t plan) { return plan ? plan->path : HYENA_PATH_AUTO; }

size_t hyena_spectrum_bytes(hyena_plan_t plan) {
    if (!plan) return 0;
    return (size_t)(plan->order - 1) * (size_t)plan->D * ((size_t)1 << plan->logT) * sizeof(float2);
}

size_t hyena_workspace_bytes(hyena_plan_t plan, int64_t B) {
    if (!plan || B < 1) return 0;
    if (plan->path == HYENA_PATH_LDS) return 0;
    const size_t per_row = ws_per_row(plan);
    int64_t rows = B * plan->D;
    if (pipe_rows(plan, rows, (size_t)-1) > 0) {
        const int64_t R = rows < kPipeRows ? rows : kPipeRows;
        return (size_t)(2 * plan->order - 1) * (size_t)R * per_row;
    }
    int64_t want = (int64_t)(kChunkTargetBytes / per_row);
    if (want < 1) want = 1;
    if (want > rows) want = rows;
    return (size_t)want * per_row;
}

hyena_status_t hyena_filter_spectrum_batched(hyena_plan_t plan, int64_t B, const float* h, void* spec,
                                             hipStream_t stream) {
    if (!plan || B < 1 || !h || !spec) return HYENA_ERR_INVALID_ARG;
    if (!aligned16(h) || !aligned16(spec)) return HYENA_ERR_INVALID_ARG;
    if (B > (int64_t(1) << 24) || B * (plan->order - 1) * plan->D > (int64_t(1) << 24)) return HYENA_ERR_INVALID_ARG;
    if (check_device(plan) != HYENA_OK) return HYENA_ERR_DEVICE;
    const int64_t rows = B * (plan->order - 1) * plan->D;
    hipError_t e;
    if (plan->path == HYENA_PATH_LDS)
        e = hy::launch_lds_spectrum(plan->logT, h, (float2*)spec, rows, plan->tw, plan->wpair, stream, plan->circular);
    else if (plan->path == HYENA_PATH_PARTITIONED)
        // each filter row is L / Q consecutive blocks of Q taps: LDS spectra of Q-sample rows
        e = hy::launch_lds_spectrum(hy::kPartLogQ, h, (float2*)spec, rows << (plan->logT - hy::kPartLogQ), plan->tw,
                                    plan->wpair, stream, false);
    else
        e = hy::launch_fs_spectrum(plan->logT, h, (float2*)spec, rows, plan->fs, stream, plan->circular);
    return e == hipSuccess ? HYENA_OK : HYENA_ERR_DEVICE;
}

hyena_status_t hyena_filter_spectrum(hyena_plan_t plan, const float* h, void* spec, hipStream_t stream) {
    return hyena_filter_spectrum_batched(plan, 1, h, spec, stream);
}

}  // extern "C"

namespace {

// Shared body of hyena_forward and hyena_forward_timed. With `ms`, HIP events are
// recorded around every launch on `stream`, the call waits for them, and the
// elapsed milliseconds are summed per kernel family (see hyena_forward_timed).
hyena_status_t forward_impl(hyena_plan_t plan, int64_t B, const void* u_proj, const float* short_w,
                            const void* spec, const float* bias, void* y, void* workspace, size_t workspace_bytes,
                            hipStream_t stream, float* ms, bool per_sample = false) {
    if (!plan || B < 1 || !u_proj || !short_w || !spec || !bias || !y) return HYENA_ERR_INVALID_ARG;
    if (!aligned16(u_proj) || !aligned16(spec) || !aligned16(y) || !aligned16(short_w) || !aligned16(bias))
        return HYENA_ERR_INVALID_ARG;
    // grid sizes are 32-bit: B*D rows times at most L/16 column blocks
    if (B > (int64_t(1) << 24) || B * plan->D > (int64_t(1) << 26)) return HYENA_ERR_INVALID_ARG;
    const bool bf16 = plan->dtype == HYENA_BF16;
    const int64_t rows = B * plan->D;
    // sample b reads spectrum b when every sample has its own filters
    const int64_t sbs = per_sample ? (int64_t)(plan->order - 1) * plan->D * (int64_t(1) << plan->logT) : 0;
    const bool part = plan->path == HYENA_PATH_PARTITIONED;
    const bool chunked = plan->path == HYENA_PATH_FOURSTEP || part;
    int64_t chunk = 0, pipe = 0;
    if (chunked) {
        if (!workspace || !aligned16(workspace)) return HYENA_ERR_WORKSPACE;
        pipe = pipe_rows(plan, rows, workspace_bytes);
        chunk = pipe > 0 ? pipe : chunk_rows(plan, rows, workspace_bytes);
        if (chunk < 1) return HYENA_ERR_WORKSPACE;
    }
    if (check_device(plan) != HYENA_OK) return HYENA_ERR_DEVICE;

    // launches per chunk: four-step 2N-1, partitioned 2(N-1); pipelined: one per
    // chunk plus 2N-2
    const int per_chunk = part ? 2 * (plan->order - 1) : 2 * plan->order - 1;
    const int64_t nchunks = chunked ? (rows + chunk - 1) / chunk : 1;
    const int64_t nlaunch = pipe > 0 ? nchunks + 2 * plan->order - 2 : chunked ? nchunks * per_chunk : 1;
    std::vector<hipEvent_t> ev;
    if (ms) {
        for (int i = 0; i < 6; ++i) ms[i] = 0.f;
        const int64_t n = pipe > 0 ? nlaunch + 1 : chunked ? nchunks * (per_chunk + 1) : 2;
        if (n > 4096) return HYENA_ERR_INVALID_ARG;  // timing is for bounded chunk counts
        ev.resize((size_t)n, nullptr);
        for (auto& e : ev)
            if (hipEventCreate(&e) != hipSuccess) {
                for (auto& f : ev)
                    if (f) (void)hipEventDestroy(f);
                return HYENA_ERR_DEVICE;
            }
    }
    hyena_status_t st = HYENA_OK;
    if (plan->path == HYENA_PATH_LDS) {
        if ((int64_t)B * 8 * ((plan->D + 7) / 8) > 0x7fffffff) return HYENA_ERR_INVALID_ARG;
        hy::LdsArgs a{u_proj, short_w, (const float2*)spec, bias, y, plan->tw, plan->wpair,
                      (int)B, (int)plan->D, plan->order, bf16, sbs, plan->circular};
        if (ms) (void)hipEventRecord(ev[0], stream);
        if (hy::launch_lds_forward(plan->logT, a, stream) != hipSuccess) st = HYENA_ERR_DEVICE;
        if (ms) (void)hipEventRecord(ev[1], stream);
    } else if (part) {
        // window spectra of the chunk's rows first, then the gated outputs of a step
        const int64_t T = int64_t(1) << plan->logT;
        float* vb = plan->order > 2 ? (float*)((float2*)workspace + chunk * T) : nullptr;
        hy::PartArgs a{u_proj, short_w, (const float2*)spec, bias, y, (float2*)workspace, vb, plan->tw, plan->wpair,
                       (int)plan->D, plan->order, (int)(T >> hy::kPartLogQ), bf16, sbs};
        int64_t ci = 0;
        for (int64_t r0 = 0; r0 < rows && st == HYENA_OK; r0 += chunk, ++ci) {
            const int64_t n = (rows - r0) < chunk ? (rows - r0) : chunk;
            hipEvent_t* marks = ms ? ev.data() + ci * (per_chunk + 1) : nullptr;
            if (hy::launch_part_forward_chunk(a, r0, n, stream, marks) != hipSuccess) st = HYENA_ERR_DEVICE;
        }
    } else if (pipe > 0) {
        hy::FsArgs a{u_proj, short_w, (const float2*)spec, bias, y, (float2*)workspace, plan->fs,
                     (int)plan->D, plan->order, bf16, sbs, plan->circular};
        if (hy::launch_fs_forward_pipelined(plan->logT, a, rows, pipe, stream, ms ? ev.data() : nullptr) !=
            hipSuccess)
            st = HYENA_ERR_DEVICE;
    } else {
        hy::FsArgs a{u_proj, short_w, (const float2*)spec, bias, y, (float2*)workspace, plan->fs,
                     (int)plan->D, plan->order, bf16, sbs, plan->circular};
        int64_t ci = 0;
        for (int64_t r0 = 0; r0 < rows && st == HYENA_OK; r0 += chunk, ++ci) {
            const int64_t n = (rows - r0) < chunk ? (rows - r0) : chunk;
            hipEvent_t* marks = ms ? ev.data() + ci * (per_chunk + 1) : nullptr;
            if (hy::launch_fs_forward_chunk(plan->logT, a, r0, n, stream, marks) != hipSuccess)
                st = HYENA_ERR_DEVICE;
        }
    }
    if (ms) {
        if (st == HYENA_OK && hipEventSynchronize(ev.back()) != hipSuccess) st = HYENA_ERR_DEVICE;
        if (st == HYENA_OK) {
            float t = 0.f;
            if (!chunked) {
                (void)hipEventElapsedTime(&t, ev[0], ev[1]);
                ms[0] = t;
            } else if (pipe > 0) {
                for (int64_t i = 0; i < nlaunch; ++i) {
                    (void)hipEventElapsedTime(&t, ev[i], ev[i + 1]);
                    ms[5] += t;
                }
            } else if (part) {
                for (int64_t c = 0; c < nchunks; ++c) {
                    hipEvent_t* m = ev.data() + c * (per_chunk + 1);
                    for (int i = 0; i < per_chunk; ++i) {
                        (void)hipEventElapsedTime(&t, m[i], m[i + 1]);
                        ms[1 + (i & 1)] += t;  // pass 1, pass 2 alternate
                    }
                }
            } else {
                for (int64_t c = 0; c < nchunks; ++c) {
                    hipEvent_t* m = ev.data() + c * (per_chunk + 1);
                    for (int i = 0; i < per_chunk; ++i) {
                        (void)hipEventElapsedTime(&t, m[i], m[i + 1]);
                        // launch 0 is pass A; then pass B / pass C alternate
                        const int fam = i == 0 ? 1 : (i % 2 == 1 ? 2 : 3);
                        ms[fam] += t;
                    }
                }
            }
            (void)hipEventElapsedTime(&t, ev.front(), ev.back());
            ms[4] = t;
        }
        for (auto& e : ev) (void)hipEventDestroy(e);
    }
    return st;
}

}  // namespace

// ----------------------------------------------- forward without allocation
//
// The four-step and partitioned paths keep their tiles in a workspace. For
// callers that cannot allocate, hyena_forward_noalloc uses this file-scope
// device array instead. Host code never passes the array's name to a kernel or
// a copy (on the host it is only a stand-in for the symbol): the device address
// is looked up once per device with hipGetSymbolAddress, with that device
// current, and kept in g_scratch_ptr.
static constexpr size_t kScratchBytes = HYENA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device, or nullptr.
void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

hyena_status_t hyena_forward_noalloc(hyena_plan_t plan, int64_t B, const void* u_proj, const float* short_w,
                                     const void* spec, const float* bias, void* y, hipStream_t stream) {
    if (!plan) return HYENA_ERR_INVALID_ARG;
    if (plan->path == HYENA_PATH_LDS)  // no scratch on the LDS path
        return forward_impl(plan, B, u_proj, short_w, spec, bias, y, nullptr, 0, stream, nullptr);
    // the smallest workspace the path accepts: one row's tiles
    if (ws_per_row(plan) > kScratchBytes) return HYENA_ERR_WORKSPACE;
    if (check_device(plan) != HYENA_OK) return HYENA_ERR_DEVICE;
    void* ws = scratch_on_current_device();
    if (!ws) return HYENA_ERR_DEVICE;
    return forward_impl(plan, B, u_proj, short_w, spec, bias, y, ws, kScratchBytes, stream, nullptr);
}

hyena_status_t hyena_forward(hyena_plan_t plan, int64_t B, const void* u_proj, const float* short_w,
                             const void* spec, const float* bias, void* y, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    return forward_impl(plan, B, u_proj, short_w, spec, bias, y, workspace, workspace_bytes, stream, nullptr);
}

hyena_status_t hyena_forward_per_sample(hyena_plan_t plan, int64_t B, const void* u_proj, const float* short_w,
                                        const void* spec, const float* bias, void* y, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
    return forward_impl(plan, B, u_proj, short_w, spec, bias, y, workspace, workspace_bytes, stream, nullptr, true);
}

hyena_status_t hyena_forward_timed(hyena_plan_t plan, int64_t B, const void* u_proj, const float* short_w,
                                   const void* spec, const float* bias, void* y, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream, float* ms) {
    if (!ms) return HYENA_ERR_INVALID_ARG;
    return forward_impl(plan, B, u_proj, short_w, spec, bias, y, workspace, workspace_bytes, stream, ms);
}

}  // extern "C"
