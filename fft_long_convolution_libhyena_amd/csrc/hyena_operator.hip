// The whole Hyena operator forward around the hot path (HyenaDNA walkthrough,
// section 2.1, HyenaOperator.forward): the input projection, the (B, L, D) ->
// (B, D, L) transpose, the hot path (hyena_forward), the transpose back and the
// output projection. The two projections are plain dense GEMMs and run in
// hipBLASLt (bf16 or fp32 operands, fp32 accumulation); the rearranges cost
// nothing because both GEMMs read and write the layouts the path uses directly:
//   in_proj : u_proj[b] (row-major [(N+1)D][L]) = W_in x[b]^T + b_in
//             column-major view: U (L x C) = X^T (L x D) * W_in^T (D x C) + 1 b_in^T
//   out_proj: out[b] (row-major [L][D])      = y[b]^T W_out^T + b_out
//             column-major view: O (D x L) = W_out (D x D) * Y (D x L) + b_out 1^T
// The output bias is hipBLASLt's bias epilogue (one value per row of O). The
// input bias varies along the columns of U, where that epilogue does not apply,
// so it enters as the C operand (beta = 1) of a bias matrix that a small kernel
// fills once per call. Each sequence b is one ordinary (non-batched) GEMM call:
// the weights and the bias matrix are shared by all b, and sharing them through
// a batch stride of 0 is not a documented hipBLASLt mode.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>
#include <stdint.h>

#include <mutex>
#include <new>
#include <vector>

#include "../../include/hyena.h"
#include "plan.hpp"

namespace {

constexpr size_t kLtWorkspace = 32u << 20;  // scratch offered to hipBLASLt

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

template <class T>
__global__ void k_bias_matrix(const T* __restrict__ b_in, T* __restrict__ cb, int64_t L, int64_t C) {
    // cb[c*L + t] = b_in[c]: column c of the column-major L x C matrix is b_in[c]
    const int64_t n = L * C;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        cb[i] = b_in[i / L];
}

struct Gemm {
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr, d = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    size_t ws = 0;
    std::vector<hipblasLtMatmulAlgo_t> cand;  // heuristic candidates, timed on first use
    void release() {
        if (desc) hipblasLtMatmulDescDestroy(desc);
        for (auto* l : {&a, &b, &c, &d})
            if (*l) hipblasLtMatrixLayoutDestroy(*l);
        desc = nullptr;
        a = b = c = d = nullptr;
    }
};

// Per-plan operator state: the hipBLASLt handle and the descriptors of both GEMMs
// (one sequence each). Built on first use, under the mutex; the first call also
// times the heuristic's candidate kernels on its own buffers and keeps the fastest.
struct OpState {
    std::mutex mu;
    hipblasLtHandle_t lt = nullptr;
    bool built = false, tuned = false;
    Gemm in, out;
    ~OpState() {
        in.release();
        out.release();
        if (lt) hipblasLtDestroy(lt);
    }
};

void op_free(void* p) { delete static_cast<OpState*>(p); }

bool layout(hipblasLtMatrixLayout_t* l, hipDataType t, uint64_t rows, uint64_t cols, int64_t ld) {
    return hipblasLtMatrixLayoutCreate(l, t, rows, cols, ld) == HIPBLAS_STATUS_SUCCESS;
}

constexpr int kCandidates = 16;

bool pick_algo(hipblasLtHandle_t lt, Gemm& g) {
    hipblasLtMatmulPreference_t pref = nullptr;
    if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return false;
    const uint64_t maxws = kLtWorkspace;
    hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &maxws, sizeof(maxws));
    hipblasLtMatmulHeuristicResult_t res[kCandidates];
    int n = 0;
    const hipblasStatus_t st =
        hipblasLtMatmulAlgoGetHeuristic(lt, g.desc, g.a, g.b, g.c, g.d, pref, kCandidates, res, &n);
    hipblasLtMatmulPreferenceDestroy(pref);
    if (st != HIPBLAS_STATUS_SUCCESS) return false;
    g.cand.clear();
    for (int i = 0; i < n; ++i)
        if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize <= kLtWorkspace) g.cand.push_back(res[i].algo);
    if (g.cand.empty()) return false;
    g.algo = g.cand[0];  // the heuristic's first choice until timed
    return true;
}

// Times every candidate of g on the given operands (one warm-up and three timed
// calls each, HIP events on `stream`) and keeps the fastest. The operands are the
// call's own buffers; the output is rewritten by the real call afterwards.
void tune(hipblasLtHandle_t lt, Gemm& g, const void* alpha, const void* A, const void* B, const void* beta,
          const void* C, void* Dm, void* ws, hipStream_t stream) {
    if (g.cand.size() < 2) return;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        if (e0) (void)hipEventDestroy(e0);
        return;
    }
    float best = 1e30f;
    for (const auto& algo : g.cand) {
        if (hipblasLtMatmul(lt, g.desc, alpha, A, g.a, B, g.b, beta, C, g.c, Dm, g.d, &algo, ws, kLtWorkspace,
                            stream) != HIPBLAS_STATUS_SUCCESS)
            continue;
        (void)hipEventRecord(e0, stream);
        bool ok = true;
        for (int r = 0; r < 3 && ok; ++r)
            ok = hipblasLtMatmul(lt, g.desc, alpha, A, g.a, B, g.b, beta, C, g.c, Dm, g.d, &algo, ws, kLtWorkspace,
                                 stream) == HIPBLAS_STATUS_SUCCESS;
        (void)hipEventRecord(e1, stream);
        if (!ok || hipEventSynchronize(e1) != hipSuccess) continue;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, e0, e1) == hipSuccess && ms < best) {
            best = ms;
            g.algo = algo;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
}

// Descriptors of both GEMMs for one sequence (column-major views, see the file header).
bool build(OpState& s, const hyena_plan_s* plan) {
    s.in.release();
    s.out.release();
    s.built = s.tuned = false;
    const bool bf16 = plan->dtype == HYENA_BF16;
    const hipDataType dt = bf16 ? HIP_R_16BF : HIP_R_32F;
    const int64_t L = plan->L, D = plan->D, C = (int64_t)(plan->order + 1) * plan->D;
    const hipblasOperation_t T = HIPBLAS_OP_T, N = HIPBLAS_OP_N;
    // in_proj: U (L x C, ld L) = op_T(X: D x L, ld D) * W (D x C, ld D) + CB (L x C, ld L)
    Gemm& g1 = s.in;
    if (hipblasLtMatmulDescCreate(&g1.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) return false;
    if (hipblasLtMatmulDescSetAttribute(g1.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &T, sizeof(T)) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatmulDescSetAttribute(g1.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &N, sizeof(N)) != HIPBLAS_STATUS_SUCCESS)
        return false;
    if (!layout(&g1.a, dt, D, L, D) || !layout(&g1.b, dt, D, C, D) || !layout(&g1.c, dt, L, C, L) ||
        !layout(&g1.d, dt, L, C, L))
        return false;
    if (!pick_algo(s.lt, g1)) return false;
    // out_proj: O (D x L, ld D) = op_T(Wo: D x D, ld D) * op_T(Y: L x D, ld L) + b_out (bias epilogue, one
    //           value per row of O)
    Gemm& g2 = s.out;
    if (hipblasLtMatmulDescCreate(&g2.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) return false;
    const hipblasLtEpilogue_t epi = HIPBLASLT_EPILOGUE_BIAS;
    if (hipblasLtMatmulDescSetAttribute(g2.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &T, sizeof(T)) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatmulDescSetAttribute(g2.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &T, sizeof(T)) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatmulDescSetAttribute(g2.desc, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof(epi)) !=
            HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatmulDescSetAttribute(g2.desc, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &dt, sizeof(dt)) !=
            HIPBLAS_STATUS_SUCCESS)
        return false;
    if (!layout(&g2.a, dt, D, D, D) || !layout(&g2.b, dt, L, D, L) || !layout(&g2.c, dt, D, L, D) ||
        !layout(&g2.d, dt, D, L, D))
        return false;
    // the bias pointer takes part in the heuristic's choice of kernel; a placeholder is set here
    const void* placeholder = reinterpret_cast<const void*>(uintptr_t(256));
    hipblasLtMatmulDescSetAttribute(g2.desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &placeholder, sizeof(placeholder));
    if (!pick_algo(s.lt, g2)) return false;
    s.built = true;
    return true;
}

struct Carve {
    void* u;
    void* y;
    void* cb;
    void* lt;
    void* path;
    size_t path_bytes;
    size_t total;
};

Carve carve(const hyena_plan_s* plan, int64_t B, void* base) {
    const size_t s = plan->dtype == HYENA_BF16 ? 2 : 4;
    const size_t L = (size_t)plan->L, D = (size_t)plan->D, C = (size_t)(plan->order + 1) * D;
    Carve c{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        void* p = base ? static_cast<char*>(base) + off : nullptr;
        off += align256(bytes);
        return p;
    };
    c.u = take((size_t)B * C * L * s);
    c.y = take((size_t)B * D * L * s);
    c.cb = take(L * C * s);
    c.lt = take(kLtWorkspace);
    c.path_bytes = hyena_workspace_bytes(const_cast<hyena_plan_s*>(plan), B);
    c.path = c.path_bytes ? take(c.path_bytes) : nullptr;
    c.total = off;
    return c;
}

hyena_status_t operator_impl(hyena_plan_t plan, int64_t B, const void* x, const void* w_in, const void* b_in,
                             const float* short_w, const void* spec, const float* bias, const void* w_out,
                             const void* b_out, void* out, void* workspace, size_t workspace_bytes,
                             hipStream_t stream, float* ms) {
    using hy::aligned16;
    if (!plan || B < 1 || !x || !w_in || !b_in || !short_w || !spec || !bias || !w_out || !b_out || !out)
        return HYENA_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_in) || !aligned16(b_in) || !aligned16(w_out) || !aligned16(b_out) ||
        !aligned16(out))
        return HYENA_ERR_INVALID_ARG;
    if (B > (int64_t(1) << 24) || B * plan->D > (int64_t(1) << 26) || plan->L * plan->D > (int64_t(1) << 31))
        return HYENA_ERR_INVALID_ARG;
    if (!workspace || !aligned16(workspace) || workspace_bytes < hyena_operator_workspace_bytes(plan, B))
        return HYENA_ERR_WORKSPACE;
    if (hy::check_device(plan) != HYENA_OK) return HYENA_ERR_DEVICE;

    // the per-plan operator state is attached on first use; calls on one plan are
    // serialised by its mutex
    {
        static std::mutex create_mu;
        std::lock_guard<std::mutex> g(create_mu);
        if (!plan->op) {
            OpState* s = new (std::nothrow) OpState();
            if (!s) return HYENA_ERR_DEVICE;
            if (hipblasLtCreate(&s->lt) != HIPBLAS_STATUS_SUCCESS) {
                delete s;
                return HYENA_ERR_DEVICE;
            }
            plan->op_free = op_free;
            plan->op = s;
        }
    }
    OpState& s = *static_cast<OpState*>(plan->op);
    std::lock_guard<std::mutex> lock(s.mu);
    if (!s.built && !build(s, plan)) return HYENA_ERR_UNSUPPORTED;

    const Carve c = carve(plan, B, workspace);
    const bool bf16 = plan->dtype == HYENA_BF16;
    const size_t es = bf16 ? 2 : 4;
    const int64_t L = plan->L, D = plan->D, C = (int64_t)(plan->order + 1) * plan->D;
    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    if (ms) {
        for (auto& e : ev)
            if (hipEventCreate(&e) != hipSuccess) {
                for (auto& f : ev)
                    if (f) (void)hipEventDestroy(f);
                return HYENA_ERR_DEVICE;
            }
        (void)hipEventRecord(ev[0], stream);
    }
    hyena_status_t st = HYENA_OK;
    const float one = 1.f, zero = 0.f;
    // input projection, with b_in broadcast through the C operand
    const int64_t n = L * C;
    const unsigned grid = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    if (bf16)
        hipLaunchKernelGGL(k_bias_matrix<uint16_t>, dim3(grid), dim3(256), 0, stream, (const uint16_t*)b_in,
                           (uint16_t*)c.cb, L, C);
    else
        hipLaunchKernelGGL(k_bias_matrix<float>, dim3(grid), dim3(256), 0, stream, (const float*)b_in, (float*)c.cb,
                           L, C);
    if (hipGetLastError() != hipSuccess) st = HYENA_ERR_DEVICE;
    if (st == HYENA_OK && !s.tuned) {
        // first call on this plan: time the candidates on sequence 0's operands
        tune(s.lt, s.in, &one, x, w_in, &one, c.cb, c.u, c.lt, stream);
        hipblasLtMatmulDescSetAttribute(s.out.desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &b_out, sizeof(b_out));
        tune(s.lt, s.out, &one, w_out, c.y, &zero, out, out, c.lt, stream);
        s.tuned = true;
    }
    for (int64_t b = 0; b < B && st == HYENA_OK; ++b) {
        const char* xb = static_cast<const char*>(x) + (size_t)b * L * D * es;
        char* ub = static_cast<char*>(c.u) + (size_t)b * C * L * es;
        if (hipblasLtMatmul(s.lt, s.in.desc, &one, xb, s.in.a, w_in, s.in.b, &one, c.cb, s.in.c, ub, s.in.d,
                            &s.in.algo, c.lt, kLtWorkspace, stream) != HIPBLAS_STATUS_SUCCESS)
            st = HYENA_ERR_DEVICE;
    }
    if (ms) (void)hipEventRecord(ev[1], stream);
    // the hot path
    if (st == HYENA_OK)
        st = hyena_forward(plan, B, c.u, short_w, spec, bias, c.y, c.path, c.path_bytes, stream);
    if (ms) (void)hipEventRecord(ev[2], stream);
    // output projection with the bias epilogue
    if (st == HYENA_OK)
        hipblasLtMatmulDescSetAttribute(s.out.desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &b_out, sizeof(b_out));
    for (int64_t b = 0; b < B && st == HYENA_OK; ++b) {
        const char* yb = static_cast<const char*>(c.y) + (size_t)b * D * L * es;
        char* ob = static_cast<char*>(out) + (size_t)b * L * D * es;
        if (hipblasLtMatmul(s.lt, s.out.desc, &one, w_out, s.out.a, yb, s.out.b, &zero, ob, s.out.c, ob, s.out.d,
                            &s.out.algo, c.lt, kLtWorkspace, stream) != HIPBLAS_STATUS_SUCCESS)
            st = HYENA_ERR_DEVICE;
    }
    if (ms) {
        (void)hipEventRecord(ev[3], stream);
        if (st == HYENA_OK && hipEventSynchronize(ev[3]) != hipSuccess) st = HYENA_ERR_DEVICE;
        if (st == HYENA_OK) {
            for (int i = 0; i < 3; ++i) (void)hipEventElapsedTime(&ms[i], ev[i], ev[i + 1]);
            (void)hipEventElapsedTime(&ms[3], ev[0], ev[3]);
        }
        for (auto& e : ev) (void)hipEventDestroy(e);
    }
    return st;
}

}  // namespace

extern "C" {

size_t hyena_operator_workspace_bytes(hyena_plan_t plan, int64_t B) {
    if (!plan || B < 1) return 0;
    return carve(plan, B, nullptr).total;
}

hyena_status_t hyena_operator_forward(hyena_plan_t plan, int64_t B, const void* x, const void* w_in,
                                      const void* b_in, const float* short_w, const void* spec, const float* bias,
                                      const void* w_out, const void* b_out, void* out, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    return operator_impl(plan, B, x, w_in, b_in, short_w, spec, bias, w_out, b_out, out, workspace,
                         workspace_bytes, stream, nullptr);
}

hyena_status_t hyena_operator_forward_timed(hyena_plan_t plan, int64_t B, const void* x, const void* w_in,
                                            const void* b_in, const float* short_w, const void* spec,
                                            const float* bias, const void* w_out, const void* b_out, void* out,
                                            void* workspace, size_t workspace_bytes, hipStream_t stream,
                                            float* ms) {
    if (!ms) return HYENA_ERR_INVALID_ARG;
    return operator_impl(plan, B, x, w_in, b_in, short_w, spec, bias, w_out, b_out, out, workspace,
                         workspace_bytes, stream, ms);
}

}  // extern "C"
