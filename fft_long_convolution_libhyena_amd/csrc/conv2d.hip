// Gated 2-D long convolution for gfx950 (HyenaND summary, methodology: global
// convolution evaluated by an N-d FFT on the native grid, the input zero-padded to
// double the grid in every dimension for the non-circular mode; the gate and the
// bias skip as in one step of the HyenaDNA walkthrough's recurrence, section 2.1).
// For every (b, d) image s = v * g (H x W), with the kernel k given on the doubled
// grid (2H x 2W; rows >= H and columns >= W are the negative offsets):
//   c[p][q] = sum_{i<2H, j<2W} k[i][j] s_pad[(p - i) mod 2H][(q - j) mod 2W],
//   y = (c + bias * s) * x,          p < H, q < W.
//
// The real 2H x 2W transform is carried as a 2H x W complex transform of the
// image packed along w (z[h][m] = s[h][2m] + i s[h][2m+1]); its zero padding
// leaves rows h >= H and packed columns m >= W/2 empty. Three passes over a tile
// of 2H x W/2 complex values per image (the empty columns are never stored):
//  A  column FFTs over h (length 2H, first radix pass pruned: rows >= H are 0);
//  B  for the row pair {kh, 2H - kh} (and {0, H}): row FFTs over m (length W,
//     pruned: m >= W/2 is 0), the pair step that turns Z into the real spectrum
//     S (bin (kh, kw) pairs with (-kh, -kw); the twiddle is W_{2W}^kw), the
//     multiply by the kernel spectrum plus the bias, the repack and the inverse
//     rows, of which only m < W/2 is kept;
//  C  inverse column FFTs, rows h < H kept, the gate, y.
// There is no twiddle between the column and the row transforms: this is the
// 2-D transform, not the 1-D four-step. The kernel spectrum is stored as the
// [2H][W+1] bins of the doubled-grid real transform (numpy's rfft2 layout),
// scaled by 1/(4 * 2H * W) so that the pair step also applies the inverse
// normalisation, like the 1-D path's spectrum.
// The pass kernels are shared with the 3-D step (conv_nd.hpp). A circular plan
// (periodic grid, kernel on the H x W grid itself) runs the same passes on
// transforms of the grid's own size: columns of length H, rows of W/2 packed
// points, nothing pruned and every output kept.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <new>
#include <vector>

#include "../../include/hyena.h"
#include "conv_nd.hpp"
#include "plan.hpp"
#include "tables.hpp"

struct hyena_plan2d_s {
    int64_t H = 0, W = 0, D = 0;
    int logH = 0, logW = 0;
    bool circular = false;
    // transform geometry: column transforms of 2^(lc+1) points, row transforms of
    // 2^lr packed points, rows paired as PairMap2{pm}
    int lc = 0, lr = 0, pm = 0;
    hyena_dtype_t dtype = HYENA_F32;
    int device = -1;
    float2* dtab = nullptr;
    const float2* tw1 = nullptr;    // Stockham tables, length 2H (columns)
    const float2* tw2 = nullptr;    // Stockham tables, length W (rows)
    const float2* wpair = nullptr;  // W_{2W}^kw, kw < W
};

namespace hy {
namespace {

constexpr int kC2MinLogH = 4, kC2MaxLogH = 9;  // H = 16 .. 512
constexpr int kC2MinLogW = 5, kC2MaxLogW = 9;  // W = 32 .. 512
constexpr size_t kC2ChunkBytes = 128u << 20;   // tiles in flight per launch

// Spectrum pass 1: column FFTs of the packed doubled-grid kernel (no padding: all
// 2H rows and W packed columns hold data), into spec rows of pitch W + 1.
template <int LOGH>
__global__ void __launch_bounds__(C2Col<LOGH>::THREADS)
k_c2_spec_col(const float* __restrict__ k, float2* __restrict__ spec, const float2* __restrict__ tw1, int W,
              int64_t nrows) {
    using C = C2Col<LOGH>;
    constexpr int C1 = C::C1, T1 = C::T1, CB = kC2CB;
    __shared__ float2 lds[C1 * C::CP];
    int64_t r;
    int cb;
    if (!xcd_row_map(blockIdx.x, nrows, W / CB, r, cb)) return;
    const int c = threadIdx.x % CB, t = threadIdx.x / CB;
    const int m = cb * CB + c;
    const float* kr = k + r * (int64_t)C1 * 2 * W;
    float2 a[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) a[e] = load_pair(kr + (int64_t)(t + T1 * e) * 2 * W, (uint32_t)m);
    fft_strided<C1, false, false>(a, t, tw1, ColAcc<C::CP>{lds + c});
    float2* sr = spec + r * (int64_t)C1 * (W + 1);
#pragma unroll
    for (int e = 0; e < 16; ++e) sr[(int64_t)(t + T1 * e) * (W + 1) + m] = a[e];
}

// ---------------------------------------------------------------- launchers

template <int LOGH>
void launch_spec_col(const float* k, float2* spec, const float2* tw1, int W, int64_t nrows, hipStream_t st) {
    const unsigned grid = (unsigned)xcd_grid(nrows, W / kC2CB);
    hipLaunchKernelGGL((k_c2_spec_col<LOGH>), dim3(grid), dim3(C2Col<LOGH>::THREADS), 0, st, k, spec, tw1, W,
                       nrows);
}

hipError_t spec_cols(int logH, const float* k, float2* spec, const float2* tw1, int W, int64_t nrows,
                     hipStream_t st) {
    switch (logH) {
        case 4: launch_spec_col<4>(k, spec, tw1, W, nrows, st); break;
        case 5: launch_spec_col<5>(k, spec, tw1, W, nrows, st); break;
        case 6: launch_spec_col<6>(k, spec, tw1, W, nrows, st); break;
        case 7: launch_spec_col<7>(k, spec, tw1, W, nrows, st); break;
        case 8: launch_spec_col<8>(k, spec, tw1, W, nrows, st); break;
        case 9: launch_spec_col<9>(k, spec, tw1, W, nrows, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hyena_status_t check2d(const hyena_plan2d_t plan) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return HYENA_ERR_DEVICE;
    return dev == plan->device ? HYENA_OK : HYENA_ERR_DEVICE;
}

}  // namespace
}  // namespace hy

extern "C" {

hyena_status_t hyena_plan2d_create_ex(hyena_plan2d_t* out, int64_t H, int64_t W, int64_t D, hyena_dtype_t dtype,
                                      uint32_t flags) {
    if (!out) return HYENA_ERR_INVALID_ARG;
    if (flags & ~(uint32_t)HYENA_FLAG_CIRCULAR) return HYENA_ERR_INVALID_ARG;
    if (H < 1 || W < 1 || D < 1) return HYENA_ERR_INVALID_ARG;
    if (dtype != HYENA_F32 && dtype != HYENA_BF16) return HYENA_ERR_INVALID_ARG;
    if (!hy::pow2(H) || !hy::pow2(W) || D > (int64_t(1) << 24)) return HYENA_ERR_UNSUPPORTED;
    const bool circ = (flags & HYENA_FLAG_CIRCULAR) != 0;
    const int logH = hy::log2i(H), logW = hy::log2i(W);
    // circular: transforms of the grid's own size (H columns, W/2 packed points)
    const int lc = circ ? logH - 1 : logH, lr = circ ? logW - 1 : logW;
    if (lc < hy::kC2MinLogH || lc > hy::kC2MaxLogH || lr < hy::kC2MinLogW || lr > hy::kC2MaxLogW)
        return HYENA_ERR_UNSUPPORTED;
    const int64_t Wr = int64_t(1) << lr;  // packed row transform length
    std::vector<float2> tab;
    const size_t o_tw1 = hy::append_stockham(tab, lc + 1);
    const size_t o_tw2 = hy::append_stockham(tab, lr);
    const size_t o_wp = tab.size();
    for (int64_t k = 0; k < Wr; ++k) tab.push_back(hy::wfwd(k, 2 * Wr));
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return HYENA_ERR_DEVICE;
    float2* dtab = nullptr;
    if (hipMalloc((void**)&dtab, tab.size() * sizeof(float2)) != hipSuccess) return HYENA_ERR_DEVICE;
    if (hipMemcpy(dtab, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(dtab);
        return HYENA_ERR_DEVICE;
    }
    hyena_plan2d_s* plan = new (std::nothrow) hyena_plan2d_s();
    if (!plan) {
        (void)hipFree(dtab);
        return HYENA_ERR_DEVICE;
    }
    plan->H = H;
    plan->W = W;
    plan->D = D;
    plan->logH = logH;
    plan->logW = logW;
    plan->circular = circ;
    plan->lc = lc;
    plan->lr = lr;
    plan->pm = circ ? (int)(H / 2) : (int)H;
    plan->dtype = dtype;
    plan->device = dev;
    plan->dtab = dtab;
    plan->tw1 = dtab + o_tw1;
    plan->tw2 = dtab + o_tw2;
    plan->wpair = dtab + o_wp;
    *out = plan;
    return HYENA_OK;
}

hyena_status_t hyena_plan2d_create(hyena_plan2d_t* out, int64_t H, int64_t W, int64_t D, hyena_dtype_t dtype) {
    return hyena_plan2d_create_ex(out, H, W, D, dtype, 0);
}

hyena_status_t hyena_plan2d_destroy(hyena_plan2d_t plan) {
    if (!plan) return HYENA_OK;
    const hyena_status_t st = (plan->dtab && hipFree(plan->dtab) != hipSuccess) ? HYENA_ERR_DEVICE : HYENA_OK;
    delete plan;
    return st;
}

size_t hyena_spectrum2d_bytes(hyena_plan2d_t plan) {
    if (!plan) return 0;
    return (size_t)plan->D * ((size_t)2 << plan->lc) * (((size_t)1 << plan->lr) + 1) * sizeof(float2);
}

// the tile of one image: the column transform's rows x W/2 packed columns
static size_t tile2d_bytes(const hyena_plan2d_t plan) {
    return ((size_t)2 << plan->lc) * (size_t)(plan->W / 2) * sizeof(float2);
}

size_t hyena_workspace2d_bytes(hyena_plan2d_t plan, int64_t B) {
    if (!plan || B < 1) return 0;
    const size_t per = tile2d_bytes(plan);
    int64_t want = (int64_t)(hy::kC2ChunkBytes / per);
    if (want < 1) want = 1;
    if (want > B * plan->D) want = B * plan->D;
    return (size_t)want * per;
}

hyena_status_t hyena_filter_spectrum2d_batched(hyena_plan2d_t plan, int64_t B, const float* k, void* spec,
                                               hipStream_t stream) {
    using hy::aligned16;
    if (!plan || B < 1 || !k || !spec || !aligned16(k) || !aligned16(spec)) return HYENA_ERR_INVALID_ARG;
    if (B > (int64_t(1) << 24) || B * plan->D > (int64_t(1) << 24)) return HYENA_ERR_INVALID_ARG;
    if (hy::check2d(plan) != HYENA_OK) return HYENA_ERR_DEVICE;
    const int64_t n = B * plan->D;  // the B kernel sets are B*D consecutive kernels
    float2* sp = (float2*)spec;
    // kernel rows of 2^(lr+1) samples (2W zero-padded, W circular)
    hipError_t e = hy::spec_cols(plan->lc, k, sp, plan->tw1, 1 << plan->lr, n, stream);
    if (e == hipSuccess)
        e = hy::rows(plan->lr, 1, sp, nullptr, nullptr, plan->tw2, plan->wpair, hy::PairMap2{plan->pm}, plan->pm,
                     (int)plan->D, 0, n, false, stream);
    return e == hipSuccess ? HYENA_OK : HYENA_ERR_DEVICE;
}

hyena_status_t hyena_filter_spectrum2d(hyena_plan2d_t plan, const float* k, void* spec, hipStream_t stream) {
    return hyena_filter_spectrum2d_batched(plan, 1, k, spec, stream);
}

static hyena_status_t conv2d_impl(hyena_plan2d_t plan, int64_t B, const void* v, const void* g, const void* x,
                                  const void* spec, const float* bias, void* y, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream, bool per_sample) {
    using hy::aligned16;
    if (!plan || B < 1 || !v || !spec || !bias || !y) return HYENA_ERR_INVALID_ARG;
    if (!aligned16(v) || !aligned16(spec) || !aligned16(bias) || !aligned16(y) || (g && !aligned16(g)) ||
        (x && !aligned16(x)))
        return HYENA_ERR_INVALID_ARG;
    if (B > (int64_t(1) << 24) || B * plan->D > (int64_t(1) << 24)) return HYENA_ERR_INVALID_ARG;
    const size_t per = tile2d_bytes(plan);
    if (!workspace || !aligned16(workspace) || workspace_bytes < per) return HYENA_ERR_WORKSPACE;
    if (hy::check2d(plan) != HYENA_OK) return HYENA_ERR_DEVICE;
    const int64_t nr = B * plan->D;
    int64_t chunk = (int64_t)(workspace_bytes / per);
    if (chunk > nr) chunk = nr;
    if (chunk > 65536) chunk = 65536;
    const bool bf16 = plan->dtype == HYENA_BF16;
    const int W = (int)plan->W;
    float2* tile = (float2*)workspace;
    for (int64_t r0 = 0; r0 < nr; r0 += chunk) {
        const int64_t n = nr - r0 < chunk ? nr - r0 : chunk;
        const bool circ = plan->circular;
        hipError_t e =
            hy::cols(plan->lc, true, bf16, v, g, nullptr, tile, nullptr, plan->tw1, W, r0, n, stream, circ);
        if (e == hipSuccess)
            e = hy::rows(plan->lr, 0, tile, (const float2*)spec, bias, plan->tw2, plan->wpair, hy::PairMap2{plan->pm},
                         plan->pm, (int)plan->D, r0, n, per_sample, stream, circ);
        if (e == hipSuccess)
            e = hy::cols(plan->lc, false, bf16, nullptr, nullptr, x, tile, y, plan->tw1, W, r0, n, stream, circ);
        if (e != hipSuccess) return HYENA_ERR_DEVICE;
    }
    return HYENA_OK;
}

hyena_status_t hyena_conv2d_forward(hyena_plan2d_t plan, int64_t B, const void* v, const void* g, const void* x,
                                    const void* spec, const float* bias, void* y, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    return conv2d_impl(plan, B, v, g, x, spec, bias, y, workspace, workspace_bytes, stream, false);
}

hyena_status_t hyena_conv2d_forward_per_sample(hyena_plan2d_t plan, int64_t B, const void* v, const void* g,
                                               const void* x, const void* spec, const float* bias, void* y,
                                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return conv2d_impl(plan, B, v, g, x, spec, bias, y, workspace, workspace_bytes, stream, true);
}

}  // extern "C"
