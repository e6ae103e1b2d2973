// Gated 3-D long convolution for gfx950 (HyenaND summary, methodology: global
// convolution evaluated by an N-d FFT on the native grid, the input zero-padded
// to double the grid in every dimension for the non-circular mode; the gate and
// the bias skip as in one step of the HyenaDNA walkthrough's recurrence, section
// 2.1). For every (b, d) volume s = v * g (A x H x W), with the kernel k given on
// the doubled grid (2A x 2H x 2W; indices >= the axis length are the negative
// offsets):
//   c[a][p][q] = sum_{l, i, j} k[l][i][j] s_pad[(a-l) mod 2A][(p-i) mod 2H][(q-j) mod 2W],
//   y = (c + bias * s) * x,          a < A, p < H, q < W.
//
// The real 2A x 2H x 2W transform is carried as a 2A x 2H x W complex transform
// of the volume packed along w, in five passes over two tiles per volume (the
// pass kernels are the 2-D step's, conv_nd.hpp):
//  A1 column FFTs over a (length 2A, first radix pass pruned) of the gated
//     volume seen as an A x (H*W) image: tile 1 = [ka][h][m], m < W/2;
//  A2 column FFTs over h (length 2H, pruned) of every (volume, ka) slab:
//     tile 2 = [ka][kh][m];
//  B  row FFTs over m (length W, pruned) with the pair step: row (ka, kh) pairs
//     with (-ka, -kh), bin kw with -kw; the multiply by the kernel spectrum plus
//     the bias, the repack and the inverse rows, m < W/2 kept;
//  C2 inverse column FFTs over kh, h < H kept, back to tile 1;
//  C1 inverse column FFTs over ka, a < A kept, the gate, y.
// The kernel spectrum is the [2A][2H][W+1] bins of the doubled grid's real
// transform (numpy's rfftn layout), scaled by 1/(4 * 2A * 2H * W): column FFTs
// over a and over h of the packed kernel, then the row pass in spectrum mode.
// A circular plan (periodic grid, kernel on the A x H x W grid itself) runs the
// same passes on transforms of the grid's own size, nothing pruned, every
// output kept, the height transforms in place on one tile.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <new>
#include <vector>

#include "../../include/hyena.h"
#include "conv_nd.hpp"
#include "plan.hpp"
#include "tables.hpp"

struct hyena_plan3d_s {
    int64_t A = 0, H = 0, W = 0, D = 0;
    int logA = 0, logH = 0, logW = 0;
    bool circular = false;
    // transform geometry: depth transforms of 2^(la+1) points, height transforms of
    // 2^lh points, row transforms of 2^lr packed points, rows paired as PairMap3{pa, ph}
    int la = 0, lh = 0, lr = 0, pa = 0, ph = 0;
    hyena_dtype_t dtype = HYENA_F32;
    int device = -1;
    float2* dtab = nullptr;
    const float2* twa = nullptr;    // Stockham tables, length 2A
    const float2* twh = nullptr;    // Stockham tables, length 2H
    const float2* tww = nullptr;    // Stockham tables, length W
    const float2* wpair = nullptr;  // W_{2W}^kw, kw < W
};

namespace hy {
namespace {

constexpr int kC3MinLog = 4, kC3MaxLog = 9;     // A, H = 16 .. 512
constexpr int kC3MinLogW = 5, kC3MaxLogW = 9;   // W = 32 .. 512
constexpr int kC3MaxLogVol = 24;                // A * H * W <= 2^24
constexpr size_t kC3ChunkBytes = 192u << 20;    // tiles in flight per launch

enum { kColFwdPruned = 0, kColInvHalf = 1, kColFwdFull = 2, kColInvFull = 3 };

template <int LOGN, bool INV, bool PRUNE, bool HALF>
void launch_ccol_t(const float2* in, float2* out, const float2* tw, int64_t nslabs, int ncols, int64_t in_slab,
                   int64_t in_pitch, int in_cw, int in_cp, int64_t out_slab, int64_t out_pitch, int out_cw,
                   int out_cp, hipStream_t st) {
    const unsigned grid = (unsigned)xcd_grid(nslabs, ncols / kC2CB);
    hipLaunchKernelGGL((k_cnd_col<LOGN, INV, PRUNE, HALF>), dim3(grid), dim3(kC2CB * (1 << LOGN) / 16), 0, st, in,
                       out, tw, nslabs, ncols, in_slab, in_pitch, in_cw, in_cp, out_slab, out_pitch, out_cw, out_cp);
}

template <int LOGN>
void launch_ccol_n(int kind, const float2* in, float2* out, const float2* tw, int64_t nslabs, int ncols,
                   int64_t in_slab, int64_t in_pitch, int in_cw, int in_cp, int64_t out_slab, int64_t out_pitch,
                   int out_cw, int out_cp, hipStream_t st) {
    if (kind == kColFwdPruned)
        launch_ccol_t<LOGN, false, true, false>(in, out, tw, nslabs, ncols, in_slab, in_pitch, in_cw, in_cp, out_slab,
                                                out_pitch, out_cw, out_cp, st);
    else if (kind == kColInvHalf)
        launch_ccol_t<LOGN, true, false, true>(in, out, tw, nslabs, ncols, in_slab, in_pitch, in_cw, in_cp, out_slab,
                                               out_pitch, out_cw, out_cp, st);
    else if (kind == kColInvFull)
        launch_ccol_t<LOGN, true, false, false>(in, out, tw, nslabs, ncols, in_slab, in_pitch, in_cw, in_cp,
                                                out_slab, out_pitch, out_cw, out_cp, st);
    else
        launch_ccol_t<LOGN, false, false, false>(in, out, tw, nslabs, ncols, in_slab, in_pitch, in_cw, in_cp,
                                                 out_slab, out_pitch, out_cw, out_cp, st);
}

// Column pass of length 2^logN over complex slabs (see k_cnd_col).
hipError_t ccol(int logN, int kind, const float2* in, float2* out, const float2* tw, int64_t nslabs, int ncols,
                int64_t in_slab, int64_t in_pitch, int in_cw, int in_cp, int64_t out_slab, int64_t out_pitch,
                int out_cw, int out_cp, hipStream_t st) {
#define C3_CASE(n)                                                                                              \
    case n:                                                                                                     \
        launch_ccol_n<n>(kind, in, out, tw, nslabs, ncols, in_slab, in_pitch, in_cw, in_cp, out_slab, out_pitch, \
                         out_cw, out_cp, st);                                                                   \
        break;
    switch (logN) {
        C3_CASE(5)
        C3_CASE(6)
        C3_CASE(7)
        C3_CASE(8)
        C3_CASE(9)
        C3_CASE(10)
        default: return hipErrorInvalidValue;
    }
#undef C3_CASE
    return hipGetLastError();
}

hyena_status_t check3d(const hyena_plan3d_t plan) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return HYENA_ERR_DEVICE;
    return dev == plan->device ? HYENA_OK : HYENA_ERR_DEVICE;
}

// Complex values of tile 1 (depth transformed: 2^(la+1) x H x W/2) and tile 2
// (height transformed too: 2^(la+1) x 2^lh x W/2) of one volume. A circular plan
// transforms height in place: tile 2 is tile 1.
size_t tile1_elems(const hyena_plan3d_t p) { return ((size_t)2 << p->la) * (size_t)p->H * (size_t)(p->W / 2); }
size_t tile2_elems(const hyena_plan3d_t p) { return ((size_t)2 << p->la) * ((size_t)1 << p->lh) * (size_t)(p->W / 2); }
size_t vol_ws_bytes(const hyena_plan3d_t p) {
    return (tile1_elems(p) + (p->circular ? 0 : tile2_elems(p))) * sizeof(float2);
}

}  // namespace
}  // namespace hy

extern "C" {

hyena_status_t hyena_plan3d_create_ex(hyena_plan3d_t* out, int64_t A, int64_t H, int64_t W, int64_t D,
                                      hyena_dtype_t dtype, uint32_t flags) {
    if (!out) return HYENA_ERR_INVALID_ARG;
    if (flags & ~(uint32_t)HYENA_FLAG_CIRCULAR) return HYENA_ERR_INVALID_ARG;
    if (A < 1 || H < 1 || W < 1 || D < 1) return HYENA_ERR_INVALID_ARG;
    if (dtype != HYENA_F32 && dtype != HYENA_BF16) return HYENA_ERR_INVALID_ARG;
    if (!hy::pow2(A) || !hy::pow2(H) || !hy::pow2(W) || D > (int64_t(1) << 24)) return HYENA_ERR_UNSUPPORTED;
    const bool circ = (flags & HYENA_FLAG_CIRCULAR) != 0;
    const int logA = hy::log2i(A), logH = hy::log2i(H), logW = hy::log2i(W);
    // circular: transforms of the grid's own size (A, H, W/2 packed points)
    const int la = circ ? logA - 1 : logA, lh = circ ? logH : logH + 1, lr = circ ? logW - 1 : logW;
    if (la < hy::kC3MinLog || la > hy::kC3MaxLog || lh < hy::kC3MinLog + 1 || lh > hy::kC3MaxLog + 1 ||
        lr < hy::kC3MinLogW || lr > hy::kC3MaxLogW || logA + logH + logW > hy::kC3MaxLogVol)
        return HYENA_ERR_UNSUPPORTED;
    const int64_t Wr = int64_t(1) << lr;  // packed row transform length
    std::vector<float2> tab;
    const size_t o_twa = hy::append_stockham(tab, la + 1);
    const size_t o_twh = hy::append_stockham(tab, lh);
    const size_t o_tww = hy::append_stockham(tab, lr);
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
    hyena_plan3d_s* plan = new (std::nothrow) hyena_plan3d_s();
    if (!plan) {
        (void)hipFree(dtab);
        return HYENA_ERR_DEVICE;
    }
    plan->A = A;
    plan->H = H;
    plan->W = W;
    plan->D = D;
    plan->logA = logA;
    plan->logH = logH;
    plan->logW = logW;
    plan->circular = circ;
    plan->la = la;
    plan->lh = lh;
    plan->lr = lr;
    plan->pa = circ ? (int)(A / 2) : (int)A;
    plan->ph = circ ? (int)(H / 2) : (int)H;
    plan->dtype = dtype;
    plan->device = dev;
    plan->dtab = dtab;
    plan->twa = dtab + o_twa;
    plan->twh = dtab + o_twh;
    plan->tww = dtab + o_tww;
    plan->wpair = dtab + o_wp;
    *out = plan;
    return HYENA_OK;
}

hyena_status_t hyena_plan3d_create(hyena_plan3d_t* out, int64_t A, int64_t H, int64_t W, int64_t D,
                                   hyena_dtype_t dtype) {
    return hyena_plan3d_create_ex(out, A, H, W, D, dtype, 0);
}

hyena_status_t hyena_plan3d_destroy(hyena_plan3d_t plan) {
    if (!plan) return HYENA_OK;
    const hyena_status_t st = (plan->dtab && hipFree(plan->dtab) != hipSuccess) ? HYENA_ERR_DEVICE : HYENA_OK;
    delete plan;
    return st;
}

size_t hyena_spectrum3d_bytes(hyena_plan3d_t plan) {
    if (!plan) return 0;
    return (size_t)plan->D * ((size_t)2 << plan->la) * ((size_t)1 << plan->lh) * (((size_t)1 << plan->lr) + 1) *
           sizeof(float2);
}

size_t hyena_workspace3d_bytes(hyena_plan3d_t plan, int64_t B) {
    if (!plan || B < 1) return 0;
    const size_t per = hy::vol_ws_bytes(plan);
    int64_t want = (int64_t)(hy::kC3ChunkBytes / per);
    if (want < 1) want = 1;
    if (want > B * plan->D) want = B * plan->D;
    return (size_t)want * per;
}

hyena_status_t hyena_filter_spectrum3d_batched(hyena_plan3d_t plan, int64_t B, const float* k, void* spec,
                                               hipStream_t stream) {
    using hy::aligned16;
    if (!plan || B < 1 || !k || !spec || !aligned16(k) || !aligned16(spec)) return HYENA_ERR_INVALID_ARG;
    if (B > (int64_t(1) << 24) || B * plan->D > (int64_t(1) << 24)) return HYENA_ERR_INVALID_ARG;
    if (hy::check3d(plan) != HYENA_OK) return HYENA_ERR_DEVICE;
    // the B kernel sets are B*D consecutive kernels, each [Ta][Th][Wr] complex when
    // packed (Ta, Th, Wr: the depth, height and packed row transform lengths)
    const int64_t D = B * plan->D;
    const int64_t Ta = int64_t(2) << plan->la, Th = int64_t(1) << plan->lh, Wr = int64_t(1) << plan->lr;
    float2* sp = (float2*)spec;
    // over depth: packed kernel rows [ka][h][m < Wr] into spectrum rows of pitch Wr + 1
    hipError_t e = hy::ccol(plan->la + 1, hy::kColFwdFull, (const float2*)k, sp, plan->twa, D, (int)(Th * Wr),
                            Ta * Th * Wr, Th * Wr, (int)(Th * Wr), (int)(Th * Wr), Ta * Th * (Wr + 1), Th * (Wr + 1),
                            (int)Wr, (int)(Wr + 1), stream);
    // over height, in place, for every (kernel, ka) slab
    if (e == hipSuccess)
        e = hy::ccol(plan->lh, hy::kColFwdFull, sp, sp, plan->twh, D * Ta, (int)Wr, Th * (Wr + 1), Wr + 1, (int)Wr,
                     (int)Wr, Th * (Wr + 1), Wr + 1, (int)Wr, (int)Wr, stream);
    if (e == hipSuccess)
        e = hy::rows(plan->lr, 1, sp, nullptr, nullptr, plan->tww, plan->wpair, hy::PairMap3{plan->pa, plan->ph},
                     2 * plan->pa * plan->ph, (int)plan->D, 0, D, false, stream);
    return e == hipSuccess ? HYENA_OK : HYENA_ERR_DEVICE;
}

hyena_status_t hyena_filter_spectrum3d(hyena_plan3d_t plan, const float* k, void* spec, hipStream_t stream) {
    return hyena_filter_spectrum3d_batched(plan, 1, k, spec, stream);
}

static hyena_status_t conv3d_impl(hyena_plan3d_t plan, int64_t B, const void* v, const void* g, const void* x,
                                  const void* spec, const float* bias, void* y, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream, bool per_sample) {
    using hy::aligned16;
    if (!plan || B < 1 || !v || !spec || !bias || !y) return HYENA_ERR_INVALID_ARG;
    if (!aligned16(v) || !aligned16(spec) || !aligned16(bias) || !aligned16(y) || (g && !aligned16(g)) ||
        (x && !aligned16(x)))
        return HYENA_ERR_INVALID_ARG;
    if (B > (int64_t(1) << 24) || B * plan->D > (int64_t(1) << 24)) return HYENA_ERR_INVALID_ARG;
    const size_t per = hy::vol_ws_bytes(plan);
    if (!workspace || !aligned16(workspace) || workspace_bytes < per) return HYENA_ERR_WORKSPACE;
    if (hy::check3d(plan) != HYENA_OK) return HYENA_ERR_DEVICE;
    const int64_t nv = B * plan->D;
    int64_t chunk = (int64_t)(workspace_bytes / per);
    if (chunk > nv) chunk = nv;
    if (chunk > 65536) chunk = 65536;
    const bool bf16 = plan->dtype == HYENA_BF16;
    const bool circ = plan->circular;
    const int64_t Ta = int64_t(2) << plan->la, Th = int64_t(1) << plan->lh, H = plan->H, W2 = plan->W / 2;
    const int plane = (int)(H * plan->W);  // an A x (H*W) image for the passes over depth
    float2* t1 = (float2*)workspace;
    float2* t2 = circ ? t1 : t1 + chunk * (int64_t)hy::tile1_elems(plan);
    const hy::PairMap3 pm{plan->pa, plan->ph};
    for (int64_t r0 = 0; r0 < nv; r0 += chunk) {
        const int64_t n = nv - r0 < chunk ? nv - r0 : chunk;
        hipError_t e =
            hy::cols(plan->la, true, bf16, v, g, nullptr, t1, nullptr, plan->twa, plane, r0, n, stream, circ);
        if (e == hipSuccess)
            e = hy::ccol(plan->lh, circ ? hy::kColFwdFull : hy::kColFwdPruned, t1, t2, plan->twh, n * Ta, (int)W2,
                         H * W2, W2, (int)W2, (int)W2, Th * W2, W2, (int)W2, (int)W2, stream);
        if (e == hipSuccess)
            e = hy::rows(plan->lr, 0, t2, (const float2*)spec, bias, plan->tww, plan->wpair, pm,
                         2 * plan->pa * plan->ph, (int)plan->D, r0, n, per_sample, stream, circ);
        if (e == hipSuccess)
            e = hy::ccol(plan->lh, circ ? hy::kColInvFull : hy::kColInvHalf, t2, t1, plan->twh, n * Ta, (int)W2,
                         Th * W2, W2, (int)W2, (int)W2, H * W2, W2, (int)W2, (int)W2, stream);
        if (e == hipSuccess)
            e = hy::cols(plan->la, false, bf16, nullptr, nullptr, x, t1, y, plan->twa, plane, r0, n, stream, circ);
        if (e != hipSuccess) return HYENA_ERR_DEVICE;
    }
    return HYENA_OK;
}

hyena_status_t hyena_conv3d_forward(hyena_plan3d_t plan, int64_t B, const void* v, const void* g, const void* x,
                                    const void* spec, const float* bias, void* y, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    return conv3d_impl(plan, B, v, g, x, spec, bias, y, workspace, workspace_bytes, stream, false);
}

hyena_status_t hyena_conv3d_forward_per_sample(hyena_plan3d_t plan, int64_t B, const void* v, const void* g,
                                               const void* x, const void* spec, const float* bias, void* y,
                                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return conv3d_impl(plan, B, v, g, x, spec, bias, y, workspace, workspace_bytes, stream, true);
}

}  // extern "C"
