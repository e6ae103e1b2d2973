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
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <new>
#include <vector>

#include "../../include/hyena.h"
#include "fft_core.hpp"
#include "fourstep.hpp"
#include "pair.hpp"
#include "plan.hpp"
#include "tables.hpp"

struct hyena_plan2d_s {
    int64_t H = 0, W = 0, D = 0;
    int logH = 0, logW = 0;
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
constexpr int kC2CB = 16;                      // columns per pass A / C workgroup
constexpr size_t kC2ChunkBytes = 128u << 20;   // tiles in flight per launch

template <int LOGH>
struct C2Col {
    static constexpr int H = 1 << LOGH;
    static constexpr int C1 = 2 * H;       // column transform length
    static constexpr int T1 = C1 / 16;     // threads per column
    static constexpr int CP = kC2CB + 1;   // LDS pitch of the column tile
    static constexpr int THREADS = kC2CB * T1;
};

template <int LOGW>
struct C2Row {
    static constexpr int W = 1 << LOGW;
    static constexpr int T2 = W / 16;                     // threads per row
    static constexpr int U0 = 2048 / W;
    static constexpr int UNITS = U0 > 16 ? 16 : U0;       // row pairs per workgroup (an image has H >= 16)
    static constexpr int THREADS = UNITS * 2 * T2;
    static constexpr int RP = W + W / 16;                 // padded LDS row
};

// Pass A: column FFTs of the packed gated image; tile row kh, column m < W/2.
template <int LOGH, class TIO>
__global__ void __launch_bounds__(C2Col<LOGH>::THREADS)
k_c2_colfwd(const TIO* __restrict__ v, const TIO* __restrict__ g, float2* __restrict__ tile,
            const float2* __restrict__ tw1, int W, int64_t row0, int64_t nrows) {
    using C = C2Col<LOGH>;
    constexpr int H = C::H, C1 = C::C1, T1 = C::T1, CB = kC2CB;
    __shared__ float2 lds[C1 * C::CP];
    const int half = W / 2;
    int64_t r;
    int cb;
    if (!xcd_row_map(blockIdx.x, nrows, half / CB, r, cb)) return;
    const int c = threadIdx.x % CB, t = threadIdx.x / CB;
    const int m = cb * CB + c;
    const int64_t img = (row0 + r) * (int64_t)H * W;
    const TIO* vr = v + img;
    const TIO* gr = g ? g + img : nullptr;
    float2 a[16];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int h = t + T1 * e;  // < H
        float2 s = load_pair(vr + (int64_t)h * W, (uint32_t)m);
        if (gr) s = emul(s, load_pair(gr + (int64_t)h * W, (uint32_t)m));
        a[e] = s;
    }
#pragma unroll
    for (int e = 8; e < 16; ++e) a[e] = make_float2(0.f, 0.f);
    fft_strided<C1, false, true>(a, t, tw1, ColAcc<C::CP>{lds + c});
    float2* tr = tile + r * (int64_t)C1 * half;
#pragma unroll
    for (int e = 0; e < 16; ++e) tr[(int64_t)(t + T1 * e) * half + m] = a[e];
}

// Pass C: inverse column FFTs, rows h < H, the gate, y.
template <int LOGH, class TIO>
__global__ void __launch_bounds__(C2Col<LOGH>::THREADS)
k_c2_colinv(const float2* __restrict__ tile, const TIO* __restrict__ x, TIO* __restrict__ y,
            const float2* __restrict__ tw1, int W, int64_t row0, int64_t nrows) {
    using C = C2Col<LOGH>;
    constexpr int H = C::H, C1 = C::C1, T1 = C::T1, CB = kC2CB;
    __shared__ float2 lds[C1 * C::CP];
    const int half = W / 2;
    int64_t r;
    int cb;
    if (!xcd_row_map(blockIdx.x, nrows, half / CB, r, cb)) return;
    const int c = threadIdx.x % CB, t = threadIdx.x / CB;
    const int m = cb * CB + c;
    const float2* tr = tile + r * (int64_t)C1 * half;
    float2 a[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) a[e] = tr[(int64_t)(t + T1 * e) * half + m];
    fft_strided<C1, true, false>(a, t, tw1, ColAcc<C::CP>{lds + c});
    const int64_t img = (row0 + r) * (int64_t)H * W;
    const TIO* xr = x ? x + img : nullptr;
    TIO* yr = y + img;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int h = t + T1 * e;
        float2 o = a[e];
        if (xr) o = emul(o, load_pair(xr + (int64_t)h * W, (uint32_t)m));
        store_pair(yr + (int64_t)h * W, (uint32_t)m, o);
    }
}

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

// Pass B (MODE 0) and spectrum pass 2 (MODE 1). A unit is the row pair
// {p, 2H - p} (p >= 1) or {0, H} (p = 0); a workgroup holds UNITS units.
// MODE 0: tile rows (pitch W/2, columns >= W/2 are 0) -> row FFT -> pair step
//   with the kernel spectrum plus bias -> inverse rows -> columns < W/2 back.
// MODE 1: spec rows (pitch W + 1, all W packed columns) -> row FFT -> the real
//   spectrum's bins 0..W of both rows, scaled, written over the same rows.
template <int LOGW, int MODE>
__global__ void __launch_bounds__(C2Row<LOGW>::THREADS)
k_c2_row(float2* __restrict__ buf, const float2* __restrict__ spec, const float* __restrict__ bias,
         const float2* __restrict__ tw2, const float2* __restrict__ wpair, int logH, int D, int64_t row0,
         int64_t nrows) {
    using R = C2Row<LOGW>;
    constexpr int W = R::W, T2 = R::T2, U = R::UNITS, RP = R::RP, HW = W / 2;
    __shared__ float2 lds[2 * U * RP];
    const int H = 1 << logH, C1 = 2 * H;
    int64_t r;
    int ug;
    if (!xcd_row_map(blockIdx.x, nrows, H / U, r, ug)) return;
    const int tau = threadIdx.x;
    const int rho = tau / T2, t = tau % T2;
    const int p_row = ug * U + rho / 2;
    const int kh = (rho & 1) == 0 ? p_row : (p_row == 0 ? H : C1 - p_row);
    const RowAcc racc{lds + rho * RP};
    // MODE 0 works on the chunk's tile; MODE 1 in place on the spectrum rows
    const int64_t pitch = MODE == 0 ? HW : W + 1;
    float2* img = MODE == 0 ? buf + r * (int64_t)C1 * HW : buf + (row0 + r) * (int64_t)C1 * (W + 1);
    float2* rowp = img + (int64_t)kh * pitch;
    float2 a[16];
    if constexpr (MODE == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = rowp[t + T2 * e];
#pragma unroll
        for (int e = 8; e < 16; ++e) a[e] = make_float2(0.f, 0.f);
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) a[e] = rowp[t + T2 * e];
    }
    fft_strided<W, false, MODE == 0>(a, t, tw2, racc);
    __syncthreads();
    lds_store_strided<T2>(racc, t, a);
    __syncthreads();

    // pair step: 2*T2 threads per unit, W pairs per unit
    const int unit = tau / (2 * T2), tp = tau % (2 * T2);
    const int p = ug * U + unit;
    const RowAcc au[2] = {RowAcc{lds + (2 * unit) * RP}, RowAcc{lds + (2 * unit + 1) * RP}};
    const int64_t flat = row0 + r;
    const int d = (int)(flat % D);
    const float2* S = MODE == 0 ? spec + (int64_t)d * C1 * (W + 1) : nullptr;
    const float nscale = 1.0f / (8.0f * (float)H * (float)W);  // 1 / (4 * 2H * W)
    const float bs = MODE == 0 ? bias[d] * nscale : 0.f;
    const float sc = 0.5f * nscale;  // the unpacked values are twice the spectrum
    auto hs = [&](int row, int bin) { return hadd(S[(int64_t)row * (W + 1) + bin], bs); };
    auto put = [&](int row, int bin, float2 val) { img[(int64_t)row * (W + 1) + bin] = fmul2(val, sc); };
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int j = tp + 2 * T2 * e;  // < W
        if (p > 0) {
            const int kw = j, kw2 = (W - kw) & (W - 1);
            const int ka = p, kb = C1 - p;
            const float2 Za = au[0][kw], Zb = au[1][kw2];
            if constexpr (MODE == 0) {
                float2 Ya, Yb;
                pair_conv(Za, Zb, hs(ka, kw), hs(kb, W - kw), wpair[kw], Ya, Yb);
                au[0][kw] = Ya;
                au[1][kw2] = Yb;
            } else {
                float2 Aa, Ab;
                pair_unpack(Za, Zb, wpair[kw], Aa, Ab);
                put(ka, kw, Aa);
                put(kb, W - kw, Ab);
                if (kw == 0) {  // bins (kb, 0) and (ka, W) by Hermitian symmetry
                    put(kb, 0, make_float2(Aa.x, -Aa.y));
                    put(ka, W, make_float2(Ab.x, -Ab.y));
                }
            }
        } else {
            // unit {0, H}: rows 0 and H each pair with themselves; j < W/2 serves
            // row 0, j >= W/2 row H; j = 0 (W/2) also takes the self-paired bins
            const int sel = j < HW ? 0 : 1;
            const int kr = sel == 0 ? 0 : H;
            const int kw = j & (HW - 1);
            const RowAcc& ro = au[sel];
            if (kw == 0) {
                const float2 Z0 = ro[0], Zh = ro[HW];
                if constexpr (MODE == 0) {
                    float2 Y0, Yx, Yh, Yy;
                    pair_conv(Z0, Z0, hs(kr, 0), hs(kr, W), make_float2(1.f, 0.f), Y0, Yx);
                    pair_conv(Zh, Zh, hs(kr, HW), hs(kr, HW), wpair[HW], Yh, Yy);
                    ro[0] = Y0;
                    ro[HW] = Yh;
                } else {
                    float2 A0, AW, Ah, Ax;
                    pair_unpack(Z0, Z0, make_float2(1.f, 0.f), A0, AW);
                    pair_unpack(Zh, Zh, wpair[HW], Ah, Ax);
                    put(kr, 0, A0);
                    put(kr, W, AW);
                    put(kr, HW, Ah);
                }
            } else {
                const float2 Za = ro[kw], Zb = ro[W - kw];
                if constexpr (MODE == 0) {
                    float2 Ya, Yb;
                    pair_conv(Za, Zb, hs(kr, kw), hs(kr, W - kw), wpair[kw], Ya, Yb);
                    ro[kw] = Ya;
                    ro[W - kw] = Yb;
                } else {
                    float2 Aa, Ab;
                    pair_unpack(Za, Zb, wpair[kw], Aa, Ab);
                    put(kr, kw, Aa);
                    put(kr, W - kw, Ab);
                }
            }
        }
    }
    if constexpr (MODE == 0) {
        __syncthreads();
        lds_load_strided<T2>(racc, t, a);
        fft_strided<W, true, false>(a, t, tw2, racc);
#pragma unroll
        for (int e = 0; e < 8; ++e) rowp[t + T2 * e] = a[e];
    }
}

// ---------------------------------------------------------------- launchers

template <int LOGH>
void launch_cols(bool fwd, bool bf16, const void* v, const void* g, const void* x, float2* tile, void* y,
                 const float2* tw1, int W, int64_t row0, int64_t nrows, hipStream_t st) {
    using C = C2Col<LOGH>;
    const unsigned grid = (unsigned)xcd_grid(nrows, (W / 2) / kC2CB);
    if (fwd) {
        if (bf16)
            hipLaunchKernelGGL((k_c2_colfwd<LOGH, uint16_t>), dim3(grid), dim3(C::THREADS), 0, st,
                               (const uint16_t*)v, (const uint16_t*)g, tile, tw1, W, row0, nrows);
        else
            hipLaunchKernelGGL((k_c2_colfwd<LOGH, float>), dim3(grid), dim3(C::THREADS), 0, st, (const float*)v,
                               (const float*)g, tile, tw1, W, row0, nrows);
    } else {
        if (bf16)
            hipLaunchKernelGGL((k_c2_colinv<LOGH, uint16_t>), dim3(grid), dim3(C::THREADS), 0, st, tile,
                               (const uint16_t*)x, (uint16_t*)y, tw1, W, row0, nrows);
        else
            hipLaunchKernelGGL((k_c2_colinv<LOGH, float>), dim3(grid), dim3(C::THREADS), 0, st, tile,
                               (const float*)x, (float*)y, tw1, W, row0, nrows);
    }
}

template <int LOGH>
void launch_spec_col(const float* k, float2* spec, const float2* tw1, int W, int64_t nrows, hipStream_t st) {
    const unsigned grid = (unsigned)xcd_grid(nrows, W / kC2CB);
    hipLaunchKernelGGL((k_c2_spec_col<LOGH>), dim3(grid), dim3(C2Col<LOGH>::THREADS), 0, st, k, spec, tw1, W,
                       nrows);
}

template <int LOGW>
void launch_rows(int mode, float2* buf, const float2* spec, const float* bias, const float2* tw2,
                 const float2* wpair, int logH, int D, int64_t row0, int64_t nrows, hipStream_t st) {
    using R = C2Row<LOGW>;
    const unsigned grid = (unsigned)xcd_grid(nrows, (1 << logH) / R::UNITS);
    if (mode == 0)
        hipLaunchKernelGGL((k_c2_row<LOGW, 0>), dim3(grid), dim3(R::THREADS), 0, st, buf, spec, bias, tw2, wpair,
                           logH, D, row0, nrows);
    else
        hipLaunchKernelGGL((k_c2_row<LOGW, 1>), dim3(grid), dim3(R::THREADS), 0, st, buf, spec, bias, tw2, wpair,
                           logH, D, row0, nrows);
}

hipError_t cols(int logH, bool fwd, bool bf16, const void* v, const void* g, const void* x, float2* tile, void* y,
                const float2* tw1, int W, int64_t row0, int64_t nrows, hipStream_t st) {
    switch (logH) {
        case 4: launch_cols<4>(fwd, bf16, v, g, x, tile, y, tw1, W, row0, nrows, st); break;
        case 5: launch_cols<5>(fwd, bf16, v, g, x, tile, y, tw1, W, row0, nrows, st); break;
        case 6: launch_cols<6>(fwd, bf16, v, g, x, tile, y, tw1, W, row0, nrows, st); break;
        case 7: launch_cols<7>(fwd, bf16, v, g, x, tile, y, tw1, W, row0, nrows, st); break;
        case 8: launch_cols<8>(fwd, bf16, v, g, x, tile, y, tw1, W, row0, nrows, st); break;
        case 9: launch_cols<9>(fwd, bf16, v, g, x, tile, y, tw1, W, row0, nrows, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
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

hipError_t rows(int logW, int mode, float2* buf, const float2* spec, const float* bias, const float2* tw2,
                const float2* wpair, int logH, int D, int64_t row0, int64_t nrows, hipStream_t st) {
    switch (logW) {
        case 5: launch_rows<5>(mode, buf, spec, bias, tw2, wpair, logH, D, row0, nrows, st); break;
        case 6: launch_rows<6>(mode, buf, spec, bias, tw2, wpair, logH, D, row0, nrows, st); break;
        case 7: launch_rows<7>(mode, buf, spec, bias, tw2, wpair, logH, D, row0, nrows, st); break;
        case 8: launch_rows<8>(mode, buf, spec, bias, tw2, wpair, logH, D, row0, nrows, st); break;
        case 9: launch_rows<9>(mode, buf, spec, bias, tw2, wpair, logH, D, row0, nrows, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int64_t x) {
    int l = 0;
    while ((int64_t(1) << l) < x) ++l;
    return l;
}

hyena_status_t check2d(const hyena_plan2d_t plan) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return HYENA_ERR_DEVICE;
    return dev == plan->device ? HYENA_OK : HYENA_ERR_DEVICE;
}

}  // namespace
}  // namespace hy

extern "C" {

hyena_status_t hyena_plan2d_create(hyena_plan2d_t* out, int64_t H, int64_t W, int64_t D, hyena_dtype_t dtype) {
    if (!out) return HYENA_ERR_INVALID_ARG;
    if (H < 1 || W < 1 || D < 1) return HYENA_ERR_INVALID_ARG;
    if (dtype != HYENA_F32 && dtype != HYENA_BF16) return HYENA_ERR_INVALID_ARG;
    if (!hy::pow2(H) || !hy::pow2(W) || D > (int64_t(1) << 24)) return HYENA_ERR_UNSUPPORTED;
    const int logH = hy::log2i(H), logW = hy::log2i(W);
    if (logH < hy::kC2MinLogH || logH > hy::kC2MaxLogH || logW < hy::kC2MinLogW || logW > hy::kC2MaxLogW)
        return HYENA_ERR_UNSUPPORTED;
    std::vector<float2> tab;
    hy::append_stockham(tab, logH + 1);
    const size_t o_tw2 = tab.size();
    hy::append_stockham(tab, logW);
    const size_t o_wp = tab.size();
    for (int64_t k = 0; k < W; ++k) tab.push_back(hy::wfwd(k, 2 * W));
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
    plan->dtype = dtype;
    plan->device = dev;
    plan->dtab = dtab;
    plan->tw1 = dtab;
    plan->tw2 = dtab + o_tw2;
    plan->wpair = dtab + o_wp;
    *out = plan;
    return HYENA_OK;
}

hyena_status_t hyena_plan2d_destroy(hyena_plan2d_t plan) {
    if (!plan) return HYENA_OK;
    const hyena_status_t st = (plan->dtab && hipFree(plan->dtab) != hipSuccess) ? HYENA_ERR_DEVICE : HYENA_OK;
    delete plan;
    return st;
}

size_t hyena_spectrum2d_bytes(hyena_plan2d_t plan) {
    if (!plan) return 0;
    return (size_t)plan->D * (size_t)(2 * plan->H) * (size_t)(plan->W + 1) * sizeof(float2);
}

size_t hyena_workspace2d_bytes(hyena_plan2d_t plan, int64_t B) {
    if (!plan || B < 1) return 0;
    const size_t per = (size_t)plan->H * (size_t)plan->W * sizeof(float2);  // 2H x W/2 complex
    int64_t want = (int64_t)(hy::kC2ChunkBytes / per);
    if (want < 1) want = 1;
    if (want > B * plan->D) want = B * plan->D;
    return (size_t)want * per;
}

hyena_status_t hyena_filter_spectrum2d(hyena_plan2d_t plan, const float* k, void* spec, hipStream_t stream) {
    using hy::aligned16;
    if (!plan || !k || !spec || !aligned16(k) || !aligned16(spec)) return HYENA_ERR_INVALID_ARG;
    if (hy::check2d(plan) != HYENA_OK) return HYENA_ERR_DEVICE;
    const int W = (int)plan->W;
    float2* sp = (float2*)spec;
    hipError_t e = hy::spec_cols(plan->logH, k, sp, plan->tw1, W, plan->D, stream);
    if (e == hipSuccess)
        e = hy::rows(plan->logW, 1, sp, nullptr, nullptr, plan->tw2, plan->wpair, plan->logH, (int)plan->D, 0,
                     plan->D, stream);
    return e == hipSuccess ? HYENA_OK : HYENA_ERR_DEVICE;
}

hyena_status_t hyena_conv2d_forward(hyena_plan2d_t plan, int64_t B, const void* v, const void* g, const void* x,
                                    const void* spec, const float* bias, void* y, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    using hy::aligned16;
    if (!plan || B < 1 || !v || !spec || !bias || !y) return HYENA_ERR_INVALID_ARG;
    if (!aligned16(v) || !aligned16(spec) || !aligned16(bias) || !aligned16(y) || (g && !aligned16(g)) ||
        (x && !aligned16(x)))
        return HYENA_ERR_INVALID_ARG;
    if (B > (int64_t(1) << 24) || B * plan->D > (int64_t(1) << 24)) return HYENA_ERR_INVALID_ARG;
    const size_t per = (size_t)plan->H * (size_t)plan->W * sizeof(float2);
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
        hipError_t e = hy::cols(plan->logH, true, bf16, v, g, nullptr, tile, nullptr, plan->tw1, W, r0, n, stream);
        if (e == hipSuccess)
            e = hy::rows(plan->logW, 0, tile, (const float2*)spec, bias, plan->tw2, plan->wpair, plan->logH,
                         (int)plan->D, r0, n, stream);
        if (e == hipSuccess)
            e = hy::cols(plan->logH, false, bf16, nullptr, nullptr, x, tile, y, plan->tw1, W, r0, n, stream);
        if (e != hipSuccess) return HYENA_ERR_DEVICE;
    }
    return HYENA_OK;
}

}  // extern "C"
