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

// Slab pass (plans whose height x row slab pair fits in LDS): the height
// transforms, the row pass and the inverse height transforms of one pair of depth
// slices in one launch, on chip. Workgroup j of a volume takes slices {j, 2A - j}
// (j = 0: the two self-paired slices 0 and A; A here is half the depth transform):
// their tile-1 values go through column FFTs over h (length Th) into an LDS array of
// 2 Th padded rows, then row FFTs over m (length W), the pair step with the kernel
// spectrum plus the bias exactly as in the row pass (row (ka, kh) with (-ka, -kh),
// bin kw with -kw), inverse rows and inverse columns back into tile 1. The same
// transforms as passes A2, B and C2, without tile 2. Zero-padded plans: tile-1 rows
// h < Th/2 and columns m < W/2 hold data, the first radix passes are pruned and
// only those outputs are kept. CIRC (circular plans): every row and column holds
// data, nothing is pruned, everything is kept.
template <int LOGTH, int LOGW, bool CIRC>
struct C3Slab {
    static constexpr int Th = 1 << LOGTH, W = 1 << LOGW, HP = Th / 2, WH = W / 2;
    static constexpr int HR = CIRC ? Th : HP, NC = CIRC ? W : WH;  // tile-1 rows and columns per slice
    static constexpr int LD = CIRC ? 16 : 8;                       // values per thread holding data
    static constexpr int T1 = Th / 16, T2 = W / 16;                // threads per column / row transform
    static constexpr int NT = 2 * NC * T1;                         // the column transforms of both slices
    static constexpr int IT = 2 * Th * T2 / NT;                    // row (and pair-unit) batches
    static constexpr int RP = W + W / 16;                          // padded LDS row
    static constexpr bool OK = Th * W <= 4096 && T1 >= 1 && NT >= 64 && NT % 64 == 0 && IT * NT == 2 * Th * T2;
};

template <int LOGTH, int LOGW, bool CIRC>
__global__ void __launch_bounds__((C3Slab<LOGTH, LOGW, CIRC>::NT))
k_c3_slab(float2* __restrict__ t1, const float2* __restrict__ spec, const float* __restrict__ bias,
          const float2* __restrict__ twh, const float2* __restrict__ tww, const float2* __restrict__ wpair, int A,
          int D, int64_t row0, int64_t nrows, bool per_sample) {
    using S = C3Slab<LOGTH, LOGW, CIRC>;
    constexpr int Th = S::Th, W = S::W, HP = S::HP, WH = S::WH, HR = S::HR, NC = S::NC, LD = S::LD;
    constexpr int T1 = S::T1, T2 = S::T2, NT = S::NT, IT = S::IT, RP = S::RP;
    static_assert(S::OK, "slab pair must fit the workgroup");
    __shared__ float2 lds[2 * Th * RP];
    int64_t r;
    int j;
    if (!xcd_row_map(blockIdx.x, nrows, A, r, j)) return;
    const int tid = threadIdx.x;
    const int ka0 = j == 0 ? 0 : j, ka1 = j == 0 ? A : 2 * A - j;  // the two slices
    const int64_t slice = (int64_t)HR * NC;
    float2* vol = t1 + r * (int64_t)(2 * A) * slice;
    auto lds_at = [&](int row, int m) -> float2& { return lds[row * RP + m + m / 16]; };

    // columns over h: thread (s, t, c), c fastest so that global rows are coalesced
    const int cs = tid / (NC * T1), cc = tid % NC, ct = (tid / NC) % T1;
    const int cka = cs == 0 ? ka0 : ka1;
    const ColAcc<RP> cacc{lds + cs * Th * RP + cc + cc / 16};
    {
        float2 a[16];
        const float2* src = vol + cka * slice + cc;
#pragma unroll
        for (int e = 0; e < LD; ++e) a[e] = src[(int64_t)(ct + T1 * e) * NC];
#pragma unroll
        for (int e = LD; e < 16; ++e) a[e] = make_float2(0.f, 0.f);
        fft_strided<Th, false, !CIRC>(a, ct, twh, cacc);
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 16; ++e) lds_at(cs * Th + ct + T1 * e, cc) = a[e];
    }
    // the pair step's units (Th units of two rows, 2 T2 threads each, IT batches)
    // and their spectrum values, fetched now so that the row transforms hide them
    const int64_t flat = row0 + r;
    const int d = (int)(flat % D);
    const int NR = 2 * A * Th;  // rows of the spectrum, (ka, kh) flattened as ka * Th + kh
    const float2* Sp = spec + (per_sample ? flat : (int64_t)d) * NR * (W + 1);
    struct Unit {
        int la, lb, ga, gb;  // LDS rows and spectrum rows
        bool self;
    };
    auto unit_of = [&](int it) {
        const int u = it * (NT / (2 * T2)) + tid / (2 * T2);
        Unit q;
        if (j != 0) {
            const int kh2 = (Th - u) & (Th - 1);
            q.la = u;
            q.lb = Th + kh2;
            q.ga = ka0 * Th + u;
            q.gb = ka1 * Th + kh2;
            q.self = false;
        } else {
            const int sl = u / HP, p = u % HP;  // slice ka0 = 0 (sl 0) or ka1 = A (sl 1)
            const int ka = sl == 0 ? ka0 : ka1;
            const int kb = p == 0 ? HP : Th - p;
            q.la = sl * Th + p;
            q.lb = sl * Th + kb;
            q.ga = ka * Th + p;
            q.gb = ka * Th + kb;
            q.self = p == 0;
        }
        return q;
    };
    const int tp = tid % (2 * T2);
    // per pair slot: the spectrum values at (row a, kw) and (row b, W - kw); for the
    // self-paired rows (row of jj, kw) and (same row, W - kw), kw = 0 taking bins 0 and W
    float2 sa[IT][8], sb[IT][8];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const Unit q = unit_of(it);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int jj = tp + 2 * T2 * e;
            int rowa = q.ga, rowb = q.gb, bina = jj, binb = W - jj;
            if (q.self) {
                const int kw = jj & (WH - 1);
                rowa = rowb = jj < WH ? q.ga : q.gb;
                bina = kw;
                binb = W - kw;
            }
            sa[it][e] = Sp[(int64_t)rowa * (W + 1) + bina];
            sb[it][e] = Sp[(int64_t)rowb * (W + 1) + binb];
        }
    }
    // rows over m, IT batches of the 2 Th rows
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int R = it * (NT / T2) + tid / T2, t = tid % T2;
        const RowAcc racc{lds + R * RP};
        float2 a[16];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < LD; ++e) a[e] = racc[t + T2 * e];
#pragma unroll
        for (int e = LD; e < 16; ++e) a[e] = make_float2(0.f, 0.f);
        fft_strided<W, false, !CIRC>(a, t, tww, racc);
        __syncthreads();
        lds_store_strided<T2>(racc, t, a);
    }
    __syncthreads();
    // pair step
    const float nscale = 1.0f / (4.0f * (float)NR * (float)W);
    const float bs = bias[d] * nscale;
    auto hs = [&](int row, int bin) { return hadd(Sp[(int64_t)row * (W + 1) + bin], bs); };
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const Unit q = unit_of(it);
        const RowAcc au0{lds + q.la * RP}, au1{lds + q.lb * RP};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int jj = tp + 2 * T2 * e;  // < W
            const float2 ha = hadd(sa[it][e], bs), hb = hadd(sb[it][e], bs);
            if (!q.self) {
                const int kw = jj, kw2 = (W - kw) & (W - 1);
                float2 Ya, Yb;
                pair_conv(au0[kw], au1[kw2], ha, hb, wpair[kw], Ya, Yb);
                au0[kw] = Ya;
                au1[kw2] = Yb;
            } else {
                // two self-paired rows: jj < W/2 serves row la, jj >= W/2 row lb;
                // kw = 0 also takes the self-paired bins 0, W/2 and W of its row
                const int sel = jj < WH ? 0 : 1;
                const int gr = sel == 0 ? q.ga : q.gb;
                const RowAcc ro = sel == 0 ? au0 : au1;
                const int kw = jj & (WH - 1);
                if (kw == 0) {
                    const float2 Z0 = ro[0], Zh = ro[WH];
                    const float2 Hh = hs(gr, WH);
                    float2 Y0, Yx, Yh, Yy;
                    pair_conv(Z0, Z0, ha, hb, make_float2(1.f, 0.f), Y0, Yx);  // bins 0 and W
                    pair_conv(Zh, Zh, Hh, Hh, wpair[WH], Yh, Yy);
                    ro[0] = Y0;
                    ro[WH] = Yh;
                } else {
                    float2 Ya, Yb;
                    pair_conv(ro[kw], ro[W - kw], ha, hb, wpair[kw], Ya, Yb);
                    ro[kw] = Ya;
                    ro[W - kw] = Yb;
                }
            }
        }
    }
    // inverse rows (zero-padded: columns m < W/2 kept)
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int R = it * (NT / T2) + tid / T2, t = tid % T2;
        const RowAcc racc{lds + R * RP};
        float2 a[16];
        __syncthreads();
        lds_load_strided<T2>(racc, t, a);
        fft_strided<W, true, false>(a, t, tww, racc);
        __syncthreads();
#pragma unroll
        for (int e = 0; e < LD; ++e) racc[t + T2 * e] = a[e];
    }
    __syncthreads();
    // inverse columns over kh (zero-padded: rows h < Th/2 kept), back to tile 1
    {
        float2 a[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) a[e] = lds_at(cs * Th + ct + T1 * e, cc);
        fft_strided<Th, true, false>(a, ct, twh, cacc);
        float2* dst = vol + cka * slice + cc;
#pragma unroll
        for (int e = 0; e < LD; ++e) dst[(int64_t)(ct + T1 * e) * NC] = a[e];
    }
}

template <int LOGTH, int LOGW, bool CIRC>
hipError_t launch_slab_t(float2* t1, const float2* spec, const float* bias, const float2* twh, const float2* tww,
                         const float2* wpair, int A, int D, int64_t row0, int64_t n, bool per_sample,
                         hipStream_t st) {
    using S = C3Slab<LOGTH, LOGW, CIRC>;
    if constexpr (!S::OK) {
        return hipErrorInvalidValue;
    } else {
        hipLaunchKernelGGL((k_c3_slab<LOGTH, LOGW, CIRC>), dim3((unsigned)xcd_grid(n, A)), dim3(S::NT), 0, st, t1,
                           spec, bias, twh, tww, wpair, A, D, row0, n, per_sample);
        return hipGetLastError();
    }
}

// Whether a plan with height transforms of 2^lh and row transforms of 2^lr packed
// points takes the slab pass (the slice pair fits one workgroup's LDS).
bool slab_ok(int lh, int lr) {
    const int sum = lh + lr;
    return lh >= 5 && lr >= 5 && sum >= 10 && sum <= 12;
}

hipError_t slab(int lh, int lr, bool circ, float2* t1, const float2* spec, const float* bias, const float2* twh,
                const float2* tww, const float2* wpair, int A, int D, int64_t row0, int64_t n, bool per_sample,
                hipStream_t st) {
#define C3_SLAB(a, b)                                                                                              \
    if (lh == a && lr == b)                                                                                        \
        return circ ? launch_slab_t<a, b, true>(t1, spec, bias, twh, tww, wpair, A, D, row0, n, per_sample, st)   \
                    : launch_slab_t<a, b, false>(t1, spec, bias, twh, tww, wpair, A, D, row0, n, per_sample, st);
    C3_SLAB(5, 5) C3_SLAB(5, 6) C3_SLAB(5, 7) C3_SLAB(6, 5) C3_SLAB(6, 6) C3_SLAB(7, 5)
#undef C3_SLAB
    return hipErrorInvalidValue;
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
#ifndef HY_C3_SLAB
#define HY_C3_SLAB 1
#endif
// Whether the plan's forward takes the slab pass (then only tile 1 is used).
bool uses_slab(const hyena_plan3d_t p) { return HY_C3_SLAB && slab_ok(p->lh, p->lr); }
size_t vol_ws_bytes(const hyena_plan3d_t p) {
    return (tile1_elems(p) + (p->circular || uses_slab(p) ? 0 : tile2_elems(p))) * sizeof(float2);
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
    const bool use_slab = hy::uses_slab(plan);
    for (int64_t r0 = 0; r0 < nv; r0 += chunk) {
        const int64_t n = nv - r0 < chunk ? nv - r0 : chunk;
        hipError_t e =
            hy::cols(plan->la, true, bf16, v, g, nullptr, t1, nullptr, plan->twa, plane, r0, n, stream, circ);
        if (e == hipSuccess && use_slab) {
            e = hy::slab(plan->lh, plan->lr, circ, t1, (const float2*)spec, bias, plan->twh, plan->tww, plan->wpair,
                         plan->pa, (int)plan->D, r0, n, per_sample, stream);
        } else {
            if (e == hipSuccess)
                e = hy::ccol(plan->lh, circ ? hy::kColFwdFull : hy::kColFwdPruned, t1, t2, plan->twh, n * Ta,
                             (int)W2, H * W2, W2, (int)W2, (int)W2, Th * W2, W2, (int)W2, (int)W2, stream);
            if (e == hipSuccess)
                e = hy::rows(plan->lr, 0, t2, (const float2*)spec, bias, plan->tww, plan->wpair, pm,
                             2 * plan->pa * plan->ph, (int)plan->D, r0, n, per_sample, stream, circ);
            if (e == hipSuccess)
                e = hy::ccol(plan->lh, circ ? hy::kColInvFull : hy::kColInvHalf, t2, t1, plan->twh, n * Ta,
                             (int)W2, Th * W2, W2, (int)W2, (int)W2, H * W2, W2, (int)W2, (int)W2, stream);
        }
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
