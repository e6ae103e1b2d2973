// Device code shared by the gated 2-D and 3-D long convolutions (conv2d.hip,
// conv3d.hip; HyenaND summary, methodology: global convolution on the native
// N-d grid by an N-d FFT, the input zero-padded to double the grid in every
// dimension). The real transform of the doubled grid is carried as a complex
// transform of the data packed along the last (contiguous) axis w:
// z[..][m] = s[..][2m] + i s[..][2m+1], W complex columns of which the first
// W/2 hold data. Every axis before w is transformed by column passes over a
// tile whose rows are the other axes' indices; the w axis by the row pass,
// which also carries the pair step: bin (k_1, .., k_w) of the real spectrum
// pairs with (-k_1, .., -k_w), so a row pairs with the row of the negated
// indices (the map types below), and the twiddle is W_{2W}^kw as in 1-D.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fft_core.hpp"
#include "fourstep.hpp"
#include "pair.hpp"

namespace hy {
namespace {

constexpr int kC2CB = 16;  // columns per column-pass workgroup

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
    static constexpr int UNITS = U0 > 16 ? 16 : U0;       // row pairs per workgroup (an image has >= 16)
    static constexpr int THREADS = UNITS * 2 * T2;
    static constexpr int RP = W + W / 16;                 // padded LDS row
};

// First column pass of an image of H rows of W real samples: column FFTs (length
// 2H, first radix pass pruned) of the packed gated image; tile row kh, column
// m < W/2. (3-D: H is the depth axis and W the flattened H x W plane.)
// CIRC (circular mode): the image has 2H rows, all transformed (no padding).
template <int LOGH, class TIO, bool CIRC = false>
__global__ void __launch_bounds__(C2Col<LOGH>::THREADS)
k_c2_colfwd(const TIO* __restrict__ v, const TIO* __restrict__ g, float2* __restrict__ tile,
            const float2* __restrict__ tw1, int W, int64_t row0, int64_t nrows) {
    using C = C2Col<LOGH>;
    constexpr int C1 = C::C1, T1 = C::T1, CB = kC2CB;
    constexpr int H = CIRC ? C1 : C::H;  // image rows
    constexpr int LD = CIRC ? 16 : 8;    // values per thread holding data
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
    for (int e = 0; e < LD; ++e) {
        const int h = t + T1 * e;  // < H
        float2 s = load_pair(vr + (int64_t)h * W, (uint32_t)m);
        if (gr) s = emul(s, load_pair(gr + (int64_t)h * W, (uint32_t)m));
        a[e] = s;
    }
#pragma unroll
    for (int e = LD; e < 16; ++e) a[e] = make_float2(0.f, 0.f);
    fft_strided<C1, false, !CIRC>(a, t, tw1, ColAcc<C::CP>{lds + c});
    float2* tr = tile + r * (int64_t)C1 * half;
#pragma unroll
    for (int e = 0; e < 16; ++e) tr[(int64_t)(t + T1 * e) * half + m] = a[e];
}

// Last column pass: inverse column FFTs, rows h < H, the gate, y.
// CIRC: the image has 2H rows, all kept.
template <int LOGH, class TIO, bool CIRC = false>
__global__ void __launch_bounds__(C2Col<LOGH>::THREADS)
k_c2_colinv(const float2* __restrict__ tile, const TIO* __restrict__ x, TIO* __restrict__ y,
            const float2* __restrict__ tw1, int W, int64_t row0, int64_t nrows) {
    using C = C2Col<LOGH>;
    constexpr int C1 = C::C1, T1 = C::T1, CB = kC2CB;
    constexpr int H = CIRC ? C1 : C::H;
    constexpr int LD = CIRC ? 16 : 8;
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
    for (int e = 0; e < LD; ++e) {
        const int h = t + T1 * e;
        float2 o = a[e];
        if (xr) o = emul(o, load_pair(xr + (int64_t)h * W, (uint32_t)m));
        store_pair(yr + (int64_t)h * W, (uint32_t)m, o);
    }
}

// Column FFTs of complex slabs: slab s holds rows of pitch *_pitch; column c of
// the pass sits at (c / cw) * cp + c % cw inside a row (cw = cp: plain columns;
// a wrap lets the columns of a flattened 2-D plane land in rows of another
// pitch). PRUNE: input rows >= N/2 are zero and not read. HALF_OUT: only output
// rows < N/2 are written (the kept half of an inverse). In and out may be the
// same buffer: a workgroup reads all of its columns before writing them.
template <int LOGN, bool INV, bool PRUNE, bool HALF_OUT>
__global__ void __launch_bounds__(kC2CB * (1 << LOGN) / 16)
k_cnd_col(const float2* in, float2* out, const float2* __restrict__ tw, int64_t nslabs, int ncols,
          int64_t in_slab, int64_t in_pitch, int in_cw, int in_cp, int64_t out_slab, int64_t out_pitch, int out_cw,
          int out_cp) {
    constexpr int N = 1 << LOGN, T1 = N / 16, CB = kC2CB, CP = CB + 1;
    __shared__ float2 lds[N * CP];
    int64_t s;
    int cb;
    if (!xcd_row_map(blockIdx.x, nslabs, ncols / CB, s, cb)) return;
    const int c = threadIdx.x % CB, t = threadIdx.x / CB;
    const int col = cb * CB + c;
    const float2* ip = in + s * in_slab + (int64_t)(col / in_cw) * in_cp + col % in_cw;
    float2* op = out + s * out_slab + (int64_t)(col / out_cw) * out_cp + col % out_cw;
    float2 a[16];
#pragma unroll
    for (int e = 0; e < (PRUNE ? 8 : 16); ++e) a[e] = ip[(int64_t)(t + T1 * e) * in_pitch];
#pragma unroll
    for (int e = PRUNE ? 8 : 16; e < 16; ++e) a[e] = make_float2(0.f, 0.f);
    fft_strided<N, INV, PRUNE>(a, t, tw, ColAcc<CP>{lds + c});
#pragma unroll
    for (int e = 0; e < (HALF_OUT ? 8 : 16); ++e) op[(int64_t)(t + T1 * e) * out_pitch] = a[e];
}

// Row pairing of the doubled 2-D grid: row kh pairs with 2H - kh; rows 0 and H
// pair with themselves and form one unit.
struct PairMap2 {
    int H;
    __device__ int rows() const { return 2 * H; }
    __device__ int units() const { return H; }
    __device__ void unit(int u, int& ra, int& rb, bool& self) const {
        self = u == 0;
        ra = u;
        rb = u == 0 ? H : 2 * H - u;
    }
};

// Row pairing of the doubled 3-D grid, rows (ka, kh) flattened as ka * 2H + kh:
// (ka, kh) pairs with (-ka mod 2A, -kh mod 2H). Units 0 .. 2H-1 are the depth
// slices ka = 0 and ka = A, which pair with themselves (the 2-D pairing inside
// the slice); the rest pair slice ka in [1, A) with slice 2A - ka.
struct PairMap3 {
    int A, H;
    __device__ int rows() const { return 4 * A * H; }
    __device__ int units() const { return 2 * A * H; }
    __device__ void unit(int u, int& ra, int& rb, bool& self) const {
        const int H2 = 2 * H;
        if (u < H2) {
            const int base = u < H ? 0 : A * H2;
            const int p = u < H ? u : u - H;
            self = p == 0;
            ra = base + p;
            rb = base + (p == 0 ? H : H2 - p);
        } else {
            const int v = u - H2;
            const int ka = v / H2 + 1, kh = v & (H2 - 1);
            self = false;
            ra = ka * H2 + kh;
            rb = (2 * A - ka) * H2 + ((H2 - kh) & (H2 - 1));
        }
    }
};

// Row pass (MODE 0) and last spectrum pass (MODE 1). A workgroup holds UNITS
// row pairs of one image (MODE 0) or one channel's spectrum (MODE 1).
// MODE 0: tile rows (pitch W/2, columns >= W/2 are 0) -> row FFT -> pair step
//   with the kernel spectrum plus bias -> inverse rows -> columns < W/2 back.
// MODE 1: spectrum rows (pitch W + 1, all W packed columns) -> row FFT -> the
//   real spectrum's bins 0..W of both rows, scaled, written over the same rows.
// The stored spectrum is scaled by 1/(4 * rows * W), rows * W being the complex
// transform's size, so that the pair step also applies the inverse normalisation.
// per_sample (MODE 0): image b*D + d reads spectrum b*D + d (a kernel set per
// sample) instead of spectrum d.
// CIRC (circular mode, MODE 0): the tile rows hold all W packed columns; the
// row transform is not pruned and every column is kept.
template <int LOGW, int MODE, class MAP, bool CIRC = false>
__global__ void __launch_bounds__(C2Row<LOGW>::THREADS)
k_cnd_row(float2* __restrict__ buf, const float2* __restrict__ spec, const float* __restrict__ bias,
          const float2* __restrict__ tw2, const float2* __restrict__ wpair, MAP map, int D, int64_t row0,
          int64_t nrows, bool per_sample) {
    using R = C2Row<LOGW>;
    constexpr int W = R::W, T2 = R::T2, U = R::UNITS, RP = R::RP, HW = W / 2;
    constexpr int TP = CIRC ? W : HW;  // tile pitch (MODE 0)
    constexpr int LD = CIRC ? 16 : 8;  // values per thread holding data (MODE 0)
    __shared__ float2 lds[2 * U * RP];
    const int NR = map.rows();
    int64_t r;
    int ug;
    if (!xcd_row_map(blockIdx.x, nrows, map.units() / U, r, ug)) return;
    const int tau = threadIdx.x;
    const int rho = tau / T2, t = tau % T2;
    int my_a, my_b;
    bool my_self;
    map.unit(ug * U + rho / 2, my_a, my_b, my_self);
    const int kh = (rho & 1) == 0 ? my_a : my_b;
    const RowAcc racc{lds + rho * RP};
    // MODE 0 works on the chunk's tile; MODE 1 in place on the spectrum rows
    const int64_t pitch = MODE == 0 ? TP : W + 1;
    float2* img = MODE == 0 ? buf + r * (int64_t)NR * TP : buf + (row0 + r) * (int64_t)NR * (W + 1);
    float2* rowp = img + (int64_t)kh * pitch;
    float2 a[16];
    if constexpr (MODE == 0) {
#pragma unroll
        for (int e = 0; e < LD; ++e) a[e] = rowp[t + T2 * e];
#pragma unroll
        for (int e = LD; e < 16; ++e) a[e] = make_float2(0.f, 0.f);
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) a[e] = rowp[t + T2 * e];
    }
    // pair-step role: 2*T2 threads per unit, W pairs per unit
    const int unit = tau / (2 * T2), tp = tau % (2 * T2);
    int ka, kb;
    bool self;
    map.unit(ug * U + unit, ka, kb, self);
    const int64_t flat = row0 + r;
    const int d = (int)(flat % D);
    const float2* S = MODE == 0 ? spec + (per_sample ? flat : (int64_t)d) * NR * (W + 1) : nullptr;
    // MODE 0: the spectrum values of this thread's pair slots, fetched before the
    // row transform so that it hides their latency: (row a, kw) and (row b, W - kw);
    // for self-paired rows (the slot's row, kw) and (same row, W - kw), kw = 0
    // taking bins 0 and W
    [[maybe_unused]] float2 sa[8], sb[8];
    if constexpr (MODE == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = tp + 2 * T2 * e;
            int rowa = ka, rowb = kb, bina = j, binb = W - j;
            if (self) {
                rowa = rowb = j < HW ? ka : kb;
                bina = j & (HW - 1);
                binb = W - bina;
            }
            sa[e] = S[(int64_t)rowa * (W + 1) + bina];
            sb[e] = S[(int64_t)rowb * (W + 1) + binb];
        }
    }
    fft_strided<W, false, MODE == 0 && !CIRC>(a, t, tw2, racc);
    __syncthreads();
    lds_store_strided<T2>(racc, t, a);
    __syncthreads();

    const RowAcc au[2] = {RowAcc{lds + (2 * unit) * RP}, RowAcc{lds + (2 * unit + 1) * RP}};
    const float nscale = 1.0f / (4.0f * (float)NR * (float)W);
    const float bs = MODE == 0 ? bias[d] * nscale : 0.f;
    const float sc = 0.5f * nscale;  // the unpacked values are twice the spectrum
    auto hs = [&](int row, int bin) { return hadd(S[(int64_t)row * (W + 1) + bin], bs); };
    auto put = [&](int row, int bin, float2 val) { img[(int64_t)row * (W + 1) + bin] = fmul2(val, sc); };
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int j = tp + 2 * T2 * e;  // < W
        if (!self) {
            const int kw = j, kw2 = (W - kw) & (W - 1);
            const float2 Za = au[0][kw], Zb = au[1][kw2];
            if constexpr (MODE == 0) {
                float2 Ya, Yb;
                pair_conv(Za, Zb, hadd(sa[e], bs), hadd(sb[e], bs), wpair[kw], Ya, Yb);
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
            // two self-paired rows: j < W/2 serves row ka, j >= W/2 row kb;
            // kw = 0 also takes the self-paired bins 0, W/2 and W of its row
            const int sel = j < HW ? 0 : 1;
            const int kr = sel == 0 ? ka : kb;
            const int kw = j & (HW - 1);
            const RowAcc& ro = au[sel];
            if (kw == 0) {
                const float2 Z0 = ro[0], Zh = ro[HW];
                if constexpr (MODE == 0) {
                    float2 Y0, Yx, Yh, Yy;
                    pair_conv(Z0, Z0, hadd(sa[e], bs), hadd(sb[e], bs), make_float2(1.f, 0.f), Y0, Yx);
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
                    pair_conv(Za, Zb, hadd(sa[e], bs), hadd(sb[e], bs), wpair[kw], Ya, Yb);
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
        for (int e = 0; e < LD; ++e) rowp[t + T2 * e] = a[e];
    }
}

// ------------------------------------------------------------- launch helpers

template <int LOGH, bool CIRC>
void launch_cols_c(bool fwd, bool bf16, const void* v, const void* g, const void* x, float2* tile, void* y,
                   const float2* tw1, int W, int64_t row0, int64_t nrows, hipStream_t st) {
    using C = C2Col<LOGH>;
    const unsigned grid = (unsigned)xcd_grid(nrows, (W / 2) / kC2CB);
    if (fwd) {
        if (bf16)
            hipLaunchKernelGGL((k_c2_colfwd<LOGH, uint16_t, CIRC>), dim3(grid), dim3(C::THREADS), 0, st,
                               (const uint16_t*)v, (const uint16_t*)g, tile, tw1, W, row0, nrows);
        else
            hipLaunchKernelGGL((k_c2_colfwd<LOGH, float, CIRC>), dim3(grid), dim3(C::THREADS), 0, st,
                               (const float*)v, (const float*)g, tile, tw1, W, row0, nrows);
    } else {
        if (bf16)
            hipLaunchKernelGGL((k_c2_colinv<LOGH, uint16_t, CIRC>), dim3(grid), dim3(C::THREADS), 0, st, tile,
                               (const uint16_t*)x, (uint16_t*)y, tw1, W, row0, nrows);
        else
            hipLaunchKernelGGL((k_c2_colinv<LOGH, float, CIRC>), dim3(grid), dim3(C::THREADS), 0, st, tile,
                               (const float*)x, (float*)y, tw1, W, row0, nrows);
    }
}

template <int LOGH>
void launch_cols(bool fwd, bool bf16, const void* v, const void* g, const void* x, float2* tile, void* y,
                 const float2* tw1, int W, int64_t row0, int64_t nrows, bool circ, hipStream_t st) {
    if (circ) launch_cols_c<LOGH, true>(fwd, bf16, v, g, x, tile, y, tw1, W, row0, nrows, st);
    else launch_cols_c<LOGH, false>(fwd, bf16, v, g, x, tile, y, tw1, W, row0, nrows, st);
}

// First (fwd) or last (!fwd) column pass with transforms of length 2^(logH+1):
// over images of 2^logH rows (zero-padded) or 2^(logH+1) rows (circ) of W samples.
inline hipError_t cols(int logH, bool fwd, bool bf16, const void* v, const void* g, const void* x, float2* tile,
                       void* y, const float2* tw1, int W, int64_t row0, int64_t nrows, hipStream_t st,
                       bool circ = false) {
    switch (logH) {
        case 4: launch_cols<4>(fwd, bf16, v, g, x, tile, y, tw1, W, row0, nrows, circ, st); break;
        case 5: launch_cols<5>(fwd, bf16, v, g, x, tile, y, tw1, W, row0, nrows, circ, st); break;
        case 6: launch_cols<6>(fwd, bf16, v, g, x, tile, y, tw1, W, row0, nrows, circ, st); break;
        case 7: launch_cols<7>(fwd, bf16, v, g, x, tile, y, tw1, W, row0, nrows, circ, st); break;
        case 8: launch_cols<8>(fwd, bf16, v, g, x, tile, y, tw1, W, row0, nrows, circ, st); break;
        case 9: launch_cols<9>(fwd, bf16, v, g, x, tile, y, tw1, W, row0, nrows, circ, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int LOGW, class MAP>
void launch_rows(int mode, float2* buf, const float2* spec, const float* bias, const float2* tw2,
                 const float2* wpair, MAP map, int units, int D, int64_t row0, int64_t nrows, bool per_sample,
                 bool circ, hipStream_t st) {
    using R = C2Row<LOGW>;
    const unsigned grid = (unsigned)xcd_grid(nrows, units / R::UNITS);
    if (mode == 1)
        hipLaunchKernelGGL((k_cnd_row<LOGW, 1, MAP>), dim3(grid), dim3(R::THREADS), 0, st, buf, spec, bias, tw2,
                           wpair, map, D, row0, nrows, false);
    else if (circ)
        hipLaunchKernelGGL((k_cnd_row<LOGW, 0, MAP, true>), dim3(grid), dim3(R::THREADS), 0, st, buf, spec, bias,
                           tw2, wpair, map, D, row0, nrows, per_sample);
    else
        hipLaunchKernelGGL((k_cnd_row<LOGW, 0, MAP>), dim3(grid), dim3(R::THREADS), 0, st, buf, spec, bias, tw2,
                           wpair, map, D, row0, nrows, per_sample);
}

// Row pass with transforms of 2^logW packed points (MODE 0: the forward's tile,
// half of each row holding data, or all of it when circ; MODE 1: the spectrum).
template <class MAP>
hipError_t rows(int logW, int mode, float2* buf, const float2* spec, const float* bias, const float2* tw2,
                const float2* wpair, MAP map, int units, int D, int64_t row0, int64_t nrows, bool per_sample,
                hipStream_t st, bool circ = false) {
#define CND_ROWS(n)                                                                                         \
    case n:                                                                                                 \
        launch_rows<n>(mode, buf, spec, bias, tw2, wpair, map, units, D, row0, nrows, per_sample, circ, st); \
        break;
    switch (logW) {
        CND_ROWS(5)
        CND_ROWS(6)
        CND_ROWS(7)
        CND_ROWS(8)
        CND_ROWS(9)
        default: return hipErrorInvalidValue;
    }
#undef CND_ROWS
    return hipGetLastError();
}

inline bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
inline int log2i(int64_t x) {
    int l = 0;
    while ((int64_t(1) << l) < x) ++l;
    return l;
}

}  // namespace
}  // namespace hy
