// Four-step path of the Hyena forward hot path for gfx950, and the run-time
// dispatch of both paths over transform sizes.
//
// What is computed (HyenaDNA walkthrough, section 2.1, HyenaOperator.forward;
// section 2.2, HyenaFilter.forward and its fftconv call): a causal width-3
// depthwise conv of every u_proj channel, a split into gates x_0..x_{N-1} and
// the value v, then for o = 0..N-2: v <- v * x_{N-1-o}; v <- conv(v, h[o]) +
// bias[o] * v; finally y = v * x_0. The long convolution is evaluated in the
// frequency domain of a transform of length 2L (zero padding to double length,
// as in the HyenaND summary's boundary handling), which the FFT makes
// O(L log L) (Hyena Hierarchy concept page, section 3.2, FFT acceleration).
//
// Real 2L-point transforms are carried as L-point complex transforms of the
// packed sequence z[m] = a[2m] + i a[2m+1]. The second half of z is the zero
// padding (never loaded, pruned in the first radix pass), and only the first
// half of the inverse is kept. Bins k and L-k are combined in one "pair step"
// that unpacks the forward spectrum, multiplies by the filter spectrum plus the
// bias (the skip term bias*v is the convolution of v with bias*delta, whose
// spectrum is the constant bias) and repacks for the inverse. The stored
// filter spectrum is scaled by 2^-(log2 L + 2) (exact) so that the pair step
// also applies the inverse normalisation.
//
// Two paths:
//  * LDS path (L <= 16384): one workgroup per (b, d) row keeps the whole
//    transform on chip for all N-1 steps; only u_proj, the spectrum and y touch
//    HBM.
//  * Four-step path (any L >= 256, used for L >= 32768): L = L1 * L2 with
//    m = L2*m1 + m2 and k = k1 + L1*k2. Pass A takes column FFTs over m1,
//    pass B takes row FFTs over m2 (with the L-point twiddle), the pair step and
//    the inverse rows, pass C takes the inverse columns and the gate. Pass C of
//    step o is fused with pass A of step o+1. Rows are processed in chunks
//    whose tiles live in the workspace; at order 2 the chunks are pipelined
//    (k_fs_pipe: one launch runs pass C of chunk k-2, pass B of chunk k-1 and
//    pass A of chunk k), otherwise each chunk takes 2N-1 launches of its own.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fft_core.hpp"
#include "fourstep.hpp"
#include "kernels.hpp"
#include "pair.hpp"


namespace hy {

// defined in lds_path_*.hip
template <int LOGL>
hipError_t launch_lds_forward_t(const LdsArgs& a, hipStream_t st);
template <int LOGL>
hipError_t launch_lds_spectrum_t(const float* h, float2* spec, int64_t rows, const float2* tw, const float2* wpair,
                                 hipStream_t st, bool circ);

// ================================================================== launchers

hipError_t launch_lds_forward(int logL, const LdsArgs& a, hipStream_t st) {
    switch (logL) {
        case 4: return launch_lds_forward_t<4>(a, st);
        case 5: return launch_lds_forward_t<5>(a, st);
        case 6: return launch_lds_forward_t<6>(a, st);
        case 7: return launch_lds_forward_t<7>(a, st);
        case 8: return launch_lds_forward_t<8>(a, st);
        case 9: return launch_lds_forward_t<9>(a, st);
        case 10: return launch_lds_forward_t<10>(a, st);
        case 11: return launch_lds_forward_t<11>(a, st);
        case 12: return launch_lds_forward_t<12>(a, st);
        case 13: return launch_lds_forward_t<13>(a, st);
        case 14: return launch_lds_forward_t<14>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_lds_spectrum(int logL, const float* h, float2* spec, int64_t rows, const float2* tw,
                               const float2* wpair, hipStream_t st, bool circ) {
    switch (logL) {
        case 4: return launch_lds_spectrum_t<4>(h, spec, rows, tw, wpair, st, circ);
        case 5: return launch_lds_spectrum_t<5>(h, spec, rows, tw, wpair, st, circ);
        case 6: return launch_lds_spectrum_t<6>(h, spec, rows, tw, wpair, st, circ);
        case 7: return launch_lds_spectrum_t<7>(h, spec, rows, tw, wpair, st, circ);
        case 8: return launch_lds_spectrum_t<8>(h, spec, rows, tw, wpair, st, circ);
        case 9: return launch_lds_spectrum_t<9>(h, spec, rows, tw, wpair, st, circ);
        case 10: return launch_lds_spectrum_t<10>(h, spec, rows, tw, wpair, st, circ);
        case 11: return launch_lds_spectrum_t<11>(h, spec, rows, tw, wpair, st, circ);
        case 12: return launch_lds_spectrum_t<12>(h, spec, rows, tw, wpair, st, circ);
        case 13: return launch_lds_spectrum_t<13>(h, spec, rows, tw, wpair, st, circ);
        case 14: return launch_lds_spectrum_t<14>(h, spec, rows, tw, wpair, st, circ);
        default: return hipErrorInvalidValue;
    }
}

// Launches the passes of one chunk of rows. With `marks`, an event is recorded
// before the first launch and after every launch (1 + 2*(N-1) launches).
template <int LOG1, int LOG2, bool CIRC>
static hipError_t fs_forward_chunk_c(const FsArgs& a, int64_t row0, int64_t nrows, hipStream_t st,
                                     hipEvent_t* marks) {
    using Cfg = FsCfg<LOG1, LOG2>;
    int mi = 0;
    auto mark = [&]() {
        if (marks) (void)hipEventRecord(marks[mi++], st);
    };
    mark();
    const unsigned gcol = (unsigned)xcd_grid(nrows, Cfg::L2 / Cfg::CB);
    const unsigned grow = (unsigned)xcd_grid(nrows, Cfg::L1 / 2 / Cfg::UNITS);
    const dim3 bcol(Cfg::COL_THREADS), brow(Cfg::ROW_THREADS);
    if (a.bf16)
        hipLaunchKernelGGL((k_fs_colfwd<LOG1, LOG2, uint16_t, 0, CIRC>), dim3(gcol), bcol, 0, st, (const uint16_t*)a.u,
                           a.w3, (const float*)nullptr, a.ws, a.tb, a.D, a.N, row0, nrows);
    else
        hipLaunchKernelGGL((k_fs_colfwd<LOG1, LOG2, float, 0, CIRC>), dim3(gcol), bcol, 0, st, (const float*)a.u, a.w3,
                           (const float*)nullptr, a.ws, a.tb, a.D, a.N, row0, nrows);
    mark();
    for (int o = 0; o < a.N - 1; ++o) {
        hipLaunchKernelGGL((k_fs_row<LOG1, LOG2, 0>), dim3(grow), brow, 0, st, a.ws, a.spec, a.bias, a.tb, a.D, o,
                           row0, nrows, a.sbs);
        mark();
        const bool last = (o == a.N - 2);
        if (a.bf16) {
            if (last)
                hipLaunchKernelGGL((k_fs_colinv<LOG1, LOG2, uint16_t, true, CIRC>), dim3(gcol), bcol, 0, st, a.ws,
                                   (const uint16_t*)a.u, a.w3, (uint16_t*)a.y, a.tb, a.D, a.N, o, row0, nrows);
            else
                hipLaunchKernelGGL((k_fs_colinv<LOG1, LOG2, uint16_t, false, CIRC>), dim3(gcol), bcol, 0, st, a.ws,
                                   (const uint16_t*)a.u, a.w3, (uint16_t*)a.y, a.tb, a.D, a.N, o, row0, nrows);
        } else {
            if (last)
                hipLaunchKernelGGL((k_fs_colinv<LOG1, LOG2, float, true, CIRC>), dim3(gcol), bcol, 0, st, a.ws,
                                   (const float*)a.u, a.w3, (float*)a.y, a.tb, a.D, a.N, o, row0, nrows);
            else
                hipLaunchKernelGGL((k_fs_colinv<LOG1, LOG2, float, false, CIRC>), dim3(gcol), bcol, 0, st, a.ws,
                                   (const float*)a.u, a.w3, (float*)a.y, a.tb, a.D, a.N, o, row0, nrows);
        }
        mark();
    }
    return hipGetLastError();
}

template <int LOG1, int LOG2>
static hipError_t fs_forward_chunk(const FsArgs& a, int64_t row0, int64_t nrows, hipStream_t st,
                                   hipEvent_t* marks) {
    return a.circ ? fs_forward_chunk_c<LOG1, LOG2, true>(a, row0, nrows, st, marks)
                  : fs_forward_chunk_c<LOG1, LOG2, false>(a, row0, nrows, st, marks);
}

// Pipelined launches over chunks of R rows (see k_fs_pipe): launch k runs stage s
// on chunk k - s for every stage s < 2N-1 whose chunk exists.
template <int LOG1, int LOG2, class TIO, bool CIRC>
static hipError_t fs_forward_pipe_t(const FsArgs& a, int64_t rows, int64_t R, hipStream_t st, hipEvent_t* marks) {
    using P = FsPipeCfg<LOG1, LOG2>;
    if constexpr (!P::OK) {
        return hipErrorInvalidValue;
    } else {
        constexpr int64_t L = (int64_t)FsCfg<LOG1, LOG2>::L1 * FsCfg<LOG1, LOG2>::L2;
        const int S = 2 * a.N - 1;
        const int64_t nch = (rows + R - 1) / R;
        if (marks) (void)hipEventRecord(marks[0], st);
        for (int64_t k = 0; k < nch + S - 1; ++k) {
            FsPipe pp{};
            int64_t blk = 0;
            // oldest chunk first: its workgroups are dispatched first
            for (int s = S - 1; s >= 0; --s) {
                const int64_t c = k - s;
                if (c < 0 || c >= nch) continue;
                FsStage& g = pp.s[pp.n++];
                g.row0 = c * R;
                g.nrows = (rows - g.row0) < R ? (rows - g.row0) : R;
                g.slot = a.ws + (c % S) * R * L;
                g.blk0 = (uint32_t)blk;
                if (s == 0) {
                    g.kind = 0;
                    g.o = 0;
                } else if (s % 2 == 1) {
                    g.kind = 1;
                    g.o = (s - 1) / 2;
                } else {
                    g.o = (s - 2) / 2;
                    g.kind = g.o == a.N - 2 ? 3 : 2;
                }
                blk += xcd_grid(g.nrows, g.kind == 1 ? P::ROW_PER_ROW : P::COL_PER_ROW);
            }
            if (blk > 0x7fffffff) return hipErrorInvalidValue;
            if (a.N > 2)
                hipLaunchKernelGGL((k_fs_pipe<LOG1, LOG2, TIO, CIRC, true>), dim3((unsigned)blk), dim3(P::THREADS), 0,
                                   st, (const TIO*)a.u, a.w3, a.spec, a.bias, (TIO*)a.y, a.tb, a.D, a.N, a.sbs, pp);
            else
                hipLaunchKernelGGL((k_fs_pipe<LOG1, LOG2, TIO, CIRC, false>), dim3((unsigned)blk), dim3(P::THREADS), 0,
                                   st, (const TIO*)a.u, a.w3, a.spec, a.bias, (TIO*)a.y, a.tb, a.D, a.N, a.sbs, pp);
            if (marks) (void)hipEventRecord(marks[k + 1], st);
        }
        return hipGetLastError();
    }
}

template <int LOG1, int LOG2>
static hipError_t fs_forward_pipe(const FsArgs& a, int64_t rows, int64_t R, hipStream_t st, hipEvent_t* marks) {
    if (a.bf16)
        return a.circ ? fs_forward_pipe_t<LOG1, LOG2, uint16_t, true>(a, rows, R, st, marks)
                      : fs_forward_pipe_t<LOG1, LOG2, uint16_t, false>(a, rows, R, st, marks);
    return a.circ ? fs_forward_pipe_t<LOG1, LOG2, float, true>(a, rows, R, st, marks)
                  : fs_forward_pipe_t<LOG1, LOG2, float, false>(a, rows, R, st, marks);
}

template <int LOG1, int LOG2>
static hipError_t fs_spectrum_t(const float* h, float2* spec, int64_t rows, const FsTables& tb, hipStream_t st,
                                bool circ) {
    using Cfg = FsCfg<LOG1, LOG2>;
    const unsigned gcol = (unsigned)xcd_grid(rows, Cfg::L2 / Cfg::CB);
    const unsigned grow = (unsigned)xcd_grid(rows, Cfg::L1 / 2 / Cfg::UNITS);
    if (circ)
        hipLaunchKernelGGL((k_fs_colfwd<LOG1, LOG2, float, 1, true>), dim3(gcol), dim3(Cfg::COL_THREADS), 0, st,
                           (const float*)nullptr, (const float*)nullptr, h, spec, tb, 1, 2, (int64_t)0, rows);
    else
        hipLaunchKernelGGL((k_fs_colfwd<LOG1, LOG2, float, 1, false>), dim3(gcol), dim3(Cfg::COL_THREADS), 0, st,
                           (const float*)nullptr, (const float*)nullptr, h, spec, tb, 1, 2, (int64_t)0, rows);
    hipLaunchKernelGGL((k_fs_row<LOG1, LOG2, 1>), dim3(grow), dim3(Cfg::ROW_THREADS), 0, st, spec,
                       (const float2*)nullptr, (const float*)nullptr, tb, 1, 0, (int64_t)0, rows, (int64_t)0);
    return hipGetLastError();
}

void fs_split(int logL, int* log1, int* log2) {
    switch (logL) {
#define X(LG, A, B) \
    case LG: *log1 = A; *log2 = B; return;
        HY_FS_CASES(X)
#undef X
        default: *log1 = logL / 2; *log2 = logL - logL / 2;
    }
}

hipError_t launch_fs_forward_chunk(int logL, const FsArgs& a, int64_t row0, int64_t nrows, hipStream_t st,
                                   hipEvent_t* marks) {
    switch (logL) {
#define X(LG, A, B) \
    case LG: return fs_forward_chunk<A, B>(a, row0, nrows, st, marks);
        HY_FS_CASES(X)
#undef X
        default: return hipErrorInvalidValue;
    }
}

bool fs_pipe_supported(int logL) {
    switch (logL) {
#define X(LG, A, B) \
    case LG: return FsPipeCfg<A, B>::OK;
        HY_FS_CASES(X)
#undef X
        default: return false;
    }
}

hipError_t launch_fs_forward_pipelined(int logL, const FsArgs& a, int64_t rows, int64_t R, hipStream_t st,
                                       hipEvent_t* marks) {
    if (R < 1 || rows < 1 || a.N < 2 || 2 * a.N - 1 > kFsMaxStages) return hipErrorInvalidValue;
    switch (logL) {
#define X(LG, A, B) \
    case LG: return fs_forward_pipe<A, B>(a, rows, R, st, marks);
        HY_FS_CASES(X)
#undef X
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fs_spectrum(int logL, const float* h, float2* spec, int64_t rows, const FsTables& tb,
                              hipStream_t st, bool circ) {
    switch (logL) {
#define X(LG, A, B) \
    case LG: return fs_spectrum_t<A, B>(h, spec, rows, tb, st, circ);
        HY_FS_CASES(X)
#undef X
        default: return hipErrorInvalidValue;
    }
}

int fs_row_units(int logL) {
    switch (logL) {
#define X(LG, A, B) \
    case LG: return FsCfg<A, B>::UNITS;
        HY_FS_CASES(X)
#undef X
        default: return 0;
    }
}

}  // namespace hy
