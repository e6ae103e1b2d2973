// Four-step path device code shared by the forward (fourstep.hip) and the
// backward (fourstep_backward.hip): the three passes' bodies and kernels, and the
// table of transform splits. See fourstep.hip for what each pass computes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fft_core.hpp"
#include "kernels.hpp"
#include "pair.hpp"

namespace hy {

// ============================================================ four-step path
//
// Workgroups are spread over the 8 XCDs round-robin by hardware; the mapping
// below gives every row of a chunk to one XCD (row % 8) in all three passes, so
// the neighbouring column blocks that share conv3 halo lines, and the passes that
// re-read a row's tile, meet in the same L2.
__device__ __forceinline__ bool xcd_row_map(int64_t bid, int64_t nrows, int per_row, int64_t& row, int& sub) {
    const int xcd = (int)(bid & 7);
    const int64_t s = bid >> 3;
    sub = (int)(s % per_row);
    row = (s / per_row) * 8 + xcd;
    return row < nrows;
}
__host__ __device__ constexpr int64_t xcd_grid(int64_t nrows, int per_row) { return ((nrows + 7) / 8) * 8 * per_row; }

// The four-step twiddle W_L^(k1*m2) for k1 = t + T1*e: W_L^(t*m2) * W_L^(T1*e*m2),
// from two tables laid out [t][m2] and [e][m2] so that the 16 columns of a pass A
// or pass C workgroup read consecutive entries.
template <int L2>
__device__ __forceinline__ float2 twiddle_base(const FsTables& tb, int t, int m2) {
    return tb.tbase[(uint32_t)t * L2 + m2];
}
template <int L2>
__device__ __forceinline__ float2 twiddle_step(const FsTables& tb, float2 base, int e, int m2) {
    return cmul(base, tb.tstep[(uint32_t)e * L2 + m2]);
}

// Pass A: column FFTs over m1 of the packed gated input (MODE 0) or of a filter
// row (MODE 1), written to the row-major [k1][m2] tile `slot` of row `flat`.
// CIRC: rows of 2L samples with no zero padding (circular mode): all of every
// column holds data and the first radix pass is not pruned.
template <int LOG1, int LOG2, class TIO, int MODE, bool CIRC = false>
__device__ __forceinline__ void fs_colfwd_body(float2* lds, const TIO* __restrict__ u, const float* __restrict__ w3,
                                               const float* __restrict__ h, float2* __restrict__ slot,
                                               const FsTables& tb, int D, int N, int64_t flat, int cb) {
    using Cfg = FsCfg<LOG1, LOG2>;
    constexpr int L1 = Cfg::L1, L2 = Cfg::L2, T1 = Cfg::T1, CB = Cfg::CB;
    constexpr int64_t L = (int64_t)L1 * L2;
    constexpr int64_t S = CIRC ? 2 * L : L;  // samples per input row
    constexpr int LD = CIRC ? 16 : 8;        // column slots holding data
    const int c = threadIdx.x % CB, t = threadIdx.x / CB;
    const int m2 = cb * CB + c;
    float2 v[16];
    if constexpr (MODE == 0) {
        const uint32_t b = (uint32_t)flat / (uint32_t)D, d = (uint32_t)flat - b * (uint32_t)D;
        const int64_t C = (int64_t)(N + 1) * D;
        const int64_t cv = N * D + d, cx = (N - 1) * D + d;
        const TIO* rv = u + (b * C + cv) * S;
        const TIO* rx = u + (b * C + cx) * S;
#pragma unroll
        for (int e = 0; e < LD; ++e) {
            const uint32_t m = (uint32_t)(t + T1 * e) * L2 + m2;
            v[e] = gated_pair(rv, rx, m, w3 + 3 * cv, w3 + 3 * cx);
        }
    } else {
        const float* hr = h + flat * S;
#pragma unroll
        for (int e = 0; e < LD; ++e) v[e] = load_pair(hr, (uint32_t)(t + T1 * e) * L2 + m2);
    }
#pragma unroll
    for (int e = LD; e < 16; ++e) v[e] = make_float2(0.f, 0.f);
    fft_strided<L1, false, !CIRC>(v, t, tb.tw1, ColAcc<Cfg::CP>{lds + c});
    // four-step twiddle W_L^(k1*m2), applied here so that pass B carries none
    const float2 base = twiddle_base<L2>(tb, t, m2);
#pragma unroll
    for (int e = 0; e < 16; ++e) slot[(uint32_t)(t + T1 * e) * L2 + m2] = cmul(v[e], twiddle_step<L2>(tb, base, e, m2));
}

template <int LOG1, int LOG2, class TIO, int MODE, bool CIRC = false>
__global__ void __launch_bounds__((FsCfg<LOG1, LOG2>::COL_THREADS))
k_fs_colfwd(const TIO* __restrict__ u, const float* __restrict__ w3, const float* __restrict__ h,
            float2* __restrict__ ws, FsTables tb, int D, int N, int64_t row0, int64_t nrows) {
    using Cfg = FsCfg<LOG1, LOG2>;
    __shared__ float2 lds[Cfg::L1 * Cfg::CP];
    int64_t r;
    int cb;
    if (!xcd_row_map(blockIdx.x, nrows, Cfg::L2 / Cfg::CB, r, cb)) return;
    const int64_t L = (int64_t)Cfg::L1 * Cfg::L2;
    float2* slot = (MODE == 0) ? ws + r * L : ws + (row0 + r) * L;
    fs_colfwd_body<LOG1, LOG2, TIO, MODE, CIRC>(lds, u, w3, h, slot, tb, D, N, row0 + r, cb);
}

// Where one pair slot of pass B lives: LDS rows/indices of its two bins, the
// offsets of their spectrum values in the [k1][k2] spectrum tile, and W_{2L}^k.
struct PairSlot {
    int ra, ia, rb, ib;  // LDS row slot (0 = row a, 1 = row b of the unit) and index
    int offa, offb;      // spectrum offsets
    float2 w;
    int kind;  // 0 general pair, 1 the two self-contained bins k = 0 and k = L/2
};

template <int L1, int L2>
__device__ __forceinline__ PairSlot pair_slot(int p, int k2, const FsTables& tb) {
    PairSlot ps;
    ps.kind = 0;
    if (p != 0) {
        // k = p + L1*k2 pairs with L - k = (L1-p) + L1*(L2-1-k2)
        ps.ra = 0; ps.ia = k2; ps.rb = 1; ps.ib = L2 - 1 - k2;
        ps.offa = p * L2 + ps.ia;
        ps.offb = (L1 - p) * L2 + ps.ib;
        ps.w = cmul(tb.pa[p], tb.pb[k2]);
    } else if (k2 == 0) {
        // k = 0 (with L) and k = L/2, both in row 0
        ps.kind = 1;
        ps.ra = 0; ps.ia = 0; ps.rb = 0; ps.ib = L2 / 2;
        ps.offa = 0;
        ps.offb = L2 / 2;
        ps.w = tb.pb[L2 / 2];
    } else if (k2 < L2 / 2) {
        // row 0: k = L1*k2 pairs with L1*(L2-k2)
        ps.ra = 0; ps.ia = k2; ps.rb = 0; ps.ib = L2 - k2;
        ps.offa = ps.ia;
        ps.offb = ps.ib;
        ps.w = tb.pb[k2];
    } else {
        // row L1/2: k = L1/2 + L1*j pairs with L1/2 + L1*(L2-1-j)
        const int j = k2 - L2 / 2;
        ps.ra = 1; ps.ia = j; ps.rb = 1; ps.ib = L2 - 1 - j;
        ps.offa = (L1 / 2) * L2 + ps.ia;
        ps.offb = (L1 / 2) * L2 + ps.ib;
        ps.w = cmul(tb.pa[L1 / 2], tb.pb[j]);
    }
    return ps;
}

// Pass B: row FFTs over m2 (the tile already carries the W_L^(k1*m2) twiddle),
// the pair step, then (MODE 0) the spectrum multiply and the inverse rows, in
// place; or (MODE 1) the scaled spectrum written in place. Backward modes:
// MODE 2 is MODE 0 with the result written to the tile `aux` (the column-
// transformed gated input in `slot` is kept for the adjoint); MODE 3 takes the
// row as A_dv, applies conj(H + bias) instead of H + bias (the correlation that is
// the adjoint of the convolution) and also takes the product A_dv * conj(A_g)
// through the same repack and inverse rows into the tile `pt` of the row, A_g
// being the row transform of the kept column-transformed gated input in `aux`
// (the same arithmetic as in MODE 2, so the same values).
// A unit is the row pair {p, L1-p} (p >= 1) or {0, L1/2} (p = 0).
template <int LOG1, int LOG2, int MODE>
__device__ __forceinline__ void fs_row_body(float2* lds, float2* __restrict__ slot, const float2* __restrict__ spec,
                                            const float* __restrict__ bias, const FsTables& tb, int D, int o,
                                            int64_t flat, int ug, float2* __restrict__ aux = nullptr,
                                            float2* __restrict__ pt = nullptr, int64_t sbs = 0) {
    constexpr bool CONV = MODE == 0 || MODE == 2 || MODE == 3;  // multiply by the filter spectrum
    using Cfg = FsCfg<LOG1, LOG2>;
    constexpr int L1 = Cfg::L1, L2 = Cfg::L2, T2 = Cfg::T2, U = Cfg::UNITS, RP = Cfg::RP;
    constexpr int64_t L = (int64_t)L1 * L2;
    const int tau = threadIdx.x;
    const int rho = tau / T2, t = tau % T2;
    const int p_row = ug * U + rho / 2;
    const int k1 = (rho & 1) == 0 ? p_row : (p_row == 0 ? L1 / 2 : L1 - p_row);
    float2* rowp = slot + (uint32_t)k1 * L2;
    const RowAcc racc{lds + rho * RP};

    // pair-step role of this thread: 2*T2 threads per unit, L2 pairs per unit
    const int unit = tau / (2 * T2), tp = tau % (2 * T2);
    const int p = ug * U + unit;
    const float2* Hrow = nullptr;
    float bs = 0.f;
    float2 ha[8], hb[8];
    float2 qa[8], qb[8];  // MODE 3: the repacked dh product of this thread's pairs
    if constexpr (CONV) {
        const uint32_t b = (uint32_t)flat / (uint32_t)D, d = (uint32_t)flat - b * (uint32_t)D;
        Hrow = spec + (int64_t)b * sbs + ((int64_t)o * D + d) * L;
        bs = bias[(int64_t)o * D + d] * (1.0f / (4.0f * (float)L));
    }

    // row ri (0 or 1) of this thread's unit, computed rather than taken from an array,
    // so that a run-time ri leaves a plain LDS address (no private array)
    auto au = [&](int ri) { return RowAcc{lds + (2 * unit + ri) * RP}; };

    float2 v[16];
    [[maybe_unused]] float2 ga[8], gb[8];  // MODE 3: A_g at this thread's pairs
    if constexpr (MODE == 3) {
        // A_g: the forward rows of the kept gated input, unpacked at this thread's pairs
        const float2* grow = aux + (uint32_t)k1 * L2;
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = grow[(uint32_t)(t + T2 * e)];
        fft_strided<L2, false, false>(v, t, tb.tw2, racc);
        __syncthreads();
        lds_store_strided<T2>(racc, t, v);
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const PairSlot ps = pair_slot<L1, L2>(p, tp + 2 * T2 * e, tb);
            const float2 Za = au(ps.ra)[ps.ia];
            const float2 Zb = au(ps.rb)[ps.ib];
            if (ps.kind == 0) {
                pair_unpack(Za, Zb, ps.w, ga[e], gb[e]);
            } else {
                float2 A0, AL, Ad;  // bins 0 and L (real), then L/2
                pair_unpack(Za, Za, make_float2(1.f, 0.f), A0, AL);
                ga[e] = make_float2(A0.x, AL.x);
                pair_unpack(Zb, Zb, ps.w, gb[e], Ad);
            }
        }
        // the next transform begins with a barrier before it writes the LDS
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = rowp[(uint32_t)(t + T2 * e)];
    if constexpr (CONV) {
        // the spectrum is needed only after the forward rows; fetch it now
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const PairSlot ps = pair_slot<L1, L2>(p, tp + 2 * T2 * e, tb);
            ha[e] = Hrow[(uint32_t)ps.offa];
            hb[e] = Hrow[(uint32_t)ps.offb];
        }
    }
    fft_strided<L2, false, false>(v, t, tb.tw2, racc);
    __syncthreads();
    lds_store_strided<T2>(racc, t, v);
    __syncthreads();

    const float sc = 1.0f / (8.0f * (float)L);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const PairSlot ps = pair_slot<L1, L2>(p, tp + 2 * T2 * e, tb);
        const float2 Za = au(ps.ra)[ps.ia];
        const float2 Zb = au(ps.rb)[ps.ib];
        if constexpr (MODE == 0) {
            float2 Yk, Ym;
            if (ps.kind == 0) {
                pair_conv(Za, Zb, hadd(ha[e], bs), hadd(hb[e], bs), ps.w, Yk, Ym);
                au(ps.ra)[ps.ia] = Yk;
                au(ps.rb)[ps.ib] = Ym;
            } else {
                // bin 0 pairs with bin L (spectrum slot 0 holds (H[0], H[L]))
                pair_conv(Za, Za, make_float2(ha[e].x + bs, 0.f), make_float2(ha[e].y + bs, 0.f),
                          make_float2(1.f, 0.f), Yk, Ym);
                au(ps.ra)[ps.ia] = Yk;
                const float2 Hh = hadd(hb[e], bs);  // bin L/2 pairs with itself
                pair_conv(Zb, Zb, Hh, Hh, ps.w, Yk, Ym);
                au(ps.rb)[ps.ib] = Yk;
            }
        } else if constexpr (MODE == 2 || MODE == 3) {
            // conj(H + bias) in MODE 3; bins 0 and L of slot 0 are real either way
            auto hmul = [](float2 a, float2 h) { return MODE == 2 ? cmul(a, h) : cmulc(a, h); };
            float2 Yk, Ym;
            if (ps.kind == 0) {
                float2 Ak, Am;
                pair_unpack(Za, Zb, ps.w, Ak, Am);
                if constexpr (MODE == 3) {
                    const float2 Pk = cmulc(Ak, ga[e]), Pm = cmulc(Am, gb[e]);
                    pair_repack(fmul2(Pk, sc), fmul2(Pm, sc), ps.w, qa[e], qb[e]);
                }
                pair_repack(hmul(Ak, hadd(ha[e], bs)), hmul(Am, hadd(hb[e], bs)), ps.w, Yk, Ym);
                au(ps.ra)[ps.ia] = Yk;
                au(ps.rb)[ps.ib] = Ym;
            } else {
                float2 A0, AL;  // bins 0 and L (real)
                pair_unpack(Za, Za, make_float2(1.f, 0.f), A0, AL);
                [[maybe_unused]] float2 Yd;
                if constexpr (MODE == 3) {
                    const float2 g0 = ga[e];
                    pair_repack(make_float2(A0.x * g0.x * sc, 0.f), make_float2(AL.x * g0.y * sc, 0.f),
                                make_float2(1.f, 0.f), qa[e], Yd);
                }
                pair_repack(make_float2(A0.x * (ha[e].x + bs), 0.f), make_float2(AL.x * (ha[e].y + bs), 0.f),
                            make_float2(1.f, 0.f), Yk, Ym);
                au(ps.ra)[ps.ia] = Yk;
                float2 Ah, Ad;  // bin L/2 pairs with itself
                pair_unpack(Zb, Zb, ps.w, Ah, Ad);
                if constexpr (MODE == 3) {
                    const float2 Ph = cmulc(Ah, gb[e]);
                    pair_repack(fmul2(Ph, sc), fmul2(Ph, sc), ps.w, qb[e], Yd);
                }
                const float2 Ch = hmul(Ah, hadd(hb[e], bs));
                pair_repack(Ch, Ch, ps.w, Yk, Ym);
                au(ps.rb)[ps.ib] = Yk;
            }
        } else {
            float2 Ak, Am;
            if (ps.kind == 0) {
                pair_unpack(Za, Zb, ps.w, Ak, Am);
                slot[(uint32_t)ps.offa] = fmul2(Ak, sc);
                slot[(uint32_t)ps.offb] = fmul2(Am, sc);
            } else {
                pair_unpack(Za, Za, make_float2(1.f, 0.f), Ak, Am);
                slot[0] = make_float2(Ak.x * sc, Am.x * sc);
                pair_unpack(Zb, Zb, ps.w, Ak, Am);
                slot[(uint32_t)ps.offb] = fmul2(Ak, sc);
            }
        }
    }
    if constexpr (CONV) {
        __syncthreads();
        lds_load_strided<T2>(racc, t, v);
        fft_strided<L2, true, false>(v, t, tb.tw2, racc);
        float2* orow = MODE == 2 ? aux + (uint32_t)k1 * L2 : rowp;
#pragma unroll
        for (int e = 0; e < 16; ++e) orow[(uint32_t)(t + T2 * e)] = v[e];
    }
    if constexpr (MODE == 3) {
        // the dh product through the same inverse rows, into the row's dh tile
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const PairSlot ps = pair_slot<L1, L2>(p, tp + 2 * T2 * e, tb);
            au(ps.ra)[ps.ia] = qa[e];
            au(ps.rb)[ps.ib] = qb[e];
        }
        __syncthreads();
        lds_load_strided<T2>(racc, t, v);
        fft_strided<L2, true, false>(v, t, tb.tw2, racc);
        float2* prow = pt + (uint32_t)k1 * L2;
#pragma unroll
        for (int e = 0; e < 16; ++e) prow[(uint32_t)(t + T2 * e)] = v[e];
    }
}

template <int LOG1, int LOG2, int MODE>
__global__ void __launch_bounds__((FsCfg<LOG1, LOG2>::ROW_THREADS))
k_fs_row(float2* __restrict__ ws, const float2* __restrict__ spec, const float* __restrict__ bias, FsTables tb,
         int D, int o, int64_t row0, int64_t nrows, int64_t sbs) {
    using Cfg = FsCfg<LOG1, LOG2>;
    __shared__ float2 lds[2 * Cfg::UNITS * Cfg::RP];
    int64_t r;
    int ug;
    if (!xcd_row_map(blockIdx.x, nrows, Cfg::L1 / 2 / Cfg::UNITS, r, ug)) return;
    const int64_t L = (int64_t)Cfg::L1 * Cfg::L2;
    float2* slot = (MODE == 0) ? ws + r * L : ws + (row0 + r) * L;
    fs_row_body<LOG1, LOG2, MODE>(lds, slot, spec, bias, tb, D, o, row0 + r, ug, nullptr, nullptr, sbs);
}

// Pass C: the conjugate four-step twiddle, inverse column FFTs over k1, then
// the gate. The last step stores y;
// otherwise the gated result is the next step's input and its forward column
// FFTs (pass A of step o+1) run here, written back in place.
template <int LOG1, int LOG2, class TIO, bool LAST, bool CIRC = false>
__device__ __forceinline__ void fs_colinv_body(float2* lds, float2* __restrict__ slot, const TIO* __restrict__ u,
                                               const float* __restrict__ w3, TIO* __restrict__ y, const FsTables& tb,
                                               int D, int N, int o, int64_t flat, int cb) {
    using Cfg = FsCfg<LOG1, LOG2>;
    constexpr int L1 = Cfg::L1, L2 = Cfg::L2, T1 = Cfg::T1, CB = Cfg::CB;
    constexpr int64_t L = (int64_t)L1 * L2;
    constexpr int64_t S = CIRC ? 2 * L : L;  // samples per row of u_proj and y
    constexpr int LD = CIRC ? 16 : 8;        // column slots holding data
    const uint32_t b = (uint32_t)flat / (uint32_t)D, d = (uint32_t)flat - b * (uint32_t)D;
    const int c = threadIdx.x % CB, t = threadIdx.x / CB;
    const int m2 = cb * CB + c;
    const ColAcc<Cfg::CP> cacc{lds + c};
    float2 v[16];
    const float2 base = twiddle_base<L2>(tb, t, m2);
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = cmulc(slot[(uint32_t)(t + T1 * e) * L2 + m2], twiddle_step<L2>(tb, base, e, m2));
    fft_strided<L1, true, false>(v, t, tb.tw1, cacc);
    const int64_t C = (int64_t)(N + 1) * D;
    const int64_t cg = (int64_t)(LAST ? 0 : N - 2 - o) * D + d;
    const TIO* rg = u + (b * C + cg) * S;
    const float* wg = w3 + 3 * cg;
    if constexpr (LAST) {
        TIO* yr = y + (b * D + d) * S;
#pragma unroll
        for (int e = 0; e < LD; ++e) {
            const uint32_t m = (uint32_t)(t + T1 * e) * L2 + m2;
            store_pair(yr, m, emul(v[e], conv3_pair(rg, m, wg[0], wg[1], wg[2])));
        }
    } else {
#pragma unroll
        for (int e = 0; e < LD; ++e) {
            const uint32_t m = (uint32_t)(t + T1 * e) * L2 + m2;
            v[e] = emul(v[e], conv3_pair(rg, m, wg[0], wg[1], wg[2]));
        }
#pragma unroll
        for (int e = LD; e < 16; ++e) v[e] = make_float2(0.f, 0.f);
        fft_strided<L1, false, !CIRC>(v, t, tb.tw1, cacc);
#pragma unroll
        for (int e = 0; e < 16; ++e)
            slot[(uint32_t)(t + T1 * e) * L2 + m2] = cmul(v[e], twiddle_step<L2>(tb, base, e, m2));
    }
}

template <int LOG1, int LOG2, class TIO, bool LAST, bool CIRC = false>
__global__ void __launch_bounds__((FsCfg<LOG1, LOG2>::COL_THREADS))
k_fs_colinv(float2* __restrict__ ws, const TIO* __restrict__ u, const float* __restrict__ w3, TIO* __restrict__ y,
            FsTables tb, int D, int N, int o, int64_t row0, int64_t nrows) {
    using Cfg = FsCfg<LOG1, LOG2>;
    __shared__ float2 lds[Cfg::L1 * Cfg::CP];
    int64_t r;
    int cb;
    if (!xcd_row_map(blockIdx.x, nrows, Cfg::L2 / Cfg::CB, r, cb)) return;
    const int64_t L = (int64_t)Cfg::L1 * Cfg::L2;
    fs_colinv_body<LOG1, LOG2, TIO, LAST, CIRC>(lds, ws + r * L, u, w3, y, tb, D, N, o, row0 + r, cb);
}

// ============================================================ pipelined launches
//
// The passes of consecutive chunks of rows are independent, so one launch can
// run pass A of chunk k, the passes of step 0 of chunk k-1, ... together: stage s
// of a launch takes chunk k - s. Each chunk owns one tile slot of a ring of
// 2N-1 slots, so the tile a stage writes is read by the next stage of the same
// chunk in the next launch; the launch boundary is the only synchronisation.
// This keeps every launch full (no per-pass tail per chunk) and keeps the time
// between a tile's write and its re-read to one launch.
struct FsStage {
    float2* slot;   // the chunk's tile slot (nrows tiles of L complex values)
    int64_t row0;   // first flat (b, d) row of the chunk
    int64_t nrows;  // rows of the chunk
    uint32_t blk0;  // first workgroup of this stage in the launch
    int kind;       // 0 pass A, 1 pass B, 2 pass C followed by another step, 3 pass C of the last step
    int o;          // the step of a pass B or pass C
};
constexpr int kFsMaxStages = 15;  // 2 * 8 - 1 stages at order 8
struct FsPipe {
    FsStage s[kFsMaxStages];
    int n;  // stages in this launch
};

template <int LOG1, int LOG2>
struct FsPipeCfg {
    using Cfg = FsCfg<LOG1, LOG2>;
    // one block size for every stage: the column and row passes must agree
    static constexpr bool OK = Cfg::COL_THREADS == Cfg::ROW_THREADS;
    static constexpr int THREADS = Cfg::COL_THREADS;
    static constexpr int LDS_COL = Cfg::L1 * Cfg::CP;
    static constexpr int LDS_ROW = 2 * Cfg::UNITS * Cfg::RP;
    static constexpr int LDS = LDS_COL > LDS_ROW ? LDS_COL : LDS_ROW;
    static constexpr int COL_PER_ROW = Cfg::L2 / Cfg::CB;         // pass A / C workgroups per row
    static constexpr int ROW_PER_ROW = Cfg::L1 / 2 / Cfg::UNITS;  // pass B workgroups per row
};

// MID: the launch may hold a pass C followed by another step (order > 2); that
// body needs more registers than the others, so order-2 launches leave it out.
template <int LOG1, int LOG2, class TIO, bool CIRC, bool MID>
__global__ void __launch_bounds__((FsPipeCfg<LOG1, LOG2>::THREADS))
k_fs_pipe(const TIO* __restrict__ u, const float* __restrict__ w3, const float2* __restrict__ spec,
          const float* __restrict__ bias, TIO* __restrict__ y, FsTables tb, int D, int N, int64_t sbs, FsPipe pp) {
    using P = FsPipeCfg<LOG1, LOG2>;
    static_assert(P::OK, "pipelined launches need equal column and row block sizes");
    __shared__ float2 lds[P::LDS];
    constexpr int64_t L = (int64_t)FsCfg<LOG1, LOG2>::L1 * FsCfg<LOG1, LOG2>::L2;
    const uint32_t bid = blockIdx.x;
    int i = 0;
    while (i + 1 < pp.n && bid >= pp.s[i + 1].blk0) ++i;  // workgroup-uniform
    const FsStage& g = pp.s[i];
    const int64_t local = (int64_t)(bid - g.blk0);
    int64_t r;
    int sub;
    if (g.kind == 1) {
        if (!xcd_row_map(local, g.nrows, P::ROW_PER_ROW, r, sub)) return;
        fs_row_body<LOG1, LOG2, 0>(lds, g.slot + r * L, spec, bias, tb, D, g.o, g.row0 + r, sub, nullptr, nullptr,
                                   sbs);
        return;
    }
    if (!xcd_row_map(local, g.nrows, P::COL_PER_ROW, r, sub)) return;
    if (g.kind == 0)
        fs_colfwd_body<LOG1, LOG2, TIO, 0, CIRC>(lds, u, w3, nullptr, g.slot + r * L, tb, D, N, g.row0 + r, sub);
    else if (MID && g.kind == 2)
        fs_colinv_body<LOG1, LOG2, TIO, false, CIRC>(lds, g.slot + r * L, u, w3, y, tb, D, N, g.o, g.row0 + r, sub);
    else
        fs_colinv_body<LOG1, LOG2, TIO, true, CIRC>(lds, g.slot + r * L, u, w3, y, tb, D, N, g.o, g.row0 + r, sub);
}

// log2 L -> (log2 L1, log2 L2). Square splits up to L1 = 512, whose pass A/C
// tile (512 x 17 complex) still leaves room for two workgroups per CU.
#ifndef HY_FS_LOG1_16
#define HY_FS_LOG1_16 8
#endif
#ifndef HY_FS_LOG1_20
#define HY_FS_LOG1_20 9
#endif
#define HY_FS_CASES(X)                                                                                   \
    X(8, 4, 4) X(9, 4, 5) X(10, 5, 5) X(11, 5, 6) X(12, 6, 6) X(13, 6, 7) X(14, 7, 7) X(15, 7, 8)          \
        X(16, HY_FS_LOG1_16, 16 - HY_FS_LOG1_16) X(17, 8, 9) X(18, 9, 9) X(19, 9, 10)                     \
        X(20, HY_FS_LOG1_20, 20 - HY_FS_LOG1_20)

}  // namespace hy
