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
//    step o is fused with pass A of step o+1.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fft_core.hpp"
#include "kernels.hpp"
#include "pair.hpp"

#ifndef HY_EXPERIMENTAL_FUSED
#define HY_EXPERIMENTAL_FUSED 0
#endif

namespace hy {

// defined in lds_path_*.hip
template <int LOGL>
hipError_t launch_lds_forward_t(const LdsArgs& a, hipStream_t st);
template <int LOGL>
hipError_t launch_lds_spectrum_t(const float* h, float2* spec, int64_t rows, const float2* tw, const float2* wpair,
                                 hipStream_t st);

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
template <int LOG1, int LOG2, class TIO, int MODE>
__device__ __forceinline__ void fs_colfwd_body(float2* lds, const TIO* __restrict__ u, const float* __restrict__ w3,
                                               const float* __restrict__ h, float2* __restrict__ slot,
                                               const FsTables& tb, int D, int N, int64_t flat, int cb) {
    using Cfg = FsCfg<LOG1, LOG2>;
    constexpr int L1 = Cfg::L1, L2 = Cfg::L2, T1 = Cfg::T1, CB = Cfg::CB;
    constexpr int64_t L = (int64_t)L1 * L2;
    const int c = threadIdx.x % CB, t = threadIdx.x / CB;
    const int m2 = cb * CB + c;
    float2 v[16];
    if constexpr (MODE == 0) {
        const uint32_t b = (uint32_t)flat / (uint32_t)D, d = (uint32_t)flat - b * (uint32_t)D;
        const int64_t C = (int64_t)(N + 1) * D;
        const int64_t cv = N * D + d, cx = (N - 1) * D + d;
        const TIO* rv = u + (b * C + cv) * L;
        const TIO* rx = u + (b * C + cx) * L;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t m = (uint32_t)(t + T1 * e) * L2 + m2;
            v[e] = gated_pair(rv, rx, m, w3 + 3 * cv, w3 + 3 * cx);
        }
    } else {
        const float* hr = h + flat * L;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = load_pair(hr, (uint32_t)(t + T1 * e) * L2 + m2);
    }
#pragma unroll
    for (int e = 8; e < 16; ++e) v[e] = make_float2(0.f, 0.f);
    fft_strided<L1, false, true>(v, t, tb.tw1, ColAcc<Cfg::CP>{lds + c});
    // four-step twiddle W_L^(k1*m2), applied here so that pass B carries none
    const float2 base = twiddle_base<L2>(tb, t, m2);
#pragma unroll
    for (int e = 0; e < 16; ++e) slot[(uint32_t)(t + T1 * e) * L2 + m2] = cmul(v[e], twiddle_step<L2>(tb, base, e, m2));
}

template <int LOG1, int LOG2, class TIO, int MODE>
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
    fs_colfwd_body<LOG1, LOG2, TIO, MODE>(lds, u, w3, h, slot, tb, D, N, row0 + r, cb);
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
// place; or (MODE 1) the scaled spectrum written in place.
// A unit is the row pair {p, L1-p} (p >= 1) or {0, L1/2} (p = 0).
template <int LOG1, int LOG2, int MODE>
__device__ __forceinline__ void fs_row_body(float2* lds, float2* __restrict__ slot, const float2* __restrict__ spec,
                                            const float* __restrict__ bias, const FsTables& tb, int D, int o,
                                            int64_t flat, int ug) {
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
    if constexpr (MODE == 0) {
        const uint32_t d = (uint32_t)flat % (uint32_t)D;
        Hrow = spec + ((int64_t)o * D + d) * L;
        bs = bias[(int64_t)o * D + d] * (1.0f / (4.0f * (float)L));
    }

    float2 v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = rowp[(uint32_t)(t + T2 * e)];
    if constexpr (MODE == 0) {
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

    const RowAcc au[2] = {RowAcc{lds + (2 * unit) * RP}, RowAcc{lds + (2 * unit + 1) * RP}};
    const float sc = 1.0f / (8.0f * (float)L);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const PairSlot ps = pair_slot<L1, L2>(p, tp + 2 * T2 * e, tb);
        const float2 Za = au[ps.ra][ps.ia];
        const float2 Zb = au[ps.rb][ps.ib];
        if constexpr (MODE == 0) {
            float2 Yk, Ym;
            if (ps.kind == 0) {
                pair_conv(Za, Zb, hadd(ha[e], bs), hadd(hb[e], bs), ps.w, Yk, Ym);
                au[ps.ra][ps.ia] = Yk;
                au[ps.rb][ps.ib] = Ym;
            } else {
                // bin 0 pairs with bin L (spectrum slot 0 holds (H[0], H[L]))
                pair_conv(Za, Za, make_float2(ha[e].x + bs, 0.f), make_float2(ha[e].y + bs, 0.f),
                          make_float2(1.f, 0.f), Yk, Ym);
                au[ps.ra][ps.ia] = Yk;
                const float2 Hh = hadd(hb[e], bs);  // bin L/2 pairs with itself
                pair_conv(Zb, Zb, Hh, Hh, ps.w, Yk, Ym);
                au[ps.rb][ps.ib] = Yk;
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
    if constexpr (MODE == 0) {
        __syncthreads();
        lds_load_strided<T2>(racc, t, v);
        fft_strided<L2, true, false>(v, t, tb.tw2, racc);
#pragma unroll
        for (int e = 0; e < 16; ++e) rowp[(uint32_t)(t + T2 * e)] = v[e];
    }
}

template <int LOG1, int LOG2, int MODE>
__global__ void __launch_bounds__((FsCfg<LOG1, LOG2>::ROW_THREADS))
k_fs_row(float2* __restrict__ ws, const float2* __restrict__ spec, const float* __restrict__ bias, FsTables tb,
         int D, int o, int64_t row0, int64_t nrows) {
    using Cfg = FsCfg<LOG1, LOG2>;
    __shared__ float2 lds[2 * Cfg::UNITS * Cfg::RP];
    int64_t r;
    int ug;
    if (!xcd_row_map(blockIdx.x, nrows, Cfg::L1 / 2 / Cfg::UNITS, r, ug)) return;
    const int64_t L = (int64_t)Cfg::L1 * Cfg::L2;
    float2* slot = (MODE == 0) ? ws + r * L : ws + (row0 + r) * L;
    fs_row_body<LOG1, LOG2, MODE>(lds, slot, spec, bias, tb, D, o, row0 + r, ug);
}

// Pass C: the conjugate four-step twiddle, inverse column FFTs over k1, then
// the gate. The last step stores y;
// otherwise the gated result is the next step's input and its forward column
// FFTs (pass A of step o+1) run here, written back in place.
template <int LOG1, int LOG2, class TIO, bool LAST>
__device__ __forceinline__ void fs_colinv_body(float2* lds, float2* __restrict__ slot, const TIO* __restrict__ u,
                                               const float* __restrict__ w3, TIO* __restrict__ y, const FsTables& tb,
                                               int D, int N, int o, int64_t flat, int cb) {
    using Cfg = FsCfg<LOG1, LOG2>;
    constexpr int L1 = Cfg::L1, L2 = Cfg::L2, T1 = Cfg::T1, CB = Cfg::CB;
    constexpr int64_t L = (int64_t)L1 * L2;
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
    const TIO* rg = u + (b * C + cg) * L;
    const float* wg = w3 + 3 * cg;
    if constexpr (LAST) {
        TIO* yr = y + (b * D + d) * L;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t m = (uint32_t)(t + T1 * e) * L2 + m2;
            store_pair(yr, m, emul(v[e], conv3_pair(rg, m, wg[0], wg[1], wg[2])));
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t m = (uint32_t)(t + T1 * e) * L2 + m2;
            v[e] = emul(v[e], conv3_pair(rg, m, wg[0], wg[1], wg[2]));
        }
#pragma unroll
        for (int e = 8; e < 16; ++e) v[e] = make_float2(0.f, 0.f);
        fft_strided<L1, false, true>(v, t, tb.tw1, cacc);
#pragma unroll
        for (int e = 0; e < 16; ++e)
            slot[(uint32_t)(t + T1 * e) * L2 + m2] = cmul(v[e], twiddle_step<L2>(tb, base, e, m2));
    }
}

template <int LOG1, int LOG2, class TIO, bool LAST>
__global__ void __launch_bounds__((FsCfg<LOG1, LOG2>::COL_THREADS))
k_fs_colinv(float2* __restrict__ ws, const TIO* __restrict__ u, const float* __restrict__ w3, TIO* __restrict__ y,
            FsTables tb, int D, int N, int o, int64_t row0, int64_t nrows) {
    using Cfg = FsCfg<LOG1, LOG2>;
    __shared__ float2 lds[Cfg::L1 * Cfg::CP];
    int64_t r;
    int cb;
    if (!xcd_row_map(blockIdx.x, nrows, Cfg::L2 / Cfg::CB, r, cb)) return;
    const int64_t L = (int64_t)Cfg::L1 * Cfg::L2;
    fs_colinv_body<LOG1, LOG2, TIO, LAST>(lds, ws + r * L, u, w3, y, tb, D, N, o, row0 + r, cb);
}

// ====================================================== fused persistent path
//
// One launch for a whole order-2 forward. Workgroups are dispatched to the 8 XCDs
// round-robin; each reads its XCD from the XCC_ID hardware register and serves
// that XCD's rows (r = xcd + 8*i) through the XCD's own ticket counter. Each
// ticket names one work item (a pass A column block, a pass B unit group or a
// pass C column block of one row). Tickets are issued per step s as
//   [A items of group s][B items of group s-1][C items of group s-2],
// and an item only waits for items holding earlier tickets (B waits for its
// row's A items, C for its row's B items, A of group j for C of group j - S,
// whose tile slot it reuses), so every wait ends even when not all workgroups
// are resident. Tiles live in a ring of S * G rows per XCD sized to stay in that
// XCD's L2, and every hand-off happens between CUs of one XCD: a producer waits
// for its stores to complete (they are then in the L2), then bumps a counter with
// an atomic in the same L2; a consumer polls the counter with atomics, then
// invalidates its L1 before reading the tile. Waits are bounded in time (see
// kWaitTicks, kKernelTicks): an expired wait records an error in the control
// block and the kernel runs to its end.
// Time bounds, on the 100 MHz real-time counter: one wait may last 20 ms, and no
// workgroup takes a new ticket more than 1 s after it started.
constexpr uint64_t kWaitTicks = 2000000;
constexpr uint64_t kKernelTicks = 100000000;

// One 128-byte line per XCD: [0] ticket counter, [1] error flag, [2] waits that
// had to poll, [3] longest wait in real-time ticks. Each line is only touched by
// the workgroups of its XCD, so it lives in that XCD's L2.
struct FusedCtl {
    uint32_t x[8][32];
};

__device__ __forceinline__ uint32_t hw_xcc_id() {
    return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (15 << 11)) & 7u;  // HW_REG_XCC_ID
}

__device__ __forceinline__ uint64_t rt_now() { return __builtin_amdgcn_s_memrealtime(); }

// read a counter where its increments are performed: an atomic add of a value
// the compiler cannot see is zero (it would turn an add of 0 into a plain load)
__device__ __forceinline__ uint32_t ctr_read(uint32_t* ctr, uint32_t zero) {
    return __hip_atomic_fetch_add(ctr, zero, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// all threads of the block: make this block's global stores visible in the L2,
// then count the item as done
__device__ __forceinline__ void fused_signal(uint32_t* ctr) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// all threads of the block: wait until *ctr >= target, then drop stale L1 lines.
// A wait that outlasts kWaitTicks sets the XCD's error flag; once the flag is set
// every wait of that XCD returns at once (the forward's output is then invalid).
__device__ __forceinline__ void fused_wait(uint32_t* ctr, uint32_t target, uint32_t* line, uint32_t zero) {
    if (threadIdx.x == 0) {
        uint32_t* err = line + 1;
        if (ctr_read(ctr, zero) < target) {
            const uint64_t t0 = rt_now();
            uint32_t polls = 0;
            for (;;) {
                __builtin_amdgcn_s_sleep(8);
                if (ctr_read(ctr, zero) >= target) break;
                if ((++polls & 15u) == 0 && ctr_read(err, zero) != 0) break;
                if (rt_now() - t0 > kWaitTicks) {
                    __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
            __hip_atomic_fetch_add(line + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_max(line + 3, (uint32_t)(rt_now() - t0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

template <int LOG1, int LOG2>
struct FusedCfg {
    using Cfg = FsCfg<LOG1, LOG2>;
    static constexpr int NA = Cfg::L2 / Cfg::CB;              // pass A / C items per row
    static constexpr int NB = Cfg::L1 / 2 / Cfg::UNITS;       // pass B items per row
    static constexpr int THREADS = Cfg::COL_THREADS;
    static_assert(Cfg::COL_THREADS == Cfg::ROW_THREADS, "one block shape for all passes");
    static constexpr int LDS_A = Cfg::L1 * Cfg::CP;
    static constexpr int LDS_B = 2 * Cfg::UNITS * Cfg::RP;
    static constexpr int LDS = LDS_A > LDS_B ? LDS_A : LDS_B;
};

template <int LOG1, int LOG2, class TIO>
__global__ void __launch_bounds__((FusedCfg<LOG1, LOG2>::THREADS))
k_fs_fused(const TIO* __restrict__ u, const float* __restrict__ w3, const float2* __restrict__ spec,
           const float* __restrict__ bias, TIO* __restrict__ y, FsTables tb, FusedCtl* __restrict__ ctl,
           uint32_t* __restrict__ cnt, float2* __restrict__ ring, int D, int64_t nrows, int G, int S, int ngmax,
           uint32_t zero) {
    using F = FusedCfg<LOG1, LOG2>;
    constexpr int NA = F::NA, NB = F::NB;
    constexpr int64_t L = (int64_t)FsCfg<LOG1, LOG2>::L1 * FsCfg<LOG1, LOG2>::L2;
    __shared__ float2 lds[F::LDS];
    __shared__ uint32_t s_ticket;
    const uint32_t x = hw_xcc_id();
    const uint32_t nr = (uint32_t)nrows;
    const uint32_t nx = nr > x ? (nr - 1 - x) / 8 + 1 : 0;  // rows of this XCD
    const uint32_t ng = (nx + G - 1) / G;
    const uint32_t seg_a = G * NA, seg_b = G * NB, seg = 2 * seg_a + seg_b;
    const uint32_t total = (ng + 2) * seg;
    // per-XCD counters: A and B per local row, C per group
    uint32_t* cA = cnt + (size_t)x * (2 * (size_t)ngmax * G + ngmax + 64);
    uint32_t* cB = cA + (size_t)ngmax * G;
    uint32_t* cC = cB + (size_t)ngmax * G;
    float2* xring = ring + (size_t)x * S * G * L;
    const uint64_t kstart = rt_now();
    for (;;) {
        if (threadIdx.x == 0) {
            if (rt_now() - kstart > kKernelTicks) {
                __hip_atomic_fetch_or(&ctl->x[x][1], 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                s_ticket = 0xffffffffu;  // give up: no further tickets
            } else {
                s_ticket = __hip_atomic_fetch_add(&ctl->x[x][0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads();
        const uint32_t tk = __builtin_amdgcn_readfirstlane(s_ticket);
        __syncthreads();
        if (tk >= total) break;
        const uint32_t step = tk / seg;
        uint32_t rem = tk - step * seg;
        if (rem < seg_a) {  // pass A of group `step`
            const uint32_t j = step;
            if (j >= ng) continue;
            const uint32_t rl = rem / NA, sub = rem % NA;
            const uint32_t i = j * G + rl;
            if (j >= (uint32_t)S) fused_wait(cC + (j - S), seg_a, ctl->x[x], zero);
            if (i < nx) {
                float2* slot = xring + ((size_t)(j % S) * G + rl) * L;
                fs_colfwd_body<LOG1, LOG2, TIO, 0>(lds, u, w3, nullptr, slot, tb, D, 2, x + 8 * i, (int)sub);
                fused_signal(cA + i);
            }
        } else if (rem < seg_a + seg_b) {  // pass B of group step-1
            if (step < 1 || step - 1 >= ng) continue;
            const uint32_t j = step - 1;
            rem -= seg_a;
            const uint32_t rl = rem / NB, sub = rem % NB;
            const uint32_t i = j * G + rl;
            if (i >= nx) continue;
            fused_wait(cA + i, NA, ctl->x[x], zero);
            float2* slot = xring + ((size_t)(j % S) * G + rl) * L;
            fs_row_body<LOG1, LOG2, 0>(lds, slot, spec, bias, tb, D, 0, x + 8 * i, (int)sub);
            fused_signal(cB + i);
        } else {  // pass C of group step-2
            if (step < 2 || step - 2 >= ng) continue;
            const uint32_t j = step - 2;
            rem -= seg_a + seg_b;
            const uint32_t rl = rem / NA, sub = rem % NA;
            const uint32_t i = j * G + rl;
            if (i < nx) {
                fused_wait(cB + i, NB, ctl->x[x], zero);
                float2* slot = xring + ((size_t)(j % S) * G + rl) * L;
                fs_colinv_body<LOG1, LOG2, TIO, true>(lds, slot, u, w3, y, tb, D, 2, 0, x + 8 * i, (int)sub);
            }
            fused_signal(cC + j);
        }
    }
}

// zero the control block and counters (a fill kernel, so the forward can be
// captured in a graph)
__global__ void k_fill_u32(uint32_t* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}

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
                               const float2* wpair, hipStream_t st) {
    switch (logL) {
        case 4: return launch_lds_spectrum_t<4>(h, spec, rows, tw, wpair, st);
        case 5: return launch_lds_spectrum_t<5>(h, spec, rows, tw, wpair, st);
        case 6: return launch_lds_spectrum_t<6>(h, spec, rows, tw, wpair, st);
        case 7: return launch_lds_spectrum_t<7>(h, spec, rows, tw, wpair, st);
        case 8: return launch_lds_spectrum_t<8>(h, spec, rows, tw, wpair, st);
        case 9: return launch_lds_spectrum_t<9>(h, spec, rows, tw, wpair, st);
        case 10: return launch_lds_spectrum_t<10>(h, spec, rows, tw, wpair, st);
        case 11: return launch_lds_spectrum_t<11>(h, spec, rows, tw, wpair, st);
        case 12: return launch_lds_spectrum_t<12>(h, spec, rows, tw, wpair, st);
        case 13: return launch_lds_spectrum_t<13>(h, spec, rows, tw, wpair, st);
        case 14: return launch_lds_spectrum_t<14>(h, spec, rows, tw, wpair, st);
        default: return hipErrorInvalidValue;
    }
}

// Launches the passes of one chunk of rows. With `marks`, an event is recorded
// before the first launch and after every launch (1 + 2*(N-1) launches).
template <int LOG1, int LOG2>
static hipError_t fs_forward_chunk(const FsArgs& a, int64_t row0, int64_t nrows, hipStream_t st,
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
        hipLaunchKernelGGL((k_fs_colfwd<LOG1, LOG2, uint16_t, 0>), dim3(gcol), bcol, 0, st, (const uint16_t*)a.u,
                           a.w3, (const float*)nullptr, a.ws, a.tb, a.D, a.N, row0, nrows);
    else
        hipLaunchKernelGGL((k_fs_colfwd<LOG1, LOG2, float, 0>), dim3(gcol), bcol, 0, st, (const float*)a.u, a.w3,
                           (const float*)nullptr, a.ws, a.tb, a.D, a.N, row0, nrows);
    mark();
    for (int o = 0; o < a.N - 1; ++o) {
        hipLaunchKernelGGL((k_fs_row<LOG1, LOG2, 0>), dim3(grow), brow, 0, st, a.ws, a.spec, a.bias, a.tb, a.D, o,
                           row0, nrows);
        mark();
        const bool last = (o == a.N - 2);
        if (a.bf16) {
            if (last)
                hipLaunchKernelGGL((k_fs_colinv<LOG1, LOG2, uint16_t, true>), dim3(gcol), bcol, 0, st, a.ws,
                                   (const uint16_t*)a.u, a.w3, (uint16_t*)a.y, a.tb, a.D, a.N, o, row0, nrows);
            else
                hipLaunchKernelGGL((k_fs_colinv<LOG1, LOG2, uint16_t, false>), dim3(gcol), bcol, 0, st, a.ws,
                                   (const uint16_t*)a.u, a.w3, (uint16_t*)a.y, a.tb, a.D, a.N, o, row0, nrows);
        } else {
            if (last)
                hipLaunchKernelGGL((k_fs_colinv<LOG1, LOG2, float, true>), dim3(gcol), bcol, 0, st, a.ws,
                                   (const float*)a.u, a.w3, (float*)a.y, a.tb, a.D, a.N, o, row0, nrows);
            else
                hipLaunchKernelGGL((k_fs_colinv<LOG1, LOG2, float, false>), dim3(gcol), bcol, 0, st, a.ws,
                                   (const float*)a.u, a.w3, (float*)a.y, a.tb, a.D, a.N, o, row0, nrows);
        }
        mark();
    }
    return hipGetLastError();
}

template <int LOG1, int LOG2>
static hipError_t fs_spectrum_t(const float* h, float2* spec, int64_t rows, const FsTables& tb, hipStream_t st) {
    using Cfg = FsCfg<LOG1, LOG2>;
    const unsigned gcol = (unsigned)xcd_grid(rows, Cfg::L2 / Cfg::CB);
    const unsigned grow = (unsigned)xcd_grid(rows, Cfg::L1 / 2 / Cfg::UNITS);
    hipLaunchKernelGGL((k_fs_colfwd<LOG1, LOG2, float, 1>), dim3(gcol), dim3(Cfg::COL_THREADS), 0, st,
                       (const float*)nullptr, (const float*)nullptr, h, spec, tb, 1, 2, (int64_t)0, rows);
    hipLaunchKernelGGL((k_fs_row<LOG1, LOG2, 1>), dim3(grow), dim3(Cfg::ROW_THREADS), 0, st, spec,
                       (const float2*)nullptr, (const float*)nullptr, tb, 1, 0, (int64_t)0, rows);
    return hipGetLastError();
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

hipError_t launch_fs_spectrum(int logL, const float* h, float2* spec, int64_t rows, const FsTables& tb,
                              hipStream_t st) {
    switch (logL) {
#define X(LG, A, B) \
    case LG: return fs_spectrum_t<A, B>(h, spec, rows, tb, st);
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

namespace hy {

// ------------------------------------------------------ fused path launchers

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

static int64_t fused_ngmax(int64_t nrows, int G) { return ((nrows + 7) / 8 + G - 1) / G; }

static size_t fused_counter_words(int64_t nrows, int G) {
    const int64_t ngmax = fused_ngmax(nrows, G);
    return 8 * (size_t)(2 * ngmax * G + ngmax + 64);
}

size_t fused_workspace_bytes(int logL, int64_t nrows, int G, int S) {
    const size_t L = (size_t)1 << logL;
    return align256(sizeof(FusedCtl)) + align256(fused_counter_words(nrows, G) * 4) +
           (size_t)8 * S * G * L * sizeof(float2);
}

template <int LOG1, int LOG2>
static hipError_t fused_launch_t(const FsArgs& a, int64_t nrows, int G, int S, int blocks, hipStream_t st) {
    using F = FusedCfg<LOG1, LOG2>;
    char* base = (char*)a.ws;
    FusedCtl* ctl = (FusedCtl*)base;
    uint32_t* cnt = (uint32_t*)(base + align256(sizeof(FusedCtl)));
    float2* ring = (float2*)(base + align256(sizeof(FusedCtl)) + align256(fused_counter_words(nrows, G) * 4));
    const size_t nzero = (align256(sizeof(FusedCtl)) + align256(fused_counter_words(nrows, G) * 4)) / 4;
    hipLaunchKernelGGL(k_fill_u32, dim3(64), dim3(256), 0, st, (uint32_t*)base, nzero);
    const int ngmax = (int)fused_ngmax(nrows, G);
    if (a.bf16)
        hipLaunchKernelGGL((k_fs_fused<LOG1, LOG2, uint16_t>), dim3(blocks), dim3(F::THREADS), 0, st,
                           (const uint16_t*)a.u, a.w3, a.spec, a.bias, (uint16_t*)a.y, a.tb, ctl, cnt, ring, a.D,
                           nrows, G, S, ngmax, 0u);
    else
        hipLaunchKernelGGL((k_fs_fused<LOG1, LOG2, float>), dim3(blocks), dim3(F::THREADS), 0, st,
                           (const float*)a.u, a.w3, a.spec, a.bias, (float*)a.y, a.tb, ctl, cnt, ring, a.D, nrows, G,
                           S, ngmax, 0u);
    return hipGetLastError();
}

template <int LOG1, int LOG2>
static int fused_occupancy_t() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_fs_fused<LOG1, LOG2, float>, FusedCfg<LOG1, LOG2>::THREADS,
                                                     0) != hipSuccess)
        return 0;
    return n;
}

// The fused path is switched off: its first two runs on MI355X did not finish
// (the second one with every wait bounded in time), while a CPU emulation of the
// same ticket and counter logic completes for every tested shape. Until the cause
// is found it is only built for experiments (HY_EXPERIMENTAL_FUSED=1) and plans
// asking for it get HYENA_ERR_UNSUPPORTED.
bool fused_supported(int logL) { return HY_EXPERIMENTAL_FUSED && logL == 16; }

int fused_blocks_per_cu(int logL) {
#if HY_EXPERIMENTAL_FUSED
    if (logL == 16) return fused_occupancy_t<8, 8>();
#endif
    (void)logL;
    return 0;
}

hipError_t launch_fs_fused(int logL, const FsArgs& a, int64_t nrows, int G, int S, int blocks, hipStream_t st) {
#if HY_EXPERIMENTAL_FUSED
    if (logL == 16) return fused_launch_t<8, 8>(a, nrows, G, S, blocks, st);
#endif
    (void)logL; (void)a; (void)nrows; (void)G; (void)S; (void)blocks; (void)st;
    return hipErrorInvalidValue;
}

// byte offset of XCD x's error flag in the workspace
uint32_t fused_error_offset(int x) { return (uint32_t)(x * 128 + 4); }

}  // namespace hy
