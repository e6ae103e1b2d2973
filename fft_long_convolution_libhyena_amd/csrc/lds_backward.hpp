// Backward of the Hyena forward hot path on the LDS-resident path (L <= 16384),
// for gfx950. Explicit instantiations live in lds_backward_*.hip.
//
// The forward (HyenaDNA walkthrough, section 2.1, HyenaOperator.forward; section
// 2.2, HyenaFilter.forward and fftconv) is, per (b, d) row, with uc_i the short
// conv of channel i*D + d, x_i = uc_i (i < N) and v_0 = uc_N:
//   g_o = v_o * x_{N-1-o},  v_{o+1} = conv(g_o, h_o) + bias_o * g_o  (o = 0..N-2)
//   y   = v_{N-1} * x_0.
// Given dy, the chain rule gives (a = dv_{o+1} while step o is undone)
//   dv_{N-1} = dy * x_0,  dx_0 = dy * v_{N-1}
//   dh_o += corr(a, g_o),  dbias_o += <a, g_o> = corr(a, g_o)[0],  dg_o = corr(a, h_o) + bias_o * a
//   dx_{N-1-o} = dg_o * v_o,  dv_o = dg_o * x_{N-1-o}
//   du = conv3^T(duc),  dw_j += sum_t duc[t] u[t-2+j]
// with corr(a, k)[t] = sum_{s>=t} k[s-t] a[s], the adjoint of the causal
// convolution. In the frequency domain of the zero-padded 2L-point transform a
// correlation is a product with a conjugate spectrum: dg_o comes from
// A_dv * conj(H_o + bias_o) and dh_o from sum_b A_dv * conj(A_g).
//
// Circular plans (CIRC; the HyenaND summary's circular boundary handling): the
// rows hold 2L samples and the same L-point packed transform carries them with no
// zero half; conv and corr are then circular (corr(a, k)[t] = sum_s k[(s-t) mod 2L]
// a[s]), the same products with the same conjugate spectra, and every output of
// the inverse is kept. The short conv stays causal.
//
// Two kernels. k_lds_bwd_rows: one workgroup per (b, d) row (the B rows of a
// channel on one XCD, sharing its filter spectrum in L2) recomputes the forward
// chain on chip (2(N-1) transforms), undoes it (2(N-1) transforms), writes the
// N+1 rows of du and, per step, the product spectrum A_dv * conj(A_g) and the
// row's tap sums. k_lds_bwd_finish: one workgroup per (o, d) sums those over the
// batch in a fixed order and inverts the dh spectrum (dbias is its lag-0 value);
// no atomics, so results are reproducible bit for bit.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "backward.hpp"
#include "fft_core.hpp"
#include "kernels.hpp"
#include "pair.hpp"

namespace hy {

// The same pointer, made opaque to the optimiser by an empty asm statement (no
// instruction is emitted): loads through the result are neither hoisted out of the
// batch loop nor shared with an earlier phase, and values stored through one
// phase's copy are not forwarded to another phase's loads. Otherwise every
// twiddle, spectrum value, workspace value and re-read input row of the
// workgroup would be kept live in registers from one phase to the next.
template <class P>
__device__ __forceinline__ P* fresh(P* p) {
    uint32_t zero = 0;  // offsetting by an opaque zero keeps the global address space
    asm volatile("" : "+s"(zero));
    return p + zero;
}

// Scheduling fence between phases: keeps the loads of a later phase from being
// issued (and held in registers) across an earlier transform.
__device__ __forceinline__ void phase() { __builtin_amdgcn_sched_barrier(0); }

// The thread index, made opaque in the same way at the start of every phase: the
// LDS and global addresses derived from it are then computed where they are used
// instead of once for the whole kernel (dozens of them would stay live).
template <int T>
__device__ __forceinline__ int fresh_tid(int t) {
    asm volatile("" : "+v"(t));
    __builtin_assume(t >= 0 && t < T);
    return t;
}

// Materialises a running sum where it is written: without it the compiler sinks
// the arithmetic past the next transform and keeps all its inputs live there.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

// Filter spectrum (scaled) plus scaled bias at bins k and L-k; slot 0 of the
// stored spectrum holds the two real bins 0 and L.
__device__ __forceinline__ void spec_pair(const float2* __restrict__ Hs, uint32_t k, uint32_t km, float bs,
                                          float2& Hk, float2& Hm) {
    if (k == 0) {
        const float2 h0 = Hs[0];
        Hk = make_float2(h0.x + bs, 0.f);
        Hm = make_float2(h0.y + bs, 0.f);
    } else {
        Hk = hadd(Hs[k], bs);
        Hm = hadd(Hs[km], bs);
    }
}

// Input gradient through the short conv of one channel row:
// du[t] = w2 duc[t] + w1 duc[t+1] + w0 duc[t+2]. duc[e] holds the pair
// (duc[2m], duc[2m+1]) at m = t + T*e, e < LD (LD = E/2, or E for the 2L-sample
// rows of a circular plan); the pairs go through LDS (each thread then reads its
// own pair and the next one back, so duc need not stay live).
template <int L, int E, int LD, class TIO>
__device__ __forceinline__ void short_conv_back(const RowAcc& acc, int t, const float2 (&duc)[LD],
                                                const float* __restrict__ w, TIO* __restrict__ durow) {
    constexpr int T = L / E;
    constexpr uint32_t NP = (uint32_t)LD * T;  // pairs of the row
    phase();
    t = fresh_tid<T>(t);
    __syncthreads();  // the previous readers of LDS are done
#pragma unroll
    for (int e = 0; e < LD; ++e) acc[t + T * e] = duc[e];
    __syncthreads();
    phase();
    t = fresh_tid<T>(t);
    const float w0 = w[0], w1 = w[1], w2 = w[2];
#pragma unroll
    for (int e = 0; e < LD; ++e) {
        const uint32_t m = t + T * e;
        const float2 dc = acc[m];
        const float2 nx = (m + 1 < NP) ? acc[m + 1] : make_float2(0.f, 0.f);
        store_pair(durow, m, make_float2(fmaf(w2, dc.x, fmaf(w1, dc.y, w0 * nx.x)),
                                         fmaf(w2, dc.y, fmaf(w1, nx.x, w0 * nx.y))));
    }
}

// Raw samples (2m-2, 2m-1) and (2m, 2m+1) of a channel row.
template <class TIO>
__device__ __forceinline__ void raw_pairs(const TIO* __restrict__ row, uint32_t m, float2& prev, float2& cur) {
    cur = load_pair(row, m);
    prev = m > 0 ? load_pair(row, m - 1) : make_float2(0.f, 0.f);
}

// Tap gradients of the short conv: dw[j] += duc[2m] u[2m-2+j] + duc[2m+1] u[2m-1+j].
__device__ __forceinline__ void tap_sums(float2 dc, float2 prev, float2 cur, float (&dws)[3]) {
    dws[0] = fmaf(dc.x, prev.x, fmaf(dc.y, prev.y, dws[0]));
    dws[1] = fmaf(dc.x, prev.y, fmaf(dc.y, cur.x, dws[1]));
    dws[2] = fmaf(dc.x, cur.x, fmaf(dc.y, cur.y, dws[2]));
}

// Workspace layout in float2 units (see bwd_ws_bytes), rows r = b*D + d:
//   P  [B*D][N-1][L]   per-row product spectra A_dv * conj(A_g), laid out like the
//                      filter spectrum (slot 0 holds the real bins 0 and L)
//   G  [B*D][N-2][L]   unpacked spectra A_g of steps o < N-2 (the last step's stays
//                      in registers from the recomputed forward to its undoing)
//   V  [B*D][N-2][S/2] v_o of steps 1..N-2 as sample pairs (S = L, 2L circular)
//   TW [B][(N+1)*D][3] (floats) per-row tap sums of the short conv
// G and V are written and read back by the same thread.
template <int LOGL, int N, bool CIRC = false>
struct BwdWs {
    static constexpr int64_t L = int64_t(1) << LOGL;
    static constexpr int64_t P_ROW = (N - 1) * L;
    static constexpr int64_t G_ROW = (N - 2) * L;
    static constexpr int64_t V_ROW = (N - 2) * (CIRC ? L : L / 2);
};

template <int LOGL, int N, class TIO, bool CIRC = false>
__global__ void __launch_bounds__(LdsCfg<LOGL>::THREADS)
k_lds_bwd_rows(const TIO* __restrict__ u, const float* __restrict__ w3, const float2* __restrict__ spec,
               const float* __restrict__ bias, const TIO* __restrict__ dy, TIO* __restrict__ du,
               float2* __restrict__ ws, const float2* __restrict__ tw, const float2* __restrict__ wpair, int B,
               int D, int64_t sbs) {
    constexpr int L = 1 << LOGL;
    constexpr int E = LdsCfg<LOGL>::E;
    constexpr int H = E / 2;
    constexpr int T = L / E;
    constexpr int LD = CIRC ? E : H;                  // pairs of data per thread
    constexpr int64_t S = CIRC ? 2 * (int64_t)L : L;  // samples per row
    constexpr int NV = 3 * (N + 1);  // tap sums per thread
    static_assert(T * NV * 4 <= padded_len<L>() * 8, "reduction buffer fits in the transform's LDS");
    using W = BwdWs<LOGL, N, CIRC>;
    __shared__ float2 lds[padded_len<L>()];
    const RowAcc acc{lds};
    // as in the forward: consecutive workgroups go to different XCDs, and the B
    // rows of channel d to workgroups of one XCD, whose L2 then serves the filter
    // spectrum of d to all of them
    const int bid = blockIdx.x;
    const int xcd = bid & 7, sidx = bid >> 3;
    const int b = sidx % B;
    const int d = (sidx / B) * 8 + xcd;
    if (d >= D) return;
    int t = threadIdx.x;
    const int64_t C = (int64_t)(N + 1) * D;
    const int64_t r = (int64_t)b * D + d;
    const int64_t rows = (int64_t)B * D;
    float2* const Pr = ws + r * W::P_ROW;
    float2* const Gr = ws + rows * W::P_ROW + r * W::G_ROW;
    float2* const Vr = ws + rows * (W::P_ROW + W::G_ROW) + r * W::V_ROW;
    float* const TWb = reinterpret_cast<float*>(ws + rows * (W::P_ROW + W::G_ROW + W::V_ROW)) +
                       (int64_t)b * C * 3;
    const float bscale = 1.0f / (4.0f * (float)L);

    float dws[N + 1][3];
#pragma unroll
    for (int i = 0; i <= N; ++i) dws[i][0] = dws[i][1] = dws[i][2] = 0.f;

    const TIO* ub = u + (int64_t)b * C * S;
    const TIO* urow[N + 1];
#pragma unroll
    for (int i = 0; i <= N; ++i) urow[i] = ub + ((int64_t)i * D + d) * S;
    const float* wN = w3 + 3 * ((int64_t)N * D + d);

    // -------------------------------------------------- forward chain, recomputed
    float2 v[LD];
#pragma unroll
    for (int e = 0; e < LD; ++e) v[e] = conv3_pair(urow[N], (uint32_t)(t + T * e), wN[0], wN[1], wN[2]);
    float2 ga[H], gb[H];  // A_g at k and L-k of the last step
    float2 gh = make_float2(0.f, 0.f);
#pragma unroll
    for (int o = 0; o < N - 1; ++o) {
        phase();
        t = fresh_tid<T>(t);
        const int gi = N - 1 - o;
        const float* wg = w3 + 3 * ((int64_t)gi * D + d);
        if (o >= 1) {
            float2* Vw = fresh(Vr) + (int64_t)(o - 1) * (S / 2);
#pragma unroll
            for (int e = 0; e < LD; ++e) Vw[t + T * e] = v[e];
        }
        float2 f[E];
        const TIO* xr = fresh(urow[gi]);
#pragma unroll
        for (int e = 0; e < LD; ++e) f[e] = emul(v[e], conv3_pair(xr, (uint32_t)(t + T * e), wg[0], wg[1], wg[2]));
#pragma unroll
        for (int e = LD; e < E; ++e) f[e] = make_float2(0.f, 0.f);
        phase();
        fft_strided<L, false, !CIRC>(f, t, fresh(tw), acc);
        phase();
        t = fresh_tid<T>(t);
        __syncthreads();
        lds_store_strided<T>(acc, t, f);
        __syncthreads();
        const float2* Hs = fresh(spec) + (int64_t)b * sbs + ((int64_t)o * D + d) * L;
        const float2* wp = fresh(wpair);
        const float bs = bias[(int64_t)o * D + d] * bscale;
        float2* Gw = fresh(Gr) + (int64_t)o * L;
#pragma unroll
        for (int e = 0; e < H; ++e) {
            const uint32_t k = t + T * e;
            const uint32_t km = k == 0 ? 0 : L - k;
            float2 Ak, Am, Hk, Hm, Yk, Ym;
            const float2 wk = wp[k];
            pair_unpack(acc[k], acc[km], wk, Ak, Am);
            spec_pair(Hs, k, km, bs, Hk, Hm);
            pair_repack(cmul(Ak, Hk), cmul(Am, Hm), wk, Yk, Ym);
            acc[k] = Yk;
            if (k != 0) acc[km] = Ym;
            if (o == N - 2) {
                ga[e] = Ak;
                gb[e] = Am;
            } else if (k != 0) {
                Gw[k] = Ak;
                Gw[km] = Am;
            } else {
                Gw[0] = make_float2(Ak.x, Am.x);  // bins 0 and L are real
            }
        }
        if (t == 0) {  // k = L/2 pairs with itself
            const uint32_t k = L / 2;
            float2 A, Am, Y, Yd;
            pair_unpack(acc[k], acc[k], wp[k], A, Am);
            const float2 Hh = hadd(Hs[k], bs);
            pair_repack(cmul(A, Hh), cmul(A, Hh), wp[k], Y, Yd);
            acc[k] = Y;
            if (o == N - 2) gh = A;
            else Gw[k] = A;
        }
        __syncthreads();
        lds_load_strided<T>(acc, t, f);
        phase();
        fft_strided<L, true, false>(f, t, fresh(tw), acc);
        phase();
        t = fresh_tid<T>(t);
#pragma unroll
        for (int e = 0; e < LD; ++e) v[e] = f[e];  // v_{o+1}
    }

    // ------------------------------------------------------------------ backward
    float2 a[LD], dx[LD];
    {
        const TIO* dyr = dy + r * S;
        const float* w0p = w3 + 3 * (int64_t)d;
        const TIO* x0r = fresh(urow[0]);
#pragma unroll
        for (int e = 0; e < LD; ++e) {
            const uint32_t m = t + T * e;
            const float2 g = load_pair(dyr, m);
            float2 prev, cur;
            raw_pairs(x0r, m, prev, cur);
            a[e] = emul(g, conv3_from(prev, cur, w0p[0], w0p[1], w0p[2]));
            dx[e] = emul(g, v[e]);
            tap_sums(dx[e], prev, cur, dws[0]);
        }
        pin(dws[0][0]);
        pin(dws[0][1]);
        pin(dws[0][2]);
        short_conv_back<L, E>(acc, t, dx, w0p, du + ((int64_t)b * C + d) * S);
    }
#pragma unroll
    for (int o = N - 2; o >= 0; --o) {
        phase();
        t = fresh_tid<T>(t);
        const int gi = N - 1 - o;
        const float* wg = w3 + 3 * ((int64_t)gi * D + d);
        float2 f[E];
#pragma unroll
        for (int e = 0; e < LD; ++e) f[e] = a[e];
#pragma unroll
        for (int e = LD; e < E; ++e) f[e] = make_float2(0.f, 0.f);
        phase();
        fft_strided<L, false, !CIRC>(f, t, fresh(tw), acc);
        phase();
        t = fresh_tid<T>(t);
        __syncthreads();
        lds_store_strided<T>(acc, t, f);
        __syncthreads();
        const float2* Hs = fresh(spec) + (int64_t)b * sbs + ((int64_t)o * D + d) * L;
        const float2* wp = fresh(wpair);
        const float bs = bias[(int64_t)o * D + d] * bscale;
        const float2* Gw = fresh(Gr) + (int64_t)o * L;
        float2* Pw = fresh(Pr) + (int64_t)o * L;
#pragma unroll
        for (int e = 0; e < H; ++e) {
            const uint32_t k = t + T * e;
            const uint32_t km = k == 0 ? 0 : L - k;
            float2 Ak, Am, Hk, Hm, Yk, Ym, Gk, Gm;
            const float2 wk = wp[k];
            pair_unpack(acc[k], acc[km], wk, Ak, Am);
            if (o == N - 2) {
                Gk = ga[e];
                Gm = gb[e];
            } else if (k != 0) {
                Gk = Gw[k];
                Gm = Gw[km];
            } else {
                const float2 g0 = Gw[0];
                Gk = make_float2(g0.x, 0.f);
                Gm = make_float2(g0.y, 0.f);
            }
            const float2 Pk = cmulc(Ak, Gk), Pm = cmulc(Am, Gm);
            if (k != 0) {
                Pw[k] = Pk;
                Pw[km] = Pm;
            } else {
                Pw[0] = make_float2(Pk.x, Pm.x);
            }
            spec_pair(Hs, k, km, bs, Hk, Hm);
            pair_repack(cmulc(Ak, Hk), cmulc(Am, Hm), wk, Yk, Ym);
            acc[k] = Yk;
            if (k != 0) acc[km] = Ym;
        }
        if (t == 0) {
            const uint32_t k = L / 2;
            float2 A, Am, Y, Yd;
            pair_unpack(acc[k], acc[k], wp[k], A, Am);
            Pw[k] = cmulc(A, o == N - 2 ? gh : Gw[k]);
            const float2 Hh = hadd(Hs[k], bs);
            pair_repack(cmulc(A, Hh), cmulc(A, Hh), wp[k], Y, Yd);
            acc[k] = Y;
        }
        __syncthreads();
        lds_load_strided<T>(acc, t, f);
        phase();
        fft_strided<L, true, false>(f, t, fresh(tw), acc);
        phase();
        t = fresh_tid<T>(t);
        // v_o and the gate x_{N-1-o} are fetched again here rather than held
        // across the transforms; their raw samples also give the tap sums
        {
            const TIO* vr = fresh(urow[N]);
            const TIO* xr = fresh(urow[gi]);
            const float2* Vw = fresh(Vr) + (int64_t)(o - 1) * (S / 2);
#pragma unroll
            for (int e = 0; e < LD; ++e) {
                const uint32_t m = t + T * e;
                float2 xp, xc;
                raw_pairs(xr, m, xp, xc);
                if (o == 0) {
                    float2 vp, vc;
                    raw_pairs(vr, m, vp, vc);
                    dx[e] = emul(f[e], conv3_from(vp, vc, wN[0], wN[1], wN[2]));  // dg * v_0
                    a[e] = emul(f[e], conv3_from(xp, xc, wg[0], wg[1], wg[2]));   // dv_0
                    tap_sums(a[e], vp, vc, dws[N]);
                } else {
                    dx[e] = emul(f[e], Vw[m]);                                  // dg * v_o
                    a[e] = emul(f[e], conv3_from(xp, xc, wg[0], wg[1], wg[2]));  // dv_o
                }
                tap_sums(dx[e], xp, xc, dws[gi]);
            }
            pin(dws[gi][0]);
            pin(dws[gi][1]);
            pin(dws[gi][2]);
            if (o == 0) {
                pin(dws[N][0]);
                pin(dws[N][1]);
                pin(dws[N][2]);
            }
        }
        short_conv_back<L, E>(acc, t, dx, wg, du + ((int64_t)b * C + (int64_t)gi * D + d) * S);
    }
    short_conv_back<L, E>(acc, t, a, wN, du + ((int64_t)b * C + (int64_t)N * D + d) * S);

    // ------------------------------------------- this row's tap sums, per channel
    float* red = reinterpret_cast<float*>(lds);
    __syncthreads();
#pragma unroll
    for (int i = 0; i <= N; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j) red[(3 * i + j) * T + t] = dws[i][j];
    __syncthreads();
    for (int q = t; q < NV; q += T) {
        float sum = 0.f;
        for (int k = 0; k < T; ++k) sum += red[q * T + k];
        TWb[((int64_t)(q / 3) * D + d) * 3 + (q % 3)] = sum;
    }
}

// Sums over the batch: dh[o][d] and dbias[o][d] from the product spectra, and
// (by the o = 0 workgroups) dshort_w of the N+1 channels of d from the row tap sums.
// PER_SAMPLE (a filter set per sample): one workgroup per (b, o, d) inverts sample
// b's product spectrum alone into dh[b][o][d]; dbias is left to k_lds_bwd_dbias.
template <int LOGL, int N, bool PER_SAMPLE, bool CIRC = false>
__global__ void __launch_bounds__(LdsCfg<LOGL>::THREADS)
k_lds_bwd_finish(const float2* __restrict__ ws, float* __restrict__ dw, float* __restrict__ dh,
                 float* __restrict__ dbias, const float2* __restrict__ tw, const float2* __restrict__ wpair, int B,
                 int D) {
    constexpr int L = 1 << LOGL;
    constexpr int E = LdsCfg<LOGL>::E;
    constexpr int H = E / 2;
    constexpr int T = L / E;
    constexpr int LD = CIRC ? E : H;                  // pairs of dh per thread
    constexpr int64_t S = CIRC ? 2 * (int64_t)L : L;  // taps per filter
    using W = BwdWs<LOGL, N, CIRC>;
    __shared__ float2 lds[padded_len<L>()];
    const RowAcc acc{lds};
    const int nod = (N - 1) * D;
    const int bs = PER_SAMPLE ? (int)(blockIdx.x / nod) : 0;  // the sample whose dh this is
    const int od = PER_SAMPLE ? (int)(blockIdx.x % nod) : (int)blockIdx.x;
    const int o = od / D, d = od % D;
    const int t = threadIdx.x;
    const int64_t rows = (int64_t)B * D;
    const int b_lo = PER_SAMPLE ? bs : 0, b_hi = PER_SAMPLE ? bs + 1 : B;
    // repack + the unnormalised L-point inverse of X gives the 2L-point inverse of
    // 2L*X; the products carry the factor 4 of the unpacked values: X = P / (8L)
    const float sc = 1.0f / (8.0f * (float)L);
    // the sum over the samples, each sample's values of this thread loaded together
    float2 Ck[H], Cm[H];
#pragma unroll
    for (int e = 0; e < H; ++e) Ck[e] = Cm[e] = make_float2(0.f, 0.f);
    for (int b = b_lo; b < b_hi; ++b) {
        const float2* Pw = ws + ((int64_t)b * D + d) * W::P_ROW + (int64_t)o * L;
#pragma unroll
        for (int e = 0; e < H; ++e) {
            const uint32_t k = t + T * e;
            Ck[e] = cadd(Ck[e], Pw[k]);
            if (k != 0) Cm[e] = cadd(Cm[e], Pw[L - k]);
        }
    }
#pragma unroll
    for (int e = 0; e < H; ++e) {
        const uint32_t k = t + T * e;
        const uint32_t km = k == 0 ? 0 : L - k;
        float2 Yk, Ym;
        if (k != 0) {
            pair_repack(fmul2(Ck[e], sc), fmul2(Cm[e], sc), wpair[k], Yk, Ym);
        } else {
            // slot 0 holds the real bins 0 and L
            pair_repack(make_float2(Ck[e].x * sc, 0.f), make_float2(Ck[e].y * sc, 0.f), wpair[0], Yk, Ym);
        }
        acc[k] = Yk;
        if (k != 0) acc[km] = Ym;
    }
    if (t == 0) {
        const uint32_t k = L / 2;
        float2 P = make_float2(0.f, 0.f);
        for (int b = b_lo; b < b_hi; ++b) P = cadd(P, ws[((int64_t)b * D + d) * W::P_ROW + (int64_t)o * L + k]);
        P = fmul2(P, sc);
        float2 Y, Yd;
        pair_repack(P, P, wpair[k], Y, Yd);
        acc[k] = Y;
    }
    __syncthreads();
    float2 f[E];
    lds_load_strided<T>(acc, t, f);
    fft_strided<L, true, false>(f, t, tw, acc);
    // shared filters: dh[o][d]; per sample: dh[b][o][d]
    float* dhr = dh + ((int64_t)bs * nod + od) * S;
#pragma unroll
    for (int e = 0; e < LD; ++e) store_pair(dhr, (uint32_t)(t + T * e), f[e]);
    // the bias gradient sum_b sum_t dv[t] g[t] is the lag-0 value of the same
    // correlation that gives dh
    if (!PER_SAMPLE && t == 0) dbias[od] = f[0].x;
    if (o == 0 && bs == 0) {
        const float* TW = reinterpret_cast<const float*>(ws + rows * (W::P_ROW + W::G_ROW + W::V_ROW));
        const int64_t C = (int64_t)(N + 1) * D;
        for (int q = t; q < 3 * (N + 1); q += T) {
            const int64_t idx = ((int64_t)(q / 3) * D + d) * 3 + (q % 3);
            float sum = 0.f;
            for (int b = 0; b < B; ++b) sum += TW[(int64_t)b * C * 3 + idx];
            dw[idx] = sum;
        }
    }
}

// With a filter set per sample: dbias[o][d] = sum over b (in order) of the lag-0
// values dh[b][o][d][0], each sample's share of the shared bias's gradient.
// (dh rows of S taps: L, or 2L for a circular plan)
template <int LOGL, bool CIRC>
__global__ void k_lds_bwd_dbias(const float* __restrict__ dh, float* __restrict__ dbias, int B, int nod) {
    constexpr int64_t S = (int64_t(1) << LOGL) * (CIRC ? 2 : 1);
    const int od = blockIdx.x * blockDim.x + threadIdx.x;
    if (od >= nod) return;
    float s = 0.f;
    for (int b = 0; b < B; ++b) s += dh[((int64_t)b * nod + od) * S];
    dbias[od] = s;
}

template <int LOGL, int N, bool CIRC>
inline void launch_lds_backward_c(const LdsBwdArgs& a, hipStream_t st) {
    constexpr int T = LdsCfg<LOGL>::THREADS;
    const unsigned grid = (unsigned)(a.B * 8 * ((a.D + 7) / 8));
    if (a.bf16)
        hipLaunchKernelGGL((k_lds_bwd_rows<LOGL, N, uint16_t, CIRC>), dim3(grid), dim3(T), 0, st,
                           (const uint16_t*)a.u, a.w3, a.spec, a.bias, (const uint16_t*)a.dy, (uint16_t*)a.du, a.ws,
                           a.tw, a.wpair, a.B, a.D, a.sbs);
    else
        hipLaunchKernelGGL((k_lds_bwd_rows<LOGL, N, float, CIRC>), dim3(grid), dim3(T), 0, st, (const float*)a.u,
                           a.w3, a.spec, a.bias, (const float*)a.dy, (float*)a.du, a.ws, a.tw, a.wpair, a.B, a.D,
                           a.sbs);
    if (a.per_sample) {
        const int nod = (N - 1) * a.D;
        hipLaunchKernelGGL((k_lds_bwd_finish<LOGL, N, true, CIRC>), dim3((unsigned)(a.B * nod)), dim3(T), 0, st,
                           (const float2*)a.ws, a.dw, a.dh, a.dbias, a.tw, a.wpair, a.B, a.D);
        hipLaunchKernelGGL((k_lds_bwd_dbias<LOGL, CIRC>), dim3((unsigned)((nod + 255) / 256)), dim3(256), 0, st,
                           (const float*)a.dh, a.dbias, a.B, nod);
    } else
        hipLaunchKernelGGL((k_lds_bwd_finish<LOGL, N, false, CIRC>), dim3((unsigned)((N - 1) * a.D)), dim3(T), 0,
                           st, (const float2*)a.ws, a.dw, a.dh, a.dbias, a.tw, a.wpair, a.B, a.D);
}

template <int LOGL, int N>
inline void launch_lds_backward_n(const LdsBwdArgs& a, hipStream_t st) {
    if (a.circ)
        launch_lds_backward_c<LOGL, N, true>(a, st);
    else
        launch_lds_backward_c<LOGL, N, false>(a, st);
}

template <int LOGL>
hipError_t launch_lds_backward_t(const LdsBwdArgs& a, hipStream_t st) {
    switch (a.N) {
        case 2: launch_lds_backward_n<LOGL, 2>(a, st); break;
        case 3: launch_lds_backward_n<LOGL, 3>(a, st); break;
        case 4: launch_lds_backward_n<LOGL, 4>(a, st); break;
        case 5: launch_lds_backward_n<LOGL, 5>(a, st); break;
        case 6: launch_lds_backward_n<LOGL, 6>(a, st); break;
        case 7: launch_lds_backward_n<LOGL, 7>(a, st); break;
        case 8: launch_lds_backward_n<LOGL, 8>(a, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace hy
