// Partitioned path of the Hyena forward for gfx950: the same causal long
// convolution as the zero-padded 2L transform (HyenaDNA walkthrough, section 2.2,
// fftconv; the step chain of section 2.1), evaluated with the filter cut into
// P = L/Q blocks of Q taps (uniformly partitioned overlap-save):
//
//   y[iQ + tau] = sum_{k<P} sum_{s<Q} h[kQ + s] v[(i-k)Q + tau - s]      (v = 0 before 0)
//
// Window m of v holds the samples [(m-1)Q, (m+1)Q); X_m is its 2Q-point real
// spectrum and H_k the 2Q-point spectrum of filter block k zero-padded to 2Q.
// The circular convolution of window i-k with block k equals the linear one on
// the window's second half, so output block i is the second half of the
// inverse transform of Y_i = sum_{k<=i} H_k X_{i-k}. The bias skip term is the
// convolution with bias * delta, which lies in block 0: H_0 + bias. Every
// transform is 2Q real points carried as a Q-point complex transform of the
// packed samples, with the LDS path's packing, pair step and spectrum scale
// 1/(4Q); the filter block spectra are exactly the LDS path's spectra of
// Q-sample rows, so hyena_filter_spectrum reuses that kernel.
//
// Two launches per step, both LDS-resident:
//   pass 1 (k_part_fwd): one workgroup per (row, window): conv3 + gate on load
//     (or the previous step's gated output), forward transform, unpack, X_m out;
//   pass 2 (k_part_inv): one workgroup per (row, G consecutive output blocks):
//     the block-Toeplitz sums over the row's windows (each X_j and H_k read once
//     per workgroup, the H blocks kept in a register ring), repack, G inverse
//     transforms side by side, second halves kept, next gate (or the final gate).
// Per row and step this moves s*(2 or 1)*L (u or the previous output) + 8L (X
// out) + 8L (X in) + 8L (spectrum) + s*2L (gate in, output out) bytes: no
// transposed tile, 40L bytes at order 2 against 56L for the four-step passes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fft_core.hpp"
#include "kernels.hpp"
#include "pair.hpp"

namespace hy {
namespace {

// Every workgroup of a row lands on the XCD of that row (hardware deals
// workgroup i to XCD i mod 8), so the two windows that read each input block and
// the pass 2 workgroups that share a row's windows meet in one L2.
__device__ __forceinline__ bool part_row_map(int64_t bid, int64_t nrows, int per_row, int64_t& row, int& sub) {
    const int xcd = (int)(bid & 7);
    const int64_t s = bid >> 3;
    sub = (int)(s % per_row);
    row = (s / per_row) * 8 + xcd;
    return row < nrows;
}
constexpr int64_t part_grid(int64_t nrows, int per_row) { return ((nrows + 7) / 8) * 8 * per_row; }

// Pass 1. SRC 0: v = conv3(u[v channel]) * conv3(u[x_{N-1}]) from u_proj; SRC 1:
// the previous step's gated output, fp32 rows of L samples in `vb`.
template <int LOGQ, class TIO, int SRC>
__global__ void __launch_bounds__(LdsCfg<LOGQ>::THREADS)
k_part_fwd(const TIO* __restrict__ u, const float* __restrict__ w3, const float* __restrict__ vb,
           float2* __restrict__ X, const float2* __restrict__ tw, const float2* __restrict__ wpair, int D, int N,
           int P, int64_t row0, int64_t nrows) {
    constexpr int Q = 1 << LOGQ, E = LdsCfg<LOGQ>::E, T = Q / E, H = E / 2;
    __shared__ float2 lds[padded_len<Q>()];
    const RowAcc acc{lds};
    int64_t r;
    int m;
    if (!part_row_map(blockIdx.x, nrows, P, r, m)) return;
    const int t = threadIdx.x;
    const int64_t L = (int64_t)P * Q;
    // window pair j is pair (m-1)Q/2 + j of the row; window 0 starts with Q zeros
    const int64_t base = (int64_t)(m - 1) * (Q / 2);
    float2 v[E];
    if constexpr (SRC == 0) {
        const int64_t flat = row0 + r;
        const uint32_t b = (uint32_t)flat / (uint32_t)D, d = (uint32_t)flat - b * (uint32_t)D;
        const int64_t C = (int64_t)(N + 1) * D;
        const int64_t cv = (int64_t)N * D + d, cx = (int64_t)(N - 1) * D + d;
        const TIO* rv = u + ((int64_t)b * C + cv) * L;
        const TIO* rx = u + ((int64_t)b * C + cx) * L;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (m == 0 && e < H) v[e] = make_float2(0.f, 0.f);
            else v[e] = gated_pair(rv, rx, (uint32_t)(base + t + T * e), w3 + 3 * cv, w3 + 3 * cx);
        }
    } else {
        const float* vr = vb + r * L;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (m == 0 && e < H) v[e] = make_float2(0.f, 0.f);
            else v[e] = load_pair(vr, (uint32_t)(base + t + T * e));
        }
    }
    fft_strided<Q, false, false>(v, t, tw, acc);
    __syncthreads();
    lds_store_strided<T>(acc, t, v);
    __syncthreads();
    // 2A[k] and 2A[Q-k] of the window's 2Q-point spectrum; slot 0 holds the two
    // real bins (2A[0], 2A[Q]), the layout of the filter spectra
    float2* out = X + (r * P + m) * Q;
#pragma unroll
    for (int e = 0; e < H; ++e) {
        const uint32_t k = t + T * e;
        const uint32_t km = k == 0 ? 0 : Q - k;
        float2 Ak, Am;
        pair_unpack(acc[k], acc[km], wpair[k], Ak, Am);
        if (k == 0) {
            out[0] = make_float2(Ak.x, Am.x);
        } else {
            out[k] = Ak;
            out[km] = Am;
        }
    }
    if (t == 0) {
        const uint32_t k = Q / 2;
        float2 Ak, Am;
        const float2 Z = acc[k];
        pair_unpack(Z, Z, wpair[k], Ak, Am);
        out[k] = Ak;
    }
}

// Pass 2 for output blocks i0 .. i0+G-1 of one row. LAST: the final gate x_0 and
// y out; otherwise the next gate x_{N-2-o} and the gated result out to `vb`.
template <int LOGQ, int G, class TIO, bool LAST>
__global__ void __launch_bounds__(G * LdsCfg<LOGQ>::THREADS)
k_part_inv(const float2* __restrict__ X, const float2* __restrict__ spec, const float* __restrict__ bias,
           const TIO* __restrict__ u, const float* __restrict__ w3, TIO* __restrict__ y, float* __restrict__ vb,
           const float2* __restrict__ tw, const float2* __restrict__ wpair, int D, int N, int o, int P,
           int64_t sbs, int64_t row0, int64_t nrows) {
    constexpr int Q = 1 << LOGQ, E = LdsCfg<LOGQ>::E, T = Q / E, H = E / 2;
    constexpr int NT = G * T;   // threads
    constexpr int NQ = Q / NT;  // bins per thread in the block sums
    constexpr int PL = padded_len<Q>();
    __shared__ float2 lds[G * PL];
    int64_t r;
    int grp;
    if (!part_row_map(blockIdx.x, nrows, P / G, r, grp)) return;
    const int i0 = grp * G;
    const int64_t flat = row0 + r;
    const uint32_t b = (uint32_t)flat / (uint32_t)D, d = (uint32_t)flat - b * (uint32_t)D;
    const int64_t L = (int64_t)P * Q;
    const float2* Xr = X + r * L;
    const float2* Hr = spec + (int64_t)b * sbs + ((int64_t)o * D + d) * L;
    const float bs = bias[(int64_t)o * D + d] * (1.0f / (4.0f * (float)Q));
    const int tau = threadIdx.x;

    // ---- Y_{i0+g} = sum_j H_{i0+g-j} X_j on this thread's bins s = tau + NT*q.
    // Bin slot 0 holds two real bins, multiplied componentwise.
    const bool real0 = tau == 0;
    float2 acc[G][NQ], hr[G][NQ];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int q = 0; q < NQ; ++q) acc[g][q] = make_float2(0.f, 0.f);
    // ring: at step j, block k = i0+g-j sits in hr[(g - j) mod G]; preload k = i0+1 .. i0+G-1
#pragma unroll
    for (int g = 1; g < G; ++g)
#pragma unroll
        for (int q = 0; q < NQ; ++q) hr[g][q] = Hr[(uint32_t)((i0 + g) * Q + tau + NT * q)];
#pragma unroll 1
    for (int jb = 0; jb <= i0; jb += G) {
#pragma unroll
        for (int jj = 0; jj < G; ++jj) {
            const int j = jb + jj;
            const int knew = i0 - j;  // the one block not used before this step
            const int sn = (G - jj) % G;
            if (knew > 0) {
#pragma unroll
                for (int q = 0; q < NQ; ++q) hr[sn][q] = Hr[(uint32_t)(knew * Q + tau + NT * q)];
            } else if (knew == 0) {
                // block 0 carries the bias skip term
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const float2 h = Hr[(uint32_t)(tau + NT * q)];
                    hr[sn][q] = (q == 0 && real0) ? make_float2(h.x + bs, h.y + bs) : hadd(h, bs);
                }
            } else {
#pragma unroll
                for (int q = 0; q < NQ; ++q) hr[sn][q] = make_float2(0.f, 0.f);
            }
            float2 x[NQ];
#pragma unroll
            for (int q = 0; q < NQ; ++q) x[q] = Xr[(uint32_t)(j * Q + tau + NT * q)];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int si = (g - jj + G) % G;
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const float2 h = hr[si][q];
                    float2 p = cmul(h, x[q]);
                    if (q == 0) p = real0 ? emul(h, x[q]) : p;
                    acc[g][q] = cadd(acc[g][q], p);
                }
            }
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const RowAcc A{lds + g * PL};
#pragma unroll
        for (int q = 0; q < NQ; ++q) A[(uint32_t)(tau + NT * q)] = acc[g][q];
    }
    __syncthreads();

    // ---- per output block (T threads each): repack, inverse transform, second half
    const int g = tau / T, t = tau % T;
    const RowAcc A{lds + g * PL};
#pragma unroll
    for (int e = 0; e < H; ++e) {
        const uint32_t k = t + T * e;
        float2 Yk, Ym;
        if (k == 0) {
            const float2 C = A[0];
            pair_repack(make_float2(C.x, 0.f), make_float2(C.y, 0.f), make_float2(1.f, 0.f), Yk, Ym);
            A[0] = Yk;
        } else {
            const uint32_t km = Q - k;
            pair_repack(A[k], A[km], wpair[k], Yk, Ym);
            A[k] = Yk;
            A[km] = Ym;
        }
    }
    if (t == 0) {
        const uint32_t k = Q / 2;
        const float2 C = A[k];
        float2 Yk, Ym;
        pair_repack(C, C, wpair[k], Yk, Ym);
        A[k] = Yk;
    }
    __syncthreads();
    float2 v[E];
    lds_load_strided<T>(A, t, v);
    fft_strided<Q, true, false>(v, t, tw, A);
    // v[e], e >= E/2, holds output pair (i0+g)Q/2 + t + T(e - E/2) of the row
    const int64_t C = (int64_t)(N + 1) * D;
    const int64_t cg = (int64_t)(LAST ? 0 : N - 2 - o) * D + d;
    const TIO* rg = u + ((int64_t)b * C + cg) * L;
    const float* wg = w3 + 3 * cg;
    const uint32_t ob = (uint32_t)((i0 + g) * (Q / 2) + t);
#pragma unroll
    for (int e = H; e < E; ++e) {
        const uint32_t pi = ob + T * (e - H);
        const float2 val = emul(v[e], conv3_pair(rg, pi, wg[0], wg[1], wg[2]));
        if constexpr (LAST) store_pair(y + ((int64_t)b * D + d) * L, pi, val);
        else store_pair(vb + r * L, pi, val);
    }
}

template <int LOGQ, int G, class TIO>
void part_chunk_t(const PartArgs& a, int64_t row0, int64_t n, hipStream_t st, hipEvent_t* marks) {
    constexpr int T = LdsCfg<LOGQ>::THREADS;
    int mi = 0;
    auto mark = [&]() {
        if (marks) (void)hipEventRecord(marks[mi++], st);
    };
    const TIO* u = (const TIO*)a.u;
    const unsigned g1 = (unsigned)part_grid(n, a.P), g2 = (unsigned)part_grid(n, a.P / G);
    mark();
    for (int o = 0; o < a.N - 1; ++o) {
        if (o == 0)
            hipLaunchKernelGGL((k_part_fwd<LOGQ, TIO, 0>), dim3(g1), dim3(T), 0, st, u, a.w3, (const float*)nullptr,
                               a.X, a.tw, a.wpair, a.D, a.N, a.P, row0, n);
        else
            hipLaunchKernelGGL((k_part_fwd<LOGQ, TIO, 1>), dim3(g1), dim3(T), 0, st, u, a.w3,
                               (const float*)a.vb, a.X, a.tw, a.wpair, a.D, a.N, a.P, row0, n);
        mark();
        if (o == a.N - 2)
            hipLaunchKernelGGL((k_part_inv<LOGQ, G, TIO, true>), dim3(g2), dim3(G * T), 0, st, (const float2*)a.X,
                               a.spec, a.bias, u, a.w3, (TIO*)a.y, a.vb, a.tw, a.wpair, a.D, a.N, o, a.P, a.sbs,
                               row0, n);
        else
            hipLaunchKernelGGL((k_part_inv<LOGQ, G, TIO, false>), dim3(g2), dim3(G * T), 0, st, (const float2*)a.X,
                               a.spec, a.bias, u, a.w3, (TIO*)a.y, a.vb, a.tw, a.wpair, a.D, a.N, o, a.P, a.sbs,
                               row0, n);
        mark();
    }
}

template <int G>
void part_chunk_g(const PartArgs& a, int64_t row0, int64_t n, hipStream_t st, hipEvent_t* marks) {
    if (a.bf16) part_chunk_t<kPartLogQ, G, uint16_t>(a, row0, n, st, marks);
    else part_chunk_t<kPartLogQ, G, float>(a, row0, n, st, marks);
}

}  // namespace

int part_group(int P) { return P >= HY_PART_G ? HY_PART_G : 2; }

hipError_t launch_part_forward_chunk(const PartArgs& a, int64_t row0, int64_t n, hipStream_t st, hipEvent_t* marks) {
    if (a.P < 2 || (a.P & (a.P - 1)) != 0 || a.P > (1 << (kPartMaxLog - kPartLogQ))) return hipErrorInvalidValue;
    switch (part_group(a.P)) {
        case 2: part_chunk_g<2>(a, row0, n, st, marks); break;
        case 4: part_chunk_g<4>(a, row0, n, st, marks); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace hy
