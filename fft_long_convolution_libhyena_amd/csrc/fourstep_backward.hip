// Backward of the hot path on the four-step sizes (L = L1 * L2 > 16384 by
// default), for gfx950, any order N. The chain rule is the one of
// lds_backward.hpp (HyenaDNA walkthrough, section 2.1, HyenaOperator.forward;
// section 2.2, fftconv): with g_o = v_o * x_{N-1-o} and
// v_{o+1} = conv(g_o, h_o) + bias_o * g_o,
//   dv_{N-1} = dy * x_0,  dx_0 = dy * v_{N-1},  and for o = N-2 .. 0:
//   dg_o = corr(dv_{o+1}, h_o) + bias_o * dv_{o+1},  dh_o = sum_b corr(dv_{o+1}, g_o),
//   dbias_o = dh_o[0],  dx_{N-1-o} = dg_o * v_o,  dv_o = dg_o * x_{N-1-o},
// then the short conv's transpose and tap sums for the N+1 channels. corr is taken
// through the same zero-padded spectra with conj(H + bias).
//
// Launches over all B*D rows (each row's tiles live in the workspace):
//  pass A of g_0 -> G_0; for o = 0 .. N-2: pass B mode 2 (rows of G_o, multiply,
//  inverse rows) -> T, G_o kept, then a column pass: MID (v_{o+1} -> V, the next
//  gated input by columns -> G_{o+1}) or, after the last step, HEAD (dx_0 -> S_0,
//  dv_{N-1} by columns -> T);
//  for o = N-2 .. 0: pass B mode 3 (conj(H + bias), inverse rows -> T; A_{g_o} from
//  the rows of G_o, the product A_dv conj(A_{g_o}) through the same inverse rows ->
//  the row's dh tile); dh_o by
//  columns from the fixed-order sum of a channel's dh tiles over the batch (dbias_o
//  its lag-0 value); then TAILMID (dx_{N-1-o} -> S, dv_o by columns -> T) or, at
//  o = 0, TAIL0 (dx_{N-1} and dv_0 -> S);
//  du = conv3^T of the N+1 staged channels; dshort_w from the tap sums.
// Every sum over the batch or over workgroups is taken in a fixed order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "backward.hpp"
#include "fft_core.hpp"
#include "fourstep.hpp"
#include "kernels.hpp"
#include "pair.hpp"

namespace hy {

namespace {

// Tap gradients of the short conv: dw[j] += duc[2m] u[2m-2+j] + duc[2m+1] u[2m-1+j].
__device__ __forceinline__ void fs_tap_sums(float2 dc, float2 prev, float2 cur, float (&s)[3]) {
    s[0] = fmaf(dc.x, prev.x, fmaf(dc.y, prev.y, s[0]));
    s[1] = fmaf(dc.x, prev.y, fmaf(dc.y, cur.x, s[1]));
    s[2] = fmaf(dc.x, cur.x, fmaf(dc.y, cur.y, s[2]));
}

template <class TIO>
__device__ __forceinline__ void fs_raw_pairs(const TIO* __restrict__ row, uint32_t m, float2& prev, float2& cur) {
    cur = load_pair(row, m);
    prev = m > 0 ? load_pair(row, m - 1) : make_float2(0.f, 0.f);
}

}  // namespace

// Pass B of step o on the tile T and the kept column-transformed gated input G_o:
// MODE 2 (forward recompute) transforms G_o and writes the inverse rows to T;
// MODE 3 (the adjoint) transforms T (dv), applies conj(H_o + bias_o), and takes the
// dh product with A_g, the rows of G_o transformed again, into P; both invert the
// rows in T.
template <int LOG1, int LOG2, int MODE>
__global__ void __launch_bounds__((FsCfg<LOG1, LOG2>::ROW_THREADS))
k_fs_row_bwd(float2* __restrict__ T, const float2* __restrict__ spec, const float* __restrict__ bias,
             float2* __restrict__ G, float2* __restrict__ P, FsTables tb, int D, int o, int64_t nrows, int64_t sbs) {
    using Cfg = FsCfg<LOG1, LOG2>;
    __shared__ float2 lds[2 * Cfg::UNITS * Cfg::RP];
    int64_t r;
    int ug;
    if (!xcd_row_map(blockIdx.x, nrows, Cfg::L1 / 2 / Cfg::UNITS, r, ug)) return;
    const int64_t L = (int64_t)Cfg::L1 * Cfg::L2;
    float2* trow = T + r * L;
    float2* grow = G + ((int64_t)o * nrows + r) * L;
    if constexpr (MODE == 2)
        fs_row_body<LOG1, LOG2, MODE>(lds, grow, spec, bias, tb, D, o, r, ug, trow, nullptr, sbs);
    else
        fs_row_body<LOG1, LOG2, MODE>(lds, trow, spec, bias, tb, D, o, r, ug, grow, P + r * L, sbs);
}

// Column passes of the backward (inverse columns of the tile first, then):
//  MID (forward recompute after step o < N-2): v_{o+1} is stored in V_{o+1};
//      g_{o+1} = v_{o+1} * x_{N-2-o} is transformed by columns into G_{o+1} (Tout).
//  HEAD (after the last step): with dy and x_0, dx_0 = dy * v_{N-1} goes to S_0 and
//      dv_{N-1} = dy * x_0 is transformed by columns back into the tile.
//  TAILMID (step o >= 1 of the adjoint): the columns give dg_o; with a = N-1-o,
//      dx_a = dg_o * v_o (v_o from V_o) goes to S_a and dv_o = dg_o * x_a is
//      transformed by columns back into the tile.
//  TAIL0 (step 0): dx_{N-1} = dg_0 * v_0 goes to S_{N-1} and dv_0 = dg_0 * x_{N-1}
//      to S_N (v_0 and x_{N-1} by the short conv of their raw rows).
// Every pass that finishes a channel adds its tap sums into
// part[row][column block][channel][tap].
constexpr int kColMid = 0, kColHead = 1, kColTailMid = 2, kColTail0 = 3;

template <int LOG1, int LOG2, class TIO, int KIND>
__global__ void __launch_bounds__((FsCfg<LOG1, LOG2>::COL_THREADS))
k_fs_colinv_bwd(const float2* __restrict__ T, float2* __restrict__ Tout, const TIO* __restrict__ u,
                const float* __restrict__ w3,
                const TIO* __restrict__ dy, float* __restrict__ S, float* __restrict__ V, float* __restrict__ part,
                FsTables tb, int D, int N, int o, int64_t nrows) {
    using Cfg = FsCfg<LOG1, LOG2>;
    constexpr int L1 = Cfg::L1, L2 = Cfg::L2, T1 = Cfg::T1, CB = Cfg::CB, NCB = L2 / CB;
    constexpr int NT = Cfg::COL_THREADS;
    constexpr int64_t L = (int64_t)L1 * L2;
    __shared__ float2 lds[L1 * Cfg::CP];
    int64_t r;
    int cb;
    if (!xcd_row_map(blockIdx.x, nrows, NCB, r, cb)) return;
    const uint32_t b = (uint32_t)r / (uint32_t)D, d = (uint32_t)r - b * (uint32_t)D;
    const int64_t C = (int64_t)(N + 1) * D;
    const int c = threadIdx.x % CB, t = threadIdx.x / CB;
    const int m2 = cb * CB + c;
    const ColAcc<Cfg::CP> cacc{lds + c};
    const float2* slot = T + r * L;
    float2* oslot = Tout + r * L;  // the refill's tile (T itself except for MID)
    float2 v[16];
    const float2 base = twiddle_base<L2>(tb, t, m2);
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = cmulc(slot[(uint32_t)(t + T1 * e) * L2 + m2], twiddle_step<L2>(tb, base, e, m2));
    fft_strided<L1, true, false>(v, t, tb.tw1, cacc);
    float* Sr = S + r * (N + 1) * L;  // staging rows of the N+1 channels (time domain, fp32)
    auto chan = [&](int i) { return u + ((int64_t)b * C + (int64_t)i * D + d) * L; };
    auto taps = [&](int i) { return w3 + 3 * ((int64_t)i * D + d); };
    float s0[3] = {0.f, 0.f, 0.f}, s1[3] = {0.f, 0.f, 0.f};
    int ch0 = 0;  // channel of s0 (s1 is channel N, TAIL0 only)
    bool refill = true;
    if constexpr (KIND == kColMid) {
        const int a = N - 2 - o;
        const TIO* xr = chan(a);
        const float* wx = taps(a);
        float* Vr = V + ((int64_t)o * nrows + r) * L;  // V_{o+1} at slot o
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t m = (uint32_t)(t + T1 * e) * L2 + m2;
            store_pair(Vr, m, v[e]);
            v[e] = emul(v[e], conv3_pair(xr, m, wx[0], wx[1], wx[2]));
        }
    } else if constexpr (KIND == kColHead) {
        const TIO* dyr = dy + r * L;
        const TIO* x0r = chan(0);
        const float* wx = taps(0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t m = (uint32_t)(t + T1 * e) * L2 + m2;
            const float2 g = load_pair(dyr, m);
            float2 prev, cur;
            fs_raw_pairs(x0r, m, prev, cur);
            const float2 dx = emul(g, v[e]);  // dy * v_{N-1}
            store_pair(Sr, m, dx);
            fs_tap_sums(dx, prev, cur, s0);
            v[e] = emul(g, conv3_from(prev, cur, wx[0], wx[1], wx[2]));  // dv_{N-1} = dy * x_0
        }
    } else if constexpr (KIND == kColTailMid) {
        const int a = N - 1 - o;
        ch0 = a;
        const TIO* xr = chan(a);
        const float* wx = taps(a);
        const float* Vr = V + ((int64_t)(o - 1) * nrows + r) * L;  // v_o
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t m = (uint32_t)(t + T1 * e) * L2 + m2;
            float2 xp, xc;
            fs_raw_pairs(xr, m, xp, xc);
            const float2 dx = emul(v[e], load_pair(Vr, m));  // dg_o * v_o
            store_pair(Sr + (int64_t)a * L, m, dx);
            fs_tap_sums(dx, xp, xc, s0);
            v[e] = emul(v[e], conv3_from(xp, xc, wx[0], wx[1], wx[2]));  // dv_o = dg_o * x_a
        }
    } else {
        refill = false;
        ch0 = N - 1;
        const TIO* x1r = chan(N - 1);
        const TIO* vr = chan(N);
        const float* wx = taps(N - 1);
        const float* wv = taps(N);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t m = (uint32_t)(t + T1 * e) * L2 + m2;
            float2 xp, xc, vp, vc;
            fs_raw_pairs(x1r, m, xp, xc);
            fs_raw_pairs(vr, m, vp, vc);
            const float2 dx1 = emul(v[e], conv3_from(vp, vc, wv[0], wv[1], wv[2]));  // dg_0 * v_0
            const float2 dv0 = emul(v[e], conv3_from(xp, xc, wx[0], wx[1], wx[2]));  // dg_0 * x_{N-1}
            store_pair(Sr + (int64_t)(N - 1) * L, m, dx1);
            store_pair(Sr + (int64_t)N * L, m, dv0);
            fs_tap_sums(dx1, xp, xc, s0);
            fs_tap_sums(dv0, vp, vc, s1);
        }
    }
    if (refill) {  // (uniform) the next transform's input goes back into the tile
#pragma unroll
        for (int e = 8; e < 16; ++e) v[e] = make_float2(0.f, 0.f);
        fft_strided<L1, false, true>(v, t, tb.tw1, cacc);
#pragma unroll
        for (int e = 0; e < 16; ++e)
            oslot[(uint32_t)(t + T1 * e) * L2 + m2] = cmul(v[e], twiddle_step<L2>(tb, base, e, m2));
    }
    if constexpr (KIND == kColMid) return;
    // this workgroup's tap sums
    constexpr int NQ = KIND == kColTail0 ? 6 : 3;
    static_assert(NQ * NT * 4 <= L1 * Cfg::CP * 8, "reduction buffer fits in the column tile's LDS");
    float* red = reinterpret_cast<float*>(lds);
    const int tid = threadIdx.x;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        red[q * NT + tid] = s0[q];
        if constexpr (KIND == kColTail0) red[(3 + q) * NT + tid] = s1[q];
    }
    __syncthreads();
    if (tid < NQ) {
        float sum = 0.f;
        for (int k = 0; k < NT; ++k) sum += red[tid * NT + k];
        // taps of channel ch0 at 3*ch0 + 0..2; TAIL0 also channel N right after (N = ch0 + 1)
        part[(r * NCB + cb) * 3 * (N + 1) + 3 * ch0 + tid] = sum;
    }
}

// du[b][i*D + d][t] = w2 S_i[t] + w1 S_i[t+1] + w0 S_i[t+2] for the N+1 channels,
// four consecutive t per thread (one 16-byte load of S, the next two values for
// the taps that reach past them, one wide store).
__device__ __forceinline__ void store_quad(float* __restrict__ row, int64_t q, float4 v) {
    reinterpret_cast<float4*>(row)[q] = v;
}
__device__ __forceinline__ void store_quad(uint16_t* __restrict__ row, int64_t q, float4 v) {
    reinterpret_cast<uint2*>(row)[q] = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

template <class TIO>
__global__ void __launch_bounds__(256)
k_fs_bwd_du(const float* __restrict__ S, const float* __restrict__ w3, TIO* __restrict__ du, int D, int N,
            int64_t L, int64_t rows) {
    const int64_t quads = L / 4;
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= quads) return;
    const int nc = N + 1;
    for (int64_t ri = blockIdx.y; ri < rows * nc; ri += gridDim.y) {
        const int64_t r = ri / nc;
        const int i = (int)(ri - r * nc);
        const int64_t b = r / D, d = r - b * D;
        const float* s = S + ri * L;
        const float4 c = reinterpret_cast<const float4*>(s)[q];
        const float2 nx = q + 1 < quads ? reinterpret_cast<const float2*>(s)[2 * q + 2] : make_float2(0.f, 0.f);
        const float* w = w3 + 3 * ((int64_t)i * D + d);
        const float w0 = w[0], w1 = w[1], w2 = w[2];
        store_quad(du + (b * nc * D + (int64_t)i * D + d) * L, q,
                   make_float4(fmaf(w2, c.x, fmaf(w1, c.y, w0 * c.z)), fmaf(w2, c.y, fmaf(w1, c.z, w0 * c.w)),
                               fmaf(w2, c.z, fmaf(w1, c.w, w0 * nx.x)), fmaf(w2, c.w, fmaf(w1, nx.x, w0 * nx.y))));
    }
}

// dh by columns from the rows' dh tiles (pass B's inverse rows of the products):
// the fixed-order sum of the nb tiles tstride apart (the samples of a channel; one
// tile with a filter set per sample), conjugate twiddle, inverse columns, the first
// half is dh; the workgroup holding column 0 also writes dbias = dh[0].
template <int LOG1, int LOG2>
__global__ void __launch_bounds__((FsCfg<LOG1, LOG2>::COL_THREADS))
k_fs_dh_col(const float2* __restrict__ Tdh, float* __restrict__ dh, float* __restrict__ dbias, FsTables tb, int D,
            int Dch, int64_t bstride, int nb, int64_t tstride) {
    using Cfg = FsCfg<LOG1, LOG2>;
    constexpr int L1 = Cfg::L1, L2 = Cfg::L2, T1 = Cfg::T1, CB = Cfg::CB, NCB = L2 / CB;
    constexpr int64_t L = (int64_t)L1 * L2;
    __shared__ float2 lds[L1 * Cfg::CP];
    int64_t dd;
    int cb;
    if (!xcd_row_map(blockIdx.x, D, NCB, dd, cb)) return;
    const int c = threadIdx.x % CB, t = threadIdx.x / CB;
    const int m2 = cb * CB + c;
    const float2* slot = Tdh + dd * L;
    float2 v[16];
    const float2 base = twiddle_base<L2>(tb, t, m2);
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = slot[(uint32_t)(t + T1 * e) * L2 + m2];
    for (int b = 1; b < nb; ++b) {  // the other samples' tiles, each loaded together
        const float2* sb = slot + b * tstride;
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = cadd(v[e], sb[(uint32_t)(t + T1 * e) * L2 + m2]);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = cmulc(v[e], twiddle_step<L2>(tb, base, e, m2));
    fft_strided<L1, true, false>(v, t, tb.tw1, ColAcc<Cfg::CP>{lds + c});
    // row dd of the tile is filter d = dd mod Dch of sample b = dd / Dch
    const int64_t b = dd / Dch;
    float* dhr = dh + b * bstride + (dd - b * Dch) * L;
#pragma unroll
    for (int e = 0; e < 8; ++e) store_pair(dhr, (uint32_t)(t + T1 * e) * L2 + m2, v[e]);
    if (t == 0 && m2 == 0) dbias[dd] = v[0].x;  // lag 0
}

// dbias[d] = sum over the samples of the per-sample lag-0 values (fixed order).
__global__ void k_fs_dbias_sum(const float* __restrict__ lag, float* __restrict__ dbias, int B, int D) {
    const int d = blockIdx.x * blockDim.x + threadIdx.x;
    if (d >= D) return;
    float s = 0.f;
    for (int b = 0; b < B; ++b) s += lag[(int64_t)b * D + d];
    dbias[d] = s;
}

// dshort_w[i*D + d][j] = sum over b and column blocks of the tap sums (fixed order).
__global__ void k_fs_bwd_dw(const float* __restrict__ part, float* __restrict__ dw, int B, int D, int N, int ncb) {
    const int d = blockIdx.x, q = threadIdx.x;  // q = 3*channel + tap
    const int nq = 3 * (N + 1);
    if (q >= nq) return;
    float s = 0.f;
    for (int b = 0; b < B; ++b) {
        const float* pr = part + ((int64_t)b * D + d) * ncb * nq;
        for (int k = 0; k < ncb; ++k) s += pr[k * nq + q];
    }
    dw[((int64_t)(q / 3) * D + d) * 3 + (q % 3)] = s;
}

template <int LOG1, int LOG2, class TIO>
static void fs_backward_launch(const FsBwdArgs& a, hipStream_t st) {
    using Cfg = FsCfg<LOG1, LOG2>;
    constexpr int NCB = Cfg::L2 / Cfg::CB;
    const int N = a.N;
    const int64_t L = (int64_t)Cfg::L1 * Cfg::L2, rows = (int64_t)a.B * a.D;
    const FsBwdWs w = fs_bwd_ws(a.ws, a.B, a.D, L, NCB, N, a.per_sample);
    const unsigned gcol = (unsigned)xcd_grid(rows, NCB);
    const unsigned grow = (unsigned)xcd_grid(rows, Cfg::L1 / 2 / Cfg::UNITS);
    const dim3 bcol(Cfg::COL_THREADS), brow(Cfg::ROW_THREADS);
    const TIO* u = (const TIO*)a.u;
    const TIO* dy = (const TIO*)a.dy;
    // forward recompute: pass A of g_0, then per step pass B (keeping G_o) and a
    // column pass (MID: store v_{o+1}, next input; HEAD after the last step)
    hipLaunchKernelGGL((k_fs_colfwd<LOG1, LOG2, TIO, 0>), dim3(gcol), bcol, 0, st, u, a.w3, (const float*)nullptr,
                       w.G, a.tb, a.D, N, (int64_t)0, rows);
    for (int o = 0; o < N - 1; ++o) {
        hipLaunchKernelGGL((k_fs_row_bwd<LOG1, LOG2, 2>), dim3(grow), brow, 0, st, w.T, a.spec, a.bias, w.G,
                           (float2*)nullptr, a.tb, a.D, o, rows, a.sbs);
        if (o < N - 2)
            hipLaunchKernelGGL((k_fs_colinv_bwd<LOG1, LOG2, TIO, kColMid>), dim3(gcol), bcol, 0, st,
                               (const float2*)w.T, w.G + (int64_t)(o + 1) * rows * L, u, a.w3, dy, w.S, w.V, w.part,
                               a.tb, a.D, N, o, rows);
        else
            hipLaunchKernelGGL((k_fs_colinv_bwd<LOG1, LOG2, TIO, kColHead>), dim3(gcol), bcol, 0, st,
                               (const float2*)w.T, w.T, u, a.w3, dy, w.S, w.V, w.part, a.tb, a.D, N, o, rows);
    }
    // the adjoint, last step first: pass B (dh product, conj(H + bias)), dh of the
    // step, then the column pass that finishes the step's gate channel
    for (int o = N - 2; o >= 0; --o) {
        hipLaunchKernelGGL((k_fs_row_bwd<LOG1, LOG2, 3>), dim3(grow), brow, 0, st, w.T, a.spec, a.bias, w.G,
                           w.Tdh, a.tb, a.D, o, rows, a.sbs);
        if (!a.per_sample) {
            // the fixed-order batch sum of the rows' dh tiles, then dh[o][d] and its lag 0
            hipLaunchKernelGGL((k_fs_dh_col<LOG1, LOG2>), dim3((unsigned)xcd_grid(a.D, NCB)), bcol, 0, st,
                               (const float2*)w.Tdh, a.dh + (int64_t)o * a.D * L, a.dbias + (int64_t)o * a.D, a.tb,
                               a.D, a.D, (int64_t)0, a.B, (int64_t)a.D * L);
        } else {
            // every row's own dh tile: dh[b][o][d]; dbias sums the samples' lag 0
            hipLaunchKernelGGL((k_fs_dh_col<LOG1, LOG2>), dim3((unsigned)xcd_grid(rows, NCB)), bcol, 0, st,
                               (const float2*)w.Tdh, a.dh + (int64_t)o * a.D * L, w.lag, a.tb, (int)rows, a.D,
                               (int64_t)(N - 1) * a.D * L, 1, (int64_t)0);
            hipLaunchKernelGGL(k_fs_dbias_sum, dim3((unsigned)((a.D + 255) / 256)), dim3(256), 0, st,
                               (const float*)w.lag, a.dbias + (int64_t)o * a.D, a.B, a.D);
        }
        if (o > 0)
            hipLaunchKernelGGL((k_fs_colinv_bwd<LOG1, LOG2, TIO, kColTailMid>), dim3(gcol), bcol, 0, st,
                               (const float2*)w.T, w.T, u, a.w3, dy, w.S, w.V, w.part, a.tb, a.D, N, o, rows);
        else
            hipLaunchKernelGGL((k_fs_colinv_bwd<LOG1, LOG2, TIO, kColTail0>), dim3(gcol), bcol, 0, st,
                               (const float2*)w.T, w.T, u, a.w3, dy, w.S, w.V, w.part, a.tb, a.D, N, o, rows);
    }
    const int64_t quads = L / 4;
    const int64_t nrc = rows * (N + 1);
    const unsigned gy = (unsigned)(nrc < 65535 ? nrc : 65535);
    hipLaunchKernelGGL((k_fs_bwd_du<TIO>), dim3((unsigned)((quads + 255) / 256), gy), dim3(256), 0, st,
                       (const float*)w.S, a.w3, (TIO*)a.du, a.D, N, L, rows);
    hipLaunchKernelGGL(k_fs_bwd_dw, dim3((unsigned)a.D), dim3(64), 0, st, (const float*)w.part, a.dw, a.B, a.D, N,
                       NCB);
}

template <int LOG1, int LOG2>
static hipError_t fs_backward_t(const FsBwdArgs& a, hipStream_t st) {
    if (a.bf16) fs_backward_launch<LOG1, LOG2, uint16_t>(a, st);
    else fs_backward_launch<LOG1, LOG2, float>(a, st);
    return hipGetLastError();
}

hipError_t launch_fs_backward(int logL, const FsBwdArgs& a, hipStream_t st) {
    if (a.N < 2 || a.N > 8) return hipErrorInvalidValue;
    switch (logL) {
#define X(LG, A, B) \
    case LG: return fs_backward_t<A, B>(a, st);
        HY_FS_CASES(X)
#undef X
        default: return hipErrorInvalidValue;
    }
}

size_t fs_bwd_ws_bytes(int logL, int64_t B, int64_t D, int N, bool per_sample) {
    int l1 = 0, l2 = 0;
    fs_split(logL, &l1, &l2);
    const int64_t L = int64_t(1) << logL;
    const int ncb = (1 << l2) / HY_FS_CB;
    return fs_bwd_ws(nullptr, B, D, L, ncb, N, per_sample).bytes;
}

}  // namespace hy
