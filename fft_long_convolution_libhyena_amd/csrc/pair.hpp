// Pair step of the packed real transform and small elementwise helpers shared by
// both kernel families.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fft_core.hpp"

namespace hy {

// ------------------------------------------------------------------ pair step
//
// Zk = Z[k], Zm = Z[L-k] of the packed L-point forward transform; w = W_{2L}^k.
// Returns 2*A[k] and 2*A[L-k], A being the 2L-point spectrum of the real input:
//   E = (Z[k] + conj Z[L-k]) / 2, O = (Z[k] - conj Z[L-k]) / 2i,
//   A[k] = E + W^k O, A[L-k] = conj(E - W^k O).
__device__ __forceinline__ void pair_unpack(float2 Zk, float2 Zm, float2 w, float2& Ak, float2& Am) {
    const float2 Ep = make_float2(Zk.x + Zm.x, Zk.y - Zm.y);  // Zk + conj(Zm)
    const float2 Dp = make_float2(Zk.x - Zm.x, Zk.y + Zm.y);  // Zk - conj(Zm)
    const float2 Op = make_float2(Dp.y, -Dp.x);                // -i * Dp
    const float2 P = cmul(w, Op);
    Ak = cadd(Ep, P);
    Am = make_float2(Ep.x - P.x, P.y - Ep.y);  // conj(Ep - P)
}

// Repack of a real signal's 2L-point spectrum values C[k], C[L-k] into the
// packed L-point spectrum that the inverse transform takes:
//   Y[k] = Ec + i Oc, Ec = (C[k] + conj C[L-k])/2, Oc = (C[k] - conj C[L-k]) W^-k / 2,
//   Y[L-k] = conj(Ec) + i conj(Oc).
// (Computed without the halves: the scale is folded into the stored spectra.)
__device__ __forceinline__ void pair_repack(float2 Ck, float2 Cm, float2 w, float2& Yk, float2& Ym) {
    const float2 Ec = make_float2(Ck.x + Cm.x, Ck.y - Cm.y);
    const float2 Dc = make_float2(Ck.x - Cm.x, Ck.y + Cm.y);
    const float2 Oc = cmulc(Dc, w);
    Yk = make_float2(Ec.x - Oc.y, Ec.y + Oc.x);
    Ym = make_float2(Ec.x + Oc.y, Oc.x - Ec.y);
}

// Spectrum multiply and repack for the inverse. Hk, Hm are the scaled filter
// spectrum plus scaled bias at k and L-k; C = A*H.
__device__ __forceinline__ void pair_conv(float2 Zk, float2 Zm, float2 Hk, float2 Hm, float2 w, float2& Yk,
                                          float2& Ym) {
    float2 Ak, Am;
    pair_unpack(Zk, Zm, w, Ak, Am);
    pair_repack(cmul(Ak, Hk), cmul(Am, Hm), w, Yk, Ym);
}

__device__ __forceinline__ float2 fmul2(float2 a, float s) { return make_float2(a.x * s, a.y * s); }
__device__ __forceinline__ float2 hadd(float2 h, float b) { return make_float2(h.x + b, h.y); }
__device__ __forceinline__ float2 emul(float2 a, float2 b) { return make_float2(a.x * b.x, a.y * b.y); }

template <class TIO>
__device__ __forceinline__ float2 gated_pair(const TIO* __restrict__ rv, const TIO* __restrict__ rx, uint32_t m,
                                             const float* wv, const float* wx) {
    const float2 a = conv3_pair(rv, m, wv[0], wv[1], wv[2]);
    const float2 g = conv3_pair(rx, m, wx[0], wx[1], wx[2]);
    return emul(a, g);
}

}  // namespace hy
