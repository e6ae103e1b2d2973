// Device-side FFT building blocks for gfx950 (CDNA4, wave64).
//
// A length-N complex transform (N = 2^s, 16 <= N <= 16384) is carried by T = N/E
// threads (E = 16 or 32 values per thread). Between passes every thread holds E
// values in registers in the "strided" layout: thread t holds element t + T*e
// for e = 0..E-1. Each pass is a
// Stockham (self-sorting) radix-R step: butterfly j reads x[j + r*N/R], scales
// input r by W_{NS*R}^{r*(j mod NS)} and writes output r to
// (j/NS)*NS*R + (j mod NS) + r*NS, where NS is the product of the radices of the
// earlier passes. With N/E threads and E values per thread (E/R butterflies per
// thread), the inputs of every pass are exactly the strided layout, and so are
// the outputs of the last pass,
// so a transform takes natural order in and gives natural order out with only
// (passes - 1) round trips through LDS. Radices are 16 (as 4x4) for every pass
// except a final 2/4/8 pass when s is not a multiple of 4.
//
// Twiddles come from tables built on the host in fp64 and rounded once to fp32
// (pass 0 needs none; pass p >= 1 holds W_{NS*R}^{r*k} at [(r-1)*NS + k], so the
// lanes of a wave read consecutive values); inverse transforms use their
// conjugates. The in-register DFT constants are fp32 roundings of cos/sin of
// multiples of pi/8. No fast sin/cos intrinsics are used anywhere.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace hy {

// Raw buffer access to read-only tables: a resource descriptor built from a
// uniform base (gfx9 layout: no stride, byte-sized records, 32-bit data format),
// a per-lane byte offset and a scalar byte offset.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
__device__ __forceinline__ BufRsrc buf_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ float2 buf_load_f2(BufRsrc rs, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)voff, (int)soff, 0));
}

// Element i of an array at a workgroup-uniform base, addressed by a 32-bit byte
// offset (i * sizeof(T) below 2^32): the access then takes the scalar base plus a
// per-lane 32-bit offset, with no 64-bit address arithmetic per lane.
template <class T>
__device__ __forceinline__ const T& ld32(const T* __restrict__ base, uint32_t i) {
    return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + i * (uint32_t)sizeof(T));
}

__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
// a * b
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
    return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}
// a * conj(b)
__device__ __forceinline__ float2 cmulc(float2 a, float2 b) {
    return make_float2(fmaf(a.x, b.x, a.y * b.y), fmaf(a.y, b.x, -a.x * b.y));
}
// multiply by the twiddle w (forward) or its conjugate (inverse)
template <bool INV>
__device__ __forceinline__ float2 twmul(float2 a, float2 w) { return INV ? cmulc(a, w) : cmul(a, w); }
// multiply by -i (forward) / +i (inverse)
template <bool INV>
__device__ __forceinline__ float2 mul_mi(float2 a) {
    return INV ? make_float2(-a.y, a.x) : make_float2(a.y, -a.x);
}

constexpr float kC8 = 0.70710678118654752440f;   // cos(pi/4)
constexpr float kC16 = 0.92387953251128675613f;  // cos(pi/8)
constexpr float kS16 = 0.38268343236508977173f;  // sin(pi/8)

// multiply by W8^1 = (1 - i)/sqrt2 (forward) or its conjugate
template <bool INV>
__device__ __forceinline__ float2 mul_w8_1(float2 a) {
    return INV ? make_float2((a.x - a.y) * kC8, (a.x + a.y) * kC8)
               : make_float2((a.x + a.y) * kC8, (a.y - a.x) * kC8);
}
// multiply by W8^3 = (-1 - i)/sqrt2 (forward) or its conjugate
template <bool INV>
__device__ __forceinline__ float2 mul_w8_3(float2 a) {
    return INV ? make_float2(-(a.x + a.y) * kC8, (a.x - a.y) * kC8)
               : make_float2((a.y - a.x) * kC8, -(a.x + a.y) * kC8);
}
// multiply by W16^e for e in {1, 3, 9} through a general complex product
template <bool INV, int E>
__device__ __forceinline__ float2 mul_w16(float2 a) {
    // W16^1 = (c, -s), W16^3 = (s, -c), W16^9 = (-c, s)
    constexpr float wr = (E == 1) ? kC16 : (E == 3) ? kS16 : -kC16;
    constexpr float wi = (E == 1) ? -kS16 : (E == 3) ? -kC16 : kS16;
    return twmul<INV>(a, make_float2(wr, wi));
}

template <bool INV>
__device__ __forceinline__ void dft2(float2& a0, float2& a1) {
    float2 t = a0;
    a0 = cadd(t, a1);
    a1 = csub(t, a1);
}

template <bool INV>
__device__ __forceinline__ void dft4(float2& a0, float2& a1, float2& a2, float2& a3) {
    float2 t0 = cadd(a0, a2), t1 = csub(a0, a2);
    float2 t2 = cadd(a1, a3), t3 = mul_mi<INV>(csub(a1, a3));
    a0 = cadd(t0, t2);
    a2 = csub(t0, t2);
    a1 = cadd(t1, t3);
    a3 = csub(t1, t3);
}

// 8-point DFT in place, natural order in and out (4 x 2 split).
template <bool INV>
__device__ __forceinline__ void dft8(float2* a) {
    dft4<INV>(a[0], a[2], a[4], a[6]);
    dft4<INV>(a[1], a[3], a[5], a[7]);
    a[3] = mul_w8_1<INV>(a[3]);
    a[5] = mul_mi<INV>(a[5]);
    a[7] = mul_w8_3<INV>(a[7]);
    float2 o[8];
#pragma unroll
    for (int k1 = 0; k1 < 4; ++k1) {
        o[k1] = cadd(a[2 * k1], a[2 * k1 + 1]);
        o[k1 + 4] = csub(a[2 * k1], a[2 * k1 + 1]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = o[i];
}

// 4-point DFT whose last two inputs are known to be zero.
template <bool INV>
__device__ __forceinline__ void dft4_half(float2& a0, float2& a1, float2& a2, float2& a3) {
    const float2 m = mul_mi<INV>(a1);
    const float2 x0 = a0;
    a2 = csub(x0, a1);
    a0 = cadd(x0, a1);
    a1 = cadd(x0, m);
    a3 = csub(x0, m);
}

// 16-point DFT in place, natural order in and out (4 x 4 split):
// n = 4*n1 + n2, k = k1 + 4*k2. HALF: inputs 8..15 are zero and are not read.
template <bool INV, bool HALF = false>
__device__ __forceinline__ void dft16(float2* a) {
#pragma unroll
    for (int n2 = 0; n2 < 4; ++n2) {
        if (HALF) dft4_half<INV>(a[n2], a[n2 + 4], a[n2 + 8], a[n2 + 12]);
        else dft4<INV>(a[n2], a[n2 + 4], a[n2 + 8], a[n2 + 12]);
    }
    // a[n2 + 4*k1] *= W16^(n2*k1)
    a[5] = mul_w16<INV, 1>(a[5]);
    a[9] = mul_w8_1<INV>(a[9]);
    a[13] = mul_w16<INV, 3>(a[13]);
    a[6] = mul_w8_1<INV>(a[6]);
    a[10] = mul_mi<INV>(a[10]);
    a[14] = mul_w8_3<INV>(a[14]);
    a[7] = mul_w16<INV, 3>(a[7]);
    a[11] = mul_w8_3<INV>(a[11]);
    a[15] = mul_w16<INV, 9>(a[15]);
#pragma unroll
    for (int k1 = 0; k1 < 4; ++k1) dft4<INV>(a[4 * k1], a[4 * k1 + 1], a[4 * k1 + 2], a[4 * k1 + 3]);
    // result X[k1 + 4*k2] sits in a[4*k1 + k2]: transpose the 4x4 index
    float2 o[16];
#pragma unroll
    for (int k1 = 0; k1 < 4; ++k1)
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) o[k1 + 4 * k2] = a[4 * k1 + k2];
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = o[i];
}

template <int R, bool INV>
__device__ __forceinline__ void dft(float2* a) {
    if constexpr (R == 2) dft2<INV>(a[0], a[1]);
    else if constexpr (R == 4) dft4<INV>(a[0], a[1], a[2], a[3]);
    else if constexpr (R == 8) dft8<INV>(a);
    else dft16<INV>(a);
}

constexpr int ilog2c(int n) { return n <= 1 ? 0 : 1 + ilog2c(n >> 1); }

// Compile-time radix schedule for N = 2^LOG carried by N/E threads.
template <int N, int E = 16>
struct Sched {
    static_assert(E == 16 || E == 32, "16 or 32 values per thread");
    static constexpr int LOG = ilog2c(N);
    static constexpr int FULL = LOG / 4;            // radix-16 passes
    static constexpr int REM = LOG % 4;             // trailing radix 2^REM pass if nonzero
    static constexpr int NPASS = FULL + (REM ? 1 : 0);
    static constexpr int T = N / E;                 // threads per transform
    static constexpr int radix(int p) { return p < FULL ? 16 : (1 << REM); }
    static constexpr int ns(int p) { return 1 << (4 * p); }  // product of earlier radices
    // offset of pass p's twiddles inside this size's table
    static constexpr int twoff(int p) {
        int off = 0;
        for (int i = 1; i < p; ++i) off += (radix(i) - 1) * ns(i);
        return off;
    }
    static constexpr int twsize() { return twoff(NPASS); }
};

// LDS accessors. phys(i) is the slot of element i; off(c) is the slot distance
// of c elements when c is a multiple of 16 (so the per-thread part of an address
// is computed once and the rest becomes an instruction's immediate offset);
// small(r) is the distance of r < 16 elements from a multiple of 16.
//
// One transform stored contiguously with one pad slot per 16 elements, which
// spreads power-of-two strides over the banks.
struct RowAcc {
    float2* base;
    __device__ __forceinline__ uint32_t phys(uint32_t i) const { return i + (i >> 4); }
    static constexpr uint32_t off(uint32_t c) { return c + c / 16; }
    static constexpr uint32_t small(uint32_t r) { return r; }
    __device__ __forceinline__ float2& operator[](uint32_t i) const { return base[phys(i)]; }
    __device__ __forceinline__ float2& at(uint32_t slot) const { return base[slot]; }
};
// One column of a [len][PITCH] tile: element i of the column at base + i*PITCH.
template <int PITCH>
struct ColAcc {
    float2* base;  // already offset by the column
    __device__ __forceinline__ uint32_t phys(uint32_t i) const { return i * PITCH; }
    static constexpr uint32_t off(uint32_t c) { return c * PITCH; }
    static constexpr uint32_t small(uint32_t r) { return r * PITCH; }
    __device__ __forceinline__ float2& operator[](uint32_t i) const { return base[phys(i)]; }
    __device__ __forceinline__ float2& at(uint32_t slot) const { return base[slot]; }
};

template <int N>
__host__ __device__ constexpr int padded_len() { return N + N / 16; }

// v[e] <-> element t + T*e of an LDS-resident transform.
template <int T, int E, class Acc>
__device__ __forceinline__ void lds_store_strided(const Acc& acc, int t, const float2 (&v)[E]) {
    if constexpr (T % 16 == 0) {
        const uint32_t b = acc.phys(t);
#pragma unroll
        for (int e = 0; e < E; ++e) acc.at(b + Acc::off(T * e)) = v[e];
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) acc[t + T * e] = v[e];
    }
}
template <int T, int E, class Acc>
__device__ __forceinline__ void lds_load_strided(const Acc& acc, int t, float2 (&v)[E]) {
    if constexpr (T % 16 == 0) {
        const uint32_t b = acc.phys(t);
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = acc.at(b + Acc::off(T * e));
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = acc[t + T * e];
    }
}

// One Stockham pass P of a length-N transform (see the file header).
template <int N, int E, int P, bool INV, bool HALF_IN, bool LAST, class Acc>
__device__ __forceinline__ void fft_pass(float2 (&v)[E], int t, const float2* __restrict__ tw, const Acc& acc) {
    using S = Sched<N, E>;
    constexpr int T = S::T;
    constexpr int R = S::radix(P);
    constexpr int NS = S::ns(P);
    constexpr int Q = E / R;
    if constexpr (P > 0) {
        __syncthreads();
        lds_load_strided<T>(acc, t, v);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const uint32_t j = t + T * q;
        const uint32_t k = j & (NS - 1);
        float2 a[R];
#pragma unroll
        for (int r = 0; r < R; ++r) a[r] = v[q + r * Q];
        if constexpr (NS > 1) {
            // buffer loads: one per-lane offset for all R - 1 twiddles, the row of
            // each r a scalar offset (no per-lane 64-bit addresses)
            const BufRsrc rs = buf_rsrc(tw);
            const uint32_t vo = k * 8u;
#pragma unroll
            for (int r = 1; r < R; ++r)
                a[r] = twmul<INV>(a[r], buf_load_f2(rs, vo, (uint32_t)(S::twoff(P) + (r - 1) * NS) * 8u));
        }
        if constexpr (HALF_IN && P == 0 && R == 16)
            dft16<INV, true>(a);  // a[8..15] are the zero padding
        else
            dft<R, INV>(a);
#pragma unroll
        for (int r = 0; r < R; ++r) v[q + r * Q] = a[r];
    }
    if constexpr (!LAST) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const uint32_t j = t + T * q;
            const uint32_t k = j & (NS - 1);
            const uint32_t pb = acc.phys((j / NS) * NS * R + k);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                // NS >= 16: r*NS is a multiple of 16; NS == 1: the base is 16*j and r < 16
                const uint32_t o = NS >= 16 ? Acc::off(r * NS) : Acc::small(r);
                acc.at(pb + o) = v[q + r * Q];
            }
        }
    }
}

template <int N, int E, bool INV, bool HALF_IN, class Acc, int... Ps>
__device__ __forceinline__ void fft_all_passes(float2 (&v)[E], int t, const float2* __restrict__ tw,
                                               const Acc& acc, std::integer_sequence<int, Ps...>) {
    (fft_pass<N, E, Ps, INV, HALF_IN, Ps == Sched<N, E>::NPASS - 1>(v, t, tw, acc), ...);
}

// One length-N transform held in the strided layout v[e] = x[t + T*e] (T = N/E);
// on return v[e] = X[t + T*e] in natural order. All threads of the block must call
// this together (it synchronises the block). It begins with a barrier before its
// first LDS write, so the caller may still have been reading LDS. HALF_IN: inputs
// e >= E/2 are zero (the zero-padded second half) and are not read.
template <int N, bool INV, bool HALF_IN, int E, class Acc>
__device__ __forceinline__ void fft_strided(float2 (&v)[E], int t, const float2* __restrict__ tw, const Acc& acc) {
    static_assert(N >= 16 && (N & (N - 1)) == 0, "transform length must be a power of two >= 16");
    static_assert(N >= E, "at least one thread per transform");
    fft_all_passes<N, E, INV, HALF_IN>(v, t, tw, acc, std::make_integer_sequence<int, Sched<N, E>::NPASS>{});
}

// ---------------------------------------------------------------- element I/O

// Two consecutive samples (2m, 2m+1) of a row, widened to fp32. Rows are
// addressed by a workgroup-uniform base pointer and a 32-bit element offset.
__device__ __forceinline__ float2 load_pair(const float* __restrict__ row, uint32_t m) {
    return reinterpret_cast<const float2*>(row)[m];
}
__device__ __forceinline__ float2 load_pair(const uint16_t* __restrict__ row, uint32_t m) {
    uint32_t bits = reinterpret_cast<const uint32_t*>(row)[m];
    return make_float2(__uint_as_float(bits << 16), __uint_as_float(bits & 0xffff0000u));
}
// Two floats to packed bf16 (lo in bits 0..15), rounded to nearest even by the
// hardware conversion; a NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    // one two-lane conversion instruction (round to nearest even), lo in the low half
    typedef float F2 __attribute__((ext_vector_type(2)));
    typedef __bf16 B2 __attribute__((ext_vector_type(2)));
    const F2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, B2));
}
__device__ __forceinline__ void store_pair(float* __restrict__ row, uint32_t m, float2 v) {
    reinterpret_cast<float2*>(row)[m] = v;
}
__device__ __forceinline__ void store_pair(uint16_t* __restrict__ row, uint32_t m, float2 v) {
    reinterpret_cast<uint32_t*>(row)[m] = pack_bf16x2(v.x, v.y);
}

// A pair of samples as stored (fp32 pair or two packed bf16), for fetching ahead
// of use.
template <class TIO>
struct RawPair;
template <>
struct RawPair<float> {
    using type = float2;
    static __device__ __forceinline__ float2 zero() { return make_float2(0.f, 0.f); }
};
template <>
struct RawPair<uint16_t> {
    using type = uint32_t;
    static __device__ __forceinline__ uint32_t zero() { return 0u; }
};
__device__ __forceinline__ float2 load_raw(const float* __restrict__ row, uint32_t m) {
    return reinterpret_cast<const float2*>(row)[m];
}
__device__ __forceinline__ uint32_t load_raw(const uint16_t* __restrict__ row, uint32_t m) {
    return reinterpret_cast<const uint32_t*>(row)[m];
}
__device__ __forceinline__ float2 unpack_raw(float2 v) { return v; }
__device__ __forceinline__ float2 unpack_raw(uint32_t bits) {
    return make_float2(__uint_as_float(bits << 16), __uint_as_float(bits & 0xffff0000u));
}

// Causal width-3 depthwise conv (PyTorch Conv1d cross-correlation, padding 2)
// at samples 2m and 2m+1, from the pairs (2m-2, 2m-1) and (2m, 2m+1).
__device__ __forceinline__ float2 conv3_from(float2 prev, float2 cur, float w0, float w1, float w2) {
    float2 r;
    r.x = fmaf(w0, prev.x, fmaf(w1, prev.y, w2 * cur.x));
    r.y = fmaf(w0, prev.y, fmaf(w1, cur.x, w2 * cur.y));
    return r;
}

// The same, reading both pairs of one channel row.
template <class TIO>
__device__ __forceinline__ float2 conv3_pair(const TIO* __restrict__ row, uint32_t m, float w0, float w1,
                                             float w2) {
    const float2 cur = load_pair(row, m);
    const float2 prev = m > 0 ? load_pair(row, m - 1) : make_float2(0.f, 0.f);
    return conv3_from(prev, cur, w0, w1, w2);
}

}  // namespace hy
