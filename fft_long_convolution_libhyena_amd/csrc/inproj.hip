// Input projection of the Hyena operator fused with the short convolution, on
// the bf16 matrix cores of gfx950 (HyenaDNA walkthrough, section 2.1: the input
// projection, the rearrange to channels-first and the short depthwise filter).
// For every sequence b, channel c < C = (N+1)*D and time t < L:
//   u[b][c][t]  = sum_k x[b][t][k] w_in[c][k] + b_in[c]              (in_proj)
//   uc[b][c][t] = w3[c][0] u[b][c][t-2] + w3[c][1] u[b][c][t-1] + w3[c][2] u[b][c][t],
//                 u[b][c][t'] = 0 for t' < 0                          (short conv)
// written as uc[b][c][t] (channels first, the layout the hot path reads); the
// hot path then runs with the identity taps. One launch covers every sequence:
// the GEMM has M = B*L rows (b, t), N = C columns and K = D, with bf16 operands
// and fp32 accumulation; the short conv is applied to the fp32 sums before the
// single rounding to bf16.
//
// Tiles: 256 rows x 256 columns per workgroup of eight waves (2 x 4), each wave
// 128 x 64 as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16 (128 fp32 accumulators
// per lane, two waves per SIMD). The 256 rows of a tile are the times t0-4 ..
// t0+251 of one sequence: the leading rows are the short conv's history (two are
// needed, four keep every output group 8-byte aligned), so a tile yields 252
// outputs and tiles of a sequence start every 252 steps. K runs in chunks of 64
// staged through LDS with double buffering (the next chunk's loads are in flight
// while the current one is multiplied). The epilogue goes through LDS in two
// rounds of 128 columns: the accumulators are laid out column by column so that
// each output channel's times are contiguous, then each lane forms the short conv
// of four consecutive times from two 16-byte LDS reads and stores them as 8 bytes
// (bf16 by the hardware's round-to-nearest-even conversion).
//
// MFMA lane layout (32 x 32 x 16, bf16): lane l supplies A[m = l % 32][k = 8 (l / 32)
// + j] and B[k = 8 (l / 32) + j][n = l % 32] for j < 8, and holds D[row][col = l % 32]
// for row = 8 (i / 4) + 4 (l / 32) + i % 4, i < 16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fft_core.hpp"
#include "kernels.hpp"

namespace hy {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTM = 256;       // tile rows: four history rows and 252 outputs
constexpr int kTH = 4;         // history rows (two are needed; four keep the stores 8-byte aligned)
constexpr int kTO = kTM - kTH; // output rows per tile
constexpr int kTN = 256;       // tile columns
constexpr int kKC = 64;        // K per staged chunk
constexpr int kKP = kKC + 8;   // LDS row pitch in bf16 (144 bytes: rows start 36 banks apart)
constexpr int kThreads = 512;  // eight waves: 2 (rows) x 4 (columns), two per SIMD
constexpr int kWN = 64;        // columns per wave
constexpr int kStage = kTM * kKP;            // bf16 elements of one staged operand tile
constexpr int kEP = kTM + 4;                 // epilogue row pitch (floats) of one column
constexpr int kRoundCols = 128;              // tile columns laid out per epilogue round
constexpr int kLdsBytes = 4 * kStage * 2;    // A and B, double buffered: 147,456 bytes
static_assert(kRoundCols * kEP * 4 + kRoundCols * 16 <= kLdsBytes,
              "one epilogue round and its column parameters fit the staging buffers");

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

struct Inproj {
    const uint16_t* x;   // [B*L][D]
    const uint16_t* w;   // [C][D]
    const uint16_t* b;   // [C]
    const float* w3;     // [C][3]
    uint16_t* u;         // [B][C][L]
    int64_t L, D, C;
    int64_t tps;         // tiles per sequence
    int64_t mtiles, ntiles;
};

__global__ void __launch_bounds__(kThreads, 1) k_inproj_conv3(Inproj a) {
    extern __shared__ __align__(16) unsigned char lds_raw[];
    uint16_t* lds = reinterpret_cast<uint16_t*>(lds_raw);
    // XCD-aware order: hardware sends workgroup i to XCD i % 8; the N tiles of one M
    // tile run back to back on one XCD, so its rows of x are read from that XCD's L2
    const int64_t bid = blockIdx.x;
    const int64_t s = bid >> 3;
    const int64_t mt = (s / a.ntiles) * 8 + (bid & 7);
    const int64_t nt = s % a.ntiles;
    if (mt >= a.mtiles) return;
    const int64_t seq = mt / a.tps;
    const int64_t t0 = (mt - seq * a.tps) * kTO;  // first output time of the tile
    const int64_t c0 = nt * kTN;
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int wm = wave >> 2, wn = wave & 3;

    // global -> LDS staging: thread tid moves 16 bytes of 4 rows of each operand per
    // chunk (row tid/8 + 64 q, bytes 16 (tid % 8)). Rows outside the sequence or past
    // C read a valid row and are zeroed by a mask, so every lane takes the same path.
    const int srow = tid / 8, sseg = tid % 8;
    uint32_t xoff[4], woff[4];  // element offsets of the rows (below 2^31: checked on the host)
    uint32_t valid = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = srow + 64 * q;
        const int64_t t = t0 - kTH + r;
        const bool vx = t >= 0 && t < a.L;
        xoff[q] = (uint32_t)((seq * a.L + (vx ? t : 0)) * a.D + 8 * sseg);
        const int64_t c = c0 + r;
        const bool vw = c < a.C;
        woff[q] = (uint32_t)((vw ? c : 0) * a.D + 8 * sseg);
        valid |= (vx ? 1u : 0u) << q;
        valid |= (vw ? 1u : 0u) << (4 + q);
    }
    uint4 ra[4], rb[4];  // the next chunk, in flight while the current one is multiplied
    auto fetch = [&](int64_t k0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            ra[q] = *reinterpret_cast<const uint4*>(a.x + xoff[q] + k0);
            rb[q] = *reinterpret_cast<const uint4*>(a.w + woff[q] + k0);
        }
    };
    auto stash = [&](int buf) {
        uint16_t* A = lds + buf * 2 * kStage;
        uint16_t* Bm = A + kStage;
        auto masked = [](uint4 v, uint32_t keep) {  // keep is 0 or all ones
            return make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
        };
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            *reinterpret_cast<uint4*>(A + (srow + 64 * q) * kKP + 8 * sseg) = masked(ra[q], 0u - ((valid >> q) & 1u));
            *reinterpret_cast<uint4*>(Bm + (srow + 64 * q) * kKP + 8 * sseg) =
                masked(rb[q], 0u - ((valid >> (4 + q)) & 1u));
        }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    const int nchunks = (int)(a.D / kKC);
    fetch(0);
    stash(0);
    __syncthreads();
    const int fr = lane % 32, fk = 8 * (lane / 32);
    for (int ch = 0; ch < nchunks; ++ch) {
        const int buf = ch & 1;
        if (ch + 1 < nchunks) fetch((int64_t)(ch + 1) * kKC);
        const uint16_t* A = lds + buf * 2 * kStage + (wm * 128 + fr) * kKP + fk;
        const uint16_t* Bm = lds + buf * 2 * kStage + kStage + (wn * kWN + fr) * kKP + fk;
#pragma unroll
        for (int ks = 0; ks < kKC / 16; ++ks) {
            bf16x8 fa[4], fb[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) fa[i] = *reinterpret_cast<const bf16x8*>(A + i * 32 * kKP + 16 * ks);
#pragma unroll
            for (int j = 0; j < 2; ++j) fb[j] = *reinterpret_cast<const bf16x8*>(Bm + j * 32 * kKP + 16 * ks);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (ch + 1 < nchunks) stash(buf ^ 1);
        __syncthreads();
    }

    // epilogue in two rounds: round j lays out block j of every wave (the tile columns
    // wn*64 + 32 j .. + 31) column by column in LDS, E[col][row] over all 256 rows,
    // with each column's taps and bias beside them; then each wave forms the outputs
    // of 16 columns: lane l the four times t0 + 4l .. t0 + 4l + 3 from rows 4l .. 4l + 7
    float* E = reinterpret_cast<float*>(lds_raw);
    float4* P = reinterpret_cast<float4*>(E + kRoundCols * kEP);  // (w0, w1, w2, b_in) per column
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (j > 0) __syncthreads();  // the previous round's reads are done
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int row = wm * 128 + 32 * i + 8 * g + 4 * (lane / 32);
                const float4 v = make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                             acc[i][j][4 * g + 3]);
                *reinterpret_cast<float4*>(E + (wn * 32 + lane % 32) * kEP + row) = v;
            }
        if (tid < kRoundCols) {
            const int64_t c = c0 + (tid / 32) * kWN + 32 * j + tid % 32;
            P[tid] = c < a.C ? make_float4(a.w3[3 * c], a.w3[3 * c + 1], a.w3[3 * c + 2], bf16_to_f32(a.b[c]))
                             : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        __syncthreads();
#pragma unroll 4
        for (int cc = 0; cc < kRoundCols / 8; ++cc) {
            const int col = wave * (kRoundCols / 8) + cc;  // 0..127 in this round's layout
            const int64_t c = c0 + (col / 32) * kWN + 32 * j + col % 32;
            if (c >= a.C) continue;
            const float4 pr = P[col];
            const float w0 = pr.x, w1 = pr.y, w2 = pr.z, bias = pr.w;
            const float* Ec = E + col * kEP + 4 * lane;
            const float4 lo = *reinterpret_cast<const float4*>(Ec);      // rows 4l .. 4l+3 (history)
            const float4 hi = *reinterpret_cast<const float4*>(Ec + 4);  // rows 4l+4 .. 4l+7
            const int64_t t = t0 + 4 * lane;                             // time of row 4l + 4
            // u = acc + b_in from time 0 on, 0 before the sequence starts
            const float u2 = t >= 2 ? lo.z + bias : 0.f, u3 = t >= 1 ? lo.w + bias : 0.f;
            const float u4 = hi.x + bias, u5 = hi.y + bias, u6 = hi.z + bias, u7 = hi.w + bias;
            const float o0 = fmaf(w0, u2, fmaf(w1, u3, w2 * u4));
            const float o1 = fmaf(w0, u3, fmaf(w1, u4, w2 * u5));
            const float o2 = fmaf(w0, u4, fmaf(w1, u5, w2 * u6));
            const float o3 = fmaf(w0, u5, fmaf(w1, u6, w2 * u7));
            if (lane < kTO / 4 && t < a.L)  // L is a multiple of 4: all four times are in range
                *reinterpret_cast<uint2*>(a.u + (seq * a.C + c) * a.L + t) = make_uint2(pack_bf16x2(o0, o1),
                                                                                         pack_bf16x2(o2, o3));
        }
    }
}

}  // namespace

bool inproj_supported(int64_t D) { return D >= kKC && D % kKC == 0; }
static_assert(kTO % 4 == 0, "tiles start at multiples of four times");

hipError_t launch_inproj_conv3(const uint16_t* x, const uint16_t* w, const uint16_t* b, const float* w3,
                               uint16_t* u, int64_t B, int64_t L, int64_t D, int64_t C, hipStream_t st) {
    if (!inproj_supported(D) || L % 4 != 0) return hipErrorInvalidValue;
    // row offsets of x and w are 32-bit element offsets in the kernel
    if (B * L * D >= (int64_t(1) << 31) || C * D >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    Inproj a{x, w, b, w3, u, L, D, C, (L + kTO - 1) / kTO, 0, (C + kTN - 1) / kTN};
    a.mtiles = B * a.tps;
    const int64_t grid = ((a.mtiles + 7) / 8) * 8 * a.ntiles;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    static bool attr = false;
    if (!attr) {
        const hipError_t e = hipFuncSetAttribute((const void*)k_inproj_conv3,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        if (e != hipSuccess) return e;
        attr = true;
    }
    hipLaunchKernelGGL(k_inproj_conv3, dim3((unsigned)grid), dim3(kThreads), kLdsBytes, st, a);
    return hipGetLastError();
}

}  // namespace hy
