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
// Tiles: 256 rows x 128 columns per workgroup of four waves (2 x 2), each wave
// 128 x 64 as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16 (128 fp32 accumulators per
// lane); two workgroups share a CU (76 KB of LDS each), so one's waits overlap the
// other's matrix work. The 256 rows of a tile are the times t0-4 .. t0+251 of one
// sequence: the leading rows are the short conv's history (two are needed, four
// keep every output group 8-byte aligned), so a tile yields 252 outputs and tiles
// of a sequence start every 252 steps.
//
// K runs in chunks of 32 columns for both operands through a ring of three chunks
// in LDS, filled by buffer loads that write LDS directly (no register staging):
// while chunk c is multiplied, chunks c + 1 and c + 2 are in flight. Rows of a
// staged operand are 64 bytes with their four 16-byte segments permuted by an XOR
// of bits of the row index, so that the fragment reads (32 rows at one segment)
// spread over the LDS banks. Rows outside the sequence or past C are filled from a
// clamped, valid row; their products are never stored (times before 0 are
// zeroed, later times and channels past C are skipped).
//
// The epilogue reuses the ring in two rounds of 64 columns: the accumulators are
// laid out column by column (a padded pitch), then each lane forms the short conv
// of four consecutive times from an 8-byte and a 16-byte LDS read and stores them
// as 8 bytes (bf16 by the hardware's round-to-nearest-even conversion).
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
typedef __attribute__((address_space(3))) void* LdsPtr;

constexpr int kTM = 256;       // tile rows: four history rows and 252 outputs
constexpr int kTH = 4;         // history rows (two are needed; four keep the stores 8-byte aligned)
constexpr int kTO = kTM - kTH; // output rows per tile
constexpr int kTN = 128;       // tile columns
constexpr int kKC = 32;        // K per staged chunk: 64-byte operand rows
constexpr int kNS = 3;         // chunks in the LDS ring
constexpr int kThreads = 256;  // four waves: 2 (rows) x 2 (columns)
constexpr int kWM = 128, kWN = 64;                // rows and columns per wave
constexpr int kABytes = kTM * kKC * 2;            // staged x rows (16 KiB)
constexpr int kStageBytes = kABytes + kTN * kKC * 2;  // and w rows (24 KiB)
constexpr int kRoundCols = 64;                    // tile columns laid out per epilogue round
constexpr int kEP = kTM + 4;                      // epilogue column pitch (floats)
constexpr int kEpiBytes = kRoundCols * kEP * 4 + 16;  // with the four-float shift of the rows
constexpr int kRingBytes = kNS * kStageBytes;
constexpr int kParamOff = kRingBytes > kEpiBytes ? kRingBytes : kEpiBytes;  // (w0, w1, w2, b_in) per column
constexpr int kLdsBytes = kParamOff + kTN * 16;   // 75,776 bytes: two workgroups per CU
static_assert(kTN == 2 * kWN && kTM == 2 * kWM && kTN == 2 * kRoundCols, "tile shape");

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// slot of 16-byte segment s (0..3) in staged 64-byte row r: s ^ swizzle(r)
__device__ __forceinline__ uint32_t seg_swizzle(uint32_t r) { return (r ^ (r >> 3)) & 3u; }

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

__global__ void __launch_bounds__(kThreads, 2) k_inproj_conv3(Inproj a) {
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // uniform: LDS and column addresses stay scalar
    const int wm = wave >> 1, wn = wave & 1;
    // XCD-aware order: hardware sends workgroup i to XCD i % 8; the N tiles of one M
    // tile run back to back on one XCD, so its rows of x are read from that XCD's L2
    const int64_t bid = blockIdx.x;
    const int64_t sidx = bid >> 3;
    const int64_t mt = (sidx / a.ntiles) * 8 + (bid & 7);
    if (mt >= a.mtiles) return;
    const int64_t seq = mt / a.tps;
    const int64_t t0 = (mt - seq * a.tps) * kTO;  // first output time of the tile
    const int64_t c0 = (sidx % a.ntiles) * kTN;
    const int nchunks = (int)(a.D / kKC);

    // fills: instruction q of a wave writes 16 staged rows (1 KiB), lane l the slot
    // l % 4 of row 16 (4 q + wave) + l / 4, holding segment (l % 4) ^ swizzle(row) of
    // the source row; x rows 0..255 take q < 4, w rows 0..127 q < 2. Rows outside the
    // sequence or past C read a clamped, valid row (their products are not stored).
    // Byte offsets below 2^31 (host check).
    const BufRsrc xr = buf_rsrc(a.x + seq * a.L * a.D);
    const BufRsrc wr = buf_rsrc(a.w);
    uint32_t xoff[4], woff[2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t r = 16 * (4 * q + wave) + (lane >> 2);
        const uint32_t seg = (uint32_t)(lane & 3) ^ seg_swizzle(r);
        int64_t t = t0 - kTH + r;
        t = t < 0 ? 0 : (t >= a.L ? a.L - 1 : t);
        xoff[q] = (uint32_t)(t * a.D * 2) + 16 * seg;
        if (q < 2) {
            int64_t c = c0 + r;
            c = c >= a.C ? a.C - 1 : c;
            woff[q] = (uint32_t)(c * a.D * 2) + 16 * seg;
        }
    }
    auto fill = [&](int stage, int chunk) {
        unsigned char* st = lds_raw + stage * kStageBytes;
        const int sk = chunk * kKC * 2;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (LdsPtr)(st + 16 * (4 * q + wave) * 64), 16, (int)xoff[q],
                                                     sk, 0, 0);
#pragma unroll
        for (int q = 0; q < 2; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (LdsPtr)(st + kABytes + 16 * (4 * q + wave) * 64), 16,
                                                     (int)woff[q], sk, 0, 0);
    };
    // taps and b_in of tile column tid (channel c0 + tid)
    float4 prm = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid < kTN && c0 + tid < a.C) {
        const int64_t c = c0 + tid;
        prm = make_float4(a.w3[3 * c], a.w3[3 * c + 1], a.w3[3 * c + 2], bf16_to_f32(a.b[c]));
    }

    // fragment reads: block i of A is staged row wm*128 + 32 i + l % 32, segment
    // 2 ks + l / 32, at byte abase[i] ^ (ks << 5); block j of B the same with wn*64
    uint32_t abase[4], bbase[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t ra = wm * kWM + 32 * i + (lane & 31);
        abase[i] = ra * 64 + ((((uint32_t)lane >> 5) ^ seg_swizzle(ra)) << 4);
        if (i < 2) {
            const uint32_t rb = wn * kWN + 32 * i + (lane & 31);
            bbase[i] = kABytes + rb * 64 + ((((uint32_t)lane >> 5) ^ seg_swizzle(rb)) << 4);
        }
    }
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    bf16x8 fa[2][4], fb[2][2];
    auto frag = [&](int slot, const unsigned char* st, int ks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[slot][i] = *reinterpret_cast<const bf16x8*>(st + (abase[i] ^ (ks << 5)));
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[slot][j] = *reinterpret_cast<const bf16x8*>(st + (bbase[j] ^ (ks << 5)));
    };
    auto mma = [&](int slot) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j], acc[i][j], 0, 0, 0);
    };

    // K in a ring of three chunks: chunk c is multiplied from stage c % 3 while the
    // fills of chunks c + 1 and c + 2 are in flight. Two workgroups share a CU, so
    // one's waits overlap the other's matrix work.
    fill(0, 0);
    if (nchunks > 1) fill(1, 1);
    int stage = 0;
    for (int ch = 0; ch < nchunks; ++ch) {
        if (ch + 1 < nchunks)
            __builtin_amdgcn_s_waitcnt(0x0F76);  // vmcnt(6): all but the next chunk's six fills are in
        else
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        // everyone's fills of chunk ch are in (each wave's own wait above), and chunk ch - 1
        // is no longer read (its fragments fed this wave's last matrix products). A bare
        // barrier: the fenced one waits for every load in flight, the fills of chunk ch + 1
        // too, which would leave one chunk in flight instead of two.
        asm volatile("s_barrier" ::: "memory");
        if (ch + 2 < nchunks) fill(stage == 0 ? 2 : stage - 1, ch + 2);
        const unsigned char* st = lds_raw + stage * kStageBytes;
        frag(0, st, 0);
        frag(1, st, 1);
        mma(0);
        mma(1);
        // schedule: the six fragment reads of k-step 0, then the first six products
        // each followed by one read of k-step 1, then the remaining ten products
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // LDS reads
#pragma unroll
        for (int q = 0; q < 6; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // a matrix product
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 10, 0);
        stage = stage == kNS - 1 ? 0 : stage + 1;
    }

    // epilogue in two rounds over the ring: round h lays out block j = h of every wave
    // (tile columns wn*64 + 32 h .. + 31) column by column, E[col][4 + row] over all
    // 256 rows (column pitch 260 floats: the float4 writes of 16 consecutive columns
    // start on distinct banks); then each wave forms the outputs of 16 columns: lane l
    // the four times t0 + 4l .. t0 + 4l + 3 from rows 4l + 2 .. 4l + 7
    float* E = reinterpret_cast<float*>(lds_raw);
    float4* P = reinterpret_cast<float4*>(lds_raw + kParamOff);
    if (tid < kTN) P[tid] = prm;
    const int t = (int)t0 + 4 * lane;
    // L is a multiple of 4: all four times of a lane are in range or none is (the
    // column's buffer ends at time L; lane 63 holds no output)
    const uint32_t voff = lane < kTO / 4 ? 8u * lane : 0x80000000u;
    const uint16_t* useq = a.u + seq * a.C * a.L;
    const uint32_t colbytes = (uint32_t)(a.L - t0) * 2;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        __syncthreads();  // the last chunk's (or the previous round's) reads are done
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = wn * 32 + lane % 32;
                const int row = wm * kWM + 32 * i + 8 * g + 4 * (lane / 32);
                const f32x16& v = acc[i][h];
                *reinterpret_cast<float4*>(E + col * kEP + 4 + row) =  // rows sit four floats in
                    make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
            }
        __syncthreads();
#pragma unroll 1
        for (int cb = 0; cb < kRoundCols / 4; cb += 4) {
            // four columns at a time: their LDS reads are issued together
            typedef float F4 __attribute__((ext_vector_type(4)));
            typedef float F2 __attribute__((ext_vector_type(2)));
            F2 lo[4];
            F4 hi[4];
            float4 pr[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int col = wave * (kRoundCols / 4) + cb + e;  // 0..63 in this round's layout
                // rows 4l + 2, 4l + 3 in one 8-byte read, 4l + 4 .. 4l + 7 in one 16-byte read
                const float* Ec = E + col * kEP + 4 + 4 * lane;
                pr[e] = P[(col >> 5) * kWN + 32 * h + (col & 31)];
                lo[e] = *reinterpret_cast<const F2*>(Ec + 2);
                hi[e] = *reinterpret_cast<const F4*>(Ec + 4);
            }
            // whole vectors in registers before the selects below, so that no read is
            // narrowed or made conditional (lanes 16 bytes apart would then share banks)
            asm volatile("" : "+v"(lo[0]), "+v"(lo[1]), "+v"(lo[2]), "+v"(lo[3]), "+v"(hi[0]), "+v"(hi[1]),
                         "+v"(hi[2]), "+v"(hi[3]));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int col = wave * (kRoundCols / 4) + cb + e;
                const int64_t c = c0 + (col >> 5) * kWN + 32 * h + (col & 31);
                const float w0 = pr[e].x, w1 = pr[e].y, w2 = pr[e].z, bias = pr[e].w;
                // u = acc + b_in from time 0 on and 0 before the sequence starts, so
                // w0 u[t-2] + w1 u[t-1] + w2 u[t] = w0 x2 + w1 x3 + w2 x4 + b_in (w0 + w1 + w2)
                // with the accumulators x, and x = -b_in standing for times below 0
                const float bs = bias * (w0 + w1 + w2);
                const float x2 = t >= 2 ? lo[e].x : -bias, x3 = t >= 1 ? lo[e].y : -bias;
                const float x4 = hi[e].x, x5 = hi[e].y, x6 = hi[e].z, x7 = hi[e].w;
                const float o0 = fmaf(w0, x2, fmaf(w1, x3, fmaf(w2, x4, bs)));
                const float o1 = fmaf(w0, x3, fmaf(w1, x4, fmaf(w2, x5, bs)));
                const float o2 = fmaf(w0, x4, fmaf(w1, x5, fmaf(w2, x6, bs)));
                const float o3 = fmaf(w0, x5, fmaf(w1, x6, fmaf(w2, x7, bs)));
                if (c < a.C) {
                    const BufRsrc ur = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(useq + c * a.L + t0),
                                                                         0, (int)colbytes, 0x00020000);
                    typedef unsigned int U2 __attribute__((ext_vector_type(2)));
                    const U2 v = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
                    __builtin_amdgcn_raw_buffer_store_b64(v, ur, (int)voff, 0, 0);
                }
            }
        }
    }
}

}  // namespace

bool inproj_supported(int64_t D) { return D >= 64 && D % 64 == 0; }
static_assert(kTO % 4 == 0, "tiles start at multiples of four times");

hipError_t launch_inproj_conv3(const uint16_t* x, const uint16_t* w, const uint16_t* b, const float* w3,
                               uint16_t* u, int64_t B, int64_t L, int64_t D, int64_t C, hipStream_t st) {
    if (!inproj_supported(D) || L % 4 != 0) return hipErrorInvalidValue;
    // byte offsets of rows within a sequence of x and within w are 32-bit in the kernel
    if (L * D * 2 >= (int64_t(1) << 31) || C * D * 2 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    Inproj a{x, w, b, w3, u, L, D, C, (L + kTO - 1) / kTO, 0, (C + kTN - 1) / kTN};
    a.mtiles = B * a.tps;
    const int64_t grid = ((a.mtiles + 7) / 8) * 8 * a.ntiles;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    static bool attr = false;
    if (!attr) {
        const hipError_t e =
            hipFuncSetAttribute((const void*)k_inproj_conv3, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        if (e != hipSuccess) return e;
        attr = true;
    }
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_inproj_conv3, dim3((unsigned)grid), dim3(kThreads), kLdsBytes, st, a);
    return hipGetLastError();
}

}  // namespace hy
