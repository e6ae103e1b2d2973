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
// Tiles: 256 rows x 256 columns per workgroup of four waves (2 x 2, one per
// SIMD), each wave 128 x 128 as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16 (256 fp32
// accumulators per lane, held in the accumulation registers). The 256 rows of a
// tile are the times t0-4 .. t0+251 of one sequence: the leading rows are the
// short conv's history (two are needed, four keep every output group 8-byte
// aligned), so a tile yields 252 outputs and tiles of a sequence start every 252
// steps.
//
// The launch is persistent: one workgroup per compute unit walks its tiles (every
// G-th tile, G the grid size) through one continuous pipeline of K chunks. A chunk
// is 64 columns of K for both operands (two 32 KiB tiles), double buffered in LDS
// and filled by buffer loads that write LDS directly (no register staging): while
// chunk g is multiplied, chunk g + 1 - which at the end of a tile is the next
// tile's first chunk - is already in flight. Rows of a staged operand are 128
// bytes with their eight 16-byte segments permuted by an XOR of the row index, so
// the fragment reads (32 rows at one segment) and the fills (eight rows of eight
// segments) spread over the LDS banks. Rows outside the sequence or past C are
// filled from a clamped, valid row; their products are never stored (times before
// 0 are zeroed, later times and channels past C are skipped).
//
// The epilogue reuses the buffer of the tile's last chunk (the other one already
// holds the next tile's first chunk) in four rounds of 64 columns: the
// accumulators are laid out column by column (a padded pitch, so the buffer has a
// 1 KiB overhang), then each lane forms the short conv of four consecutive times
// from an 8-byte and a 16-byte LDS read and stores them as 8 bytes (bf16 by the
// hardware's round-to-nearest-even conversion). The taps and b_in of the tile's columns are
// loaded when the tile starts, so their latency hides behind the products.
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
constexpr int kTN = 256;       // tile columns
constexpr int kKC = 64;        // K per staged chunk: 128-byte operand rows
constexpr int kThreads = 256;  // four waves: 2 (rows) x 2 (columns), one per SIMD
constexpr int kWM = 128, kWN = 128;          // rows and columns per wave
constexpr int kOpBytes = kTM * kKC * 2;      // one staged operand tile (32 KiB)
constexpr int kStageBytes = 2 * kOpBytes;    // A and B
constexpr int kRoundCols = 64;               // tile columns laid out per epilogue round
constexpr int kEP = kTM + 4;                 // epilogue column pitch (floats)
constexpr int kBufStride = kStageBytes + 1024;   // a chunk buffer and the epilogue's overhang
constexpr int kParamOff = 2 * kBufStride;    // (w0, w1, w2, b_in) of the tile's columns
constexpr int kLdsBytes = kParamOff + kTN * 16;  // 137,216 bytes
static_assert(kTN == 2 * kWN && kTM == 2 * kWM && kTN == 4 * kRoundCols, "tile shape");
static_assert(kRoundCols * kEP * 4 <= kBufStride, "one epilogue round fits a chunk buffer and its overhang");

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// segment slot of 16-byte segment s in staged row r
__device__ __forceinline__ uint32_t seg_swizzle(uint32_t r) { return (r ^ (r >> 3)) & 7u; }

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

// Tile T of the walk: hardware sends workgroup i to XCD i % 8 and the grid is a
// multiple of 8, so every tile of a workgroup has the XCD T % 8; the N tiles of
// one M tile are consecutive in T / 8, so at any time the workgroups of one XCD
// share their rows of x and the columns of w in that XCD's L2.
struct TileAt {
    bool valid;
    int64_t seq, t0, c0;
    __device__ TileAt(const Inproj& a, int64_t T) {
        const int64_t s = T >> 3;
        const int64_t mt = (s / a.ntiles) * 8 + (T & 7);
        valid = mt < a.mtiles;
        const int64_t m = valid ? mt : 0;
        seq = m / a.tps;
        t0 = (m - seq * a.tps) * kTO;  // first output time of the tile
        c0 = (s % a.ntiles) * kTN;
    }
};

__global__ void __launch_bounds__(kThreads, 1) k_inproj_conv3(Inproj a) {
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // uniform: LDS and column addresses stay scalar
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t G = gridDim.x;
    const int nchunks = (int)(a.D / kKC);

    int64_t T = blockIdx.x;
    TileAt cur(a, T);
    if (!cur.valid) return;

    // fills: instruction q of this wave writes staged rows 32 q + 8 wave .. + 7, lane l
    // the slot l % 8 of row 32 q + 8 wave + l / 8, which holds segment
    // (l % 8) ^ swizzle(row) of the source row. Byte offsets below 2^31 (host check).
    const BufRsrc wr = buf_rsrc(a.w);
    BufRsrc xr;
    uint32_t xoff[8], woff[8];
    auto target = [&](const TileAt& tl) {
        xr = buf_rsrc(a.x + tl.seq * a.L * a.D);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t r = 32 * q + 8 * wave + (lane >> 3);
            const uint32_t seg = (uint32_t)(lane & 7) ^ seg_swizzle(r);
            int64_t t = tl.t0 - kTH + r;
            t = t < 0 ? 0 : (t >= a.L ? a.L - 1 : t);
            int64_t c = tl.c0 + r;
            c = c >= a.C ? a.C - 1 : c;
            xoff[q] = (uint32_t)(t * a.D * 2) + 16 * seg;
            woff[q] = (uint32_t)(c * a.D * 2) + 16 * seg;
        }
    };
    auto fill = [&](int buf, int chunk) {
        unsigned char* st = lds_raw + buf * kBufStride;
        const int sk = chunk * kKC * 2;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (LdsPtr)(st + (32 * q + 8 * wave) * 128), 16, (int)xoff[q],
                                                     sk, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (LdsPtr)(st + kOpBytes + (32 * q + 8 * wave) * 128), 16,
                                                     (int)woff[q], sk, 0, 0);
        }
    };
    // taps and b_in of tile column tid (channel c0 + tid), loaded when a tile starts
    auto params = [&](const TileAt& tl) {
        const int64_t c = tl.c0 + tid;
        return c < a.C ? make_float4(a.w3[3 * c], a.w3[3 * c + 1], a.w3[3 * c + 2], bf16_to_f32(a.b[c]))
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    };

    // fragment reads: block i of A is staged rows wm*128 + 32 i + l % 32, segment
    // 2 ks + l / 32; its byte address is abase[i] ^ (ks << 5) (the XOR only touches
    // the slot bits). The same for block j of B with wn.
    uint32_t abase[4], bbase[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t ra = wm * kWM + 32 * i + (lane & 31);
        const uint32_t rb = wn * kWN + 32 * i + (lane & 31);
        abase[i] = ra * 128 + ((((uint32_t)lane >> 5) ^ seg_swizzle(ra)) << 4);
        bbase[i] = kOpBytes + rb * 128 + ((((uint32_t)lane >> 5) ^ seg_swizzle(rb)) << 4);
    }
    bf16x8 fa[2][4], fb[2][4];
    auto frag = [&](int slot, const unsigned char* st, int ks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[slot][i] = *reinterpret_cast<const bf16x8*>(st + (abase[i] ^ (ks << 5)));
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[slot][j] = *reinterpret_cast<const bf16x8*>(st + (bbase[j] ^ (ks << 5)));
    };
    f32x16 acc[4][4];
    auto mma = [&](int slot) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j], acc[i][j], 0, 0, 0);
    };

    target(cur);
    float4 prm = params(cur);
    fill(0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's fills are in LDS
    __syncthreads();                     // and everyone's
    int buf = 0;                         // buffer of the chunk being multiplied
    bool more = true;                    // another tile follows the current one
    TileAt nxt(a, T + G);
    if (nchunks > 1) {
        fill(1, 1);
    } else if (nxt.valid) {
        target(nxt);
        fill(1, 0);
    }
    frag(0, lds_raw, 0);

    while (true) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
        for (int ch = 0; ch < nchunks; ++ch) {
            // Chunk ch of the tile sits in buffer buf; the next chunk of the walk is in
            // flight to the other buffer. The barrier that hands a chunk over sits before
            // the last step's 16 products, so that the barrier wait and the first
            // fragment reads of the next chunk overlap matrix work. Fragments of step ks
            // are read while the products of step ks - 1 run (register slots ks & 1).
            const unsigned char* st = lds_raw + buf * kBufStride;
#pragma unroll
            for (int ks = 0; ks < kKC / 16 - 1; ++ks) {
                frag((ks + 1) & 1, st, ks + 1);
                mma(ks & 1);
            }
            // issue order: a fragment read, then two products
#pragma unroll
            for (int n = 0; n < 3 * 8; ++n) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of buffer buf are done
            const bool last = ch + 1 == nchunks;
            if (!last || nxt.valid) {
                // the next chunk (this tile's, or the next tile's first) has landed for
                // everyone after the barrier, and nobody reads buffer buf any more
                __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
                __syncthreads();
                if (ch + 2 < nchunks) {
                    fill(buf, ch + 2);
                } else if (ch + 2 == nchunks && nxt.valid) {
                    target(nxt);  // this tile's fills are all issued
                    fill(buf, 0);
                }
                if (!last) frag(0, lds_raw + (buf ^ 1) * kBufStride, 0);
            } else {
                more = false;
                __syncthreads();  // the epilogue below overwrites buffer buf
            }
            mma((kKC / 16 - 1) & 1);
            if (!last) buf ^= 1;
        }

        // epilogue in four rounds over buffer buf: round h lays out block j = h of every
        // wave (tile columns wn*128 + 32 h .. + 31) column by column, E[col][row] over
        // all 256 rows (column pitch 260 floats: the float4 writes of 16 consecutive
        // columns start on distinct banks); then each wave forms the outputs of 16
        // columns: lane l the four times t0 + 4l .. t0 + 4l + 3 from rows 4l + 2 .. 4l + 7
        float* E = reinterpret_cast<float*>(lds_raw + buf * kBufStride);
        float4* P = reinterpret_cast<float4*>(lds_raw + kParamOff);
        P[tid] = prm;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            if (h > 0) __syncthreads();  // the previous round's reads are done
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
            // lane l: the four times t0 + 4l .. + 3 (rows 4l + 4 .. 4l + 7); a column's
            // outputs start at a scalar address, the lane adds 8 l bytes
            const int t = (int)cur.t0 + 4 * lane;
            // L is a multiple of 4: all four times of a lane are in range or none is
            // (the column's buffer ends at time L; lane 63 holds no output)
            const uint32_t voff = lane < kTO / 4 ? 8u * lane : 0x80000000u;
            const uint16_t* useq = a.u + cur.seq * a.C * a.L;
            const uint32_t colbytes = (uint32_t)(a.L - cur.t0) * 2;
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
                    const int64_t c = cur.c0 + (col >> 5) * kWN + 32 * h + (col & 31);
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
                        const BufRsrc ur =
                            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(useq + c * a.L + cur.t0), 0,
                                                              (int)colbytes, 0x00020000);
                        typedef unsigned int U2 __attribute__((ext_vector_type(2)));
                        const U2 v = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
                        __builtin_amdgcn_raw_buffer_store_b64(v, ur, (int)voff, 0, 0);
                    }
                }
            }
        }
        if (!more) break;

        // next tile: its first chunk is in buffer buf ^ 1 (waited for before the
        // epilogue); the buffer of the epilogue takes the chunk after it once every
        // wave is done with the epilogue
        buf ^= 1;
        T += G;
        cur = nxt;
        nxt = TileAt(a, T + G);
        prm = params(cur);
        __syncthreads();
        if (nchunks > 1) {
            fill(buf ^ 1, 1);
        } else if (nxt.valid) {
            target(nxt);
            fill(buf ^ 1, 0);
        }
        frag(0, lds_raw + buf * kBufStride, 0);
    }
}

}  // namespace

bool inproj_supported(int64_t D) { return D >= kKC && D % kKC == 0; }
static_assert(kTO % 4 == 0, "tiles start at multiples of four times");

hipError_t launch_inproj_conv3(const uint16_t* x, const uint16_t* w, const uint16_t* b, const float* w3,
                               uint16_t* u, int64_t B, int64_t L, int64_t D, int64_t C, hipStream_t st) {
    if (!inproj_supported(D) || L % 4 != 0) return hipErrorInvalidValue;
    // byte offsets of rows within a sequence of x and within w are 32-bit in the kernel
    if (L * D * 2 >= (int64_t(1) << 31) || C * D * 2 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    Inproj a{x, w, b, w3, u, L, D, C, (L + kTO - 1) / kTO, 0, (C + kTN - 1) / kTN};
    a.mtiles = B * a.tps;
    const int64_t slots = ((a.mtiles + 7) / 8) * 8 * a.ntiles;  // tile indices of the walk
    static int cus = 0;
    static bool attr = false;
    if (!attr) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void*)k_inproj_conv3, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    kLdsBytes);
        if (e != hipSuccess) return e;
        attr = true;
    }
    // one workgroup per compute unit, a multiple of 8 (one per XCD in turn)
    int64_t grid = (cus / 8) * 8;
    if (grid < 8) grid = 8;
    if (grid > slots) grid = slots;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_inproj_conv3, dim3((unsigned)grid), dim3(kThreads), kLdsBytes, st, a);
    return hipGetLastError();
}

}  // namespace hy
