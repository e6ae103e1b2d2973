// Output projection of the Hyena operator on the bf16 matrix cores of gfx950
// (HyenaDNA walkthrough, section 2.1: the rearrange back to tokens-first and the
// output projection). For every sequence b, time t < L and output channel n < D:
//   out[b][t][n] = sum_k y[b][k][t] w_out[n][k] + b_out[n]
// with y channels-first (the hot path's output) and out tokens-first. One launch
// covers every sequence: per sequence a GEMM with M = D rows (n), N = L columns
// (t) and K = D, bf16 operands and fp32 accumulation, rounded once to bf16.
//
// Tiles: 256 output channels x 256 times per workgroup of four waves (2 x 2, one
// per SIMD), each wave 128 x 128 as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16 (256
// fp32 accumulators per lane, in the accumulation registers). K runs in chunks of
// 64, double buffered in LDS, both operands filled by buffer loads that write LDS
// directly. The w_out rows (k contiguous) are staged as 128-byte rows with their
// eight 16-byte segments permuted by an XOR of the row (as in the input
// projection). y is k-major (t contiguous) and is staged as it is: 64 rows of 256
// times (512 bytes), the 16-byte segments of row k permuted by XOR with 4 (k % 4).
// The matrix cores take k-contiguous fragments; gfx950's transposing LDS read
// (ds_read_b64_tr_b16) gives them: within each group of 16 lanes, lane i receives
// element i % 4 of the 8-byte pieces addressed by lanes i/4, i/4 + 4, i/4 + 8 and
// i/4 + 12, so with lane r addressing row k0 + r/4 at times t0 + 4 (r % 4), lane i
// holds 4 consecutive k of time t0 + i; two such reads make a fragment. Rows past
// D and times past L are filled from a clamped, valid row and never stored.
//
// The accumulator layout puts four consecutive output channels of one time in a
// lane (D[row][col] with row = 8 (i / 4) + 4 (l / 32) + i % 4, col = l % 32 for
// lane l and element i): the epilogue adds b_out, lays the tile out in LDS as
// bf16 rows of one time and stores them as 16 bytes per lane, 1 KiB contiguous per
// store instruction.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fft_core.hpp"
#include "kernels.hpp"
#include "outproj.hpp"

namespace hy {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* LdsPtr;

constexpr int kTR = 256;       // tile rows: output channels n
constexpr int kTC = 256;       // tile columns: times t
constexpr int kKC = 64;        // K per staged chunk: 128-byte operand rows
constexpr int kThreads = 256;  // four waves: 2 (rows) x 2 (columns), one per SIMD
constexpr int kWR = 128, kWC = 128;            // rows and columns per wave
constexpr int kOpBytes = kTR * kKC * 2;        // one staged operand tile (32 KiB)
constexpr int kStageBytes = 2 * kOpBytes;      // w_out rows, then y columns
constexpr int kOP = kTR * 2 + 16;              // epilogue row pitch (bytes): one time, 256 channels
constexpr int kBiasOff = kTC * kOP;            // b_out of the tile's rows, fp32
constexpr int kLdsBytes = kBiasOff + kTR * 4;  // 136,192 bytes
static_assert(kBiasOff >= 2 * kStageBytes, "the epilogue tile covers both chunk buffers");
static_assert(kTR == 2 * kWR && kTC == 2 * kWC && kTC == kTR, "tile shape");

__device__ __forceinline__ uint32_t seg_swizzle(uint32_t r) { return (r ^ (r >> 3)) & 7u; }

struct Outproj {
    const uint16_t* y;   // [B][D][L]
    const uint16_t* w;   // [D][D]: w_out[n][k]
    const uint16_t* bo;  // [D]
    uint16_t* out;       // [B][L][D]
    int64_t L, D;
    int64_t ttiles, ntiles, tiles;  // time tiles per sequence, channel tiles, all tiles
};

__global__ void __launch_bounds__(kThreads, 1) k_outproj(Outproj a) {
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)lds_raw;
    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int wm = wave >> 1, wn = wave & 1;
    // XCD-aware order: hardware sends workgroup i to XCD i % 8; the channel tiles of
    // one time tile run back to back on one XCD and share its columns of y in L2
    const int64_t bid = blockIdx.x;
    const int64_t s = bid >> 3;
    const int64_t tt = (s / a.ntiles) * 8 + (bid & 7);  // time tile over all sequences
    if (tt >= a.tiles) return;
    const int64_t seq = tt / a.ttiles;
    const int64_t t0 = (tt - seq * a.ttiles) * kTC;
    const int64_t n0 = (s % a.ntiles) * kTR;
    const int nchunks = (int)(a.D / kKC);

    // w_out fills: instruction q of this wave writes staged rows 32 q + 8 wave .. + 7
    // (lane l: slot l % 8 of row 32 q + 8 wave + l / 8, holding segment
    // (l % 8) ^ swizzle(row) of that row of w_out)
    const BufRsrc wr = buf_rsrc(a.w);
    uint32_t woff[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const uint32_t r = 32 * q + 8 * wave + (lane >> 3);
        int64_t n = n0 + r;
        n = n >= a.D ? a.D - 1 : n;
        woff[q] = (uint32_t)(n * a.D * 2) + 16 * ((uint32_t)(lane & 7) ^ seg_swizzle(r));
    }
    // y fills: instruction q of this wave writes staged rows (k) 8 q + 2 wave and the
    // next one, 1 KiB; lane l slot l % 32 of row 8 q + 2 wave + l / 32, which holds
    // times 8 seg .. 8 seg + 7 for seg = (l % 32) ^ (4 (row % 4))
    const BufRsrc yr = buf_rsrc(a.y + seq * a.D * a.L);
    uint32_t yoff[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const uint32_t r = 8 * q + 2 * wave + (lane >> 5);
        int64_t t = t0 + 8 * ((uint32_t)(lane & 31) ^ (4 * (r & 3)));
        t = t >= a.L ? a.L - 8 : t;  // L is a multiple of 8
        yoff[q] = (uint32_t)((r * a.L + t) * 2);
    }
    auto fill = [&](int buf, int chunk) {
        unsigned char* st = lds_raw + buf * kStageBytes;
        const int skw = chunk * kKC * 2;
        const int sky = (int)((int64_t)chunk * kKC * a.L * 2);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (LdsPtr)(st + (32 * q + 8 * wave) * 128), 16, (int)woff[q],
                                                     skw, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(yr, (LdsPtr)(st + kOpBytes + (8 * q + 2 * wave) * 512), 16,
                                                     (int)yoff[q], sky, 0, 0);
        }
    };

    // fragment reads: block i of A (w_out rows) is staged rows wm*128 + 32 i + l % 32,
    // segment 2 ks + l / 32, at byte abase[i] ^ (ks << 5). Block j of B (times
    // wn*128 + 32 j ..) takes two transposing reads per step: lane l (r = l % 16)
    // addresses row k = 16 ks + 8 (l / 32) + 4 h + r / 4 (h = 0, 1) at time
    // tb = wn*128 + 32 j + 16 ((l / 16) % 2) + 4 (r % 4), i.e. byte
    // 512 k + 16 ((tb / 8) ^ 4 (k % 4)) + 8 ((tb / 4) % 2); the row's k % 4 is r / 4,
    // so the byte offset is bbase[j] + 512 (16 ks + 4 h)
    uint32_t abase[4], bbase[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t ra = wm * kWR + 32 * i + (lane & 31);
        abase[i] = ra * 128 + ((((uint32_t)lane >> 5) ^ seg_swizzle(ra)) << 4);
        const uint32_t r = lane & 15;
        const uint32_t tb = wn * kWC + 32 * i + 16 * ((lane >> 4) & 1) + 4 * (r & 3);
        const uint32_t k = 8 * (lane >> 5) + (r >> 2);
        bbase[i] = kOpBytes + 512 * k + 16 * ((tb >> 3) ^ (4 * (r >> 2))) + 8 * ((tb >> 2) & 1);
    }
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    bf16x8 fa[2][4], fb[2][4];
    auto frag = [&](int slot, const unsigned char* st, int ks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[slot][i] = *reinterpret_cast<const bf16x8*>(st + (abase[i] ^ (ks << 5)));
        // the eight transposing reads of the step in one block that also waits for
        // them (the reads' intrinsic would make every read wait for the next chunk's
        // fills in flight; those go to the other buffer)
        const uint32_t s0 = (uint32_t)(uintptr_t)(st - lds_raw) + 512u * 16u * ks;
        typedef double V2;  // 8 bytes: two registers
        V2 r[8];
        asm volatile(
            "ds_read_b64_tr_b16 %0, %8\n"
            "ds_read_b64_tr_b16 %1, %8 offset:2048\n"
            "ds_read_b64_tr_b16 %2, %9\n"
            "ds_read_b64_tr_b16 %3, %9 offset:2048\n"
            "ds_read_b64_tr_b16 %4, %10\n"
            "ds_read_b64_tr_b16 %5, %10 offset:2048\n"
            "ds_read_b64_tr_b16 %6, %11\n"
            "ds_read_b64_tr_b16 %7, %11 offset:2048\n"
            "s_waitcnt lgkmcnt(0)"
            : "=v"(r[0]), "=v"(r[1]), "=v"(r[2]), "=v"(r[3]), "=v"(r[4]), "=v"(r[5]), "=v"(r[6]), "=v"(r[7])
            : "v"(lds_base + s0 + bbase[0]), "v"(lds_base + s0 + bbase[1]), "v"(lds_base + s0 + bbase[2]),
              "v"(lds_base + s0 + bbase[3])
            : "memory");
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const V2 both[2] = {r[2 * j], r[2 * j + 1]};
            fb[slot][j] = __builtin_bit_cast(bf16x8, both);
        }
    };
    auto mma = [&](int slot) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j], acc[i][j], 0, 0, 0);
    };

    // b_out of the tile's rows
    {
        const int64_t n = n0 + tid;
        reinterpret_cast<float*>(lds_raw + kBiasOff)[tid] =
            n < a.D ? __uint_as_float((uint32_t)a.bo[n] << 16) : 0.f;
    }
    fill(0, 0);
    for (int ch = 0; ch < nchunks; ++ch) {
        const int buf = ch & 1;
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's fills of chunk ch are in LDS
        __syncthreads();                     // everyone's are, and nobody reads buffer buf ^ 1 any more
        if (ch + 1 < nchunks) fill(buf ^ 1, ch + 1);
        const unsigned char* st = lds_raw + buf * kStageBytes;
        frag(0, st, 0);
#pragma unroll
        for (int ks = 0; ks < kKC / 16; ++ks) {
            if (ks + 1 < kKC / 16) frag((ks + 1) & 1, st, ks + 1);
            mma(ks & 1);
        }
    }

    // epilogue: lane l of block (i, j) holds times wn*128 + 32 j + l % 32 and, for
    // g < 4, channels wm*128 + 32 i + 8 g + 4 (l / 32) .. + 3 of the tile: with b_out
    // added and rounded to bf16 they go to LDS as rows of one time (pitch 528 bytes,
    // so the 8-byte writes of 16 consecutive times start on distinct banks), then
    // each lane stores 16 bytes: one store instruction writes 1 KiB, two rows of 512
    // contiguous bytes of out
    __syncthreads();  // the last chunk's reads are done
    const float* bias = reinterpret_cast<const float*>(lds_raw + kBiasOff);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int rl = wm * kWR + 32 * i + 8 * g + 4 * (lane >> 5);  // tile row of the lane's first channel
            const float4 bv = *reinterpret_cast<const float4*>(bias + rl);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tl = wn * kWC + 32 * j + (lane & 31);
                const f32x16& v = acc[i][j];
                *reinterpret_cast<uint2*>(lds_raw + tl * kOP + rl * 2) =
                    make_uint2(pack_bf16x2(v[4 * g] + bv.x, v[4 * g + 1] + bv.y),
                               pack_bf16x2(v[4 * g + 2] + bv.z, v[4 * g + 3] + bv.w));
            }
        }
    __syncthreads();
    const BufRsrc orr = __builtin_amdgcn_make_buffer_rsrc(a.out + seq * a.L * a.D, 0,
                                                          (int)(a.L * a.D * 2), 0x00020000);
    const int nc = 8 * (lane & 31);  // the lane's 8 channels in the row
    // D is a multiple of 64: all 8 channels or none; times past L fall outside the buffer
    const bool on = n0 + nc < a.D;
#pragma unroll 8
    for (int q = 0; q < kTC / 8; ++q) {
        const int tl = 8 * q + 2 * wave + (lane >> 5);
        const uint4 v = *reinterpret_cast<const uint4*>(lds_raw + tl * kOP + nc * 2);
        const int64_t t = t0 + tl;
        const uint32_t off = on && t < a.L ? (uint32_t)((t * a.D + n0 + nc) * 2) : 0x80000000u;
        typedef unsigned int U4 __attribute__((ext_vector_type(4)));
        const U4 w4 = {v.x, v.y, v.z, v.w};
        __builtin_amdgcn_raw_buffer_store_b128(w4, orr, (int)off, 0, 0);
    }
}

}  // namespace

bool outproj_supported(int64_t D, int64_t L) { return D >= kKC && D % kKC == 0 && L >= 8 && L % 8 == 0; }

hipError_t launch_outproj(const uint16_t* y, const uint16_t* w, const uint16_t* bo, uint16_t* out, int64_t B,
                          int64_t L, int64_t D, hipStream_t st) {
    if (!outproj_supported(D, L)) return hipErrorInvalidValue;
    // byte offsets within one sequence of y and out, and within w_out, are 32-bit
    if (L * D * 2 >= (int64_t(1) << 31) || D * D * 2 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    Outproj a{y, w, bo, out, L, D, (L + kTC - 1) / kTC, (D + kTR - 1) / kTR, 0};
    a.tiles = B * a.ttiles;
    const int64_t grid = ((a.tiles + 7) / 8) * 8 * a.ntiles;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    static bool attr = false;
    if (!attr) {
        const hipError_t e =
            hipFuncSetAttribute((const void*)k_outproj, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        if (e != hipSuccess) return e;
        attr = true;
    }
    hipLaunchKernelGGL(k_outproj, dim3((unsigned)grid), dim3(kThreads), kLdsBytes, st, a);
    return hipGetLastError();
}

}  // namespace hy
