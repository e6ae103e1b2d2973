// Internal launch interface between the C-ABI layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hy {

// LDS path: one workgroup per (b, d) row, L/E threads holding E values each,
// the whole packed transform (L complex values plus one pad slot per 16) in LDS.
// Build-time tuning knobs of the LDS path (defaults chosen by measurement):
//   HY_LDS_E32_FROM   smallest log2 L that uses 32 values per thread (else 16)
//   HY_LDS_PREFETCH   fetch the spectrum before the forward transform (1) or in
//                     the pair step (0)
//   HY_LDS_PREFETCH_GATE  fetch the final gate's input rows before the inverse
//                     transform (1) or after it (0)
// and of the four-step path:
//   HY_FS_CB          columns per pass A / pass C workgroup
#ifndef HY_LDS_E32_FROM
#define HY_LDS_E32_FROM 14
#endif
#ifndef HY_LDS_PREFETCH
#define HY_LDS_PREFETCH 1
#endif
#ifndef HY_LDS_PREFETCH_GATE
#define HY_LDS_PREFETCH_GATE 1
#endif
#ifndef HY_FS_CB
#define HY_FS_CB 16
#endif
// HY_PART_G         output blocks per workgroup of the partitioned path's pass 2
#ifndef HY_PART_G
#define HY_PART_G 4
#endif
template <int LOGL>
struct LdsCfg {
    static constexpr int L = 1 << LOGL;
    static constexpr int E = LOGL >= HY_LDS_E32_FROM ? 32 : 16;
    static constexpr int THREADS = L / E;
    // waves per SIMD when as many workgroups share a CU as its 160 KB of LDS
    // allows (one padded transform each), capped at 8: the register budget asked
    // of the compiler is the one that keeps them all resident
    static constexpr int LDS_BYTES = (L + L / 16) * 8;
    static constexpr int BLOCKS = (160 * 1024) / LDS_BYTES;
    static constexpr int WAVES_RAW = BLOCKS * (THREADS / 64) / 4;
    static constexpr int MIN_WAVES = WAVES_RAW < 1 ? 1 : (WAVES_RAW > 8 ? 8 : WAVES_RAW);
};
constexpr int kLdsMinLog = 4;   // L = 16: one thread per 16 values
constexpr int kLdsMaxLog = 14;  // L = 16384: 139,264 bytes of LDS

// Four-step path geometry for L = L1 * L2.
template <int LOG1, int LOG2>
struct FsCfg {
    static constexpr int L1 = 1 << LOG1;
    static constexpr int L2 = 1 << LOG2;
    static constexpr int T1 = L1 / 16;                 // threads per column transform
    static constexpr int T2 = L2 / 16;                 // threads per row transform
    static constexpr int CB = HY_FS_CB;                // columns per pass A/C workgroup
    static constexpr int CP = CB + 1;                  // LDS pitch of the column tile
    static constexpr int COL_THREADS = CB * T1;
    static constexpr int U0 = 256 / (2 * T2);
    static constexpr int UNITS = U0 < 1 ? 1 : (U0 > L1 / 2 ? L1 / 2 : U0);  // row pairs per pass B workgroup
    static constexpr int ROW_THREADS = UNITS * 2 * T2;
    static constexpr int RP = L2 + L2 / 16;            // padded LDS row length
};
constexpr int kFsMinLog = 8;
constexpr int kFsMaxLog = 20;

struct LdsArgs {
    const void* u;
    const float* w3;
    const float2* spec;
    const float* bias;
    void* y;
    const float2* tw;     // Stockham twiddles for length L
    const float2* wpair;  // W_{2L}^k, k = 0..L/2
    int B, D, N;
    bool bf16;
    int64_t sbs = 0;      // spectrum batch stride (complex values): 0 = one spectrum for every b
    bool circ = false;    // circular convolution of 2L-sample rows (no zero padding)
};

struct FsTables {
    const float2* tw1;    // Stockham twiddles for length L1
    const float2* tw2;    // Stockham twiddles for length L2
    const float2* tbase;  // [t][m2] = W_L^(t*m2), t < L1/16, m2 < L2
    const float2* tstep;  // [e][m2] = W_L^((L1/16)*e*m2), e < 16, m2 < L2
    const float2* pa;     // W_{2L}^k1, k1 < L1
    const float2* pb;     // W_{2L}^(L1*k2), k2 < L2
};

struct FsArgs {
    const void* u;
    const float* w3;
    const float2* spec;
    const float* bias;
    void* y;
    float2* ws;  // nrows * L complex values
    FsTables tb;
    int D, N;
    bool bf16;
    int64_t sbs = 0;  // spectrum batch stride (complex values): 0 = one spectrum for every b
    bool circ = false;  // circular convolution of 2L-sample rows (no zero padding)
};

hipError_t launch_lds_forward(int logL, const LdsArgs& a, hipStream_t st);
hipError_t launch_lds_spectrum(int logL, const float* h, float2* spec, int64_t rows, const float2* tw,
                               const float2* wpair, hipStream_t st, bool circ = false);
hipError_t launch_fs_forward_chunk(int logL, const FsArgs& a, int64_t row0, int64_t nrows, hipStream_t st,
                                   hipEvent_t* marks = nullptr);
// Pipelined four-step forward over chunks of R rows: one launch per chunk plus
// 2N-2, the workspace holding 2N-1 tile slots of R rows each. With `marks`, an
// event is recorded before the first launch and after every launch.
bool fs_pipe_supported(int logL);
hipError_t launch_fs_forward_pipelined(int logL, const FsArgs& a, int64_t rows, int64_t R, hipStream_t st,
                                       hipEvent_t* marks = nullptr);
hipError_t launch_fs_spectrum(int logL, const float* h, float2* spec, int64_t rows, const FsTables& tb,
                              hipStream_t st, bool circ = false);
void fs_split(int logL, int* log1, int* log2);

// Partitioned path: blocks of Q = 2^kPartLogQ taps, L from 2Q to 2^kPartMaxLog.
constexpr int kPartLogQ = 12;
constexpr int kPartMinLog = kPartLogQ + 1;
constexpr int kPartMaxLog = 17;
struct PartArgs {
    const void* u;
    const float* w3;
    const float2* spec;  // [o][d][block][Q] filter block spectra (the LDS layout for Q samples)
    const float* bias;
    void* y;
    float2* X;           // window spectra of the chunk's rows, [row][window][Q]
    float* vb;           // gated output of the previous step, [row][L] (order > 2)
    const float2* tw;    // Stockham twiddles for length Q
    const float2* wpair; // W_{2Q}^k, k = 0..Q/2
    int D, N, P;         // P = L / Q
    bool bf16;
    int64_t sbs;         // spectrum batch stride (complex values): 0 = one spectrum for every b
};
hipError_t launch_part_forward_chunk(const PartArgs& a, int64_t row0, int64_t n, hipStream_t st, hipEvent_t* marks);
int part_group(int P);  // output blocks per pass 2 workgroup

int fs_row_units(int logL);

// Fused input projection and short conv on the bf16 matrix cores (inproj.hip):
// uc[b][c][t] = short_conv_c(x[b] w_in^T + b_in)[t] for C = (N+1)*D channels.
bool inproj_supported(int64_t D);
hipError_t launch_inproj_conv3(const uint16_t* x, const uint16_t* w, const uint16_t* b, const float* w3,
                               uint16_t* u, int64_t B, int64_t L, int64_t D, int64_t C, hipStream_t st);

}  // namespace hy
