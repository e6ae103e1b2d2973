/*
 * libhyena — the Hyena operator forward hot path, its backward, the whole
 * operator forward, the implicit filter generator, and the HyenaND variants
 * (per-sample filters, circular plans, gated 2-D and 3-D long convolutions), on
 * AMD MI355X (gfx950).
 *
 * The operator (HyenaDNA walkthrough, section 2.1, the Hyena operator module and
 * its forward pass; section 2.2, the long-filter module and its FFT convolution).
 * For each channel d < D and time t < L, with u the in-projected activation of
 * (N+1)*D channels:
 *   uc[c][t] = w[c][0] u[c][t-2] + w[c][1] u[c][t-1] + w[c][2] u[c][t],
 *              u[c][t'] = 0 for t' < 0 (a causal width-3 depthwise filter);
 *   x_i[d] = uc[i*D + d] for i < N (the gates), v_0[d] = uc[N*D + d] (the value);
 *   for o = 0 .. N-2 (the gates taken from x_{N-1} down to x_1):
 *       g_o     = v_o (.) x_{N-1-o}
 *       v_{o+1} = h[o] * g_o + bias[o] g_o
 *   y = v_{N-1} (.) x_0,
 * with (.) the elementwise product and * the causal per-channel long convolution
 *   (h * g)[t] = sum_{s <= t} h[s] g[t - s],
 * evaluated by FFT on the sequence zero-padded to 2L (the HyenaND summary's
 * boundary handling; the Hyena Hierarchy concept page, section 3.2, FFT
 * acceleration). hyena_operator_forward adds the module's in/out projections and
 * its (B, L, D) <-> (B, D, L) transposes around the path; dropout is the identity; the
 * short Conv1d bias is taken as zero.
 *
 * Conventions for every call:
 *  - Device pointers are plain device memory on the device that was current when
 *    the plan was created; that device must be current for every later call.
 *    The caller owns every buffer; libhyena never frees caller memory.
 *  - Tensors are dense and row-major (C order) with the shapes given below and
 *    16-byte aligned base pointers. Outputs must not alias inputs.
 *  - Calls that take a stream enqueue work on it and return without
 *    synchronising; results are ready when the stream reaches that point.
 *  - Errors are reported by return value; nothing throws across this ABI.
 *    Argument errors are detected on the host before any HIP call is made.
 *  - A plan is immutable after creation (apart from the GEMM state the operator
 *    entry points attach under a lock) and may be shared between host threads;
 *    concurrent calls need distinct workspaces and outputs.
 */
#ifndef LIBHYENA_HYENA_H
#define LIBHYENA_HYENA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct hyena_plan_s* hyena_plan_t; /* opaque */

/* Element type of u_proj and y. All parameters (short_w, h, bias) and every
 * intermediate are fp32; bf16 outputs are rounded to nearest even. */
typedef enum { HYENA_F32 = 0, HYENA_BF16 = 1 } hyena_dtype_t;

typedef enum {
    HYENA_OK = 0,
    HYENA_ERR_INVALID_ARG = 1, /* NULL pointer, bad size or shape, misaligned pointer */
    HYENA_ERR_UNSUPPORTED = 2, /* valid request outside what the library implements */
    HYENA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    HYENA_ERR_DEVICE = 4       /* no usable HIP device, allocation or launch failure */
} hyena_status_t;

/* Which kernel family runs a plan.
 *   LDS       one launch; the whole transform of a (b, d) row stays in LDS
 *             (L <= 16384).
 *   FOURSTEP  three passes per recurrence step (column FFTs, row FFTs with
 *             the spectrum multiply, inverse columns with the gate) over
 *             chunks of rows; any order, 256 <= L <= 2^20. At order 2 with
 *             L = 2^16 or 2^17 the chunks are pipelined: one launch runs the
 *             three passes on three consecutive chunks.
 *   PARTITIONED  the same causal convolution with the filter cut into
 *             blocks of Q = 4096 taps (uniformly partitioned overlap-save):
 *             two LDS-resident launches per recurrence step (transforms of
 *             2Q-sample windows of v; block-Toeplitz sums of window and
 *             filter-block spectra, inverse transforms and the gate), no
 *             transposed tile. Zero-padded plans with 8192 <= L <= 131072;
 *             hyena_backward does not take these plans.
 * AUTO picks LDS when L <= 16384 and FOURSTEP otherwise. */
typedef enum {
    HYENA_PATH_AUTO = 0,
    HYENA_PATH_LDS = 1,
    HYENA_PATH_FOURSTEP = 2,
    /* 3 is unused (HYENA_ERR_INVALID_ARG) */
    HYENA_PATH_PARTITIONED = 4
} hyena_path_t;

/* Create a plan for sequence length L, operator width D and recurrence order
 * N = `order` (N-1 long filters, N gates). Requirements: L a power of two in
 * [16, 2^20], D >= 1, 2 <= order <= 8, dtype one of hyena_dtype_t.
 * Builds the twiddle tables on the host in fp64 and uploads them to the current
 * device (the plan owns that memory; hyena_plan_destroy releases it).
 * Returns HYENA_ERR_INVALID_ARG / HYENA_ERR_UNSUPPORTED for bad arguments,
 * HYENA_ERR_DEVICE when no HIP device is usable. *out is set only on success. */
hyena_status_t hyena_plan_create(hyena_plan_t* out, int64_t L, int64_t D, int order, hyena_dtype_t dtype);

/* As hyena_plan_create, with an explicit kernel family. HYENA_PATH_LDS needs
 * L <= 16384; HYENA_PATH_FOURSTEP needs L >= 256; HYENA_PATH_PARTITIONED needs
 * 8192 <= L <= 131072 and no flags. The spectrum layout depends on the
 * path (PARTITIONED holds the 2Q-point spectra of
 * each filter's L/Q blocks, [o][d][block][Q], in the LDS layout), so a spectrum
 * must be made by a plan whose path uses the same layout as the plan that
 * consumes it. */
hyena_status_t hyena_plan_create_path(hyena_plan_t* out, int64_t L, int64_t D, int order, hyena_dtype_t dtype,
                                      hyena_path_t path);

/* Plan options (bit flags for hyena_plan_create_ex). */
enum {
    /* Circular long convolution (the HyenaND summary's boundary handling offers
     * circular convolution for periodic data besides zero padding to double the
     * grid):  conv(v, h)[t] = sum_{s < L} h[s] v[(t - s) mod L]. The L samples are
     * transformed as they are (an L-point real transform, no zero padding); the
     * short conv keeps its causal zero padding. Requires L >= 32; the LDS path
     * serves L <= 32768. hyena_backward takes circular plans on the LDS path. */
    HYENA_FLAG_CIRCULAR = 1
};

/* As hyena_plan_create_path, with option flags (0 or HYENA_FLAG_CIRCULAR).
 * HYENA_ERR_INVALID_ARG for unknown flag bits; HYENA_ERR_UNSUPPORTED for a
 * circular plan with L < 32 or on the partitioned path. */
hyena_status_t hyena_plan_create_ex(hyena_plan_t* out, int64_t L, int64_t D, int order, hyena_dtype_t dtype,
                                    hyena_path_t path, uint32_t flags);

/* Release a plan and its device tables. NULL is a no-op returning HYENA_OK.
 * The caller must ensure no enqueued work still uses the plan. */
hyena_status_t hyena_plan_destroy(hyena_plan_t plan);

/* The path a plan resolved to (HYENA_PATH_LDS, HYENA_PATH_FOURSTEP or
 * HYENA_PATH_PARTITIONED), or HYENA_PATH_AUTO for a NULL plan. */
hyena_path_t hyena_plan_path(hyena_plan_t plan);

/* Bytes of the opaque spectrum buffer: (N-1) * D * L complex fp32 values, i.e.
 * 8 * (N-1) * D * L (L/2 complex values per filter for a circular plan).
 * Returns 0 for a NULL plan. */
size_t hyena_spectrum_bytes(hyena_plan_t plan);

/* Workspace for a forward over batch B: 0 on the LDS path. On the four-step
 * path this is the recommended size, in tiles of 8*L bytes per (b, d) row held
 * in flight: at order 2 with L = 2^16 or 2^17, three tile slots of
 * min(B*D, 128) rows (the pipelined launches); otherwise up to 128 MiB of
 * tiles. Any workspace of at least 8*L bytes (one row) is accepted: a
 * pipelined forward needs three slots of min(B*D, 32) rows and otherwise runs
 * chunk by chunk, and a larger one lets more rows run per launch. The
 * partitioned path likewise, with 8*L bytes per row at order 2 and 12*L bytes
 * per row above (the gated output of a step is held for the next). The choice
 * of chunks never changes the result: every chunking gives the same bits.
 * Returns 0 for a NULL plan or B < 1. */
size_t hyena_workspace_bytes(hyena_plan_t plan, int64_t B);

/* The real FFT of the long filters, once per plan (the filter spectrum of the
 * causal convolution; HyenaDNA walkthrough section 2.2, fftconv).
 *   h    [N-1][D][L] fp32, device: filter o of channel d at h[(o*D + d)*L + t]
 *   spec device buffer of hyena_spectrum_bytes(plan) bytes, written in the
 *        plan's private layout (the 2L-point spectrum bins 0..L of each
 *        zero-padded filter, scaled by 2^-(log2 L + 2)).
 * Enqueued on `stream`. HYENA_ERR_INVALID_ARG for NULL pointers or misaligned
 * buffers; HYENA_ERR_DEVICE if the launch fails or the plan's device is not
 * current. */
hyena_status_t hyena_filter_spectrum(hyena_plan_t plan, const float* h, void* spec, hipStream_t stream);

/* Spectra of per-sample long filters, for input-dependent convolutions (the
 * HyenaND summary's methodology: kernels conditioned on each input sample, one
 * global FFT path). hyena_filter_spectrum for B filter sets at once:
 *   h    [B][N-1][D][L] fp32, device: the filters of sample b at h + b*(N-1)*D*L
 *   spec device buffer of B * hyena_spectrum_bytes(plan) bytes; sample b's
 *        spectrum starts at byte b * hyena_spectrum_bytes(plan).
 * Errors as hyena_filter_spectrum; HYENA_ERR_INVALID_ARG also for B < 1 or
 * B*(N-1)*D > 2^24. */
hyena_status_t hyena_filter_spectrum_batched(hyena_plan_t plan, int64_t B, const float* h, void* spec,
                                             hipStream_t stream);

/* The forward hot path for a batch of B sequences.
 *   u_proj  [B][(N+1)*D][L] of the plan dtype, device: channel i*D + d is gate
 *           x_i for i < N and channel N*D + d is the value v (the in-projected,
 *           rearranged activation)
 *   short_w [(N+1)*D][3] fp32, device: PyTorch Conv1d taps; uc[t] =
 *           w[0]*u[t-2] + w[1]*u[t-1] + w[2]*u[t] with u[t<0] = 0
 *   spec    from hyena_filter_spectrum of a plan with the same L, D, order, path
 *   bias    [N-1][D] fp32, device: the bias skip term of step o is bias[o][d]*v
 *   y       [B][D][L] of the plan dtype, device (output, before the transpose
 *           to [B][L][D])
 *   workspace / workspace_bytes: device scratch, at least 8*L bytes on the
 *           four-step path and 8*L (order 2) or 12*L bytes on the partitioned
 *           path (see hyena_workspace_bytes); ignored (may be NULL) on the LDS
 *           path. Contents on entry are irrelevant.
 * Enqueued on `stream`; no host synchronisation. Errors: HYENA_ERR_INVALID_ARG
 * (NULL/misaligned pointers, B < 1 or B*D*L too large), HYENA_ERR_WORKSPACE,
 * HYENA_ERR_DEVICE (launch failure, wrong current device). */
hyena_status_t hyena_forward(hyena_plan_t plan, int64_t B, const void* u_proj, const float* short_w,
                             const void* spec, const float* bias, void* y, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Parameters of the input-dependent kernel synthesis (HyenaND summary, method:
 * input-dependent kernels through registers and FiLM, kernel synthesis, kernel
 * parametrisation). With A = axes, W = width, M = layers, Z = zdim and
 * C = channels; all arrays fp32, row-major, device, 16-byte aligned:
 *   w_first  [W][A]      first layer, on the coordinates
 *   w_hidden [M-1][W][W] further layers (may be NULL when M = 1); row = output unit
 *   b_layer  [M][W]      layer biases
 *   omega    [M][W]      sine frequency of every hidden unit
 *   film_g [M][W][Z], film_gb [M][W]   FiLM scale  gamma_l = film_g[l] z + film_gb[l]
 *   film_b [M][W][Z], film_bb [M][W]   FiLM shift  beta_l  = film_b[l] z + film_bb[l]
 *   w_out [C][W], b_out [C]            affine output layer, one row per kernel
 *   win_mu [C][A], win_sigma [C][A]    Gaussian window of every kernel
 * Layer l maps h_l to h_{l+1} = sin(omega_l * (gamma_l * (W_l h_l + b_l) + beta_l))
 * with h_0 the coordinate c of a grid point; the kernel is
 *   K_k(c) = exp(-1/2 sum_i ((c_i - mu_ki) / sigma_ki)^2) * (w_out[k] . h_M + b_out[k]).
 * The grid has grid[i] points on axis i (axis 0 slowest; grid[i] for i >= axes is
 * ignored). Point j of a causal axis of n points sits at c = j / n; a signed axis
 * (bit i of signed_axes set) holds the wrapped offsets j (j < n/2) and j - n
 * (j >= n/2) at c = 2 * offset / n. 1-D Hyena filters use one causal axis of L
 * points with C = (N-1)*D (kernel o*D + d is filter o of channel d); the 2-D and
 * 3-D steps use signed axes on their kernel grid (2H x 2W, or H x W for a
 * circular plan) with C = D. */
typedef struct hyena_synth_params_s {
    int64_t axes;          /* 1, 2 or 3 */
    int64_t grid[3];       /* points per axis; at most 2^28 points in all */
    uint32_t signed_axes;  /* bit i: axis i holds signed offsets */
    int64_t width;         /* W: 8, 16, 32 or 64 */
    int64_t layers;        /* M: 1 .. 16 */
    int64_t zdim;          /* Z: 1 .. 256 */
    int64_t channels;      /* C: 1 .. 2^24 */
    const float* w_first;
    const float* w_hidden;
    const float* b_layer;
    const float* omega;
    const float* film_g;
    const float* film_gb;
    const float* film_b;
    const float* film_bb;
    const float* w_out;
    const float* b_out;
    const float* win_mu;
    const float* win_sigma;
} hyena_synth_params_t;

/* Synthesise B samples' kernels from their control vectors:
 *   z [B][Z] fp32, device: the control vector of every sample (derived by the
 *     model from its register tokens)
 *   k [B][C][grid points] fp32, device (output): kernel kk of sample b at
 *     k + (b*C + kk) * points, points in row-major grid order; for 1-D filters this
 *     is the [B][N-1][D][L] input of hyena_filter_spectrum_batched.
 * Enqueued on `stream` on the current device (no plan). HYENA_ERR_INVALID_ARG for
 * NULL or misaligned pointers, B < 1, sizes below 1 or signed bits beyond the axes;
 * HYENA_ERR_UNSUPPORTED for a width other than 8/16/32/64, more than 16 layers,
 * Z > 256, more than 2^28 grid points, B > 65535 or C > 2^24; HYENA_ERR_DEVICE if
 * the launch fails. */
hyena_status_t hyena_kernel_synthesis(const hyena_synth_params_t* params, int64_t B, const float* z, float* k,
                                      hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): hyena_forward with no
 * workspace argument and no allocation of any kind. The four-step and
 * partitioned paths keep their tiles in a scratch array of
 * HYENA_NOALLOC_SCRATCH_BYTES bytes that the library holds in device memory on
 * every GPU it runs on, from load until the process ends (the LDS path needs
 * none); chunks of rows are sized to it, so long rows run fewer rows per launch
 * than with the recommended workspace (the results are the same bits).
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (on different streams, or from different host threads without
 * ordering) race and give undefined results. The array's contents on entry are
 * irrelevant. Same arguments, results and errors as hyena_forward otherwise;
 * HYENA_ERR_WORKSPACE if one row's tiles exceed the array (not reachable with
 * the supported sizes), HYENA_ERR_DEVICE if the array's address cannot be
 * obtained on the current device. */
#define HYENA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
hyena_status_t hyena_forward_noalloc(hyena_plan_t plan, int64_t B, const void* u_proj, const float* short_w,
                                     const void* spec, const float* bias, void* y, hipStream_t stream);

/* hyena_forward with a filter set per sample (input-dependent long convolutions,
 * the HyenaND summary's methodology): sample b is convolved with the filters whose
 * spectrum hyena_filter_spectrum_batched wrote at byte b * hyena_spectrum_bytes
 * of `spec` (B spectra, B as in this call); short_w and bias stay shared. Same
 * arguments, workspace, results and errors as hyena_forward otherwise. */
hyena_status_t hyena_forward_per_sample(hyena_plan_t plan, int64_t B, const void* u_proj, const float* short_w,
                                        const void* spec, const float* bias, void* y, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream);

/* hyena_forward with per-kernel timing, for measurement. HIP events are
 * recorded on `stream` around every kernel launch of this forward; the call
 * then waits for the last event (so it is synchronous), and writes elapsed
 * milliseconds summed per kernel family into ms[6]:
 *   ms[0] the single kernel of the LDS path, ms[1] four-step pass A (column
 *   FFTs of the gated input), ms[2] pass B (row FFTs, spectrum multiply,
 *   inverse rows), ms[3] pass C (inverse columns and gate; for order > 2 it
 *   also carries the next step's pass A), ms[4] first event to last event,
 *   ms[5] the pipelined four-step launches (each runs all three passes, on
 *   different chunks). On the partitioned path ms[1] is pass 1 (window
 *   transforms) and ms[2] pass 2 (block sums, inverse transforms, gate).
 * Same arguments, results and errors as hyena_forward; HYENA_ERR_INVALID_ARG
 * also for ms == NULL or more than 4096 events. */
hyena_status_t hyena_forward_timed(hyena_plan_t plan, int64_t B, const void* u_proj, const float* short_w,
                                   const void* spec, const float* bias, void* y, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream, float* ms);

/* Bytes of workspace hyena_backward needs for batch B.
 * LDS path: per (b, d) row the N-1 product spectra that the batch sums of dh are
 * taken from, the gated-input spectra of steps 0..N-3 and the values v_1..v_{N-2}
 * (8 bytes per complex or pair value), then 3 floats of short-conv tap sums per
 * (b, channel): 8*B*D*((2N-3)*L + (N-2)*L/2) + 12*B*(N+1)*D.
 * Four-step path: per (b, d) row N+1 L-point complex tiles (the transform, the
 * N-1 gated inputs after their column transforms, the row's share of dh after the
 * inverse rows), N-2
 * fp32 rows of recomputed values and N+1 fp32 staging rows; and 12*(N+1) bytes
 * of tap sums per (row, column block); each region 256-byte aligned. A circular
 * plan (LDS path only) counts L/2-point transforms and L sample pairs per value.
 * Returns 0 for a NULL plan, B < 1, or a circular four-step plan. */
size_t hyena_backward_workspace_bytes(hyena_plan_t plan, int64_t B);

/* Backward of the forward hot path: given the upstream gradient dy of y, the
 * gradients of the same scalar loss with respect to u_proj, short_w, the long
 * filters h (time domain, i.e. through hyena_filter_spectrum) and bias. They
 * follow from the forward's definitions (HyenaDNA walkthrough, section 2.1,
 * HyenaOperator.forward; section 2.2, HyenaFilter.forward and fftconv) by the
 * chain rule; the adjoint of the causal convolution with h is the correlation
 * corr(a, h)[t] = sum_{s >= t} h[s-t] a[s], taken through the same zero-padded
 * 2L-point spectra with the filter spectrum conjugated.
 *   u_proj, short_w, spec, bias: the forward's inputs (spec from
 *           hyena_filter_spectrum of this plan)
 *   dy      [B][D][L] of the plan dtype, device
 *   du_proj [B][(N+1)*D][L] of the plan dtype, device (output; bf16 rounded to
 *           nearest even)
 *   dshort_w [(N+1)*D][3] fp32, dh [N-1][D][L] fp32, dbias [N-1][D] fp32, device
 *           (outputs; the batch sums are complete, not accumulated into the
 *           buffers' previous contents)
 *   workspace / workspace_bytes: device scratch of at least
 *           hyena_backward_workspace_bytes(plan, B); contents on entry irrelevant.
 * Both paths have a backward for every order. For a circular plan (LDS path
 * only; a circular four-step plan gives HYENA_ERR_UNSUPPORTED) the correlations
 * are circular too (corr(a, k)[t] = sum_s k[(s - t) mod L] a[s]), dh has L taps
 * per filter and the short conv's transpose keeps its causal form. Every sum over the batch
 * or over workgroups is taken in a fixed order (no atomics), so results are
 * bitwise reproducible.
 * Enqueued on `stream`. Errors: HYENA_ERR_INVALID_ARG (NULL or misaligned
 * pointers, B < 1), HYENA_ERR_UNSUPPORTED, HYENA_ERR_WORKSPACE,
 * HYENA_ERR_DEVICE (launch failure, wrong current device). Outputs must not
 * alias inputs or each other. */
hyena_status_t hyena_backward(hyena_plan_t plan, int64_t B, const void* u_proj, const float* short_w,
                              const void* spec, const float* bias, const void* dy, void* du_proj, float* dshort_w,
                              float* dh, float* dbias, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace hyena_backward_per_sample needs for batch B: as
 * hyena_backward_workspace_bytes, except on the four-step path, where B*D floats
 * of per-sample dbias terms are added. Returns 0 for a NULL plan, B < 1, or a
 * circular four-step plan. */
size_t hyena_backward_per_sample_workspace_bytes(hyena_plan_t plan, int64_t B);

/* Backward of hyena_forward_per_sample (a filter set per sample, the HyenaND
 * summary's input-dependent convolutions): spec holds the B spectra of
 * hyena_filter_spectrum_batched, and sample b's filter gradient is its own, so
 *   dh      [B][N-1][D][L] fp32, device (output): dh[b] is the gradient with
 *           respect to sample b's filters h[b] [N-1][D][L]
 * while dshort_w and dbias, whose parameters every sample shares, are batch sums
 * as in hyena_backward. Every other argument, the workspace (of at least
 * hyena_backward_per_sample_workspace_bytes(plan, B)), the fixed summation order
 * and the errors are those of hyena_backward; in addition HYENA_ERR_INVALID_ARG
 * when B*(N-1)*D*L exceeds 2^35 (dh alone would pass 128 GiB). */
hyena_status_t hyena_backward_per_sample(hyena_plan_t plan, int64_t B, const void* u_proj, const float* short_w,
                                         const void* spec, const float* bias, const void* dy, void* du_proj,
                                         float* dshort_w, float* dh, float* dbias, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace hyena_operator_forward needs for batch B: the in-projected
 * activation u_proj, the path output y, either the identity short-conv taps
 * (bf16 plans with D a multiple of 64, whose input projection is fused with the
 * short conv) or, for the other plans, x and w_in with the input-bias term
 * appended to each row (B*L + (N+1)*D rows of Dp = D + 1 rounded up to 8
 * values), 32 MiB of GEMM scratch and the path's own workspace
 * (hyena_workspace_bytes), each 256-byte aligned. Returns 0 for a NULL plan or
 * B < 1. */
size_t hyena_operator_workspace_bytes(hyena_plan_t plan, int64_t B);

/* The whole operator forward around the hot path (HyenaDNA walkthrough, section
 * 2.1, HyenaOperator.forward): in_proj, the (B, L, D) -> (B, D, L) transpose, the
 * hot path as in hyena_forward, the transpose back, out_proj:
 *   u_proj[b][c][t] = sum_k w_in[c][k] x[b][t][k] + b_in[c]
 *   out[b][t][j]    = sum_d w_out[j][d] y[b][d][t] + b_out[j]
 *   x     [B][L][D] of the plan dtype, device
 *   w_in  [(N+1)*D][D], b_in [(N+1)*D], w_out [D][D], b_out [D]: the projections'
 *         weights and biases (PyTorch nn.Linear layout), plan dtype, device
 *   short_w, spec, bias: as in hyena_forward
 *   out   [B][L][D] of the plan dtype, device (output)
 *   workspace: at least hyena_operator_workspace_bytes(plan, B) bytes.
 * bf16 plans with D a multiple of 64: the input projection runs in libhyena's own
 * bf16 matrix-core kernel, one launch over every sequence, fused with b_in and
 * the short conv (applied to the fp32 sums, then rounded once to bf16); the path
 * then runs with identity taps. Other plans: the input projection is a hipBLASLt
 * GEMM per sequence (u_proj rounded to the plan dtype) and the path applies the
 * short conv. The output projection of bf16 plans with D a multiple of 64 and L
 * a multiple of 8 runs in libhyena's own bf16 matrix-core kernel, one launch over
 * every sequence (fp32 accumulation, b_out added, rounded once); otherwise it is a
 * hipBLASLt GEMM per sequence (fp32 accumulation). hipBLASLt's heuristic choice of
 * kernel is used unless hyena_operator_tune has run on the plan. The first call
 * on a plan attaches the
 * GEMM state to it (a hipBLASLt handle and descriptors), so calls on one plan are
 * serialised internally; hyena_plan_destroy releases it. The call never waits on
 * the device.
 * Enqueued on `stream`. Errors: HYENA_ERR_INVALID_ARG (NULL or misaligned
 * pointers, B < 1, sizes too large), HYENA_ERR_WORKSPACE, HYENA_ERR_UNSUPPORTED
 * (no GEMM kernel for these shapes), HYENA_ERR_DEVICE, and those of
 * hyena_forward. Outputs must not alias inputs. */
hyena_status_t hyena_operator_forward(hyena_plan_t plan, int64_t B, const void* x, const void* w_in,
                                      const void* b_in, const float* short_w, const void* spec, const float* bias,
                                      const void* w_out, const void* b_out, void* out, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* Times hipBLASLt's candidate kernels for this plan's projection GEMMs on the
 * given buffers (a few calls each) and keeps the fastest for later calls on the
 * plan. Same arguments and errors as hyena_operator_forward; it overwrites `out`
 * and the workspace with scratch values and returns after the stream has finished
 * (a blocking call, made once before timing-sensitive use). */
hyena_status_t hyena_operator_tune(hyena_plan_t plan, int64_t B, const void* x, const void* w_in, const void* b_in,
                                   const float* short_w, const void* spec, const float* bias, const void* w_out,
                                   const void* b_out, void* out, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* hyena_operator_forward with timing: HIP events around the three stages on
 * `stream`; waits for the last one and writes milliseconds into ms[4]:
 * ms[0] input projection (with the bias or tap fill; the short conv as well on the
 * fused bf16 path), ms[1] the hot path, ms[2] output
 * projection, ms[3] total. HYENA_ERR_INVALID_ARG also for ms == NULL. */
hyena_status_t hyena_operator_forward_timed(hyena_plan_t plan, int64_t B, const void* x, const void* w_in,
                                            const void* b_in, const float* short_w, const void* spec,
                                            const float* bias, const void* w_out, const void* b_out, void* out,
                                            void* workspace, size_t workspace_bytes, hipStream_t stream,
                                            float* ms);

/* Parameters of the implicit long-filter generator (HyenaDNA walkthrough, section
 * 2.2, HyenaFilter). With E = emb_dim (odd, 3..127), K = (E-1)/2 bands,
 * W = width (8, 16, 32 or 64), M = num_inner (0..16) and C = (N-1)*D of the plan;
 * all arrays fp32, row-major, device, 16-byte aligned:
 *   band_freq [K]      frequencies f_k of the positional sine/cosine bands
 *   w_in [W][E], b_in [W]                 first Linear (PyTorch nn.Linear layout)
 *   w_inner [M][W][W], b_inner [M][W]     inner Linears (may be NULL when M = 0)
 *   sin_freq [W]       frequency of the Sin activation, shared by all its uses
 *   w_out [C][W]       output Linear, no bias; row c = o*D + d
 *   alpha [C]          modulation rates */
typedef struct hyena_filter_mlp_s {
    int64_t emb_dim;
    int64_t width;
    int64_t num_inner;
    const float* band_freq;
    const float* w_in;
    const float* b_in;
    const float* w_inner;
    const float* b_inner;
    const float* sin_freq;
    const float* w_out;
    const float* alpha;
} hyena_filter_mlp_t;

/* The implicit long filters of the plan (HyenaDNA walkthrough, section 2.2,
 * HyenaFilter.filter: positional embedding, the Linear/Sin stack, modulation; and
 * the [L, (N-1)*D] -> [N-1][D][L] reshape of section 2.1). For tau = 0..L-1, t = tau/L:
 *   z    = (t, sin(2 pi f_1 t) .. sin(2 pi f_K t), cos(2 pi f_1 t) .. cos(2 pi f_K t))
 *   a    = sin(sin_freq * (w_in z + b_in)),  then M times  a = sin(sin_freq * (w_inner[m] a + b_inner[m]))
 *   h[o][d][tau] = exp(-alpha[c] t) * sum_j w_out[c][j] a[j],   c = o*D + d
 * (the pages give the structure but not these formulas: the positional features,
 * the Sin activation and the modulation are this library's readings of them).
 *   h [N-1][D][L] fp32, device (output): the layout hyena_filter_spectrum takes.
 * The positional features are evaluated in fp64 and rounded once; the stack runs
 * in fp32; exp(-alpha t) is evaluated as 2^(alpha * (-t log2 e)) with the hardware
 * exp2 (relative error about 1e-7). Enqueued on `stream`. Errors: HYENA_ERR_INVALID_ARG (NULL plan, mlp or
 * h, NULL arrays, even or too small emb_dim, misaligned pointers),
 * HYENA_ERR_UNSUPPORTED (width not 8/16/32/64, emb_dim > 127, num_inner > 16),
 * HYENA_ERR_DEVICE. h must not alias the parameters. */
hyena_status_t hyena_implicit_filter(hyena_plan_t plan, const hyena_filter_mlp_t* mlp, float* h,
                                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * 2-D long convolution (HyenaND summary, methodology: global convolution on the
 * native N-d grid by an N-d FFT; the non-circular mode zero-pads the input to
 * double the grid in every dimension). One gated step per (b, d) image, as one
 * step of the 1-D recurrence above:
 *   s = v * g            (g optional: s = v when NULL)
 *   c[p][q] = sum_{i < 2H, j < 2W} k[i][j] s_pad[(p - i) mod 2H][(q - j) mod 2W]
 *   y = (c + bias * s) * x   (x optional),     p < H, q < W,
 * where s_pad is s zero-padded to 2H x 2W and the kernel k is given on the
 * doubled grid: rows i >= H and columns j >= W hold the negative offsets i - 2H
 * and j - 2W, so a causal kernel (zero outside [0,H) x [0,W)) and a centred one
 * are both expressible. (How the HyenaND operator synthesises its kernels and
 * what short convolution it applies on a grid are not on the pages; this is the
 * convolution step on its own.)
 * ------------------------------------------------------------------------ */
typedef struct hyena_plan2d_s* hyena_plan2d_t; /* opaque */

/* Plan for H x W images (powers of two, 16 <= H <= 512, 32 <= W <= 512) of D
 * channels; dtype of v, g, x and y as for the 1-D plans. The plan owns its
 * twiddle tables on the current device. Errors as hyena_plan_create. */
hyena_status_t hyena_plan2d_create(hyena_plan2d_t* out, int64_t H, int64_t W, int64_t D, hyena_dtype_t dtype);

/* As hyena_plan2d_create, with option flags (0 or HYENA_FLAG_CIRCULAR). A circular
 * plan convolves the grid periodically (the HyenaND summary's boundary handling
 * for periodic systems), with the kernel k[D][H][W] on the grid itself:
 *   c[p][q] = sum_{i < H, j < W} k[i][j] s[(p - i) mod H][(q - j) mod W];
 * its spectrum is D * H * (W/2 + 1) complex values (rfft2 of the H x W kernel,
 * scaled by 1/(2 * H * W)), its workspace 4*H*W bytes per image; 32 <= H <= 1024,
 * 64 <= W <= 1024. HYENA_ERR_INVALID_ARG for unknown flag bits. */
hyena_status_t hyena_plan2d_create_ex(hyena_plan2d_t* out, int64_t H, int64_t W, int64_t D, hyena_dtype_t dtype,
                                      uint32_t flags);

/* Release a 2-D plan. NULL is a no-op. */
hyena_status_t hyena_plan2d_destroy(hyena_plan2d_t plan);

/* Bytes of a 2-D kernel spectrum: D * 2H * (W + 1) complex fp32 values, the
 * doubled grid's real-transform bins (numpy.fft.rfft2 layout) of each channel,
 * scaled by 1/(4 * 2H * W). Returns 0 for a NULL plan. */
size_t hyena_spectrum2d_bytes(hyena_plan2d_t plan);

/* Workspace for hyena_conv2d_forward over batch B: any size of at least one
 * image tile (8 * H * W bytes) is accepted; this is the recommended size (up to
 * 128 MiB of tiles per launch). Returns 0 for a NULL plan or B < 1. */
size_t hyena_workspace2d_bytes(hyena_plan2d_t plan, int64_t B);

/* Kernel spectra, once per plan.
 *   k    [D][2H][2W] fp32, device: the kernels on the doubled grid
 *   spec device buffer of hyena_spectrum2d_bytes(plan) bytes (output)
 * Enqueued on `stream`. HYENA_ERR_INVALID_ARG for NULL or misaligned pointers,
 * HYENA_ERR_DEVICE for launch failures or a wrong current device. */
hyena_status_t hyena_filter_spectrum2d(hyena_plan2d_t plan, const float* k, void* spec, hipStream_t stream);

/* The gated 2-D long convolution above for B x D images.
 *   v    [B][D][H][W] of the plan dtype, device
 *   g, x [B][D][H][W] of the plan dtype, device, or NULL (no gate)
 *   spec from hyena_filter_spectrum2d of this plan; bias [D] fp32, device
 *   y    [B][D][H][W] of the plan dtype, device (output; must not alias inputs)
 *   workspace / workspace_bytes: at least 8*H*W bytes (see hyena_workspace2d_bytes)
 * Three passes per chunk of images: column FFTs of the gated image, row FFTs with
 * the spectrum multiply and the inverse rows, inverse columns with the gate; all
 * intermediates fp32. Enqueued on `stream`. Errors: HYENA_ERR_INVALID_ARG (NULL or
 * misaligned pointers, B < 1, B*D > 2^24), HYENA_ERR_WORKSPACE, HYENA_ERR_DEVICE. */
hyena_status_t hyena_conv2d_forward(hyena_plan2d_t plan, int64_t B, const void* v, const void* g, const void* x,
                                    const void* spec, const float* bias, void* y, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* Input-dependent kernels (the HyenaND summary's methodology: a kernel set per
 * input sample): hyena_filter_spectrum2d for B kernel sets at once,
 *   k    [B][D][2H][2W] fp32, device; spec: B * hyena_spectrum2d_bytes(plan) bytes,
 *        sample b's spectrum at byte b * hyena_spectrum2d_bytes(plan),
 * and the forward in which image (b, d) uses sample b's kernel d (bias shared).
 * Errors as the calls above; HYENA_ERR_INVALID_ARG also for B < 1 or B*D > 2^24. */
hyena_status_t hyena_filter_spectrum2d_batched(hyena_plan2d_t plan, int64_t B, const float* k, void* spec,
                                               hipStream_t stream);
hyena_status_t hyena_conv2d_forward_per_sample(hyena_plan2d_t plan, int64_t B, const void* v, const void* g,
                                               const void* x, const void* spec, const float* bias, void* y,
                                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * 3-D long convolution: the 2-D step above with one more grid axis (HyenaND
 * summary, methodology: the N-d FFT convolution on the native grid, zero-padded
 * to double the grid in every dimension). One gated step per (b, d) volume:
 *   s = v * g            (g optional)
 *   c[a][p][q] = sum_{l < 2A, i < 2H, j < 2W} k[l][i][j]
 *                s_pad[(a - l) mod 2A][(p - i) mod 2H][(q - j) mod 2W]
 *   y = (c + bias * s) * x   (x optional),     a < A, p < H, q < W,
 * with the kernel given on the doubled grid (an index >= the axis length holds
 * the negative offset, as in 2-D).
 * ------------------------------------------------------------------------ */
typedef struct hyena_plan3d_s* hyena_plan3d_t; /* opaque */

/* Plan for A x H x W volumes (powers of two, 16 <= A, H <= 512, 32 <= W <= 512,
 * A*H*W <= 2^24) of D channels; dtype of v, g, x and y as for the 1-D plans. The
 * plan owns its twiddle tables on the current device. Errors as
 * hyena_plan_create. */
hyena_status_t hyena_plan3d_create(hyena_plan3d_t* out, int64_t A, int64_t H, int64_t W, int64_t D,
                                   hyena_dtype_t dtype);

/* As hyena_plan3d_create, with option flags (0 or HYENA_FLAG_CIRCULAR): a
 * circular plan convolves the volume periodically with the kernel k[D][A][H][W]
 * on the grid itself; its spectrum is D * A * H * (W/2 + 1) complex values
 * (rfftn of the kernel, scaled by 1/(2 * A * H * W)), its workspace 4*A*H*W
 * bytes per volume; 32 <= A, H <= 1024, 64 <= W <= 1024. */
hyena_status_t hyena_plan3d_create_ex(hyena_plan3d_t* out, int64_t A, int64_t H, int64_t W, int64_t D,
                                      hyena_dtype_t dtype, uint32_t flags);

/* Release a 3-D plan. NULL is a no-op. */
hyena_status_t hyena_plan3d_destroy(hyena_plan3d_t plan);

/* Bytes of a 3-D kernel spectrum: D * 2A * 2H * (W + 1) complex fp32 values, the
 * doubled grid's real-transform bins (numpy.fft.rfftn layout) of each channel,
 * scaled by 1/(4 * 2A * 2H * W). Returns 0 for a NULL plan. */
size_t hyena_spectrum3d_bytes(hyena_plan3d_t plan);

/* Workspace for hyena_conv3d_forward over batch B: any size of at least one
 * volume's tiles is accepted: for a zero-padded plan 24 * A * H * W bytes, or
 * 8 * A * H * W when a depth slice's height x row transform (2H x W packed points)
 * has at most 4096 points (the slab pass keeps one tile); 4 * A * H * W bytes for a
 * circular plan. This is the recommended size (up to 192 MiB of tiles per launch).
 * Returns 0 for a NULL plan or B < 1. */
size_t hyena_workspace3d_bytes(hyena_plan3d_t plan, int64_t B);

/* Kernel spectra, once per plan.
 *   k    [D][2A][2H][2W] fp32, device: the kernels on the doubled grid
 *   spec device buffer of hyena_spectrum3d_bytes(plan) bytes (output)
 * Enqueued on `stream`. HYENA_ERR_INVALID_ARG for NULL or misaligned pointers,
 * HYENA_ERR_DEVICE for launch failures or a wrong current device. */
hyena_status_t hyena_filter_spectrum3d(hyena_plan3d_t plan, const float* k, void* spec, hipStream_t stream);

/* The gated 3-D long convolution above for B x D volumes.
 *   v    [B][D][A][H][W] of the plan dtype, device
 *   g, x [B][D][A][H][W] of the plan dtype, device, or NULL (no gate)
 *   spec from hyena_filter_spectrum3d of this plan; bias [D] fp32, device
 *   y    [B][D][A][H][W] of the plan dtype, device (output; must not alias inputs)
 *   workspace / workspace_bytes: at least one volume's tiles (hyena_workspace3d_bytes)
 * Five passes per chunk of volumes: column FFTs over a of the gated volume and
 * over h, row FFTs over w with the spectrum multiply and the inverse rows, inverse
 * columns over h and over a with the gate; all intermediates fp32. When a pair of
 * depth slices fits one workgroup's LDS (the sizes above), the middle three run as
 * one pass per slice pair on chip. Enqueued on
 * `stream`. Errors: HYENA_ERR_INVALID_ARG (NULL or misaligned pointers, B < 1,
 * B*D > 2^24), HYENA_ERR_WORKSPACE, HYENA_ERR_DEVICE. */
hyena_status_t hyena_conv3d_forward(hyena_plan3d_t plan, int64_t B, const void* v, const void* g, const void* x,
                                    const void* spec, const float* bias, void* y, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* A kernel set per input sample, as for 2-D: k [B][D][2A][2H][2W] fp32 gives B
 * spectra of hyena_spectrum3d_bytes(plan) bytes each; volume (b, d) uses sample
 * b's kernel d. */
hyena_status_t hyena_filter_spectrum3d_batched(hyena_plan3d_t plan, int64_t B, const float* k, void* spec,
                                               hipStream_t stream);
hyena_status_t hyena_conv3d_forward_per_sample(hyena_plan3d_t plan, int64_t B, const void* v, const void* g,
                                               const void* x, const void* spec, const float* bias, void* y,
                                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char* hyena_status_string(hyena_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* LIBHYENA_HYENA_H */
