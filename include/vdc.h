/*
 * vdc.h - packed variable-length width-4 depthwise causal convolution
 * followed by SiLU, training forward and backward, on AMD Instinct MI355X
 * (gfx950).  C ABI of libvdc.so.
 *
 * The operation is the one documented on the pages of
 * flashinfer.cake_causal_conv1d_train:
 *   [F] cake_causal_conv1d_train_forward  (Parameters, Returns)
 *   [B] cake_causal_conv1d_train_backward (Description, Parameters, Returns)
 *
 * Many documents are packed back to back into one [S, C] activation tensor;
 * int32 cu_seqlens[0..num_docs] holds the prefix sums of their lengths
 * (cu_seqlens[0] = 0, cu_seqlens[num_docs] = S, a repeated value is an empty
 * document).  For token t in a document starting at s, channel c:
 *
 *   p[t,c]  = sum_{k=0..3, t-3+k >= s} w[c,k] * x[t-3+k,c]  (+ b[c])
 *   y[t,c]  = bf16(SiLU(p[t,c]))                                   [F] Returns
 *
 * w[c,3] multiplies the current token and w[c,0] the token three back; the
 * bias is added after the four taps ([F] Parameters).  The backward
 * recomputes p in FP32 and forms dpre = dy * SiLU'(z), where z is p rounded
 * to BF16 (policy VDC_SILU_GRAD_BF16, the default) or p itself
 * (VDC_SILU_GRAD_FP32) ([B] Description, Parameters silu_grad_preactivation).
 * Then, with e the end of t's document ([B] Returns):
 *
 *   dx[t,c]      = bf16(sum_{k, t+3-k < e} w[c,k] * dpre[t+3-k,c])
 *   dweight[c,k] = sum_t dpre[t,c] * x[t-3+k,c]   (taps inside the document)
 *   dbias[c]     = sum_t dpre[t,c]
 *
 * dweight and dbias are reduced in a fixed order that depends only on
 * (S, C, policy), so they are bitwise reproducible for a given (S, C, device)
 * and route ([B] Returns, Description).
 *
 * General rules for every entry point below:
 *  - Pointers to tensors are DEVICE pointers; sizes are element counts.
 *    Tensors are dense and row-major; x / dy / y / dx are [S][C] bf16 and
 *    must be 16-byte aligned; weight is [C][4] and bias [C], both 16-byte
 *    aligned; dweight [C][4] and dbias [C] are 4-byte (FP32) or 2-byte
 *    (BF16) aligned; each is FP32 or BF16 as its dtype argument says;
 *    cu_seqlens is int32 [num_docs + 1].
 *  - The caller owns every buffer.  The library allocates nothing, frees
 *    nothing, keeps no per-call state, never synchronizes, and never reads
 *    device memory on the host (in particular not cu_seqlens, whose
 *    well-formedness is the caller's precondition, [F] Parameters
 *    cu_seqlens; for malformed values the kernels stay inside their buffers
 *    and the results are unspecified).
 *  - Work is only enqueued on `stream` (0 = the null stream).  Calls are
 *    safe to capture into a HIP graph once the workspace exists.
 *  - Every argument is validated on the host before anything is enqueued;
 *    on any status but VDC_OK and VDC_EHIP nothing was enqueued and no
 *    output was touched.  VDC_EHIP means the runtime refused a launch, and
 *    an earlier launch of the same call may already be enqueued.
 *  - Two calls that may run concurrently need two workspaces.
 */
#ifndef VDC_H
#define VDC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype codes of weight / bias / dweight / dbias ([F] Parameters weight,
 * bias; [B] Parameters dweight, dbias). */
enum vdc_dtype {
    VDC_F32 = 0,
    VDC_BF16 = 1
};

/* Where SiLU' is evaluated ([B] Parameters, silu_grad_preactivation). */
enum vdc_silu_grad {
    VDC_SILU_GRAD_BF16 = 0, /* at the BF16-rounded FP32 preactivation      */
    VDC_SILU_GRAD_FP32 = 1  /* at the FP32 preactivation; FP64 reduction   */
};

/* Direction argument of workspace_bytes. */
enum vdc_direction {
    VDC_FWD = 0,
    VDC_BWD = 1
};

/* Status codes returned by the entry points. */
enum vdc_status {
    VDC_OK = 0,
    VDC_EINVAL = 1,     /* bad size, missing pointer, overlapping buffers  */
    VDC_EDTYPE = 2,     /* unknown dtype or policy code                    */
    VDC_EALIGN = 3,     /* a tensor pointer is not aligned as required     */
    VDC_EWORKSPACE = 4, /* workspace missing or smaller than required      */
    VDC_ENOBIAS = 5,    /* dbias requested without a bias                  */
    VDC_EHIP = 6,       /* the HIP runtime refused a launch                */
    VDC_ESCRATCH = 7    /* conv1d_bwd_noalloc: problem exceeds its scratch  */
};

/*
 * workspace_bytes - bytes of workspace a call needs.
 *
 * [F] Parameters workspace and [B] Parameters workspace: one size that
 * serves every route of the direction.  VDC_FWD: the forward keeps no
 * counters and needs no workspace, so the answer is 0 (conv1d_fwd accepts
 * workspace = NULL).  VDC_BWD: room for the FP32 / FP64 partial rows of
 * dweight and dbias (one per band of tokens; one per workgroup of the main
 * kernel when 256 <= C < 1024; one per group of four bands when C is a
 * multiple of 256, at least 1024, and the bands are shorter than 1024
 * tokens) for every policy, at this (S, C), plus the
 * FP64 sums of the reduce's first stage when there are more than 2048
 * partial rows; the backward writes every byte it later reads, so the
 * buffer needs no zeroing ([B] Parameters workspace).
 *
 * direction: VDC_FWD or VDC_BWD.  S >= 0 tokens, C > 0 channels (a multiple
 * of 8).  Returns 0 for invalid arguments (and for every valid forward).
 */
size_t workspace_bytes(int direction, int64_t S, int64_t C);

/*
 * conv1d_fwd - training forward ([F] Returns).
 *
 * x          bf16 [S][C], 16-byte aligned, C a multiple of 8 ([F] Parameters x).
 * weight     [C][4] of dtype w_dtype (VDC_F32 / VDC_BF16) ([F] Parameters weight).
 * bias       [C] of dtype b_dtype, or NULL for no bias; b_dtype is ignored
 *            when bias is NULL ([F] Parameters bias).
 * cu_seqlens int32 [num_docs + 1] device prefix sums; num_docs >= 1 when
 *            S > 0 ([F] Parameters cu_seqlens).
 * y          bf16 [S][C] output, 16-byte aligned, must not overlap x
 *            ([F] Parameters out).
 * workspace, ws_bytes: may be NULL / 0 (workspace_bytes(VDC_FWD) is 0).
 * stream     the HIP stream the kernel is enqueued on.
 *
 * S == 0 enqueues nothing ([F] Returns).  Returns a vdc_status.
 */
int conv1d_fwd(const void *x, const void *weight, int w_dtype,
               const void *bias, int b_dtype,
               const int32_t *cu_seqlens, int64_t num_docs,
               int64_t S, int64_t C,
               void *y, void *workspace, size_t ws_bytes,
               hipStream_t stream);

/*
 * conv1d_bwd - training backward ([B] Description, Returns).
 *
 * x, weight, w_dtype, bias, b_dtype, cu_seqlens, num_docs, S, C: the
 *            forward's inputs, same contracts as conv1d_fwd
 *            ([B] Parameters x, weight, cu_seqlens, bias).
 * dy         bf16 [S][C] gradient of y, 16-byte aligned ([B] Parameters dy).
 * policy     VDC_SILU_GRAD_BF16 or VDC_SILU_GRAD_FP32.
 * dx         bf16 [S][C] output, 16-byte aligned; must not overlap x or dy.
 * dweight    [C][4] output of dtype dw_dtype (VDC_F32 / VDC_BF16).
 * dbias      [C] output of dtype db_dtype, or NULL; non-NULL needs a bias
 *            (VDC_ENOBIAS otherwise) ([B] Parameters dbias).
 * workspace  at least workspace_bytes(VDC_BWD, S, C) bytes, 16-byte aligned,
 *            contents irrelevant; must not overlap any other argument.
 *
 * Two launches are enqueued in stream order: the main kernel writes dx and
 * partial rows of dweight / dbias into the workspace (one per band of
 * tokens, workgroup or group of bands, as workspace_bytes describes; FP32
 * under VDC_SILU_GRAD_BF16, FP64 under VDC_SILU_GRAD_FP32), and the
 * reduce kernel sums the rows in FP64 in a fixed order and rounds once to
 * the output dtype ([B] Description).  With more than 2048 partial rows
 * (long sequences of few channels) the reduce takes two launches: sums of
 * 2048-row ranges, then their sum, in an order that again depends on
 * (S, C) only.  S == 0 launches no main kernel ([B] Returns): dweight
 * (and dbias) are set to zero with hipMemsetAsync, or, if the stream is
 * being captured into a graph, by one launch of the reduce kernel over zero
 * partial rows, so that the graph holds no memset node.
 * Returns a vdc_status.
 */
int conv1d_bwd(const void *x, const void *weight, int w_dtype,
               const void *bias, int b_dtype,
               const int32_t *cu_seqlens, int64_t num_docs,
               const void *dy, int64_t S, int64_t C, int policy,
               void *dx, void *dweight, int dw_dtype,
               void *dbias, int db_dtype,
               void *workspace, size_t ws_bytes,
               hipStream_t stream);

/*
 * conv1d_bwd_noalloc - conv1d_bwd without a workspace argument, for callers
 * that cannot allocate device memory: code being captured into a HIP
 * graph, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Arguments, validation, results and status codes are those of conv1d_bwd
 * (the same kernels, launch plan and fixed reduction order, so the outputs
 * are bitwise those of conv1d_bwd for the same inputs); the caller still
 * owns and passes every input and output.  The workspace is instead a
 * device array inside the library of conv1d_noalloc_scratch_bytes() bytes
 * (16 MiB), one copy per GPU, held until the process ends.  The first call
 * on a device looks up that device's copy (with hipGetSymbolAddress; the
 * device of `stream` is made current for the lookup and restored after),
 * so make that first call outside any stream capture; no call allocates or
 * frees anything, and later calls may be captured into a HIP graph.
 *
 * A problem whose workspace_bytes(VDC_BWD, S, C) exceeds the array returns
 * VDC_ESCRATCH before anything is enqueued.  Every launch plan whose bands
 * times C stays within 2^18 fits (at most one band per lane of a full
 * machine: for example S = 65536 at C = 4096, S = 131072 at C = 8192,
 * S = 262144 at C = 520, S = 16384 at C = 2048); plans for very long
 * sequences, whose bands the planner shortens, and C in the hundreds of
 * thousands may not (conv1d_plan and workspace_bytes tell in advance).
 *
 * All calls on one GPU share its array, and a call leaves its contents
 * behind: two calls whose work may overlap in time on one GPU (on
 * different streams, or captured into graphs replayed concurrently) race
 * and give unspecified gradients.  Calls in one stream's order are safe.
 * Nothing in the array needs to start at zero.
 */
int conv1d_bwd_noalloc(const void *x, const void *weight, int w_dtype,
                       const void *bias, int b_dtype,
                       const int32_t *cu_seqlens, int64_t num_docs,
                       const void *dy, int64_t S, int64_t C, int policy,
                       void *dx, void *dweight, int dw_dtype,
                       void *dbias, int db_dtype,
                       hipStream_t stream);

/* conv1d_noalloc_scratch_bytes - size in bytes of the device array
 * conv1d_bwd_noalloc uses as its workspace. */
size_t conv1d_noalloc_scratch_bytes(void);

/* conv1d_status_string - static English text of a vdc_status code. */
const char *conv1d_status_string(int status);

/*
 * conv1d_plan - the launch plan a call with these sizes would use
 * (introspection for tests and benchmarks; enqueues nothing).
 * Fills out[0..10] = { rows per band, bands, lanes (bands * C / channels
 * per lane), main-kernel workgroups, threads per workgroup, partial
 * element bytes (0 forward, 4 or 8 backward), reduce-kernel workgroups,
 * reduce chunks, channels per lane, first-stage reduce row ranges (0 when
 * the reduce is one launch), partial rows of the backward (0 forward:
 * one per band, per workgroup when 256 <= C < 1024, or per group of four
 * bands when C is a multiple of 256, at least 1024, with bands shorter
 * than 1024 tokens) }.
 * Returns a vdc_status.
 */
int conv1d_plan(int direction, int64_t S, int64_t C, int policy, int64_t out[11]);

/* conv1d_launch_count - kernels this process has launched through the
 * library so far (a diagnostic counter, e.g. to check that S == 0
 * launches nothing). */
uint64_t conv1d_launch_count(void);

#ifdef __cplusplus
}
#endif

#endif /* VDC_H */
