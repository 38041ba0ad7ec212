/*
 * sharded_linear.h -- C ABI of one tensor-parallel rank's linear step on gfx950 (MI355X).
 *
 * The step (llm-infra-atlas, "01 · ColumnParallelLinear / RowParallelLinear and the core
 * autograd", section 4): forward Y = X.W^T, input gradient dX = dY.W, and the weight gradient
 * fused into gradient accumulation, main_grad += dY^T.X in fp32, where main_grad is a view of a
 * flat grad_data buffer and W a view of a matching param_data buffer (llm-infra-atlas,
 * "05 · grad/param buffer", sections 4-5).  Collectives are not part of this library.
 *
 * Conventions shared by every entry point
 *   - Matrices are row-major and dense: the leading dimension is the last extent.
 *       X, dX : [T, in]     W : [out, in]     Y, dY : [T, out]     main_grad : [out, in]
 *     T = tokens (sequence x micro-batch rows flattened), in/out = the shard's features.
 *   - bf16 tensors are passed as raw 16-bit storage; main_grad and grad_data are fp32.
 *   - Device pointers must be 16-byte aligned; in and out must be multiples of 8 (32 for the
 *     MXFP8 entry points); T may be any value >= 0.  A zero extent is a no-op.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the null stream) and
 *     performs no synchronisation, no allocation and no free.  The caller owns all memory.
 *   - Arguments are validated on the host before any HIP call; on error nothing is launched.
 *   - Return value: SL_OK (0) or a negative SL_E* status; sl_status_str() names it.
 *   - Results of the GEMMs are deterministic: the same inputs give the same bits.
 *   - Tile and split choices, and so the sizes the *_workspace_bytes queries return, are the
 *     library's own unless forced through sl_set_tuning(); the library reads no environment
 *     variables.  Keep the knobs unchanged between a query and the calls whose workspace it
 *     sizes; a call that finds its workspace too small returns SL_EWORKSPACE and launches
 *     nothing.
 */
#ifndef SHARDED_LINEAR_H
#define SHARDED_LINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SL_OK = 0,
  SL_EINVAL = -1,      /* null pointer with a nonzero extent, negative extent, bad option      */
  SL_EALIGN = -2,      /* device pointer not 16-byte aligned                                   */
  SL_ESHAPE = -3,      /* in/out not a multiple of 8 (32 for MXFP8), or an extent >= 2^31       */
  SL_EWORKSPACE = -4,  /* workspace missing or smaller than sl_wgrad_workspace_bytes()          */
  SL_EHIP = -5,        /* the HIP runtime reported an error at launch                          */
  SL_ECAPACITY = -6    /* an output array given to sl_layout_build is too small                */
};

/* Name of a status code (static storage). */
const char* sl_status_str(int status);

/* ---------------------------------------------------------------------------------------------
 * Tuning knobs, for measurement and tests (not needed for correct use).  sl_set_tuning forces
 * one choice for every later call and workspace query of this process; value -1 restores the
 * built-in choice.  The previous value is stored in *previous when it is not NULL.  Ranges:
 *   SL_TUNE_FWD_CONFIG                bf16 tile configuration 0..25 of the forward (25: 256x192
 *                                     tiles, which only the forward has)
 *   SL_TUNE_{DGRAD,WGRAD}_CONFIG      bf16 tile configuration 0..24 of that product
 *   SL_TUNE_SPLITK                    split count 1..64 of the bf16 weight gradient
 *   SL_TUNE_F8_CONFIG                 block-scaled fp8 configuration 0..2 (0: 256x256, 1: 128x128,
 *                                     2: 256x128), for the weight gradient as well
 * An unknown knob or a value out of range returns SL_EINVAL and changes nothing.  The knobs are
 * process-wide atomics: safe to set from any thread, but a call that overlaps a change may see
 * either value, so change them only while no call is being planned.
 * ------------------------------------------------------------------------------------------- */
enum {
  SL_TUNE_FWD_CONFIG = 0,
  SL_TUNE_DGRAD_CONFIG = 1,
  SL_TUNE_WGRAD_CONFIG = 2,
  SL_TUNE_SPLITK = 3,
  SL_TUNE_F8_CONFIG = 4,
  SL_TUNE_COUNT = 5
};
int sl_set_tuning(int32_t knob, int32_t value, int32_t* previous);

/* ---------------------------------------------------------------------------------------------
 * Buffer layout (host only; llm-infra-atlas "05 · grad/param buffer", sections 4.1-4.3 and 5).
 *
 * Places n parameters, numel[] given in model definition order, into one flat buffer:
 *   - in reverse definition order (backprop order), so offset 0 holds the last parameter;
 *   - each parameter start rounded up to a multiple of param_align elements (64 under the
 *     distributed optimizer; the page notes the unit is elements, not bytes);
 *   - a bucket is closed right after the parameter whose end makes (end - bucket_start) reach
 *     bucket_size elements; bucket_size <= 0 puts everything in one bucket;
 *   - each bucket end is rounded up to a multiple of `divisor` (lcm(dp,128), or
 *     lcm(dp,128,65536) with the high-bus-bandwidth option, see sl_bucket_divisor), and the next
 *     bucket starts there.
 * Outputs (caller-owned host arrays): start/end/bucket_id per parameter (definition order);
 * per bucket: offset, padded numel and unpadded numel (param end - bucket start), up to
 * bucket_cap entries; *n_buckets and *total_numel.  If bucket_cap is too small the call
 * returns SL_ECAPACITY and sets *n_buckets to the number needed.  A zero-size parameter is
 * allowed; n = 0 gives total_numel 0 and no buckets.
 * ------------------------------------------------------------------------------------------- */
int sl_layout_build(int32_t n, const int64_t* numel, int64_t param_align, int64_t bucket_size,
                    int64_t divisor, int64_t* start, int64_t* end, int32_t* bucket_id,
                    int32_t bucket_cap, int64_t* bucket_offset, int64_t* bucket_numel,
                    int64_t* bucket_numel_unpadded, int32_t* n_buckets, int64_t* total_numel);

/* Default bucket size in elements, max(40,000,000, 1,000,000 * dp) (same page, section 4.3). */
int64_t sl_default_bucket_size(int64_t dp);

/* Bucket-end divisor lcm(dp, 128), or lcm(dp, 128, 65536) when high_busbw != 0 (section 4.2).
 * Returns 0 for dp <= 0. */
int64_t sl_bucket_divisor(int64_t dp, int32_t high_busbw);

/* ---------------------------------------------------------------------------------------------
 * Gradient-buffer zeroing (same page, section 6.6: grad_data is zeroed once per iteration and
 * never freed).  Writes 0.0f to grad_data[0, numel).  A fill kernel, so it is safe to record in
 * a captured HIP graph.  Also used to prepare a wgrad workspace before its first use.
 * ------------------------------------------------------------------------------------------- */
int sl_grad_buffer_zero(void* stream, float* grad_data, int64_t numel);

/* ---------------------------------------------------------------------------------------------
 * Forward GEMM: Y[T,out] = X[T,in] . W[out,in]^T, bf16 inputs, fp32 accumulation, one
 * round-to-nearest-even to bf16 (atlas page "01", section 4.1).  For a row-parallel weight Y is
 * the partial sum that the following all-reduce would add up.
 * ------------------------------------------------------------------------------------------- */
int sl_linear_fwd(void* stream, const void* X, const void* W, void* Y,
                  int64_t T, int64_t in, int64_t out);

/* ---------------------------------------------------------------------------------------------
 * Input-gradient GEMM: dX[T,in] = dY[T,out] . W[out,in], bf16 in/out, fp32 accumulation
 * (atlas page "01", section 4.2, the dgrad).
 * ------------------------------------------------------------------------------------------- */
int sl_linear_dgrad(void* stream, const void* dY, const void* W, void* dX,
                    int64_t T, int64_t in, int64_t out);

/* ---------------------------------------------------------------------------------------------
 * Weight gradient fused into accumulation: main_grad[out,in] += dY[T,out]^T . X[T,in] in fp32
 * (atlas page "01", section 4.2, gradient_accumulation_fusion).  The micro-batch gradient is
 * never rounded and never stored on its own; main_grad is read and written only inside its
 * [out, in] extent, so neighbouring views and padding of grad_data are untouched.
 *
 * workspace: device memory of at least sl_wgrad_workspace_bytes(T, in, out) bytes (0 when the
 * shape needs no split-K; workspace may then be NULL).  It holds fp32 split-K partial planes
 * [splits][out][in], written and then read within the call; its initial contents do not
 * matter.  A split call launches a second, reducing kernel on the same stream.  Calls that may
 * run concurrently must use distinct workspaces.
 * ------------------------------------------------------------------------------------------- */
size_t sl_wgrad_workspace_bytes(int64_t T, int64_t in, int64_t out);
int sl_linear_wgrad_accum(void* stream, const void* X, const void* dY, float* main_grad,
                          int64_t T, int64_t in, int64_t out,
                          void* workspace, size_t workspace_bytes);

/* ---------------------------------------------------------------------------------------------
 * The weight gradient for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, and harnesses that forbid hipMalloc.  Same operation, arguments
 * (other than the workspace), results and kernels as sl_linear_wgrad_accum; the split-K partial
 * planes go into a library-owned device array of SL_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU
 * holds from module load until the process ends.  The call allocates and frees nothing.
 *   - A shape whose plan needs more than that (sl_wgrad_workspace_bytes(T, in, out) >
 *     SL_NOALLOC_SCRATCH_BYTES) returns SL_EWORKSPACE and launches nothing.
 *   - `stream` must belong to the current device (SL_EINVAL otherwise): the array is the current
 *     device's, resolved at the first call on that device.
 *   - Every call on one GPU shares that GPU's array, and its partial planes are written and read
 *     within the call (nothing needs clearing between calls).  Calls that overlap on one GPU --
 *     on different streams, or from different host threads -- race on the array: serialise them.
 * ------------------------------------------------------------------------------------------- */
#define SL_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int sl_linear_wgrad_accum_noalloc(void* stream, const void* X, const void* dY, float* main_grad,
                                  int64_t T, int64_t in, int64_t out);

/* ---------------------------------------------------------------------------------------------
 * MXFP8 operand variants (NVIDIA Megatron-Core guide "Generalized Tensor Parallelism",
 * section 1.3: E4M3 elements with one E8M0 scale per 32 elements).  A quantised matrix M[r, c]
 * is passed as codes Mq[r, c] (uint8, E4M3FN) and scales Ms[r, c/32] (uint8, E8M0), and stands
 * for deq(q, s) = E4M3(q) * 2^(s - 127).  Blocks run along `in` for both X and W.
 *   fwd:   Y  = deq(Xq).deq(Wq)^T           (bf16 out; block-scaled fp8 MFMA when 128 | in and
 *                                            the scale pointers are 4-byte aligned)
 *   dgrad: dX = dY.deq(Wq)                  (dY, dX bf16)
 *   wgrad: main_grad += dY^T.deq(Xq)        (dY bf16, main_grad fp32)
 * Every dequantised element must be representable in bf16 (an E4M3 value times a power of two
 * whose result is a normal bf16); it then enters the GEMMs exactly.  in must be a multiple of
 * 32.  Code pointers must be 16-byte aligned; scale pointers have no alignment requirement.
 *
 * dgrad and wgrad take a device workspace of at least sl_mxfp8_workspace_bytes(T, in, out)
 * bytes: the MXFP8 operand is dequantised into its front (bf16), the rest serves the bf16
 * weight-gradient split-K planes.  Its initial contents do not matter; calls that may run
 * concurrently must use distinct workspaces.
 * ------------------------------------------------------------------------------------------- */
size_t sl_mxfp8_workspace_bytes(int64_t T, int64_t in, int64_t out);
int sl_linear_fwd_mxfp8(void* stream, const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq,
                        const uint8_t* Ws, void* Y, int64_t T, int64_t in, int64_t out);
int sl_linear_dgrad_mxfp8w(void* stream, const void* dY, const uint8_t* Wq, const uint8_t* Ws,
                           void* dX, int64_t T, int64_t in, int64_t out,
                           void* workspace, size_t workspace_bytes);
int sl_linear_wgrad_accum_mxfp8x(void* stream, const uint8_t* Xq, const uint8_t* Xs,
                                 const void* dY, float* main_grad, int64_t T, int64_t in,
                                 int64_t out, void* workspace, size_t workspace_bytes);

/* sl_mxfp8_dequantize: out[r, c] (bf16) = deq(q, s)[r, c] = E4M3(q[r, c]) * 2^(s[r, c/32] - 127)
 * for q[rows, cols] codes and s[rows, cols/32] scales (section 1.3 block of 32 above).  Exact under
 * the representability rule above (results that are not normal bf16 values are unspecified).
 * cols % 32 == 0 (SL_ESHAPE); q and out 16-byte aligned (SL_EALIGN); the caller owns all buffers.
 * This is the expansion sl_linear_dgrad_mxfp8w and sl_linear_wgrad_accum_mxfp8x perform into
 * their workspace; sl_linear_dgrad on its output gives the same dX bit for bit.
 */
int sl_mxfp8_dequantize(void* stream, const uint8_t* q, const uint8_t* s, void* out, int64_t rows,
                        int64_t cols);

/* ---------------------------------------------------------------------------------------------
 * All-MXFP8 step: the backward GEMMs in MXFP8 as well (NVIDIA Megatron-Core guide "Generalized
 * Tensor Parallelism", section 1.3: in the MXFP8 recipe each GEMM reads E4M3 elements with one
 * E8M0 scale per 32 elements along its own contraction axis; the weight gradient still
 * accumulates into fp32 main_grad, section 3.1).  A tensor read along both axes is quantised
 * twice: rowwise (blocks along the last axis) and columnwise (blocks down the columns, stored
 * transposed so that the consuming GEMM reads k contiguously).
 *   fwd:   sl_linear_fwd_mxfp8 with X, W rowwise                      (above)
 *   dgrad: dX[T,in]         = deq(dYq)[T,out] . deq(WqT)[in,out]^T    dY rowwise, W columnwise
 *   wgrad: main_grad[out,in] += deq(dYqT)[out,T] . deq(XqT)[in,T]^T   dY and X columnwise
 *
 * sl_mxfp8_quantize: x[rows, cols] bf16 (row-major, 16-byte aligned) into rowwise codes
 * q_rows[rows, cols] + scales s_rows[rows, cols/32] and/or columnwise codes q_cols[cols, rows] +
 * scales s_cols[cols, rows/32]; a NULL pair is skipped (each code pointer must come with its
 * scale pointer: SL_EINVAL otherwise).  The rowwise copy needs cols % 32 == 0, the columnwise
 * copy rows % 32 == 0 and cols % 8 == 0 (SL_ESHAPE).  The rule is the OCP MX v1.0 conversion (the pages fix only
 * the block and per-block scaling): per block X = clamp(floor(log2 amax) - 8, -127, 127),
 * scale byte X + 127, codes = E4M3 round-to-nearest-even of x / 2^X saturating at +-448 with
 * the sign kept; an all-zero block stores scale 0 and zero codes.  Inputs must be finite
 * (non-finite elements give unspecified codes).  Code pointers 16-byte aligned.
 *
 * sl_linear_dgrad_mxfp8 / sl_linear_wgrad_accum_mxfp8: the contraction extent (out for dgrad,
 * T for wgrad) must be a multiple of 128, in/out multiples of 8 (SL_ESHAPE); code pointers
 * 16-byte aligned, scale pointers 4-byte aligned (SL_EALIGN).  The weight gradient takes a
 * device workspace of at least sl_mxfp8_wgrad_workspace_bytes(T, in, out) bytes (fp32 split-K
 * planes [splits][out][in]; 0 when the shape needs no split, workspace may then be NULL); its
 * initial contents do not matter, a split call launches a second, reducing kernel on the same
 * stream, and concurrent calls need distinct workspaces.  main_grad is read and written only
 * inside its [out, in] extent.
 * ------------------------------------------------------------------------------------------- */
int sl_mxfp8_quantize(void* stream, const void* x, int64_t rows, int64_t cols, uint8_t* q_rows,
                      uint8_t* s_rows, uint8_t* q_cols, uint8_t* s_cols);
int sl_linear_dgrad_mxfp8(void* stream, const uint8_t* dYq, const uint8_t* dYs, const uint8_t* WqT,
                          const uint8_t* WsT, void* dX, int64_t T, int64_t in, int64_t out);
size_t sl_mxfp8_wgrad_workspace_bytes(int64_t T, int64_t in, int64_t out);
int sl_linear_wgrad_accum_mxfp8(void* stream, const uint8_t* dYqT, const uint8_t* dYsT,
                                const uint8_t* XqT, const uint8_t* XsT, float* main_grad,
                                int64_t T, int64_t in, int64_t out, void* workspace,
                                size_t workspace_bytes);

/* ---- NVFP4 weights -------------------------------------------------------------------------
 * NVIDIA Megatron-Core guide "Generalized Tensor Parallelism", section 1.3 (native NVFP4 param):
 * the weight shard W[out, in] is kept as NVFP4 -- packed 4-bit E2M1 codes, one E4M3 scale per
 * 16 elements along in, and one fp32 per-tensor scale t (set when the optimizer writes the
 * shard) -- and activations and gradients stay bf16:
 *   deq(W)[o][i] = E2M1(code[o][i]) * E4M3(scale[o][i/16]) * t
 *   forward: Y  = X . deq(W)^T          dgrad: dX = dY . deq(W)
 * (the weight gradient does not read W: sl_linear_wgrad_accum applies unchanged).
 *
 * sl_nvfp4_materialize: Wq[rows, cols/2] packed codes (element 2j of a row in the low nibble of
 * byte j) and Ws[rows, cols/16] E4M3 scale bytes into Wm[rows, cols] bf16 holding
 * E2M1(code) * E4M3(scale) -- exact, since every such product is a bf16 value; t is NOT applied.
 * cols % 16 == 0 (the NVFP4 alignment pad; SL_ESHAPE otherwise); Wq and Wm 16-byte aligned
 * (SL_EALIGN); the caller owns all three buffers.  A NaN scale byte (S.1111.111) gives NaN
 * weights.  Wm may be materialised once per optimizer step and reused; materialising it right
 * before each product measured faster on the 8-micro-batch MLP step, since the GEMM then reads a
 * copy that is still in the caches.
 *
 * sl_linear_fwd_nvfp4w / sl_linear_dgrad_nvfp4w: as sl_linear_fwd / sl_linear_dgrad with W = Wm
 * from sl_nvfp4_materialize and w_scale = t: the fp32 accumulators are multiplied by w_scale
 * before the bf16 rounding of Y or dX.  in % 16 == 0 (SL_ESHAPE); w_scale must be finite
 * (SL_EINVAL); the other rules are those of the bf16 entry points.
 * ------------------------------------------------------------------------------------------- */
int sl_nvfp4_materialize(void* stream, const uint8_t* Wq, const uint8_t* Ws, void* Wm, int64_t rows,
                         int64_t cols);
int sl_linear_fwd_nvfp4w(void* stream, const void* X, const void* Wm, float w_scale, void* Y,
                         int64_t T, int64_t in, int64_t out);
int sl_linear_dgrad_nvfp4w(void* stream, const void* dY, const void* Wm, float w_scale, void* dX,
                           int64_t T, int64_t in, int64_t out);

#ifdef __cplusplus
}
#endif

#endif /* SHARDED_LINEAR_H */
