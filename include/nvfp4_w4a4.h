/*
 * nvfp4_w4a4.h - C ABI of the NVFP4 W4A4 prefill linear layer for MI355X
 * (gfx950).
 *
 * The layer is the prefill path of Mix-Quant: weights and activations are
 * both quantised to NVFP4 and multiplied in a W4A4 GEMM ("Mix-Quant：面向
 * 智能体LLM的量化预填充与精确解码", paper.rainbus.top digest, sections
 * 核心方法 and 方法步骤详情 step (4); "Mix-Quant: Quantized Prefilling,
 * Precise Decoding for Agentic LLMs", r9-hu.github.io digest, section
 * Method, item 1).
 *
 * NVFP4 encoding produced and consumed here (the format of the paper.rainbus
 * digest, section 前置知识 "NVFP4 微缩放量化", and the formulas of its
 * section 方法步骤详情 step (3)):
 *
 *   alpha   one float32 per tensor:  alpha = RNE_fp32(max|x| / 2688),
 *           2688 = 6 * 448 (q_max of E2M1 times the largest E4M3 value).
 *   scales  uint8 [rows][K/16], row-major: OCP E4M3FN byte of
 *           sigma_b = RNE_E4M3(max_{i in b}|x_i| / (6 alpha)), saturating
 *           at 448, for the 16 consecutive K-elements of block b.
 *   codes   uint8 [rows][K/2], row-major: E2M1 codes (sign in bit 3) of
 *           q_i = RNE_E2M1(x_i / (alpha sigma_b)), ties to the even code,
 *           saturating at 6; element 2j in the low nibble of byte j.
 *           A block with sigma_b = 0 (or alpha = 0) gets magnitude 0.
 *   Dequantised value: xhat_i = alpha * sigma_b * q_i.
 *
 * Every division above is taken in exact real arithmetic (no float32
 * evaluation-order effects): codes and scale bytes are a pure function of
 * the BF16 inputs and alpha.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller.  BF16 data is
 *    passed as raw 16-bit patterns.  The library never allocates, keeps no
 *    state between calls and is safe to call from several host threads.
 *  - Work is enqueued on `stream` and is asynchronous; device faults surface
 *    at the caller's next synchronisation.
 *  - Arguments are validated first; on any error nothing is launched and the
 *    status code says why.  Inputs must be finite (no NaN/Inf).
 *  - Sizes are element counts.  K must be a positive multiple of 16.
 *  - Pointer alignment: BF16 inputs 16 bytes (and ld*2 a multiple of 16),
 *    codes 16 bytes for the GEMMs (8 for the quantiser's output), scales 8
 *    bytes when K % 128 == 0; outputs and alpha need only their element
 *    alignment.
 */
#ifndef NVFP4_W4A4_H
#define NVFP4_W4A4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,          /* a required pointer is NULL                */
  NVFP4_ERR_SHAPE = 2,         /* a size/stride is negative, too large, or  */
                               /* K % 16 != 0, or group offsets malformed   */
  NVFP4_ERR_ALIGN = 3,         /* a pointer or leading dimension misaligned */
  NVFP4_ERR_UNSUPPORTED = 4,   /* the current device is not gfx950          */
  NVFP4_ERR_LAUNCH = 5,        /* a HIP launch reported an error            */
  NVFP4_ERR_WORKSPACE = 6      /* workspace NULL or smaller than required   */
} nvfp4_status_t;

/* Human-readable text of a status code (static storage). */
const char* nvfp4_status_string(nvfp4_status_t status);

/* Bytes of device workspace the quantisers need (a fixed, small amount). */
size_t nvfp4_workspace_bytes(void);

/*
 * Kernel-path flags: a process-wide setting (default 0) that tests and
 * benchmarks use to reach paths the size-based choice would not take, or to
 * stop every call at the device check.  Results do not depend on the path
 * (each path is checked against the same bounds).  Not for production use;
 * changing the flags while other threads launch work is allowed but those
 * launches may use either setting.
 *   NVFP4_PATH_GEMM_GRID       the W4A4 GEMMs launch one workgroup per tile
 *                              instead of the persistent tile walk
 *   NVFP4_PATH_DECODE_DIRECT   w4a4_gemm_decode uses its register-load kernel
 *                              for every K
 *   NVFP4_PATH_REJECT_DEVICE   every entry point that would launch work
 *                              returns NVFP4_ERR_UNSUPPORTED after validating
 *                              its arguments (it can only reject a device)
 */
#define NVFP4_PATH_GEMM_GRID 1
#define NVFP4_PATH_DECODE_DIRECT 2
#define NVFP4_PATH_REJECT_DEVICE 4
void nvfp4_set_path_flags(int flags);
int nvfp4_path_flags(void);

/*
 * nvfp4_quantize_act - quantise a BF16 activation tensor X [M][K] (row
 * stride ld_x elements) to NVFP4 on the fly.
 *
 *   alpha_in   NULL: alpha is computed from X on the device (amax pass);
 *              otherwise the float32 at *alpha_in (device, finite, >= 0) is
 *              used for every row.
 *   alpha_out  device float32 receiving the alpha used (may equal alpha_in).
 *   codes      device [M][K/2];  scales  device [M][K/16].
 *   workspace  device scratch of nvfp4_workspace_bytes() bytes; the call
 *              uses it as it runs on `stream` (calls that overlap in time
 *              need separate workspaces).
 * Formulas: paper.rainbus digest, 方法步骤详情 step (3); r9-hu digest,
 * Method item 1.  M = 0 is allowed (nothing is launched unless alpha is to be
 * computed, in which case alpha_out receives 0).
 */
nvfp4_status_t nvfp4_quantize_act(const void* x_bf16, int64_t M, int64_t K,
                                  int64_t ld_x, const float* alpha_in,
                                  float* alpha_out, uint8_t* codes,
                                  uint8_t* scales, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_quantize_act_noalloc - nvfp4_quantize_act without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * The call allocates nothing: its scratch (amax partials, alpha's
 * parameters and the decision tables) is a fixed 15 616-byte array in the
 * library's device globals, one copy per device, held from the first call on
 * that device until the process ends.  The scratch is the same size for every
 * M and K, so the size limits are exactly those of nvfp4_quantize_act.  The
 * first call on a device looks the array's address up (hipGetSymbolAddress)
 * with that device current; a failure there returns NVFP4_ERR_LAUNCH.
 *
 * Every call on a device shares that device's array, and the array keeps the
 * last call's contents (each call rewrites all of it that it reads): calls
 * that overlap in time on one device race and give wrong results, so keep
 * them in order on one stream (or order their streams).  Arguments, results
 * and other errors as for nvfp4_quantize_act.
 */
nvfp4_status_t nvfp4_quantize_act_noalloc(const void* x_bf16, int64_t M, int64_t K,
                                          int64_t ld_x, const float* alpha_in,
                                          float* alpha_out, uint8_t* codes,
                                          uint8_t* scales, hipStream_t stream);

/*
 * nvfp4_quantize_weights - quantise a BF16 weight matrix (done once,
 * offline: paper.rainbus digest, 核心方法; same format as the activations)
 * into the GEMM's operand layout, N rows of K elements.
 *
 * Element (n, k) of the source is w_bf16[n * stride_n + k * stride_k], so a
 * row-major N x K matrix has (stride_n, stride_k) = (K, 1) and a row-major
 * K x N matrix has (1, N).  alpha is always computed from the whole matrix
 * (one alpha per weight tensor; a grouped layer quantises each expert with
 * its own call).  Outputs as for nvfp4_quantize_act.
 */
nvfp4_status_t nvfp4_quantize_weights(const void* w_bf16, int64_t N, int64_t K,
                                      int64_t stride_n, int64_t stride_k,
                                      float* alpha_out, uint8_t* codes,
                                      uint8_t* scales, void* workspace,
                                      size_t workspace_bytes,
                                      hipStream_t stream);

/*
 * w4a4_gemm - Y[M][N] = (alpha_a alpha_b) * sum_k (sigma q)_a[m][k] *
 * (sigma q)_b[n][k], the NVFP4 W4A4 linear layer (paper.rainbus digest,
 * 核心方法 "W4A4" and 方法步骤详情 step (4)).  Products of dequantised
 * operands are exact; they are accumulated in float32.
 *
 *   a_codes/a_scales  activation operand, [M][K/2] and [M][K/16]
 *   b_codes/b_scales  weight operand,     [N][K/2] and [N][K/16]
 *   alpha_a, alpha_b  device float32 scalars
 *   y_f32   nullable, float32 [M][ld_y];  y_bf16  nullable, BF16 [M][ld_y]
 *           (at least one non-NULL; BF16 is the RNE rounding of the float32
 *           value).  ld_y >= N.
 * M, N >= 0 (0 launches nothing), K >= 16.
 */
nvfp4_status_t w4a4_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
                         const float* alpha_a, const uint8_t* b_codes,
                         const uint8_t* b_scales, const float* alpha_b,
                         int64_t M, int64_t N, int64_t K, float* y_f32,
                         uint16_t* y_bf16, int64_t ld_y, hipStream_t stream);

/*
 * w4a4_gemm_multi - w4a4_gemm where the weight operand is several NVFP4
 * tensors stacked along N, each quantised under its own tensor scale (for
 * example the Q, K and V projections of one activation, 核心方法 "W4A4"
 * linear layers of the paper.rainbus digest, run as one launch):
 *
 *   b_codes/b_scales  the tensors' rows concatenated, [N][K/2], [N][K/16]
 *   alpha_b_rows      device float32 [N]: the tensor scale of each B row
 *
 * Output column n is scaled by alpha_a * alpha_b_rows[n]; every output is
 * bit-identical to w4a4_gemm on that row's own tensor.  Other arguments,
 * ownership and errors as for w4a4_gemm.
 */
nvfp4_status_t w4a4_gemm_multi(const uint8_t* a_codes, const uint8_t* a_scales,
                               const float* alpha_a, const uint8_t* b_codes,
                               const uint8_t* b_scales, const float* alpha_b_rows,
                               int64_t M, int64_t N, int64_t K, float* y_f32,
                               uint16_t* y_bf16, int64_t ld_y, hipStream_t stream);

/*
 * nvfp4_rmsnorm_quantize_act - RMSNorm with the activation quantiser fused
 * into it: the normalised activation is produced as NVFP4 (codes, scales,
 * alpha) without a BF16 tensor in between.  The pages' models (Qwen3-8B,
 * Qwen3.5-9B, Gemma-4; paper.rainbus digest, 实验结果) normalise each block's
 * input with RMSNorm before the quantised projections; the pages do not
 * define it, and the standard definition is taken:
 *
 *   y[m][k] = RNE_bf16( x[m][k] * r_m * gamma[k] ),
 *   r_m     = 1 / sqrt( (1/K) sum_k x[m][k]^2 + eps )       (float32)
 *
 * and y is quantised exactly as nvfp4_quantize_act quantises a BF16 tensor
 * (alpha from the amax of |y| unless alpha_in is given; 方法步骤详情 step (3)).
 *
 *   x_bf16      [M][ld_x] BF16 (16-byte aligned, ld_x * 2 a multiple of 16)
 *   gamma_bf16  [K] BF16 weights (16-byte aligned)
 *   K           a multiple of 16, at most 8192 (the row is held in registers)
 *   eps         >= 0
 *   alpha_in, alpha_out, codes, scales: as nvfp4_quantize_act
 *   workspace   device scratch of at least nvfp4_workspace_bytes() bytes;
 *               with nvfp4_rmsnorm_workspace_bytes(M) bytes or more (and
 *               alpha_in null) the amax pass of rows longer than 5120 also
 *               stores each row's r there and the quantise pass reads it
 *               instead of reading the row twice (a faster kernel, the same
 *               results)
 *   y_bf16      nullable: when set, y itself is also written, [M][ld_y]
 *               (16-byte aligned, ld_y a multiple of 8, ld_y >= K)
 * The two passes read x twice; both see the same y, whether r is summed in
 * each pass by the same arithmetic or stored by the first.  Errors and
 * ownership as for nvfp4_quantize_act.
 */
/* Workspace bytes with which nvfp4_rmsnorm_quantize_act keeps each row's r
 * between its passes (nvfp4_workspace_bytes() plus 4 bytes a row, rounded);
 * 0 for M < 0. */
size_t nvfp4_rmsnorm_workspace_bytes(int64_t M);

nvfp4_status_t nvfp4_rmsnorm_quantize_act(const void* x_bf16, const void* gamma_bf16, int64_t M,
                                          int64_t K, int64_t ld_x, float eps,
                                          const float* alpha_in, float* alpha_out,
                                          uint8_t* codes, uint8_t* scales, uint16_t* y_bf16,
                                          int64_t ld_y, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);

/*
 * w4a4_gemm_silu_mul_quantize - the gate|up projection of a gated MLP with
 * the activation and the next quantiser fused in: the W4A4 GEMM's epilogue
 * computes H = SiLU(gate) * up, the down projection's input, in BF16
 * together with the amax of |H| per tile, then H is quantised to NVFP4 with
 * alpha from those maxima (方法步骤详情 step (3)).  The pages' models
 * (Qwen3-8B and its kin; paper.rainbus digest, 实验结果) use this gated MLP
 * without defining it; the standard definition is taken.  The gate and up
 * outputs never reach memory.
 *
 *   b_codes/b_scales  the gate and up weights interleaved in 32-row blocks:
 *                     rows 64j .. 64j + 31 are gate rows 32j .. 32j + 31 and
 *                     rows 64j + 32 .. 64j + 63 the up rows of the same
 *                     units; N = 2 x hidden, a multiple of 64
 *   alpha_b_rows      device float32 [N]: the tensor scale of each B row
 *   h_bf16            [M][ld_h] BF16 (ld_h >= N/2, a multiple of 8, 16-byte
 *                     aligned): H, written, then read by the quantiser
 *   H[m][u] = RNE_bf16( g * v / (1 + exp(-g)) ), with g and v the float32
 *             gate and up outputs (alpha_a alpha_b sum ...) of unit u
 *   alpha_h_out, h_codes [M][N/4], h_scales [M][N/32]: H in NVFP4
 *   workspace  at least w4a4_gemm_silu_mul_workspace_bytes(M, N) bytes
 *             (16-byte aligned): the quantiser's tables and the tile maxima
 * Other arguments, ownership and errors as for w4a4_gemm_multi.
 */
size_t w4a4_gemm_silu_mul_workspace_bytes(int64_t M, int64_t N);
nvfp4_status_t w4a4_gemm_silu_mul_quantize(const uint8_t* a_codes, const uint8_t* a_scales,
                                           const float* alpha_a, const uint8_t* b_codes,
                                           const uint8_t* b_scales, const float* alpha_b_rows,
                                           int64_t M, int64_t N, int64_t K, uint16_t* h_bf16,
                                           int64_t ld_h, float* alpha_h_out, uint8_t* h_codes,
                                           uint8_t* h_scales, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream);

/*
 * w4a4_gemm_decode - the W4A4 GEMM at decode shape: M <= 64 token rows
 * against a whole NVFP4 weight matrix, Y = A . B^T with the same arithmetic
 * and outputs as w4a4_gemm.  This is the decode step of the uniform-NVFP4
 * configuration Mix-Quant is compared with (paper.rainbus digest, 实验结果,
 * Table 1 and the phase-wise ablation of Table 3).  At this shape the time
 * goes to reading the weight codes once, so the kernel is laid out for the
 * HBM stream rather than for the matrix cores (one workgroup per 16 output
 * columns).
 *
 *   a_codes/a_scales  the quantised token rows, [M][K/2] and [M][K/16]
 *   b_codes/b_scales  the weight, [N][K/2] and [N][K/16]
 *   alpha_b           device float32: the weight's tensor scale, or
 *   alpha_b_rows      nullable device float32 [N]: the tensor scale of each
 *                     B row (stacked weights as in w4a4_gemm_multi); when
 *                     set it is used instead of alpha_b.
 * M must lie in [0, NVFP4_DECODE_MAX_ROWS] (else NVFP4_ERR_SHAPE); larger
 * batches go to w4a4_gemm.  Scales need 2-byte alignment when K % 32 == 0.
 * Outputs are within the same bound of the exact product as w4a4_gemm's
 * (float32 sums in another order, so not bit-identical to it).  Ownership,
 * stream and other errors as for w4a4_gemm.
 */
#define NVFP4_DECODE_MAX_ROWS 64
nvfp4_status_t w4a4_gemm_decode(const uint8_t* a_codes, const uint8_t* a_scales,
                                const float* alpha_a, const uint8_t* b_codes,
                                const uint8_t* b_scales, const float* alpha_b,
                                const float* alpha_b_rows, int64_t M, int64_t N, int64_t K,
                                float* y_f32, uint16_t* y_bf16, int64_t ld_y,
                                hipStream_t stream);

/*
 * w4a4_gemm_grouped - the W4A4 GEMM of a mixture-of-experts layer: one
 * launch over num_groups experts with ragged row counts.
 *
 *   group_offsets  device int64 [num_groups + 1], non-decreasing,
 *                  group_offsets[0] = 0 and group_offsets[num_groups] = M:
 *                  GEMM rows [off[g], off[g+1]) use expert g.
 *   a_row_index    nullable device int32 [M]: GEMM row r reads operand-A row
 *                  a_row_index[r] (each in [0, a_rows)); NULL means row r.
 *                  This gathers routed tokens straight from the quantised
 *                  activation, which is bit-identical to quantising after the
 *                  gather because one alpha covers the tensor.
 *   b_codes/b_scales  [num_groups][N][K/2] and [num_groups][N][K/16]
 *   alpha_b           device float32 [num_groups]
 * The offsets are read on the device (no host synchronisation); malformed
 * offsets are out of contract.
 */
nvfp4_status_t w4a4_gemm_grouped(const uint8_t* a_codes,
                                 const uint8_t* a_scales, const float* alpha_a,
                                 int64_t a_rows, const int32_t* a_row_index,
                                 const uint8_t* b_codes,
                                 const uint8_t* b_scales, const float* alpha_b,
                                 int64_t M, int64_t N, int64_t K,
                                 int32_t num_groups,
                                 const int64_t* group_offsets, float* y_f32,
                                 uint16_t* y_bf16, int64_t ld_y,
                                 hipStream_t stream);

/*
 * w4a4_gemm_fused_act - the same layer with the activation quantiser fused
 * into the GEMM: each workgroup quantises its BF16 A tile under alpha_a while
 * it loads it, so the NVFP4 activation never goes through HBM.  alpha_a is a
 * device float32 (e.g. from nvfp4_tensor_alpha); the call first rebuilds the
 * exact decision tables for it in `workspace` (nvfp4_workspace_bytes()).
 * Results are identical to nvfp4_quantize_act(alpha_in = alpha_a) followed by
 * w4a4_gemm.  x_bf16 is [M][ld_x]; other arguments as for w4a4_gemm.
 */
nvfp4_status_t w4a4_gemm_fused_act(const void* x_bf16, int64_t ld_x,
                                   const float* alpha_a,
                                   const uint8_t* b_codes,
                                   const uint8_t* b_scales,
                                   const float* alpha_b, int64_t M, int64_t N,
                                   int64_t K, float* y_f32, uint16_t* y_bf16,
                                   int64_t ld_y, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_tensor_alpha - only the amax pass: alpha_out = RNE_fp32(max|x|/2688)
 * of a BF16 tensor [M][K] (ld_x), for callers that fuse the quantiser.
 */
nvfp4_status_t nvfp4_tensor_alpha(const void* x_bf16, int64_t M, int64_t K,
                                  int64_t ld_x, float* alpha_out,
                                  void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * bf16_gemm_baseline - the BF16 comparison GEMM (the pages compare NVFP4
 * prefill against BF16: paper.rainbus digest, 实验结果 (3), Figure 4):
 * Y[M][N] = X[M][K] . W[N][K]^T with BF16 operands, float32 accumulation.
 * num_groups >= 1; with num_groups > 1, W is [num_groups][N][K] and
 * group_offsets (device int64 [num_groups+1]) splits the rows of X as in
 * w4a4_gemm_grouped (pass NULL when num_groups == 1).  K % 16 == 0.
 */
nvfp4_status_t bf16_gemm_baseline(const void* x_bf16, const void* w_bf16,
                                  int64_t M, int64_t N, int64_t K,
                                  int32_t num_groups,
                                  const int64_t* group_offsets, float* y_f32,
                                  uint16_t* y_bf16, int64_t ld_y,
                                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_W4A4_H */
