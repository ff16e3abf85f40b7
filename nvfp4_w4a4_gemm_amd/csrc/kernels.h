// Internal interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

// Kernel-path flags set through nvfp4_set_path_flags (api.cpp).
constexpr int kPathGemmGrid = 1, kPathDecodeDirect = 2, kPathRejectDevice = 4;
int path_flags();

// ---- quantiser workspace layout (bytes) ------------------------------------
constexpr int kAmaxPartials = 1024;          // per-workgroup maxima (uint32)
constexpr size_t kWsPartials = 0;
constexpr size_t kWsParams = 4096;           // QuantParams
constexpr int kSigLutN = 2944;               // BF16 amax_b in [2^-10, 2^13)
constexpr size_t kWsSigLut = 4096 + 256;
constexpr int kCodeLutRow = 1024;            // BF16 x in [2^-3, 2^5)
constexpr int kCodeLutN = 8 * kCodeLutRow;   // one row per E4M3 mantissa
constexpr size_t kWsCodeLut = kWsSigLut + 3072;
constexpr size_t kWorkspaceBytes = kWsCodeLut + kCodeLutN;   // 15616
// RMSNorm + quantiser: one float a row after the quantiser's workspace
constexpr size_t kWsRowR = 15872;
static_assert(kWsRowR >= kWorkspaceBytes && kWsRowR % 256 == 0, "row r offset");

// BF16 bit patterns of the first entries of the two tables.
constexpr int kSigLutBase = 117 * 128;       // 2^-10
constexpr int kCodeLutBase = 124 * 128;      // 2^-3

// Written by the prepare kernel, read by the quantise kernels.
struct QuantParams {
  float alpha;       // the tensor scale used
  int32_t sig_off;   // LUT index of a block = amax bits + sig_off (clamped)
  int32_t code_off;  // code LUT index term 128 * s - kCodeLutBase
  int32_t shift;     // s: alpha * 2^s lies in [1, 2)
  int32_t slow;      // 1: exponent range needs the exact rescaling path
  int32_t pad[3];
};

struct FastDivHost {
  uint32_t d, mul, shift;
};
FastDivHost make_fast_div(uint32_t d);

// ---- quantiser -------------------------------------------------------------
hipError_t launch_amax(const uint16_t* x, int64_t rows, int64_t k,
                       int64_t stride_row, int64_t stride_k, uint8_t* ws,
                       int* n_partials, hipStream_t stream);
hipError_t launch_prepare(const uint8_t* ws_partials, int n_partials,
                          const float* alpha_in, float* alpha_out, uint8_t* ws,
                          hipStream_t stream);
hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t k,
                           int64_t stride_row, int64_t stride_k,
                           const uint8_t* ws, uint8_t* codes, uint8_t* scales,
                           hipStream_t stream);

// ---- RMSNorm with the quantiser fused in ------------------------------------
struct RmsQuantArgs {
  const uint16_t* x;         // BF16 [M][ld_x]
  const uint16_t* gamma;     // BF16 [K]
  int64_t M, K, ld_x;
  float eps;
  uint8_t* ws;               // quantiser workspace (partials, tables)
  uint8_t* codes;
  uint8_t* scales;
  uint16_t* y_out;           // nullable BF16 [M][ld_y]
  int64_t ld_y;
  bool amax_pass;            // true: the amax pass, false: the quantise pass
  float* row_r;              // nullable [M]: each row's r, written by the amax
                             // pass, read by the segment-walk quantise pass
};
constexpr int64_t kRmsMaxK = 8192;
int rmsnorm_amax_grid(int64_t M, int64_t K);   // workgroups (partials) of the amax pass
hipError_t launch_rmsnorm_quant(const RmsQuantArgs& args, hipStream_t stream);

// ---- GEMMs -----------------------------------------------------------------
struct W4A4Args {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* alpha_a;
  const int32_t* a_row_index;     // nullable gather
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  const float* alpha_b;
  const float* alpha_b_rows;      // nullable: tensor scale of each B row [N]
  int64_t M, N, K;
  int32_t num_groups;             // 1 for a dense GEMM
  const int64_t* group_offsets;   // device [num_groups + 1] or nullptr
  float* y_f32;
  uint16_t* y_bf16;
  int64_t ld_y;
  // fused activation quantisation (a_codes/a_scales unused when set)
  const uint16_t* a_bf16;
  int64_t ld_a;
  const uint8_t* ws;              // prepared decision tables for alpha_a
  // gated activation (launch_w4a4_silu): H [M][N/2] BF16 and the amax of
  // |H| bits per tile (tile blockIdx.y * gridDim.x + blockIdx.x)
  uint16_t* h_bf16;
  int64_t ld_h;
  uint32_t* h_partials;
  // set by the launcher: the output rows may be written 16 bytes at a time
  int32_t vec_f32, vec_bf16, vec_h;
};
hipError_t launch_w4a4(const W4A4Args& args, hipStream_t stream);
hipError_t launch_w4a4_fused(const W4A4Args& args, hipStream_t stream);
hipError_t launch_w4a4_silu(const W4A4Args& args, hipStream_t stream);
int64_t w4a4_silu_tiles_max(int64_t M, int64_t N);   // bound on h_partials entries
int64_t w4a4_tiles(int64_t M, int64_t N);            // workgroups of a dense launch

// Decode-shaped W4A4 GEMM (M <= 64): codes/scales/alphas as in W4A4Args.
struct DecodeArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* alpha_a;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  const float* alpha_b;           // used when alpha_b_rows is null
  const float* alpha_b_rows;      // nullable: tensor scale of each B row [N]
  int64_t M, N, K;
  float* y_f32;
  uint16_t* y_bf16;
  int64_t ld_y;
};
hipError_t launch_w4a4_decode(const DecodeArgs& args, hipStream_t stream);

struct Bf16Args {
  const uint16_t* x;
  const uint16_t* w;
  int64_t M, N, K;
  int32_t num_groups;
  const int64_t* group_offsets;
  float* y_f32;
  uint16_t* y_bf16;
  int64_t ld_y;
};
hipError_t launch_bf16(const Bf16Args& args, hipStream_t stream);

}  // namespace nvfp4
