// RMSNorm with the NVFP4 quantiser fused into it: the producer of a quantised
// projection's input writes codes and scales instead of a BF16 tensor that
// the quantiser would read twice.  The pages' models (Qwen3-8B, Qwen3.5-9B,
// Gemma-4; "Mix-Quant：面向智能体LLM的量化预填充与精确解码", paper.rainbus.top
// digest, 实验结果) normalise every attention and MLP input with RMSNorm;
// the pages do not define it, and the standard definition is taken:
//
//   y_i = RNE_bf16( x_i * r * gamma_i ),  r = 1 / sqrt( mean_j x_j^2 + eps )
//
// and y is then quantised exactly as the quantiser does (alpha = RNE_fp32(
// amax|y| / 2688), block scales and codes by the exact decision tables;
// same digest, 方法步骤详情 step (3)).
//
// Two passes over x, one wave per row (the row stays in registers):
//   1. rmsnorm_amax_kernel: r and the amax of |y| per workgroup (partials);
//   2. prepare_kernel (quantize.hip): alpha and the decision tables;
//   3. rmsnorm_quantize_kernel: r and y again, by the same code, then codes
//      and scales (and y itself when asked for).
// HBM traffic: 2 + 2 + 0.5625 bytes an element, against 2 + 2 (a separate
// RMSNorm) + 2 + 2.5625 (the quantiser) unfused.
//
// r and y are computed by one device function in both passes: fixed-order
// fused multiply-add sums of the squares per lane, a butterfly over the wave
// (every lane ends with the same sum, as float addition is commutative),
// IEEE division and square root, and y = (x * r) * gamma, so pass 3
// reproduces pass 1's y bit for bit.
#include "device_common.h"
#include "kernels.h"
#include "quant_block.h"

#include <atomic>

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;   // one wave a row

// Row chunk c (8 elements, 16 bytes) of lane l: c = l + 64 j, j < CH.
template <int CH>
struct Row {
  u32x4 x[CH];
};

template <int CH>
__device__ __forceinline__ void load_row(const uint16_t* __restrict__ xr, int nc, int lane,
                                         Row<CH>& row) {
  const u32x4* p = reinterpret_cast<const u32x4*>(xr);
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = lane + 64 * j;
    // non-temporal: a streamed read, so the tensor does not churn L2 and MALL
    row.x[j] = c < nc ? __builtin_nontemporal_load(&p[c]) : u32x4{0u, 0u, 0u, 0u};
  }
}

// r = 1 / sqrt(mean(x^2) + eps); the same value on every lane.
template <int CH>
__device__ __forceinline__ float row_inv_rms(const Row<CH>& row, int K, float eps) {
  // four independent chains (word i of every chunk), then (0 + 1) + (2 + 3)
  float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const uint32_t w[4] = {row.x[j].x, row.x[j].y, row.x[j].z, row.x[j].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xFFFF0000u);
      part[i] = __builtin_fmaf(lo, lo, part[i]);
      part[i] = __builtin_fmaf(hi, hi, part[i]);
    }
  }
  float ss = (part[0] + part[1]) + (part[2] + part[3]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  return 1.0f / __builtin_sqrtf(ss / (float)K + eps);
}

// y of one chunk (8 values, element 2i in the low half of word i).
__device__ __forceinline__ u32x4 chunk_y(const u32x4 x, const u32x4 g, float r) {
  uint32_t xw[4] = {x.x, x.y, x.z, x.w};
  const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
  // unpack the words again here rather than keep the whole row unpacked
  // from the sum of squares (which would double the row's registers)
  asm volatile("" : "+v"(xw[0]), "+v"(xw[1]), "+v"(xw[2]), "+v"(xw[3]));
  uint32_t y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // BF16 -> float32 is a shift (low half) or a mask (high half); the two
    // results are rounded to BF16 together by the hardware RNE conversion
    const float lo = (__uint_as_float(xw[i] << 16) * r) * __uint_as_float(gw[i] << 16);
    const float hi = (__uint_as_float(xw[i] & 0xFFFF0000u) * r) *
                     __uint_as_float(gw[i] & 0xFFFF0000u);
    y[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){lo, hi}, bf16x2_t));
  }
  return u32x4{y[0], y[1], y[2], y[3]};
}

// The wave's rows: blockIdx.x * 4 + wave, then every gridDim.x * 4 rows.  A
// lane always touches the same chunks, so gamma is loaded once; with kPre
// the next row's x is loaded before the current row is processed, so one
// row's HBM round trip overlaps the other's arithmetic.
// `first` runs once, after the first row's loads are issued (the quantise
// pass copies its tables there); every wave of the workgroup runs it, also a
// wave without a row.
template <int CH, bool kPre, typename First, typename Body>
__device__ __forceinline__ void for_rows(const uint16_t* __restrict__ x, int M, int nc,
                                         int64_t ld_x, int lane, First first, Body body) {
  const int stride = gridDim.x * kRowsPerBlock;
  int rowi = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  Row<CH> cur;
  if (rowi < M) load_row<CH>(x + rowi * ld_x, nc, lane, cur);
  first();
  if (rowi >= M) return;
  while (true) {
    const int nxt = rowi + stride;
    Row<CH> pre;
    if (kPre && nxt < M) load_row<CH>(x + nxt * ld_x, nc, lane, pre);
    body(rowi, cur);
    if (nxt >= M) break;
    if (kPre) cur = pre;
    else load_row<CH>(x + nxt * ld_x, nc, lane, cur);
    rowi = nxt;
  }
}

template <int CH>
__device__ __forceinline__ void load_gamma(const uint16_t* __restrict__ gamma, int nc, int lane,
                                           u32x4 (&g)[CH]) {
  const u32x4* g4 = reinterpret_cast<const u32x4*>(gamma);
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = lane + 64 * j;
    g[j] = c < nc ? g4[c] : u32x4{0u, 0u, 0u, 0u};
  }
}

template <int CH, bool kPre>
__global__ __launch_bounds__(kThreads) void rmsnorm_amax_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, int M, int K,
    int64_t ld_x, float eps, uint32_t* __restrict__ partials) {
  const int lane = threadIdx.x & 63;
  const int nc = K / 8;
  u32x4 g[CH];
  load_gamma<CH>(gamma, nc, lane, g);
  uint32_t m = 0;
  for_rows<CH, kPre>(x, M, nc, ld_x, lane, [] {}, [&](int, const Row<CH>& row) {
    const float r = row_inv_rms<CH>(row, K, eps);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const u32x4 y = chunk_y(row.x[j], g[j], r);      // zero past the row end
      m = pk_max_u16(m, pk_max_u16(pk_max_u16(y.x & 0x7FFF7FFFu, y.y & 0x7FFF7FFFu),
                                   pk_max_u16(y.z & 0x7FFF7FFFu, y.w & 0x7FFF7FFFu)));
    }
  });
  m = max(m & 0xFFFFu, m >> 16);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t red[kRowsPerBlock];
  if (lane == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = red[0];
#pragma unroll
    for (int i = 1; i < kRowsPerBlock; ++i) v = max(v, red[i]);
    partials[blockIdx.x] = v;
  }
}

template <int CH, bool kPre>
__global__ __launch_bounds__(kThreads) void rmsnorm_quantize_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, int M, int K,
    int64_t ld_x, float eps, const uint8_t* __restrict__ ws, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, uint16_t* __restrict__ y_out, int64_t ld_y) {
  __shared__ __align__(16) uint8_t lds_sig[kSigLutN];
  __shared__ __align__(16) uint8_t lds_code[kCodeLutN];
  const int lane = threadIdx.x & 63;
  const int nc = K / 8;
  u32x4 g[CH];
  load_gamma<CH>(gamma, nc, lane, g);
  const BlockTables t = tables_from(ws, lds_sig, lds_code);
  // the tables are copied while the first row's loads are in flight
  auto tables = [&] {
    load_tables_to_lds(ws, lds_sig, lds_code, threadIdx.x, kThreads);
    __syncthreads();
  };
  for_rows<CH, kPre>(x, M, nc, ld_x, lane, tables, [&](int rowi, const Row<CH>& row) {
    const float r = row_inv_rms<CH>(row, K, eps);
    uint32_t* crow = reinterpret_cast<uint32_t*>(codes + (int64_t)rowi * (K / 2));
    uint8_t* srow = scales + (int64_t)rowi * (K / 16);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = lane + 64 * j;
      // lanes 2i and 2i + 1 hold the two halves of a block (64 is even);
      // every lane of the wave takes part in the exchange (past the row's
      // end the values are zero and nothing is stored)
      const u32x4 y = chunk_y(row.x[j], g[j], r);
      const uint32_t w[4] = {y.x, y.y, y.z, y.w};
      uint32_t mag[8];
      magnitudes<4>(w, t, mag);
      uint32_t amax = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = max(amax, mag[i]);
      amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0xB1, 0xF, 0xF, false));
      CodeRow cr;
      const uint32_t sb = block_scale(amax, t, cr);
      const uint32_t o = codes8(mag, w, cr, t);
      if (c < nc) {
        crow[c] = o;
        if ((lane & 1) == 0) srow[c >> 1] = (uint8_t)sb;
        if (y_out != nullptr) reinterpret_cast<u32x4*>(y_out + rowi * ld_y)[c] = y;
      }
      __builtin_amdgcn_sched_barrier(0);               // one chunk at a time (registers)
    }
  });
}

// ---- streaming variant (rows longer than 5120) -----------------------------
// The row is not held in registers: it is read once for the sum of squares
// and chunk by chunk again for y (the second read finds it in L2), gamma is
// read per chunk (L2), so a wave needs few registers.  The sum of
// squares visits the chunks, and the words of a chunk, in the same order as
// row_inv_rms, so r (and y) are the same bits as the register variant's.
template <int CH>
__device__ __forceinline__ float stream_inv_rms(const u32x4* __restrict__ xr, int nc, int lane,
                                                int K, float eps) {
  float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = lane + 64 * j;
    const u32x4 v = c < nc ? xr[c] : u32x4{0u, 0u, 0u, 0u};
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xFFFF0000u);
      part[i] = __builtin_fmaf(lo, lo, part[i]);
      part[i] = __builtin_fmaf(hi, hi, part[i]);
    }
  }
  float ss = (part[0] + part[1]) + (part[2] + part[3]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  return 1.0f / __builtin_sqrtf(ss / (float)K + eps);
}

template <int CH>
__global__ __launch_bounds__(kThreads) void rmsnorm_amax_stream_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, int M, int K,
    int64_t ld_x, float eps, uint32_t* __restrict__ partials) {
  const int lane = threadIdx.x & 63;
  const int nc = K / 8;
  const u32x4* g4 = reinterpret_cast<const u32x4*>(gamma);
  uint32_t m = 0;
  for (int rowi = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6); rowi < M;
       rowi += gridDim.x * kRowsPerBlock) {
    const u32x4* xr = reinterpret_cast<const u32x4*>(x + rowi * ld_x);
    const float r = stream_inv_rms<CH>(xr, nc, lane, K, eps);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = lane + 64 * j;
      if (c < nc) {
        const u32x4 y = chunk_y(xr[c], g4[c], r);
        m = pk_max_u16(m, pk_max_u16(pk_max_u16(y.x & 0x7FFF7FFFu, y.y & 0x7FFF7FFFu),
                                     pk_max_u16(y.z & 0x7FFF7FFFu, y.w & 0x7FFF7FFFu)));
      }
    }
  }
  m = max(m & 0xFFFFu, m >> 16);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t red[kRowsPerBlock];
  if (lane == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = red[0];
#pragma unroll
    for (int i = 1; i < kRowsPerBlock; ++i) v = max(v, red[i]);
    partials[blockIdx.x] = v;
  }
}

template <int CH>
__global__ __launch_bounds__(kThreads) void rmsnorm_quantize_stream_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, int M, int K,
    int64_t ld_x, float eps, const uint8_t* __restrict__ ws, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, uint16_t* __restrict__ y_out, int64_t ld_y) {
  __shared__ __align__(16) uint8_t lds_sig[kSigLutN];
  __shared__ __align__(16) uint8_t lds_code[kCodeLutN];
  const int lane = threadIdx.x & 63;
  const int nc = K / 8;
  const u32x4* g4 = reinterpret_cast<const u32x4*>(gamma);
  load_tables_to_lds(ws, lds_sig, lds_code, threadIdx.x, kThreads);
  const BlockTables t = tables_from(ws, lds_sig, lds_code);
  __syncthreads();
  for (int rowi = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6); rowi < M;
       rowi += gridDim.x * kRowsPerBlock) {
    const u32x4* xr = reinterpret_cast<const u32x4*>(x + rowi * ld_x);
    const float r = stream_inv_rms<CH>(xr, nc, lane, K, eps);
    uint32_t* crow = reinterpret_cast<uint32_t*>(codes + (int64_t)rowi * (K / 2));
    uint8_t* srow = scales + (int64_t)rowi * (K / 16);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = lane + 64 * j;
      const bool ok = c < nc;
      const u32x4 y = ok ? chunk_y(xr[c], g4[c], r) : u32x4{0u, 0u, 0u, 0u};
      const uint32_t w[4] = {y.x, y.y, y.z, y.w};
      uint32_t mag[8];
      magnitudes<4>(w, t, mag);
      uint32_t amax = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = max(amax, mag[i]);
      amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0xB1, 0xF, 0xF, false));
      CodeRow cr;
      const uint32_t sb = block_scale(amax, t, cr);
      const uint32_t o = codes8(mag, w, cr, t);
      if (ok) {
        crow[c] = o;
        if ((lane & 1) == 0) srow[c >> 1] = (uint8_t)sb;
        if (y_out != nullptr) reinterpret_cast<u32x4*>(y_out + rowi * ld_y)[c] = y;
      }
    }
  }
}

template <int CH>
hipError_t launch_stream(const RmsQuantArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.M + kRowsPerBlock - 1) / kRowsPerBlock;
  if (a.amax_pass) {
    const int grid = (int)(blocks < kAmaxPartials ? blocks : kAmaxPartials);
    hipLaunchKernelGGL((rmsnorm_amax_stream_kernel<CH>), dim3(grid), dim3(kThreads), 0, stream,
                       a.x, a.gamma, (int)a.M, (int)a.K, a.ld_x, a.eps,
                       reinterpret_cast<uint32_t*>(a.ws + kWsPartials));
    return hipGetLastError();
  }
  const int grid = (int)(blocks < 2048 ? blocks : 2048);
  hipLaunchKernelGGL((rmsnorm_quantize_stream_kernel<CH>), dim3(grid), dim3(kThreads), 0, stream,
                     a.x, a.gamma, (int)a.M, (int)a.K, a.ld_x, a.eps, a.ws, a.codes, a.scales,
                     a.y_out, a.ld_y);
  return hipGetLastError();
}

template <int CH>
hipError_t launch_ch(const RmsQuantArgs& a, hipStream_t stream) {
  // two rows held (the next one loading) where registers allow
  constexpr bool kPre = CH <= 10;
  const int64_t blocks = (a.M + kRowsPerBlock - 1) / kRowsPerBlock;
  if (a.amax_pass) {
    const int grid = (int)(blocks < kAmaxPartials ? blocks : kAmaxPartials);
    hipLaunchKernelGGL((rmsnorm_amax_kernel<CH, kPre>), dim3(grid), dim3(kThreads), 0, stream, a.x,
                       a.gamma, (int)a.M, (int)a.K, a.ld_x, a.eps,
                       reinterpret_cast<uint32_t*>(a.ws + kWsPartials));
    return hipGetLastError();
  }
  // persistent: as many workgroups as fit at once (each copies the tables
  // once and walks several rows)
  static std::atomic<int> cache[64];          // per device (0: not yet known)
  int dev = 0;
  (void)hipGetDevice(&dev);
  int fit = cache[dev & 63].load(std::memory_order_relaxed);
  if (fit == 0) {
    int occ = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, rmsnorm_quantize_kernel<CH, kPre>,
                                                     kThreads, 0) != hipSuccess || occ < 1)
      occ = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      cus = 256;
    fit = occ * cus;
    cache[dev & 63].store(fit, std::memory_order_relaxed);
  }
  const int grid = (int)(blocks < fit ? blocks : fit);
  hipLaunchKernelGGL((rmsnorm_quantize_kernel<CH, kPre>), dim3(grid), dim3(kThreads), 0, stream, a.x,
                     a.gamma, (int)a.M, (int)a.K, a.ld_x, a.eps, a.ws, a.codes, a.scales,
                     a.y_out, a.ld_y);
  return hipGetLastError();
}

}  // namespace

int rmsnorm_amax_grid(int64_t M) {
  const int64_t blocks = (M + kRowsPerBlock - 1) / kRowsPerBlock;
  return (int)(blocks < kAmaxPartials ? blocks : kAmaxPartials);
}

hipError_t launch_rmsnorm_quant(const RmsQuantArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  // the row in registers: 16-byte chunks a lane = ceil(K / 512)
  const int64_t ch = (a.K + 511) / 512;
  if (ch <= 1) return launch_ch<1>(a, stream);
  if (ch <= 2) return launch_ch<2>(a, stream);
  if (ch <= 4) return launch_ch<4>(a, stream);
  if (ch <= 6) return launch_ch<6>(a, stream);
  if (ch <= 8) return launch_ch<8>(a, stream);
  if (ch <= 10) return launch_ch<10>(a, stream);
  // longer rows: two would not fit in registers; streaming the row (measured
  // 6% faster at K = 8192, slower below)
  if (ch <= 12) return launch_stream<12>(a, stream);
  return launch_stream<16>(a, stream);
}

}  // namespace nvfp4
