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
// Two passes over x, one wave per row (the row stays in registers, gamma
// sits in LDS as float32, unpacked once per workgroup):
//   1. rmsnorm_amax_kernel: r and the amax of |y| per workgroup (partials);
//   2. prepare_kernel (quantize.hip): alpha and the decision tables;
//   3. rmsnorm_quantize_kernel: r and y again, by the same code, then codes
//      and scales (and y itself when asked for).  For rows too long to hold
//      (K > 5120), when the workspace has room for one float a row, pass 1
//      also leaves each row's r there and pass 3 is
//      rmsnorm_quantize_seg_kernel: the flat quantiser's 4 KiB segment walk,
//      y from x, the stored r and gamma, instead of reading each row twice.
// HBM traffic: 2 + 2 + 0.5625 bytes an element, against 2 + 2 (a separate
// RMSNorm) + 2 + 2.5625 (the quantiser) unfused.
//
// r and y are computed by one device function in both passes: fixed-order
// two-term dot products summing the squares per lane, a fixed-order DPP
// reduction over the wave whose total one lane hands to all, IEEE division and
// square root, and y = (x * r) * gamma, so pass 3 reproduces pass 1's y bit
// for bit.
#include "device_common.h"
#include "kernels.h"
#include "quant_block.h"

#include <atomic>
#include <type_traits>

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;   // one wave a row

// Row chunk c (8 elements, 16 bytes) of lane l: c = l + 64 j, j < CH.
template <int CH>
struct Row {
  u32x4 x[CH];
};

// kFull: K = 512 CH, every chunk of every lane is in the row (no checks).
template <int CH, bool kFull>
__device__ __forceinline__ void load_row(const uint16_t* __restrict__ xr, int nc, int lane,
                                         Row<CH>& row) {
  const u32x4* p = reinterpret_cast<const u32x4*>(xr);
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = lane + 64 * j;
    // non-temporal: a streamed read, so the tensor does not churn L2 and MALL
    row.x[j] = kFull || c < nc ? __builtin_nontemporal_load(&p[c]) : u32x4{0u, 0u, 0u, 0u};
  }
}

// acc + lo^2 + hi^2 of the two BF16 values packed in w, in one two-term
// dot product (the same instruction in both passes, so the same bits)
__device__ __forceinline__ float sq2(uint32_t w, float acc) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const bf16x2v b = __builtin_bit_cast(bf16x2v, w);
  return __builtin_amdgcn_fdot2_f32_bf16(b, b, acc, false);
}

// Sum of v over the wave, the same value on every lane: DPP steps in a
// fixed order (pairs, quads, half rows, rows of 16, then rows 0+1 and
// 0+1+2+3 by row broadcasts; lane 63 ends with the total), then lane 63's
// value to all lanes.  Every step stays in the VALU (no LDS round trip).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                 0, __builtin_bit_cast(int, v), kCtrl, kRowMask, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xB1, 0xF>(v);     // quad_perm [1,0,3,2]
  v = dpp_add<0x4E, 0xF>(v);     // quad_perm [2,3,0,1]
  v = dpp_add<0x141, 0xF>(v);    // row_half_mirror
  v = dpp_add<0x140, 0xF>(v);    // row_mirror
  v = dpp_add<0x142, 0xA>(v);    // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);    // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
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
    for (int i = 0; i < 4; ++i) part[i] = sq2(w[i], part[i]);
  }
  const float ss = wave_sum((part[0] + part[1]) + (part[2] + part[3]));
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

// gamma of the held-row kernels as float32 in LDS, unpacked once per
// workgroup: chunk c's elements 0-3 at h[0][c], 4-7 at h[1][c] (the lanes of a
// wave read consecutive 16-byte slots, so no bank conflicts).  Chunks past
// the row's end hold zeros.
template <int CH>
struct GammaLds {
  float4_t h[2][64 * CH];
};

template <int CH>
__device__ __forceinline__ void fill_gamma(const uint16_t* __restrict__ gamma, int nc,
                                           GammaLds<CH>& gl) {
  const u32x4* g4 = reinterpret_cast<const u32x4*>(gamma);
  for (int c = threadIdx.x; c < 64 * CH; c += kThreads) {
    const u32x4 g = c < nc ? g4[c] : u32x4{0u, 0u, 0u, 0u};
    gl.h[0][c] = float4_t{__uint_as_float(g.x << 16), __uint_as_float(g.x & 0xFFFF0000u),
                          __uint_as_float(g.y << 16), __uint_as_float(g.y & 0xFFFF0000u)};
    gl.h[1][c] = float4_t{__uint_as_float(g.z << 16), __uint_as_float(g.z & 0xFFFF0000u),
                          __uint_as_float(g.w << 16), __uint_as_float(g.w & 0xFFFF0000u)};
  }
}

// The float32 values (x * r) * gamma of one chunk (the same arithmetic as
// chunk_y, before the rounding to BF16), gamma from LDS.
struct Chunk8f {
  float v[8];
};
__device__ __forceinline__ Chunk8f chunk_xrg(const u32x4 x, const float4_t ga, const float4_t gb,
                                             float r) {
  uint32_t xw[4] = {x.x, x.y, x.z, x.w};
  asm volatile("" : "+v"(xw[0]), "+v"(xw[1]), "+v"(xw[2]), "+v"(xw[3]));
  const float g[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
  Chunk8f o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o.v[2 * i] = (__uint_as_float(xw[i] << 16) * r) * g[2 * i];
    o.v[2 * i + 1] = (__uint_as_float(xw[i] & 0xFFFF0000u) * r) * g[2 * i + 1];
  }
  return o;
}

__device__ __forceinline__ u32x4 to_bf16x8(const Chunk8f& f) {
  uint32_t y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    y[i] = __builtin_bit_cast(uint32_t,
                              __builtin_convertvector((float2_t){f.v[2 * i], f.v[2 * i + 1]},
                                                      bf16x2_t));
  return u32x4{y[0], y[1], y[2], y[3]};
}

// The wave's rows: blockIdx.x * 4 + wave, then every gridDim.x * 4 rows.
// With kPre the next row's x is loaded before the current row is processed,
// so one row's HBM round trip overlaps the other's arithmetic.
// `first(load)` runs once and must call load() (which issues the first
// row's loads); the quantise pass issues its table loads before it.  Every
// wave of the workgroup runs it, also a wave without a row.
template <int CH, bool kPre, bool kFull, typename First, typename Body>
__device__ __forceinline__ void for_rows(const uint16_t* __restrict__ x, int M, int nc,
                                         int64_t ld_x, int lane, First first, Body body) {
  const int stride = gridDim.x * kRowsPerBlock;
  int rowi = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  Row<CH> cur;
  first([&] {
    if (rowi < M) load_row<CH, kFull>(x + rowi * ld_x, nc, lane, cur);
  });
  if (rowi >= M) return;
  if constexpr (kPre) {
    // two rows an iteration, alternating buffers, so the prefetched row is
    // never copied between registers
    Row<CH> alt;
    while (true) {
      int nxt = rowi + stride;
      if (nxt < M) load_row<CH, kFull>(x + nxt * ld_x, nc, lane, alt);
      body(rowi, cur);
      if (nxt >= M) break;
      rowi = nxt;
      nxt = rowi + stride;
      if (nxt < M) load_row<CH, kFull>(x + nxt * ld_x, nc, lane, cur);
      body(rowi, alt);
      if (nxt >= M) break;
      rowi = nxt;
    }
  } else {
    while (true) {
      const int nxt = rowi + stride;
      body(rowi, cur);
      if (nxt >= M) break;
      load_row<CH, kFull>(x + nxt * ld_x, nc, lane, cur);
      rowi = nxt;
    }
  }
}

// row_r (nullable): each row's r, for rmsnorm_quantize_seg_kernel.
template <int CH, bool kPre, bool kFull>
__global__ __launch_bounds__(kThreads) void rmsnorm_amax_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, int M, int K,
    int64_t ld_x, float eps, uint32_t* __restrict__ partials, float* __restrict__ row_r) {
  __shared__ GammaLds<CH> gl;
  const int lane = threadIdx.x & 63;
  const int nc = K / 8;
  uint32_t m = 0;       // BF16 magnitude bits (rows whose r is not finite)
  float mf = 0.0f;      // float32 magnitudes (every other row)
  auto first = [&](auto load) {
    load();
    fill_gamma<CH>(gamma, nc, gl);
    __syncthreads();
  };
  for_rows<CH, kPre, kFull>(x, M, nc, ld_x, lane, first, [&](int rowi, const Row<CH>& row) {
    const float r = row_inv_rms<CH>(row, K, eps);
    if (row_r != nullptr && lane == 0) row_r[rowi] = r;
    if (__builtin_isfinite(r)) {
      // |y| = RNE_bf16(|(x r) gamma|) and the rounding is monotonic, so the
      // largest |y| is the rounding of the largest float32 magnitude
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int c = lane + 64 * j;
        const Chunk8f f = chunk_xrg(row.x[j], gl.h[0][c], gl.h[1][c], r);   // zero past the end
#pragma unroll
        for (int i = 0; i < 8; i += 2)
          mf = __builtin_fmaxf(mf, __builtin_fmaxf(__builtin_fabsf(f.v[i]), __builtin_fabsf(f.v[i + 1])));
      }
    } else {
      // r = inf (eps = 0 and a row whose squares sum to 0): the BF16 values
      // themselves, so that a NaN y (0 * inf) reaches alpha as it would
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int c = lane + 64 * j;
        const u32x4 y = to_bf16x8(chunk_xrg(row.x[j], gl.h[0][c], gl.h[1][c], r));
        m = pk_max_u16(m, pk_max_u16(pk_max_u16(y.x & 0x7FFF7FFFu, y.y & 0x7FFF7FFFu),
                                     pk_max_u16(y.z & 0x7FFF7FFFu, y.w & 0x7FFF7FFFu)));
      }
    }
  });
  m = max(m & 0xFFFFu, m >> 16);
  m = max(m, __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){mf, 0.0f}, bf16x2_t)) &
                 0xFFFFu);
  m = wave_max_u32(m);
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
    for (int i = 0; i < 4; ++i) part[i] = sq2(w[i], part[i]);
  }
  const float ss = wave_sum((part[0] + part[1]) + (part[2] + part[3]));
  return 1.0f / __builtin_sqrtf(ss / (float)K + eps);
}

template <int CH>
__global__ __launch_bounds__(kThreads) void rmsnorm_amax_stream_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, int M, int K,
    int64_t ld_x, float eps, uint32_t* __restrict__ partials, float* __restrict__ row_r) {
  const int lane = threadIdx.x & 63;
  const int nc = K / 8;
  const u32x4* g4 = reinterpret_cast<const u32x4*>(gamma);
  uint32_t m = 0;
  for (int rowi = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6); rowi < M;
       rowi += gridDim.x * kRowsPerBlock) {
    const u32x4* xr = reinterpret_cast<const u32x4*>(x + rowi * ld_x);
    const float r = stream_inv_rms<CH>(xr, nc, lane, K, eps);
    if (row_r != nullptr && lane == 0) row_r[rowi] = r;
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
  m = wave_max_u32(m);
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

// Rows of the wave, streamed: codes, scales (and y) of each.  slow: alpha's
// exponent beyond +-100, the generic block path (which rescales first).
template <int CH>
__device__ __forceinline__ void stream_rows_quantize(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, int M, int K,
    int64_t ld_x, float eps, const BlockTables& tg, const FastTables& tf, bool slow,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint16_t* __restrict__ y_out,
    int64_t ld_y) {
  const int lane = threadIdx.x & 63;
  const int nc = K / 8;
  const u32x4* g4 = reinterpret_cast<const u32x4*>(gamma);
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
      uint32_t o, sb;
      if (slow) {
        uint32_t mag[8];
        magnitudes<4>(w, tg, mag);
        uint32_t amax = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = max(amax, mag[i]);
        amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0xB1, 0xF, 0xF, false));
        CodeRow cr;
        sb = block_scale(amax, tg, cr);
        o = codes8(mag, w, cr, tg);
      } else {
        o = quantize_half_block(w, tf, sb);
      }
      if (ok) {
        crow[c] = o;
        if ((lane & 1) == 0) srow[c >> 1] = (uint8_t)sb;
        if (y_out != nullptr) reinterpret_cast<u32x4*>(y_out + rowi * ld_y)[c] = y;
      }
    }
  }
}

template <int CH>
__global__ __launch_bounds__(kThreads) void rmsnorm_quantize_stream_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, int M, int K,
    int64_t ld_x, float eps, const uint8_t* __restrict__ ws, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, uint16_t* __restrict__ y_out, int64_t ld_y) {
  __shared__ TableLds tl;
  copy_tables_first(ws, tl, threadIdx.x, [] {});
  const QuantParams P = *reinterpret_cast<const QuantParams*>(ws + kWsParams);
  __syncthreads();
  stream_rows_quantize<CH>(x, gamma, M, K, ld_x, eps, tables_from(ws, tl.sig, tl.code),
                           fast_tables(tl, P), P.slow != 0, codes, scales, y_out, ld_y);
}

template <int CH, bool kPre, bool kFull>
__global__ __launch_bounds__(kThreads) void rmsnorm_quantize_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, int M, int K,
    int64_t ld_x, float eps, const uint8_t* __restrict__ ws, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, uint16_t* __restrict__ y_out, int64_t ld_y) {
  __shared__ TableLds tl;
  const int lane = threadIdx.x & 63;
  const int nc = K / 8;
  const QuantParams P = *reinterpret_cast<const QuantParams*>(ws + kWsParams);
  if (P.slow) {
    // alpha's exponent beyond +-100: the rows are streamed (as the streaming
    // variant does, with the same r and y bits) through the generic block
    // path, so that this rare path adds no registers to the held-row one
    copy_tables_first(ws, tl, threadIdx.x, [] {});
    __syncthreads();
    stream_rows_quantize<CH>(x, gamma, M, K, ld_x, eps, tables_from(ws, tl.sig, tl.code),
                             fast_tables(tl, P), true, codes, scales, y_out, ld_y);
    return;
  }
  __shared__ GammaLds<CH> gl;
  // the tables' loads go first, then the first row's (see copy_tables_first)
  auto tables = [&](auto load) {
    copy_tables_first(ws, tl, threadIdx.x, load);
    fill_gamma<CH>(gamma, nc, gl);
    __syncthreads();
  };
  for_rows<CH, kPre, kFull>(x, M, nc, ld_x, lane, tables, [&](int rowi, const Row<CH>& row) {
    const FastTables t = fast_tables(tl, P);
    const float r = row_inv_rms<CH>(row, K, eps);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      // lanes 2i and 2i + 1 hold the two halves of a block (64 is even);
      // every lane of the wave takes part in the exchange (past the row's
      // end the values are zero and nothing is stored)
      const int c = lane + 64 * j;
      const u32x4 y = to_bf16x8(chunk_xrg(row.x[j], gl.h[0][c], gl.h[1][c], r));
      const uint32_t w[4] = {y.x, y.y, y.z, y.w};
      uint32_t sb;
      const uint32_t o = quantize_half_block(w, t, sb);
      if (kFull || c < nc) {
        reinterpret_cast<uint32_t*>(codes + (int64_t)rowi * (K / 2))[c] = o;
        if ((lane & 1) == 0) (scales + (int64_t)rowi * (K / 16))[c >> 1] = (uint8_t)sb;
        if (y_out != nullptr) reinterpret_cast<u32x4*>(y_out + rowi * ld_y)[c] = y;
      }
      __builtin_amdgcn_sched_barrier(0);               // one chunk at a time (registers)
    }
  });
}

// Pass 3 with each row's r given (row_r, written by pass 1).  A row is cut
// into segments of 256 chunks (4 KiB; the last one may be shorter); the
// segments (row m, column segment s) are dealt to the waves in order, and
// the number of waves is a multiple of the segments a row (ns), so a wave
// keeps one column segment: its gamma chunks are loaded once, and r is one
// wave-uniform load a segment, issued with the segment's x.  Lane l takes
// chunks l, l + 64, l + 128 and l + 192 of the segment, as the flat
// quantiser does (lanes 2i and 2i + 1 hold the halves of a block: 256 s is
// even).  y = (x * r) * gamma by chunk_y, the same bits as pass 1's.
__global__ __launch_bounds__(kThreads) void rmsnorm_quantize_seg_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, int M, int K,
    int64_t ld_x, const float* __restrict__ row_r, const uint8_t* __restrict__ ws,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint16_t* __restrict__ y_out,
    int64_t ld_y) {
  __shared__ TableLds tl;
  const int tid = threadIdx.x, lane = tid & 63;
  const int nc = K / 8;
  const int ns = (nc + 255) / 256;
  const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * kRowsPerBlock + (tid >> 6));
  const int mstep = gridDim.x * kRowsPerBlock / ns;
  const int cb = 256 * (wave % ns) + lane;      // the lane's first chunk in a row
  int m = wave / ns;
  const u32x4* g4 = reinterpret_cast<const u32x4*>(gamma);
  u32x4 g[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) g[u] = cb + 64 * u < nc ? g4[cb + 64 * u] : u32x4{0u, 0u, 0u, 0u};
  auto load = [&](int mm, u32x4 (&v)[4], float& r) __attribute__((always_inline)) {
    const u32x4* xr = reinterpret_cast<const u32x4*>(x + (int64_t)mm * ld_x);
    const bool ok = mm < M;
    r = ok ? row_r[mm] : 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u)      // non-temporal, as in the other passes
      v[u] = ok && cb + 64 * u < nc ? __builtin_nontemporal_load(&xr[cb + 64 * u])
                                    : u32x4{0u, 0u, 0u, 0u};
  };
  u32x4 v[4];
  float r;
  copy_tables_first(ws, tl, tid, [&] { load(m, v, r); });
  const QuantParams P = *reinterpret_cast<const QuantParams*>(ws + kWsParams);
  __syncthreads();
  // kSlow: alpha's exponent beyond +-100, the generic block path (which
  // rescales first); otherwise the packed fast path
  auto walk = [&](auto slow) __attribute__((always_inline)) {
    constexpr bool kSlow = decltype(slow)::value;
    const BlockTables tg = tables_from(ws, tl.sig, tl.code);
    const FastTables tf = fast_tables(tl, P);
    while (m < M) {
      uint32_t* crow = reinterpret_cast<uint32_t*>(codes + (int64_t)m * (K / 2));
      uint8_t* srow = scales + (int64_t)m * (K / 16);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = cb + 64 * u;
        const u32x4 y = chunk_y(v[u], g[u], r);         // zero past the row end
        const uint32_t w[4] = {y.x, y.y, y.z, y.w};
        uint32_t o, sb;
        if constexpr (kSlow) {
          uint32_t mag[8];
          magnitudes<4>(w, tg, mag);
          uint32_t amax = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) amax = max(amax, mag[i]);
          amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0xB1, 0xF, 0xF, false));
          CodeRow cr;
          sb = block_scale(amax, tg, cr);
          o = codes8(mag, w, cr, tg);
        } else {
          o = quantize_half_block(w, tf, sb);
        }
        if (c < nc) {
          crow[c] = o;
          if ((lane & 1) == 0) srow[c >> 1] = (uint8_t)sb;
          if (y_out != nullptr) reinterpret_cast<u32x4*>(y_out + (int64_t)m * ld_y)[c] = y;
        }
      }
      m += mstep;
      load(m, v, r);
    }
  };
  if (P.slow)
    walk(std::true_type{});
  else
    walk(std::false_type{});
}

hipError_t launch_seg(const RmsQuantArgs& a, hipStream_t stream) {
  const int64_t ns = (a.K / 8 + 255) / 256;
  const int64_t need = (a.M * ns + kRowsPerBlock - 1) / kRowsPerBlock;   // a segment a wave
  int64_t grid = need < 2048 ? need : 2048;
  // waves a multiple of ns (ns <= 4 at K <= 8192; 4 waves a workgroup)
  if (ns == 3) grid = (grid + 2) / 3 * 3;
  hipLaunchKernelGGL(rmsnorm_quantize_seg_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     a.x, a.gamma, (int)a.M, (int)a.K, a.ld_x, a.row_r, a.ws, a.codes, a.scales,
                     a.y_out, a.ld_y);
  return hipGetLastError();
}

// Workgroups of kernel k that fit on the device at once (cached per device;
// one cache per kernel instantiation).
template <auto kKernel>
int resident_blocks() {
  static std::atomic<int> cache[64];          // 0: not yet known
  int dev = 0;
  (void)hipGetDevice(&dev);
  int fit = cache[dev & 63].load(std::memory_order_relaxed);
  if (fit == 0) {
    int occ = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kKernel, kThreads, 0) != hipSuccess ||
        occ < 1)
      occ = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      cus = 256;
    fit = occ * cus;
    cache[dev & 63].store(fit, std::memory_order_relaxed);
  }
  return fit;
}

template <int CH>
hipError_t launch_stream(const RmsQuantArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.M + kRowsPerBlock - 1) / kRowsPerBlock;
  if (a.amax_pass) {
    const int grid = (int)(blocks < kAmaxPartials ? blocks : kAmaxPartials);
    hipLaunchKernelGGL((rmsnorm_amax_stream_kernel<CH>), dim3(grid), dim3(kThreads), 0, stream,
                       a.x, a.gamma, (int)a.M, (int)a.K, a.ld_x, a.eps,
                       reinterpret_cast<uint32_t*>(a.ws + kWsPartials), a.row_r);
    return hipGetLastError();
  }
  const int grid = (int)(blocks < 2048 ? blocks : 2048);
  hipLaunchKernelGGL((rmsnorm_quantize_stream_kernel<CH>), dim3(grid), dim3(kThreads), 0, stream,
                     a.x, a.gamma, (int)a.M, (int)a.K, a.ld_x, a.eps, a.ws, a.codes, a.scales,
                     a.y_out, a.ld_y);
  return hipGetLastError();
}

template <int CH, bool kFull>
int amax_grid_ch(int64_t M) {
  const int64_t blocks = (M + kRowsPerBlock - 1) / kRowsPerBlock;
  // as many workgroups as fit at once, so that no second, partial wave of
  // workgroups follows (measured 5% faster at 8192 x 4096 and 16384 x 5120)
  int64_t cap = resident_blocks<rmsnorm_amax_kernel<CH, (CH <= 10), kFull>>();
  if (cap > kAmaxPartials) cap = kAmaxPartials;
  return (int)(blocks < cap ? blocks : cap);
}

template <int CH, bool kFull>
hipError_t launch_ch_full(const RmsQuantArgs& a, hipStream_t stream) {
  // two rows held (the next one loading) where registers allow
  constexpr bool kPre = CH <= 10;
  constexpr bool kPreA = CH <= 10;
  const int64_t blocks = (a.M + kRowsPerBlock - 1) / kRowsPerBlock;
  if (a.amax_pass) {
    const int grid = amax_grid_ch<CH, kFull>(a.M);
    hipLaunchKernelGGL((rmsnorm_amax_kernel<CH, kPreA, kFull>), dim3(grid), dim3(kThreads), 0,
                       stream, a.x, a.gamma, (int)a.M, (int)a.K, a.ld_x, a.eps,
                       reinterpret_cast<uint32_t*>(a.ws + kWsPartials), a.row_r);
    return hipGetLastError();
  }
  // persistent: as many workgroups as fit at once (each copies the tables
  // once and walks several rows)
  const int fit = resident_blocks<rmsnorm_quantize_kernel<CH, kPre, kFull>>();
  const int grid = (int)(blocks < fit ? blocks : fit);
  hipLaunchKernelGGL((rmsnorm_quantize_kernel<CH, kPre, kFull>), dim3(grid), dim3(kThreads), 0,
                     stream, a.x, a.gamma, (int)a.M, (int)a.K, a.ld_x, a.eps, a.ws, a.codes,
                     a.scales, a.y_out, a.ld_y);
  return hipGetLastError();
}

// kFull when every lane's CH chunks are all in the row (K = 512 CH): the
// loads and stores then need no per-chunk check
template <int CH>
hipError_t launch_ch(const RmsQuantArgs& a, hipStream_t stream) {
  return a.K == 512 * CH ? launch_ch_full<CH, true>(a, stream) : launch_ch_full<CH, false>(a, stream);
}

template <int CH>
int amax_grid_of(int64_t M, int64_t K) {
  return K == 512 * CH ? amax_grid_ch<CH, true>(M) : amax_grid_ch<CH, false>(M);
}

}  // namespace

int rmsnorm_amax_grid(int64_t M, int64_t K) {
  const int64_t ch = (K + 511) / 512;
  if (ch <= 1) return amax_grid_of<1>(M, K);
  if (ch <= 2) return amax_grid_of<2>(M, K);
  if (ch <= 4) return amax_grid_of<4>(M, K);
  if (ch <= 6) return amax_grid_of<6>(M, K);
  if (ch <= 8) return amax_grid_of<8>(M, K);
  if (ch <= 10) return amax_grid_of<10>(M, K);
  const int64_t blocks = (M + kRowsPerBlock - 1) / kRowsPerBlock;   // streaming kernels
  return (int)(blocks < kAmaxPartials ? blocks : kAmaxPartials);
}

hipError_t launch_rmsnorm_quant(const RmsQuantArgs& args, hipStream_t stream) {
  if (args.M == 0) return hipSuccess;
  // the row in registers: 16-byte chunks a lane = ceil(K / 512)
  const int64_t ch = (args.K + 511) / 512;
  // with room for each row's r, rows too long to hold in registers take the
  // segment walk (measured 20% faster than streaming the row again at
  // K = 8192); held rows sum themselves again (as fast or faster below)
  RmsQuantArgs a = args;
  if (ch <= 10) a.row_r = nullptr;
  if (!a.amax_pass && a.row_r != nullptr) return launch_seg(a, stream);
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
