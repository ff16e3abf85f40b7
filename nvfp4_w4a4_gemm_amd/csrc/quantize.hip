// NVFP4 activation/weight quantiser for gfx950.
//
// Computes, for a BF16 tensor x split into 16-element blocks b along K
// ("Mix-Quant：面向智能体LLM的量化预填充与精确解码", paper.rainbus.top
// digest, section 方法步骤详情 step (3); "Mix-Quant: Quantized Prefilling,
// Precise Decoding for Agentic LLMs", r9-hu.github.io digest, Method item 1):
//
//   alpha   = RNE_fp32(max|x| / 2688)
//   sigma_b = RNE_E4M3(max_{i in b}|x_i| / (6 alpha))       (saturating)
//   q_i     = RNE_E2M1(x_i / (alpha sigma_b))               (saturating)
//
// with every quotient taken exactly.  Three launches on the caller's stream:
//
//   amax     grid-stride max of the BF16 magnitude bits -> per-WG partials
//            (a flat walk over 16-byte chunks when the rows are contiguous).
//   prepare  a few workgroups, one table entry per thread: each reduces the
//            partials to alpha (IEEE float32 division) and builds its slice
//            of two exact decision tables for this alpha, in float64
//            (a float64 quotient of these short operands lands on the
//            correct side of every rounding midpoint and hits a midpoint only
//            when the exact quotient does):
//              sig_lut[j]  = E4M3 byte of RNE(a / (6 alpha_s)) for the BF16
//                            value a with bits kSigLutBase + j,
//              code_lut[k][i] = E2M1 code of RNE(v / (alpha_s (1 + k/8)))
//                            for the BF16 value v with bits kCodeLutBase + i,
//            where alpha_s = alpha * 2^s lies in [1, 2).
//   quantize streaming pass: one 16-element block per lane and iteration,
//            two 16-byte loads, block max from packed 16-bit compares, the
//            scale from sig_lut, and each code from code_lut indexed by the
//            element's BF16 bits shifted by the block scale's exponent.
//
// Why the tables are exact: scaling x and sigma by powers of two leaves the
// quotients unchanged, so the decision for (x, sigma = (1 + k/8) 2^e) equals
// the decision for (x 2^(s - e), 1 + k/8) at alpha_s; for a normal BF16 value
// the bits of x 2^(s-e) are bits(x) + 128 (s - e).  Values below the first
// table entry are below every rounding threshold (code/scale 0) and values
// above the last one are above every threshold (saturation), so indices are
// clamped.
#include "device_common.h"
#include "kernels.h"
#include "quant_block.h"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t block_amax_bits(const uint32_t w[8]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = pk_max_u16(m, w[i] & 0x7FFF7FFFu);
  return max(m & 0xFFFFu, m >> 16);
}

// Loads the 16 BF16 values of block (row, cb) into w[8] (2 per word).
template <bool kContig>
__device__ __forceinline__ void load_block(const uint16_t* __restrict__ x,
                                           int64_t row, uint32_t cb,
                                           int64_t stride_row,
                                           int64_t stride_k, uint32_t w[8]) {
  if (kContig) {
    const u32x4* p =
        reinterpret_cast<const u32x4*>(x + row * stride_row + (int64_t)cb * 16);
    u32x4 v0 = p[0];
    u32x4 v1 = p[1];
    w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w;
    w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
  } else {
    const uint16_t* p = x + row * stride_row + (int64_t)cb * 16 * stride_k;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t lo = p[(2 * i) * stride_k];
      uint32_t hi = p[(2 * i + 1) * stride_k];
      w[i] = lo | (hi << 16);
    }
  }
}

// Block index -> (row, block-in-row).  Contiguous tensors are walked row by
// row; the transposed (stride_k != 1) weight layout walks rows fastest so
// neighbouring lanes read neighbouring addresses.
template <bool kContig>
__device__ __forceinline__ void block_coords(uint32_t b, uint32_t rows,
                                             uint32_t kb, const FastDiv& div,
                                             int64_t& row, uint32_t& cb) {
  if (kContig) {
    uint32_t r = fast_div(b, div);   // div.d == kb
    row = r;
    cb = b - r * kb;
  } else {
    uint32_t c = fast_div(b, div);   // div.d == rows
    cb = c;
    row = b - c * rows;
  }
}

__device__ __forceinline__ uint32_t chunk_amax_bits(u32x4 v) {
  uint32_t m = pk_max_u16(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu);
  m = pk_max_u16(m, v.z & 0x7FFF7FFFu);
  return pk_max_u16(m, v.w & 0x7FFF7FFFu);
}

// Writes the workgroup's maximum of m to partials[blockIdx.x].
__device__ __forceinline__ void store_partial(uint32_t m, uint32_t* __restrict__ partials) {
  m = wave_max_u32(m);
  __shared__ uint32_t red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) r = max(r, red[i]);
    partials[blockIdx.x] = r;
  }
}

// Dense tensors (rows back to back) are walked flat in 4 KiB segments of 256
// 16-byte chunks, one segment per wave and iteration: lane l takes chunks
// l, l + 64, l + 128 and l + 192, so each load instruction covers 1 KiB and
// the wave's four loads one contiguous 4 KiB range (DRAM-page friendly).
constexpr int kSegChunks = 256;

// Max over n 16-byte chunks (n even).
__global__ __launch_bounds__(kThreads) void amax_flat_kernel(
    const u32x4* __restrict__ x, uint64_t n, uint32_t* __restrict__ partials) {
  const int lane = threadIdx.x & 63;
  const uint64_t nwaves = (uint64_t)gridDim.x * (kThreads / 64);
  uint32_t m = 0;
  uint64_t seg = (uint64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  for (; seg * kSegChunks < n; seg += nwaves) {
    const uint64_t c0 = seg * kSegChunks + lane;
    if (c0 + 192 < n) {
      // non-temporal: a streamed read, so the tensor does not churn L2 and MALL
      const u32x4 v0 = __builtin_nontemporal_load(&x[c0]), v1 = __builtin_nontemporal_load(&x[c0 + 64]),
                  v2 = __builtin_nontemporal_load(&x[c0 + 128]),
                  v3 = __builtin_nontemporal_load(&x[c0 + 192]);
      m = pk_max_u16(m, pk_max_u16(pk_max_u16(chunk_amax_bits(v0), chunk_amax_bits(v1)),
                                   pk_max_u16(chunk_amax_bits(v2), chunk_amax_bits(v3))));
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (c0 + 64 * u < n)
          m = pk_max_u16(m, chunk_amax_bits(__builtin_nontemporal_load(&x[c0 + 64 * u])));
    }
  }
  store_partial(max(m & 0xFFFFu, m >> 16), partials);
}

template <bool kContig>
__global__ __launch_bounds__(kThreads) void amax_kernel(
    const uint16_t* __restrict__ x, uint32_t rows, uint32_t kb, FastDiv div,
    int64_t stride_row, int64_t stride_k, uint32_t* __restrict__ partials) {
  const uint32_t nb = rows * kb;
  uint32_t m = 0;
  for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < nb;
       b += gridDim.x * kThreads) {
    int64_t row;
    uint32_t cb;
    block_coords<kContig>(b, rows, kb, div, row, cb);
    uint32_t w[8];
    load_block<kContig>(x, row, cb, stride_row, stride_k, w);
    m = max(m, block_amax_bits(w));
  }
  store_partial(m, partials);
}

// E4M3FN byte of the round-to-nearest-even value of v >= 0, saturating.
__device__ uint32_t e4m3_rne_byte(double v) {
  if (v >= 448.0) return 0x7E;
  if (v < 0.015625) {                       // below 2^-6: spacing 2^-9
    return (uint32_t)rint(v * 512.0);       // 8 means 2^-6 (byte 0x08)
  }
  int e = ilogb(v);                         // v in [2^e, 2^(e+1)), e >= -6
  double q = ldexp(v, 3 - e);               // [8, 16)
  uint32_t n = (uint32_t)rint(q);           // 8..16; 16 carries into e+1
  uint32_t byte = (uint32_t)(e + 7) * 8 + (n - 8);
  return byte > 0x7E ? 0x7E : byte;
}

// E2M1 magnitude code (0..7) of the round-to-nearest-even value of s >= 0.
__device__ uint32_t e2m1_rne_code(double s) {
  if (s >= 6.0) return 7;
  if (s < 2.0) return (uint32_t)rint(2.0 * s);        // 0, .5, 1, 1.5, 2
  if (s < 4.0) return (uint32_t)rint(s) + 2;          // 2, 3, 4
  return (uint32_t)rint(0.5 * s) + 4;                 // 4, 6
}

constexpr int kPrepareGrid = (kSigLutN + kCodeLutN + kThreads - 1) / kThreads;

// Thread j of the grid writes table entry j (sig_lut, then code_lut).
// Workgroup 0 also writes alpha_out and the parameters.  Every workgroup
// reads *alpha_in; alpha_out may be the same float, since the value written
// is the value read.
__global__ __launch_bounds__(kThreads) void prepare_kernel(
    const uint32_t* __restrict__ partials, int n_partials,
    const float* __restrict__ alpha_in, float* __restrict__ alpha_out,
    uint8_t* __restrict__ ws) {
  __shared__ uint32_t red[kThreads / 64];
  float alpha;
  if (alpha_in != nullptr) {
    alpha = *alpha_in;
  } else {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < n_partials; i += kThreads) m = max(m, partials[i]);
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) m = max(m, red[i]);
    // correctly rounded float32 division (IEEE): alpha = RNE(amax / 2688)
    alpha = bf16_bits_to_f32(m) / 2688.0f;
  }

  QuantParams* P = reinterpret_cast<QuantParams*>(ws + kWsParams);
  uint8_t* sig_lut = ws + kWsSigLut;
  uint8_t* code_lut = ws + kWsCodeLut;

  int s = 0;
  bool zero = !(alpha > 0.0f) || isinf(alpha);
  if (!zero) {
    int e;
    (void)frexpf(alpha, &e);                // alpha = f 2^e, f in [0.5, 1)
    s = 1 - e;                              // alpha * 2^s in [1, 2)
  }
  const bool slow = !zero && (s > 100 || s < -100);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *alpha_out = alpha;
    QuantParams p;
    p.alpha = alpha;
    p.shift = s;
    p.slow = slow ? 1 : 0;
    if (zero) {
      p.sig_off = -(1 << 28);               // every block scale is 0
      p.code_off = 0;
    } else if (slow) {
      p.sig_off = -kSigLutBase;             // bits are taken after rescaling
      p.code_off = -kCodeLutBase;
    } else {
      p.sig_off = 128 * s - kSigLutBase;
      p.code_off = 128 * s - kCodeLutBase;
    }
    p.pad[0] = p.pad[1] = p.pad[2] = 0;
    *P = p;
  }
  const double a = zero ? 1.0 : ldexp((double)alpha, s);   // exact
  const int j = blockIdx.x * kThreads + threadIdx.x;
  if (j < kSigLutN) {
    double v = (double)bf16_bits_to_f32(kSigLutBase + j) / (6.0 * a);
    sig_lut[j] = (uint8_t)e4m3_rne_byte(v);
  } else if (j < kSigLutN + kCodeLutN) {
    const int c = j - kSigLutN;
    int k = c / kCodeLutRow, i = c - k * kCodeLutRow;
    double d = a * (1.0 + 0.125 * k);                     // exact
    double q = (double)bf16_bits_to_f32(kCodeLutBase + i) / d;
    code_lut[c] = (uint8_t)e2m1_rne_code(q);
  }
}

// Dense tensor, flat segments as in amax_flat_kernel.  A 16-byte chunk is
// half a block: lanes 2c and 2c + 1 hold the two halves of one block and
// exchange their maxima (DPP quad permutation [1,0,3,2]).  Each lane writes
// the 4 code bytes of its chunk (chunk c -> codes word c), the even lane the
// scale byte (block c / 2).  n is even, so a block's two chunks are both in
// range or both out.  The tables' loads go before the first segment's (see
// copy_tables_first).
__global__ __launch_bounds__(kThreads) void quantize_flat_kernel(
    const u32x4* __restrict__ x, uint64_t n, const uint8_t* __restrict__ ws,
    uint32_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  __shared__ TableLds tl;
  const int tid = threadIdx.x, lane = tid & 63;
  const uint64_t nwaves = (uint64_t)gridDim.x * (kThreads / 64);
  auto load_seg = [&](uint64_t seg, u32x4 (&v)[4]) __attribute__((always_inline)) {
    const uint64_t c0 = seg * kSegChunks + lane;
#pragma unroll
    for (int u = 0; u < 4; ++u)      // non-temporal, as in the amax pass
      v[u] = c0 + 64 * u < n ? __builtin_nontemporal_load(&x[c0 + 64 * u]) : u32x4{0u, 0u, 0u, 0u};
  };
  uint64_t seg = (uint64_t)blockIdx.x * (kThreads / 64) + (tid >> 6);
  u32x4 v[4];
  copy_tables_first(ws, tl, tid, [&] { load_seg(seg, v); });
  const QuantParams P = *reinterpret_cast<const QuantParams*>(ws + kWsParams);
  __syncthreads();

  if (P.slow) {
    // alpha's exponent beyond +-100: the generic block path rescales first
    const BlockTables t = tables_from(ws, tl.sig, tl.code);
    for (; seg * kSegChunks < n; seg += nwaves) {
      const uint64_t c0 = seg * kSegChunks + lane;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        uint32_t mag[8];
        magnitudes<4>(w, t, mag);
        uint32_t amax = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = max(amax, mag[i]);
        amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0xB1, 0xF, 0xF, false));
        CodeRow row;
        const uint32_t sb = block_scale(amax, t, row);
        const uint32_t o = codes8(mag, w, row, t);
        const uint64_t c = c0 + 64 * u;
        if (c < n) {
          codes[c] = o;
          if ((lane & 1) == 0) scales[c >> 1] = (uint8_t)sb;
        }
      }
      load_seg(seg + nwaves, v);
    }
    return;
  }

  const FastTables t = fast_tables(tl, P);
  while (seg * kSegChunks < n) {
    const uint64_t c0 = seg * kSegChunks + lane;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      uint32_t sb;
      const uint32_t o = quantize_half_block(w, t, sb);
      const uint64_t c = c0 + 64 * u;
      if (c < n) {
        codes[c] = o;
        if ((lane & 1) == 0) scales[c >> 1] = (uint8_t)sb;
      }
    }
    seg += nwaves;
    load_seg(seg, v);
  }
}

template <bool kContig>
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const uint16_t* __restrict__ x, uint32_t rows, uint32_t kb, FastDiv div,
    int64_t stride_row, int64_t stride_k, const uint8_t* __restrict__ ws,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  __shared__ __align__(16) uint8_t lds_sig[kSigLutN];
  __shared__ __align__(16) uint8_t lds_code[kCodeLutN];
  load_tables_to_lds(ws, lds_sig, lds_code, threadIdx.x, kThreads);
  const BlockTables t = tables_from(ws, lds_sig, lds_code);
  __syncthreads();

  const uint32_t nb = rows * kb;
  const uint32_t stride = gridDim.x * kThreads;
  // codes are [rows][K/2]: block (row, cb) starts at byte 8 * (row kb + cb)
  auto one = [&](uint32_t b, const uint32_t (&w)[8], int64_t row, uint32_t cb)
      __attribute__((always_inline)) {
    uint32_t out0, out1, sb;
    quantize16(w, t, out0, out1, sb);
    const uint32_t ob = (uint32_t)row * kb + cb;
    *reinterpret_cast<u32x2*>(codes + (size_t)ob * 8) = u32x2{out0, out1};
    scales[ob] = (uint8_t)sb;
  };
  uint32_t b = blockIdx.x * kThreads + threadIdx.x;
  // two blocks per lane and iteration: four 16-byte loads in flight
  for (; b + stride < nb; b += 2 * stride) {
    int64_t r0, r1;
    uint32_t c0, c1;
    block_coords<kContig>(b, rows, kb, div, r0, c0);
    block_coords<kContig>(b + stride, rows, kb, div, r1, c1);
    uint32_t w0[8], w1[8];
    load_block<kContig>(x, r0, c0, stride_row, stride_k, w0);
    load_block<kContig>(x, r1, c1, stride_row, stride_k, w1);
    one(b, w0, r0, c0);
    one(b + stride, w1, r1, c1);
  }
  if (b < nb) {
    int64_t r0;
    uint32_t c0;
    block_coords<kContig>(b, rows, kb, div, r0, c0);
    uint32_t w0[8];
    load_block<kContig>(x, r0, c0, stride_row, stride_k, w0);
    one(b, w0, r0, c0);
  }
}

int grid_for(uint32_t nb, int per_cu_wgs) {
  int64_t need = ((int64_t)nb + kThreads - 1) / kThreads;
  int64_t cap = 256 * per_cu_wgs;
  return (int)(need < cap ? (need > 0 ? need : 1) : cap);
}

}  // namespace

FastDivHost make_fast_div(uint32_t d) {
  FastDivHost f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.shift = s;
  f.mul = (uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1);
  return f;
}

static FastDiv to_dev(const FastDivHost& h) {
  FastDiv f;
  f.d = h.d;
  f.mul = h.mul;
  f.shift = h.shift;
  return f;
}

hipError_t launch_amax(const uint16_t* x, int64_t rows, int64_t k,
                       int64_t stride_row, int64_t stride_k, uint8_t* ws,
                       int* n_partials, hipStream_t stream) {
  const uint32_t kb = (uint32_t)(k / 16);
  const uint32_t nb = (uint32_t)rows * kb;
  const bool contig = (stride_k == 1);
  int grid = grid_for(nb, 4);
  if (grid > kAmaxPartials) grid = kAmaxPartials;
  *n_partials = grid;
  uint32_t* partials = reinterpret_cast<uint32_t*>(ws + kWsPartials);
  if (contig && stride_row == k) {
    const uint64_t n = (uint64_t)rows * (uint64_t)k / 8;      // 16-byte chunks
    const int64_t segs = (int64_t)((n + kSegChunks - 1) / kSegChunks);
    const int64_t need = (segs + 3) / 4;
    grid = (int)(need < kAmaxPartials ? (need > 0 ? need : 1) : kAmaxPartials);
    *n_partials = grid;
    hipLaunchKernelGGL(amax_flat_kernel, dim3(grid), dim3(kThreads), 0, stream,
                       reinterpret_cast<const u32x4*>(x), n, partials);
    return hipGetLastError();
  }
  FastDiv div = to_dev(make_fast_div(contig ? kb : (uint32_t)rows));
  if (contig)
    hipLaunchKernelGGL(amax_kernel<true>, dim3(grid), dim3(kThreads), 0, stream,
                       x, (uint32_t)rows, kb, div, stride_row, stride_k, partials);
  else
    hipLaunchKernelGGL(amax_kernel<false>, dim3(grid), dim3(kThreads), 0, stream,
                       x, (uint32_t)rows, kb, div, stride_row, stride_k, partials);
  return hipGetLastError();
}

hipError_t launch_prepare(const uint8_t* ws_partials, int n_partials,
                          const float* alpha_in, float* alpha_out, uint8_t* ws,
                          hipStream_t stream) {
  hipLaunchKernelGGL(prepare_kernel, dim3(kPrepareGrid), dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint32_t*>(ws_partials), n_partials,
                     alpha_in, alpha_out, ws);
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t k,
                           int64_t stride_row, int64_t stride_k,
                           const uint8_t* ws, uint8_t* codes, uint8_t* scales,
                           hipStream_t stream) {
  const uint32_t kb = (uint32_t)(k / 16);
  const uint32_t nb = (uint32_t)rows * kb;
  if (nb == 0) return hipSuccess;
  const bool contig = (stride_k == 1);
  if (contig && stride_row == k) {
    const uint64_t n = (uint64_t)rows * (uint64_t)k / 8;      // 16-byte chunks
    const int64_t segs = (int64_t)((n + kSegChunks - 1) / kSegChunks);
    const int64_t need = (segs + 3) / 4;                      // one segment per wave
    const int grid = (int)(need < 2048 ? need : 2048);
    hipLaunchKernelGGL(quantize_flat_kernel, dim3(grid), dim3(kThreads), 0, stream,
                       reinterpret_cast<const u32x4*>(x), n, ws,
                       reinterpret_cast<uint32_t*>(codes), scales);
    return hipGetLastError();
  }
  const int grid = grid_for(nb, 8);
  FastDiv div = to_dev(make_fast_div(contig ? kb : (uint32_t)rows));
  if (contig) {
    hipLaunchKernelGGL((quantize_kernel<true>), dim3(grid), dim3(kThreads), 0,
                       stream, x, (uint32_t)rows, kb, div, stride_row, stride_k,
                       ws, codes, scales);
  } else {
    hipLaunchKernelGGL((quantize_kernel<false>), dim3(grid), dim3(kThreads), 0,
                       stream, x, (uint32_t)rows, kb, div, stride_row, stride_k,
                       ws, codes, scales);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
