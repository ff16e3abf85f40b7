// NVFP4 W4A4 GEMM for gfx950 (dense and grouped).
//
// Y[m][n] = alpha_a alpha_b sum_b sigma^a_{m,b} sigma^b_{n,b}
//           sum_{k in b} q^a_{m,k} q^b_{n,k}
// the W4A4 linear layer of "Mix-Quant：面向智能体LLM的量化预填充与精确解码"
// (paper.rainbus.top digest, 核心方法 and 方法步骤详情 step (4)), with the
// dequantisation xhat = alpha sigma q of its step (3).
//
// How the per-16 E4M3 scales are honoured on CDNA4.  gfx950's block-scaled
// f8f6f4 MFMAs take one power-of-two (E8M0) scale per 32 elements, which
// cannot carry a non-power-of-two scale per 16 elements.  Every product
// q * sigma, however, has at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in float16.  Each wave therefore decodes its
// FP4 fragments to float16 with the block scale folded in
// (v_cvt_scalef32_pk_f16_fp4 for the codes, then one packed f16 multiply by
// sigma * 2^-4, which keeps every nonzero value a normal float16) and feeds
// v_mfma_f32_32x32x16_f16.  Products are exact and accumulate in float32; the
// epilogue multiplies by alpha_a alpha_b 2^8.  (An FP8 operand with sigma
// folded in would round 5- and 6-bit products.)
//
// Tiling: a 256-thread workgroup computes a BM x BN tile as 2 x 2 waves of
// (BM/2) x (BN/2).  Each K-stage covers 128 elements (8 NVFP4 blocks): the
// FP4 codes (BM and BN rows of 64 bytes) and the E4M3 scales (8 bytes a row)
// go global -> registers -> LDS, double-buffered with one barrier a stage.
// A lane of a 32x32x16 MFMA fragment holds 8 consecutive K-elements of one
// row; lanes 0-31 take K-elements [0, 64) of the stage and lanes 32-63 take
// [64, 128), eight per MFMA step, so a lane reads 32 contiguous code bytes
// and 4 scale bytes per fragment and stage.  A and B use the same K order,
// which is all the contraction needs.
#include "device_common.h"
#include "kernels.h"
#include "quant_block.h"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 128;                 // K-elements per stage
constexpr int kCodePitch = 80;           // LDS bytes per row (64 + 16 pad)
constexpr int kScalePitch = 12;          // LDS bytes per row (8 + 4 pad)

// sigma (E4M3FN byte) -> float16 sigma * 2^-4, replicated in both halves.
__device__ __forceinline__ half2_t scale_pair(uint32_t sb) {
  uint32_t bits = (sb << 7) | (sb << 23);        // = sigma * 2^-8 (exact)
  half2_t h = __builtin_bit_cast(half2_t, bits);
  const half2_t sixteen = {(_Float16)16.0f, (_Float16)16.0f};
  return h * sixteen;                            // exact power-of-two scaling
}

// 8 FP4 codes (one 32-bit word) -> 8 float16 values q * sigma * 2^-4.
__device__ __forceinline__ half8_t decode8(uint32_t w, half2_t s) {
  half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  half8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

struct TileCoord {
  int64_t m0, m_end;      // rows [m0, min(m0 + BM, m_end)) of this tile
  int64_t n0;
  int group;
};

// Maps the workgroup to (group, row tile, column tile).  Dense GEMMs have one
// group.  Grouped GEMMs launch an upper bound of row tiles (ceil(M/BM) +
// groups) and walk the device-side offsets; surplus workgroups return.
template <int BM>
__device__ __forceinline__ bool tile_coord(int tile_m, const int64_t* offsets,
                                           int num_groups, int64_t M,
                                           TileCoord& tc) {
  if (offsets == nullptr) {
    tc.group = 0;
    tc.m0 = (int64_t)tile_m * BM;
    tc.m_end = M;
    return tc.m0 < M;
  }
  int64_t before = 0;
  for (int g = 0; g < num_groups; ++g) {
    int64_t lo = offsets[g], hi = offsets[g + 1];
    int64_t nt = (hi - lo + BM - 1) / BM;
    if (tile_m < before + nt) {
      tc.group = g;
      tc.m0 = lo + (tile_m - before) * BM;
      tc.m_end = hi;
      return true;
    }
    before += nt;
  }
  return false;
}

// kFused: operand A arrives as BF16 and each workgroup quantises its tile
// into LDS with the exact tables (quant_block.h) instead of loading codes.
template <int BM, int BN, bool kKAligned, bool kFused>
__global__ __launch_bounds__(kThreads, 1) void w4a4_gemm_kernel(W4A4Args p) {
  constexpr int WM = BM / 2, WN = BN / 2;      // wave tile
  constexpr int TM = WM / 32, TN = WN / 32;    // 32x32 fragments per wave
  constexpr int kStageBytes = (BM + BN) * kCodePitch + (BM + BN) * kScalePitch;
  constexpr int kTableBytes = kFused ? kSigLutN + kCodeLutN : 16;
  __shared__ __align__(16) uint8_t lds[2 * kStageBytes];
  __shared__ __align__(16) uint8_t lds_tables[kTableBytes];

  TileCoord tc;
  if (!tile_coord<BM>(blockIdx.x, p.group_offsets, p.num_groups, p.M, tc)) return;
  tc.n0 = (int64_t)blockIdx.y * BN;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;
  const int64_t K = p.K;
  const int64_t kc = K / 2, ks = K / 16;       // row pitch of codes / scales

  const uint8_t* b_codes = p.b_codes + (int64_t)tc.group * p.N * kc;
  const uint8_t* b_scales = p.b_scales + (int64_t)tc.group * p.N * ks;

  // ---- global -> register loader ------------------------------------------
  // codes: row r = i * 64 + tid / 4 (i = 0..BM/64-1), 16-byte chunk tid % 4
  constexpr int kARowIters = BM / 64, kBRowIters = BN / 64;
  const int ld_chunk = tid & 3;
  const uint8_t* a_row_ptr[kARowIters];
  const uint8_t* b_row_ptr[kBRowIters];
#pragma unroll
  for (int i = 0; i < kARowIters; ++i) {
    int64_t r = tc.m0 + i * 64 + (tid >> 2);
    r = r < tc.m_end ? r : tc.m_end - 1;
    if (!kFused && p.a_row_index) r = p.a_row_index[r];
    a_row_ptr[i] = kFused ? nullptr : p.a_codes + r * kc + ld_chunk * 16;
  }
#pragma unroll
  for (int i = 0; i < kBRowIters; ++i) {
    int64_t r = tc.n0 + i * 64 + (tid >> 2);
    r = r < p.N ? r : p.N - 1;
    b_row_ptr[i] = b_codes + r * kc + ld_chunk * 16;
  }
  // scales: row tid of A (and of B), 8 bytes a stage
  const uint8_t* a_scale_ptr = nullptr;
  const uint8_t* b_scale_ptr = nullptr;
  if (!kFused && tid < BM) {
    int64_t r = tc.m0 + tid;
    r = r < tc.m_end ? r : tc.m_end - 1;
    if (p.a_row_index) r = p.a_row_index[r];
    a_scale_ptr = p.a_scales + r * ks;
  }
  // fused A: thread -> (row, run of blocks) of the stage's BM x 8 blocks
  constexpr int kQBlocks = BM / 32;                // blocks per thread
  const int q_row = tid % BM, q_blk0 = (tid / BM) * kQBlocks;
  const uint16_t* q_src = nullptr;
  BlockTables tables;
  if (kFused) {
    int64_t r = tc.m0 + q_row;
    r = r < tc.m_end ? r : tc.m_end - 1;
    q_src = p.a_bf16 + r * p.ld_a;
    load_tables_to_lds(p.ws, lds_tables, lds_tables + kSigLutN, tid, kThreads);
    tables = tables_from(p.ws, lds_tables, lds_tables + kSigLutN);
    __syncthreads();
  }
  if (tid < BN) {
    int64_t r = tc.n0 + tid;
    r = r < p.N ? r : p.N - 1;
    b_scale_ptr = b_scales + r * ks;
  }

  u32x4 ra[kARowIters], rb[kBRowIters];
  u32x2 rsa = {0u, 0u}, rsb = {0u, 0u};

  auto load_stage = [&](int kt) __attribute__((always_inline)) {
    const int64_t kbyte = (int64_t)kt * (kBK / 2);         // code byte offset
    if (kKAligned) {
#pragma unroll
      for (int i = 0; i < kARowIters; ++i)
        if (!kFused) ra[i] = *reinterpret_cast<const u32x4*>(a_row_ptr[i] + kbyte);
#pragma unroll
      for (int i = 0; i < kBRowIters; ++i)
        rb[i] = *reinterpret_cast<const u32x4*>(b_row_ptr[i] + kbyte);
      if (!kFused && tid < BM) rsa = *reinterpret_cast<const u32x2*>(a_scale_ptr + kt * 8);
      if (tid < BN) rsb = *reinterpret_cast<const u32x2*>(b_scale_ptr + kt * 8);
    } else {
      // K % 128 != 0: 8-byte pieces (16 elements = one block) with a bound
      const int64_t k0 = (int64_t)kt * kBK + ld_chunk * 32;
      const bool v0 = k0 < K, v1 = k0 + 16 < K;
#pragma unroll
      for (int i = 0; i < kARowIters; ++i) {
        if (kFused) break;
        const u32x2* q = reinterpret_cast<const u32x2*>(a_row_ptr[i] + kbyte);
        u32x2 x0 = v0 ? q[0] : u32x2{0u, 0u};
        u32x2 x1 = v1 ? q[1] : u32x2{0u, 0u};
        ra[i] = u32x4{x0.x, x0.y, x1.x, x1.y};
      }
#pragma unroll
      for (int i = 0; i < kBRowIters; ++i) {
        const u32x2* q = reinterpret_cast<const u32x2*>(b_row_ptr[i] + kbyte);
        u32x2 x0 = v0 ? q[0] : u32x2{0u, 0u};
        u32x2 x1 = v1 ? q[1] : u32x2{0u, 0u};
        rb[i] = u32x4{x0.x, x0.y, x1.x, x1.y};
      }
      uint32_t sa[2] = {0, 0}, sb[2] = {0, 0};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t blk = (int64_t)kt * 8 + j;
        if (blk < ks) {
          if (!kFused && tid < BM) sa[j >> 2] |= (uint32_t)a_scale_ptr[blk] << (8 * (j & 3));
          if (tid < BN) sb[j >> 2] |= (uint32_t)b_scale_ptr[blk] << (8 * (j & 3));
        }
      }
      rsa = u32x2{sa[0], sa[1]};
      rsb = u32x2{sb[0], sb[1]};
    }
  };

  auto store_stage = [&](int buf, int kt) __attribute__((always_inline)) {
    uint8_t* base = lds + buf * kStageBytes;
    uint8_t* a_lds = base;
    uint8_t* b_lds = base + BM * kCodePitch;
    uint8_t* as_lds = base + (BM + BN) * kCodePitch;
    uint8_t* bs_lds = as_lds + BM * kScalePitch;
    if (kFused) {
#pragma unroll
      for (int j = 0; j < kQBlocks; ++j) {
        const int blk = q_blk0 + j;
        const int64_t k0 = (int64_t)kt * kBK + blk * 16;
        uint32_t o0 = 0, o1 = 0, sbyte = 0;
        if (k0 < K) {
          const u32x4* q = reinterpret_cast<const u32x4*>(q_src + k0);
          const u32x4 v0 = q[0], v1 = q[1];
          const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
          quantize16(w, tables, o0, o1, sbyte);
        }
        *reinterpret_cast<u32x2*>(a_lds + q_row * kCodePitch + blk * 8) = u32x2{o0, o1};
        as_lds[q_row * kScalePitch + blk] = (uint8_t)sbyte;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kARowIters; ++i)
        *reinterpret_cast<u32x4*>(a_lds + (i * 64 + (tid >> 2)) * kCodePitch + ld_chunk * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < kBRowIters; ++i)
      *reinterpret_cast<u32x4*>(b_lds + (i * 64 + (tid >> 2)) * kCodePitch + ld_chunk * 16) = rb[i];
    if (!kFused && tid < BM) {
      uint32_t* q = reinterpret_cast<uint32_t*>(as_lds + tid * kScalePitch);
      q[0] = rsa.x;
      q[1] = rsa.y;
    }
    if (tid < BN) {
      uint32_t* q = reinterpret_cast<uint32_t*>(bs_lds + tid * kScalePitch);
      q[0] = rsb.x;
      q[1] = rsb.y;
    }
  };

  float16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (int)((K + kBK - 1) / kBK);
  const int fr = lane & 31, fh = lane >> 5;

  load_stage(0);
  store_stage(0, 0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_stage(kt + 1);

    const uint8_t* base = lds + buf * kStageBytes;
    const uint8_t* a_lds = base;
    const uint8_t* b_lds = base + BM * kCodePitch;
    const uint8_t* as_lds = base + (BM + BN) * kCodePitch;
    const uint8_t* bs_lds = as_lds + BM * kScalePitch;

    u32x4 ac[TM][2], bc[TN][2];
    uint32_t asc[TM], bsc[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wm + i * 32 + fr;
      const u32x4* q = reinterpret_cast<const u32x4*>(a_lds + row * kCodePitch + fh * 32);
      ac[i][0] = q[0];
      ac[i][1] = q[1];
      asc[i] = *reinterpret_cast<const uint32_t*>(as_lds + row * kScalePitch + fh * 4);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int row = wn + j * 32 + fr;
      const u32x4* q = reinterpret_cast<const u32x4*>(b_lds + row * kCodePitch + fh * 32);
      bc[j][0] = q[0];
      bc[j][1] = q[1];
      bsc[j] = *reinterpret_cast<const uint32_t*>(bs_lds + row * kScalePitch + fh * 4);
    }

#pragma unroll
    for (int s = 0; s < 8; ++s) {
      half8_t af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const u32x4 c = ac[i][s >> 2];
        const uint32_t w = (s & 3) == 0 ? c.x : (s & 3) == 1 ? c.y : (s & 3) == 2 ? c.z : c.w;
        af[i] = decode8(w, scale_pair((asc[i] >> (8 * (s >> 1))) & 0xFF));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const u32x4 c = bc[j][s >> 2];
        const uint32_t w = (s & 3) == 0 ? c.x : (s & 3) == 1 ? c.y : (s & 3) == 2 ? c.z : c.w;
        bf[j] = decode8(w, scale_pair((bsc[j] >> (8 * (s >> 1))) & 0xFF));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }

    if (kt + 1 < nk) store_stage(buf ^ 1, kt + 1);
    __syncthreads();
  }

  // ---- epilogue ------------------------------------------------------------
  const float scale = (*p.alpha_a) * p.alpha_b[tc.group] * 256.0f;
  const int64_t row_lim = tc.m0 + BM < tc.m_end ? tc.m0 + BM : tc.m_end;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = tc.n0 + wn + j * 32 + fr;
      if (col >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = tc.m0 + wm + i * 32 + 8 * (r >> 2) + 4 * fh + (r & 3);
        if (row < row_lim) {
          const float v = acc[i][j][r] * scale;
          if (p.y_f32) p.y_f32[row * p.ld_y + col] = v;
          if (p.y_bf16) p.y_bf16[row * p.ld_y + col] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
    }
  }
}

template <int BM, int BN, bool kFused>
hipError_t launch_tiles(const W4A4Args& a, hipStream_t stream) {
  int tiles_m;
  if (a.group_offsets == nullptr) {
    tiles_m = (int)((a.M + BM - 1) / BM);
  } else {
    tiles_m = (int)((a.M + BM - 1) / BM) + a.num_groups;
  }
  const int tiles_n = (int)((a.N + BN - 1) / BN);
  dim3 grid(tiles_m, tiles_n);
  if (a.K % kBK == 0)
    hipLaunchKernelGGL((w4a4_gemm_kernel<BM, BN, true, kFused>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((w4a4_gemm_kernel<BM, BN, false, kFused>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w4a4(const W4A4Args& a, hipStream_t stream) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  // 256 x 256 tiles when they fill the 256 CUs, else 128 x 128.
  const int64_t big = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  if (big >= 256) return launch_tiles<256, 256, false>(a, stream);
  return launch_tiles<128, 128, false>(a, stream);
}

hipError_t launch_w4a4_fused(const W4A4Args& a, hipStream_t stream) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  const int64_t big = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  if (big >= 256) return launch_tiles<256, 256, true>(a, stream);
  return launch_tiles<128, 128, true>(a, stream);
}

}  // namespace nvfp4
