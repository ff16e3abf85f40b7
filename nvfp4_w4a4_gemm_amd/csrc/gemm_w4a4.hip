// NVFP4 W4A4 GEMM for gfx950 (dense, grouped, and with the activation
// quantiser fused into the operand load).
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
// (v_cvt_scalef32_pk_f16_fp4 gives the codes times 16, one packed f16
// multiply applies sigma * 2^-8; every nonzero product is a normal float16)
// and feeds v_mfma_f32_32x32x16_f16.  Products are exact and accumulate in
// float32; the epilogue multiplies by alpha_a alpha_b 2^8.  (An FP8 operand
// with sigma folded in would round 5- and 6-bit products.)
//
// Tiling: a 256-thread workgroup computes a BM x BN tile as 2 x 2 waves of
// (BM/2) x (BN/2).  Each K-stage covers 128 elements (8 NVFP4 blocks).  The
// FP4 codes (64 bytes a row) and E4M3 scales (8 bytes a row) of a stage go
// straight from global memory to LDS with buffer_load ... lds (no staging
// registers); a ring of kRing stages keeps loads kRing - 1 stages ahead with
// one barrier a stage.  A lane of a 32x32x16 MFMA fragment holds 8
// consecutive K-elements of one row; lanes 0-31 take K-elements [0, 64) of
// the stage and lanes 32-63 take [64, 128), eight per MFMA step, so a lane
// reads 32 code bytes (two 16-byte chunks) and 4 scale bytes per fragment and
// stage.  A and B use the same K order, which is all the contraction needs.
// LDS rows are not padded; the 16-byte chunk c of row r sits at position
// c ^ ((r >> 2) & 3), so that the 16 rows a ds_read_b128 serves at a time
// (16 lanes) cover all 64 banks once.
#include "device_common.h"
#include "kernels.h"
#include "quant_block.h"

#include <atomic>
#include <type_traits>

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 128;                 // K-elements per stage
constexpr int kCodeRow = 64;             // LDS bytes of codes per row and stage
constexpr int kScaleRow = 8;             // LDS bytes of scales per row and stage

// global -> LDS DMA of 16 bytes (codes) or 4 bytes (scales) per lane: lane l
// writes lds + l * bytes; lds must be the same for the whole wave.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voff,
                                      int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voff,
                                     int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (__attribute__((address_space(3))) void*)lds, 4, voff, soff, 0, 0);
}

__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

// s_waitcnt immediate (gfx9 encoding): vector-memory count n, no expcnt
// wait, LDS/scalar count 0.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// Byte offset of 16-byte chunk c of row r inside a code tile.
__device__ __forceinline__ int chunk_off(int row, int c) {
  return row * kCodeRow + ((c ^ swz(row)) << 4);
}

// sigma (E4M3FN byte) -> float16 sigma * 2^-8 in both halves: the byte's
// exponent and mantissa fields land in the f16 fields (a subnormal E4M3 byte
// becomes a subnormal f16), i.e. bits (sb << 7) | (sb << 23).
__device__ __forceinline__ uint32_t scale_pair_bits(uint32_t sb) {
  return sb * 0x00800080u;
}

// 8 FP4 codes (one 32-bit word) -> 8 float16 values q * sigma * 2^-4: the
// conversion applies the power of two 16 (its scale operand's exponent), the
// packed multiply the scale; both products are exact.
__device__ __forceinline__ half8_t decode8(uint32_t w, uint32_t s_bits) {
  const half2_t s = __builtin_bit_cast(half2_t, s_bits);
  half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 16.0f, 0);
  half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 16.0f, 1);
  half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 16.0f, 2);
  half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 16.0f, 3);
  p0 = p0 * s;
  p1 = p1 * s;
  p2 = p2 * s;
  p3 = p3 * s;
  half8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer (stride 0); dword 3 selects the plain 32-bit data format
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// A float at a wave-uniform address, by a scalar load (the constant address
// space: the value is not written while the kernel runs).
__device__ __forceinline__ float load_uniform(const float* ptr) {
  return *reinterpret_cast<const __attribute__((address_space(4))) float*>(
      reinterpret_cast<uintptr_t>(ptr));
}

struct TileCoord {
  int64_t m0, m_end;      // rows [m0, min(m0 + BM, m_end)) of this tile
  int64_t n0;
  int group;
};

// Maps the workgroup to (group, row tile).  Dense GEMMs have one group.
// Grouped GEMMs launch an upper bound of row tiles (ceil(M/BM) + groups) and
// walk the device-side offsets; surplus workgroups return.
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

// kKAligned: K % 128 == 0 (stages are whole; codes and scales go by DMA).
// kFused: operand A arrives as BF16 and each workgroup quantises its tile
// into LDS with the exact tables (quant_block.h) instead of loading codes.
// kRing: LDS stages in the ring (3 or 4; loads run kRing - 1 stages ahead and
// the next stage's fragments are read while this one computes).  kOcc: waves
// per SIMD the register budget is sized for.  kSilu: B is a gate|up weight
// interleaved in 32-row blocks (gate rows, then the up rows of the same 32
// units) and the epilogue writes H = SiLU(gate) * up in BF16 ([M][N/2])
// and the tile's amax of |H| instead of the projections' outputs.
// SiLU(g) * u = g u / (1 + e^-g), with no overflow and no loss in the
// float32 subnormal range.  With e = exp(-|g|) <= 1 and E = e 2^64 (normal
// for |g| < 131, formed by the hardware exp2 as 2^(64 - |g| log2 e)):
// g >= 0: H = g u / (1 + e); g < 0: H = (g u / (1 + e)) E 2^-64, the power
// of two applied last so that the product keeps float32's relative
// precision until the final rounding even where H is a float32 subnormal.
// exp2 and the reciprocal are 1-ulp hardware approximations; with the
// rounding of |g| log2 e the relative error of H stays below about 2^-17.
__device__ __forceinline__ float silu_mul(float g, float u) {
  constexpr float kLog2e = 1.44269504f;
  const float big_e = __builtin_amdgcn_exp2f(__builtin_fmaf(fabsf(g), -kLog2e, 64.0f));
  const float q = (g * u) * __builtin_amdgcn_rcpf(1.0f + big_e * 0x1p-64f);
  return g >= 0.0f ? q : (q * big_e) * 0x1p-64f;
}

template <int BM, int BN, bool kKAligned, bool kFused, int kRing, int kOcc, bool kSilu = false,
          bool kPersist = false>
__global__ __launch_bounds__(kThreads, kOcc) void w4a4_gemm_kernel(W4A4Args p) {
  constexpr int WM = BM / 2, WN = BN / 2;      // wave tile
  constexpr int TM = WM / 32, TN = WN / 32;    // 32x32 fragments per wave
  constexpr int kCodesA = 0, kCodesB = BM * kCodeRow;
  constexpr int kScalesA = (BM + BN) * kCodeRow, kScalesB = kScalesA + BM * kScaleRow;
  constexpr int kStageBytes = (BM + BN) * (kCodeRow + kScaleRow);
  constexpr int kTableBytes = kFused ? kSigLutN + kCodeLutN : 16;
  __shared__ __align__(16) uint8_t lds[kRing * kStageBytes];
  __shared__ __align__(16) uint8_t lds_tables[kTableBytes];

  // kPersist: workgroup b walks the linear tiles b, b + gridDim.x, ... (row
  // tile fastest, as the 2-D grid orders them); the last three stages of a
  // tile load the next tile's first three, so its prologue is hidden.
  // tc is the tile being computed, tl the tile whose stages are being loaded.
  const int tiles_m = (int)((p.M + BM - 1) / BM);
  const int tiles_n = (int)((p.N + BN - 1) / BN);
  const int n_tiles = tiles_m * tiles_n;
  int tile = kPersist ? (int)blockIdx.x : (int)(blockIdx.y * gridDim.x + blockIdx.x);
  auto dense_coord = [&](int t, TileCoord& c) __attribute__((always_inline)) {
    c.group = 0;
    c.m0 = (int64_t)(t % tiles_m) * BM;
    c.m_end = p.M;
    c.n0 = (int64_t)(t / tiles_m) * BN;
  };
  TileCoord tc;
  if constexpr (kPersist) {
    dense_coord(tile, tc);
  } else if (p.group_offsets == nullptr) {
    if (!tile_coord<BM>(blockIdx.x, p.group_offsets, p.num_groups, p.M, tc)) return;
    tc.n0 = (int64_t)blockIdx.y * BN;
  } else {
    // grouped: column tile fastest, and the workgroups of one XCD take
    // consecutive tiles, so that at a time an XCD holds a few row tiles of
    // one group against that group's column tiles (a few operand panels in
    // its L2, not a weight panel of every group: measured 3-6% faster at the
    // 64-expert shapes).  The workgroups resident at a time are about a
    // window of 256 consecutive linear ids, id i on XCD i % 8; within each
    // whole window XCD x takes tiles 32x .. 32x + 31 of it.  The grid's row
    // tiles are an upper bound; surplus tiles return.
    int lin = (int)(blockIdx.y * gridDim.x + blockIdx.x);
    const int base = lin & ~255;
    if (base + 256 <= (int)(gridDim.x * gridDim.y)) lin = base + (lin & 7) * 32 + ((lin & 255) >> 3);
    if (!tile_coord<BM>(lin / tiles_n, p.group_offsets, p.num_groups, p.M, tc)) return;
    tc.n0 = (int64_t)(lin % tiles_n) * BN;
  }
  TileCoord tl = tc;

  const int tid = threadIdx.x;
  // the wave index is uniform: keep it (and the DMA LDS addresses) in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;
  const int64_t K = p.K;
  const int64_t kc = K / 2, ks = K / 16;       // row pitch of codes / scales

  const uint8_t* b_codes = p.b_codes + (int64_t)tc.group * p.N * kc;
  const uint8_t* b_scales = p.b_scales + (int64_t)tc.group * p.N * ks;

  auto a_src_row = [&](int r) __attribute__((always_inline)) {
    int64_t g = tl.m0 + r;
    g = g < tl.m_end ? g : tl.m_end - 1;       // past the tile: clamp (not stored)
    // (the tile walk runs without a row gather: no index load, whose wait
    // would drain the DMA in flight, in its loop)
    if (!kFused && !kPersist && p.a_row_index) g = p.a_row_index[g];
    return g;
  };
  auto b_src_row = [&](int r) __attribute__((always_inline)) {
    int64_t g = tl.n0 + r;
    return g < p.N ? g : p.N - 1;
  };

  // ---- loader: DMA (K % 128 == 0) ---------------------------------------
  // Code tile of R rows: WG instruction g (of R/16) moves rows [16g, 16g+16):
  // lane l -> row 16g + l/4, LDS chunk position l % 4, global chunk
  // (l % 4) ^ swz(row).  Wave w issues instructions g = w, w + 4, ...
  // Scale tile: WG instruction g (of R/32) moves rows [32g, 32g+32): lane l
  // -> row 32g + l/2, dword l % 2.
  constexpr int kACodeIns = BM / 64, kBCodeIns = BN / 64;      // per wave
  constexpr int kAScaleIns = BM / 128, kBScaleIns = BN / 128;  // per wave
  // DMA instructions a wave issues per stage
  constexpr int kDmaPerStage =
      kKAligned ? (kFused ? 0 : kACodeIns + kAScaleIns) + kBCodeIns + kBScaleIns : 0;
  static_assert(BM % 128 == 0 && BN % 128 == 0, "tile sizes");
  static_assert(kRing == 3 || kRing == 4, "ring depth");
  uint32_t a_cv[kACodeIns], b_cv[kBCodeIns], a_sv[kAScaleIns], b_sv[kBScaleIns];
  // DMA source offsets of the rows of tile tl
  auto set_offsets = [&]() __attribute__((always_inline)) {
#pragma unroll
  for (int i = 0; i < kACodeIns; ++i) {
    const int row = (i * 4 + wave) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz(row);
    a_cv[i] = kFused ? 0u : (uint32_t)(a_src_row(row) * kc + c * 16);
  }
#pragma unroll
  for (int i = 0; i < kBCodeIns; ++i) {
    const int row = (i * 4 + wave) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz(row);
    b_cv[i] = (uint32_t)(b_src_row(row) * kc + c * 16);
  }
#pragma unroll
  for (int i = 0; i < kAScaleIns; ++i) {
    const int row = (i * 4 + wave) * 32 + (lane >> 1);
    a_sv[i] = kFused ? 0u : (uint32_t)(a_src_row(row) * ks + (lane & 1) * 4);
  }
#pragma unroll
  for (int i = 0; i < kBScaleIns; ++i) {
    const int row = (i * 4 + wave) * 32 + (lane >> 1);
    b_sv[i] = (uint32_t)(b_src_row(row) * ks + (lane & 1) * 4);
  }
  };
  set_offsets();
  const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(p.a_codes, 0xFFFFFFFFu);
  const __amdgpu_buffer_rsrc_t rs_as = make_rsrc(p.a_scales, 0xFFFFFFFFu);
  const __amdgpu_buffer_rsrc_t rs_b = make_rsrc(b_codes, (uint32_t)(p.N * kc));
  const __amdgpu_buffer_rsrc_t rs_bs = make_rsrc(b_scales, (uint32_t)(p.N * ks));

  // With a 4-deep ring the DMA of a stage is spread over the first six MFMA
  // groups of an iteration (kDmaPer instructions each) instead of being
  // issued in one burst, so a wave never stalls its MFMA issue on a full
  // memory queue.  These loads are branch-free: past the last stage they
  // reload stage nk - 1 into the slot being refilled, which no wave reads
  // again (it is neither the stage being computed nor the next two).
  constexpr bool kSpread = kKAligned && !kFused && kRing == 4;
  constexpr int kDmaGroups = 6;
  constexpr int kDmaPer = (kDmaPerStage + kDmaGroups - 1) / kDmaGroups;
  constexpr int kDmaBeforeWait = 3 * kDmaPer < kDmaPerStage ? 3 * kDmaPer : kDmaPerStage;
  auto dma_one = [&](uint8_t* base, int kcode, int kscale, int idx) __attribute__((always_inline)) {
    if (idx < kACodeIns) {
      dma16(rs_a, base + kCodesA + (idx * 4 + wave) * 1024, a_cv[idx], kcode);
    } else if (idx < kACodeIns + kAScaleIns) {
      const int i = idx - kACodeIns;
      dma4(rs_as, base + kScalesA + (i * 4 + wave) * 256, a_sv[i], kscale);
    } else if (idx < kACodeIns + kAScaleIns + kBCodeIns) {
      const int i = idx - kACodeIns - kAScaleIns;
      dma16(rs_b, base + kCodesB + (i * 4 + wave) * 1024, b_cv[i], kcode);
    } else {
      const int i = idx - kACodeIns - kAScaleIns - kBCodeIns;
      dma4(rs_bs, base + kScalesB + (i * 4 + wave) * 256, b_sv[i], kscale);
    }
  };

  // ---- loader: registers (K % 128 != 0) ----------------------------------
  // 16-byte chunk tid % 4 of rows i * 64 + tid / 4, read in 8-byte pieces
  // with a bound; scales of row tid byte by byte.
  const int ld_chunk = tid & 3;

  // fused A: thread -> (row, run of blocks) of the stage's BM x 8 blocks
  constexpr int kQBlocks = BM / 32;                // blocks per thread
  const int q_row = tid % BM, q_blk0 = (tid / BM) * kQBlocks;
  const uint16_t* q_src = nullptr;
  BlockTables tables;
  if (kFused) {
    q_src = p.a_bf16 + a_src_row(q_row) * p.ld_a;
    load_tables_to_lds(p.ws, lds_tables, lds_tables + kSigLutN, tid, kThreads);
    tables = tables_from(p.ws, lds_tables, lds_tables + kSigLutN);
    __syncthreads();
  }

  // Issues the loads of stage kt into ring slot buf (DMA, or registers then
  // LDS stores for the unaligned and fused paths, which complete here).
  auto fill_stage = [&](int buf, int kt) __attribute__((always_inline)) {
    uint8_t* base = lds + buf * kStageBytes;
    if (kSpread) {
#pragma unroll
      for (int idx = 0; idx < kDmaPerStage; ++idx)
        dma_one(base, kt * (kBK / 2), kt * 8, idx);
    } else if (kKAligned) {
      const int kcode = kt * (kBK / 2), kscale = kt * 8;
      if (!kFused) {
#pragma unroll
        for (int i = 0; i < kACodeIns; ++i)
          dma16(rs_a, base + kCodesA + (i * 4 + wave) * 1024, a_cv[i], kcode);
#pragma unroll
        for (int i = 0; i < kAScaleIns; ++i)
          dma4(rs_as, base + kScalesA + (i * 4 + wave) * 256, a_sv[i], kscale);
      }
#pragma unroll
      for (int i = 0; i < kBCodeIns; ++i)
        dma16(rs_b, base + kCodesB + (i * 4 + wave) * 1024, b_cv[i], kcode);
#pragma unroll
      for (int i = 0; i < kBScaleIns; ++i)
        dma4(rs_bs, base + kScalesB + (i * 4 + wave) * 256, b_sv[i], kscale);
    } else {
      const int64_t kbyte = (int64_t)kt * (kBK / 2);
      const int64_t k0 = (int64_t)kt * kBK + ld_chunk * 32;
      const bool v0 = k0 < K, v1 = k0 + 16 < K;
      if (!kFused) {
#pragma unroll
        for (int i = 0; i < BM / 64; ++i) {
          const int row = i * 64 + (tid >> 2);
          const u32x2* q = reinterpret_cast<const u32x2*>(p.a_codes + a_src_row(row) * kc + ld_chunk * 16 + kbyte);
          const u32x2 x0 = v0 ? q[0] : u32x2{0u, 0u};
          const u32x2 x1 = v1 ? q[1] : u32x2{0u, 0u};
          *reinterpret_cast<u32x4*>(base + kCodesA + chunk_off(row, ld_chunk)) = u32x4{x0.x, x0.y, x1.x, x1.y};
        }
      }
#pragma unroll
      for (int i = 0; i < BN / 64; ++i) {
        const int row = i * 64 + (tid >> 2);
        const u32x2* q = reinterpret_cast<const u32x2*>(b_codes + b_src_row(row) * kc + ld_chunk * 16 + kbyte);
        const u32x2 x0 = v0 ? q[0] : u32x2{0u, 0u};
        const u32x2 x1 = v1 ? q[1] : u32x2{0u, 0u};
        *reinterpret_cast<u32x4*>(base + kCodesB + chunk_off(row, ld_chunk)) = u32x4{x0.x, x0.y, x1.x, x1.y};
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t blk = (int64_t)kt * 8 + j;
        if (!kFused && tid < BM)
          base[kScalesA + tid * kScaleRow + j] = blk < ks ? p.a_scales[a_src_row(tid) * ks + blk] : 0;
        if (tid < BN)
          base[kScalesB + tid * kScaleRow + j] = blk < ks ? b_scales[b_src_row(tid) * ks + blk] : 0;
      }
    }
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
        *reinterpret_cast<u32x2*>(base + kCodesA + chunk_off(q_row, blk >> 1) + 8 * (blk & 1)) =
            u32x2{o0, o1};
        base[kScalesA + q_row * kScaleRow + blk] = (uint8_t)sbyte;
      }
    }
  };

  float16_t acc[TM][TN];
  const int nk = (int)((K + kBK - 1) / kBK);
  // ring slot of stage st of the tile being computed
  int ring0 = 0;
  auto slot = [&](int st) __attribute__((always_inline)) { return (ring0 + st) % kRing; };
  bool has_next = false;      // kPersist: the last stages load the next tile
  const int fr = lane & 31, fh = lane >> 5;

  // Raw fragments of one stage in two halves (code words of steps 0-3 and
  // of steps 4-7), the scale bytes, and two sets of decoded operands: step
  // s+1 is decoded while the MFMAs of step s issue.  The second halves and
  // the scales have two sets each, for even and odd stages: the next
  // stage's are read while this stage's steps 4-7 still decode with its own.
  struct Half1 {
    u32x4 a[TM], b[TN];
  };
  struct Scales {
    uint32_t a[TM], b[TN];
  };
  u32x4 ac0[TM], bc0[TN];
  Half1 h1_even, h1_odd;
  Scales sc_even, sc_odd;
  half8_t a_cur[TM], b_cur[TN], a_nxt[TM], b_nxt[TN];

  // This lane's fragment reads inside a ring slot.  Rows wm + 32 i + fr
  // share the swizzle of row fr (wm and 32 i are multiples of 16), so
  // fragment i lies a compile-time 32 i rows past fragment 0 and one base
  // address per array and stage serves every fragment.
  static_assert(WM % 16 == 0 && WN % 16 == 0, "fragment rows share the swizzle of fr");
  const int fr_sw = swz(fr);
  const uint32_t off_a0 = kCodesA + (wm + fr) * kCodeRow + (((2 * fh) ^ fr_sw) << 4);
  const uint32_t off_a1 = kCodesA + (wm + fr) * kCodeRow + (((2 * fh + 1) ^ fr_sw) << 4);
  const uint32_t off_b0 = kCodesB + (wn + fr) * kCodeRow + (((2 * fh) ^ fr_sw) << 4);
  const uint32_t off_b1 = kCodesB + (wn + fr) * kCodeRow + (((2 * fh + 1) ^ fr_sw) << 4);
  const uint32_t off_as = kScalesA + (wm + fr) * kScaleRow + fh * 4;
  const uint32_t off_bs = kScalesB + (wn + fr) * kScaleRow + fh * 4;

  auto read_half0 = [&](int buf, Scales& sn) __attribute__((always_inline)) {
    const uint8_t* base = lds + buf * kStageBytes;
    const uint8_t* pa = base + off_a0;
    const uint8_t* pas = base + off_as;
    const uint8_t* pb = base + off_b0;
    const uint8_t* pbs = base + off_bs;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      ac0[i] = *reinterpret_cast<const u32x4*>(pa + i * 32 * kCodeRow);
      sn.a[i] = *reinterpret_cast<const uint32_t*>(pas + i * 32 * kScaleRow);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      bc0[j] = *reinterpret_cast<const u32x4*>(pb + j * 32 * kCodeRow);
      sn.b[j] = *reinterpret_cast<const uint32_t*>(pbs + j * 32 * kScaleRow);
    }
  };
  auto read_half1 = [&](int buf, Half1& h) __attribute__((always_inline)) {
    const uint8_t* base = lds + buf * kStageBytes;
    const uint8_t* pa = base + off_a1;
    const uint8_t* pb = base + off_b1;
#pragma unroll
    for (int i = 0; i < TM; ++i) h.a[i] = *reinterpret_cast<const u32x4*>(pa + i * 32 * kCodeRow);
#pragma unroll
    for (int j = 0; j < TN; ++j) h.b[j] = *reinterpret_cast<const u32x4*>(pb + j * 32 * kCodeRow);
  };
  auto word = [](const u32x4 c, int s) __attribute__((always_inline)) {
    return (s & 3) == 0 ? c.x : (s & 3) == 1 ? c.y : (s & 3) == 2 ? c.z : c.w;
  };
  // decoded operands of step s of a stage whose second half and scales are
  // h1 and sc (its first half is in ac0/bc0)
  auto decode_step = [&](int s, half8_t (&ad)[TM], half8_t (&bd)[TN], const Half1& h1,
                         const Scales& sc) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      ad[i] = decode8(word(s < 4 ? ac0[i] : h1.a[i], s),
                      scale_pair_bits((sc.a[i] >> (8 * (s >> 1))) & 0xFF));
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bd[j] = decode8(word(s < 4 ? bc0[j] : h1.b[j], s),
                      scale_pair_bits((sc.b[j] >> (8 * (s >> 1))) & 0xFF));
  };
  auto mfma_step = [&](const half8_t (&ad)[TM], const half8_t (&bd)[TN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ad[i], bd[j], acc[i][j], 0, 0, 0);
  };
  // one MFMA, then five of the next step's decode instructions (about a
  // sixteenth of them), and so on; the group's share of the stage DMA goes
  // after its first MFMAs, and LDS reads (ds_lo <= MFMA index < ds_hi) one
  // per MFMA, so no burst of loads holds up the in-order issue of the next
  // MFMA
  auto interleave = [&](int n_dma = 0, int ds_lo = 0, int ds_hi = 0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM * TN; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < n_dma) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      if (i >= ds_lo && i < ds_hi) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // DMA group g (0..5) of the stage loaded during iteration kt
  auto dma_group = [&](int kt, int g) __attribute__((always_inline)) {
    if (!kSpread) return 0;
    int ahead = kt + kRing - 1;
    uint8_t* base = lds + slot(ahead) * kStageBytes;
    ahead = ahead < nk ? ahead : (has_next ? ahead - nk : nk - 1);
    int n = 0;
#pragma unroll
    for (int idx = g * kDmaPer; idx < (g + 1) * kDmaPer && idx < kDmaPerStage; ++idx, ++n)
      dma_one(base, ahead * (kBK / 2), ahead * 8, idx);
    return n;
  };
  constexpr int kHalf0Reads = 2 * (TM + TN), kHalf1Reads = TM + TN;

  // prologue: kRing - 1 stages in LDS
#pragma unroll
  for (int st = 0; st < kRing - 1; ++st)
    if (st < nk) fill_stage(slot(st), st);
  if constexpr (kKAligned && !kFused) {
    // wait for stage 0 only; stages 1 .. kRing - 2 stay in flight
    const int issued = nk < kRing - 1 ? nk : kRing - 1;
    if (kRing == 4 && issued >= 3) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kDmaPerStage));
    else if (issued >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kDmaPerStage));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
  } else {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  for (;;) {                                   // tiles (one unless kPersist)
  read_half0(slot(0), sc_even);
  read_half1(slot(0), h1_even);
  decode_step(0, a_cur, b_cur, h1_even, sc_even);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Stage kt, whose second half and scales are in h1/sc; the next stage's
  // go to h1n/sn.
  auto k_stage = [&](int kt, const Half1& h1, const Scales& sc, Half1& h1n, Scales& sn)
      __attribute__((always_inline)) {
    if constexpr (kPersist) {
      // from here on the DMA loads the next tile's stages 0, 1, 2 (the slots
      // after this tile's last stage), if there is a next tile
      if (kt == nk - (kRing - 1)) {
        has_next = tile + (int)gridDim.x < n_tiles;
        if (has_next) {
          dense_coord(tile + (int)gridDim.x, tl);
          set_offsets();
        }
      }
    }
    const int ahead = kt + kRing - 1;           // the stage loaded this iteration
    if (!kSpread && ahead < nk) fill_stage(slot(ahead), ahead);
    // the next stage's slot: read even on the last iteration, where it holds
    // the next tile's stage 0 (kPersist) or is unused
    const int nbuf = slot(kt + 1);
    int nd = dma_group(kt, 0);
    decode_step(1, a_nxt, b_nxt, h1, sc);  mfma_step(a_cur, b_cur);  interleave(nd);
    nd = dma_group(kt, 1);
    decode_step(2, a_cur, b_cur, h1, sc);  mfma_step(a_nxt, b_nxt);  interleave(nd);
    nd = dma_group(kt, 2);
    decode_step(3, a_nxt, b_nxt, h1, sc);  mfma_step(a_cur, b_cur);  interleave(nd);
    // Stage kt + 1 must have landed (every wave's loads) before its
    // fragments are read; the loads of stages kt + 2 .. kt + kRing - 1 stay in
    // flight.  The barrier also ends every wave's reads of stage kt (all
    // issued in the previous iteration and complete at lgkmcnt 0), so the
    // next iteration may refill its slot.
    {
      if (kSpread) {
        // after kt + 1's loads: all of kt + 2's and the first part of kt + 3's
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kDmaPerStage + kDmaBeforeWait));
      } else {
        const int in_flight = nk - kt - 2;    // stages loaded after kt + 1
        if (kRing >= 4 && in_flight >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kDmaPerStage));
        else if (in_flight >= 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kDmaPerStage));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      }
      __builtin_amdgcn_s_barrier();
    }
    // the next stage: its first half and scales during step 4, its second
    // half (other registers than this stage's) during step 5
    read_half0(nbuf, sn);
    nd = dma_group(kt, 3);
    decode_step(4, a_cur, b_cur, h1, sc);  mfma_step(a_nxt, b_nxt);
    interleave(nd, 0, kHalf0Reads);
    read_half1(nbuf, h1n);
    nd = dma_group(kt, 4);
    decode_step(5, a_nxt, b_nxt, h1, sc);  mfma_step(a_cur, b_cur);
    interleave(nd, kDmaPer, kDmaPer + kHalf1Reads);
    nd = dma_group(kt, 5);
    decode_step(6, a_cur, b_cur, h1, sc);  mfma_step(a_nxt, b_nxt);  interleave(nd);
    decode_step(7, a_nxt, b_nxt, h1, sc);  mfma_step(a_cur, b_cur);  interleave();
    // step 7: decode the next stage's step 0 under this stage's last MFMAs
    decode_step(0, a_cur, b_cur, h1n, sn);
    mfma_step(a_nxt, b_nxt);
    interleave();
    // the next stage's step-0 operands are complete here (keeps their decode
    // under this stage's MFMAs rather than at the top of the next stage)
#pragma unroll
    for (int i = 0; i < TM; ++i) asm volatile("" ::"v"(a_cur[i]));
#pragma unroll
    for (int j = 0; j < TN; ++j) asm volatile("" ::"v"(b_cur[j]));
  };
  // two stages an iteration, so that the register sets alternate statically
  // (an exit between the two would make the accumulators' registers differ
  // at the two exits); an odd last stage follows the loop.  The tile walk is
  // launched for an even number of stages only, which keeps that extra copy
  // of the stage (and the registers it needs) out of it.
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    k_stage(kt, h1_even, sc_even, h1_odd, sc_odd);
    k_stage(kt + 1, h1_odd, sc_odd, h1_even, sc_even);
  }
  if constexpr (!kPersist) {
    if (kt < nk) k_stage(kt, h1_even, sc_even, h1_odd, sc_odd);
  }

  // ---- epilogue ------------------------------------------------------------
  // The accumulators leave through LDS, 16 rows of the wave's tile (a band)
  // at a time.  Each value is read once and scaled; the lanes write it in the
  // MFMA layout to a float32 band and/or a BF16 band (rounded two rows at a
  // time by the hardware's RNE conversion), then each lane reads back 16
  // contiguous bytes of one output row and stores them.  Each wave has a
  // region of its own in the (now idle) ring; a wave's LDS operations
  // complete in order, so a band needs no barrier between writes and reads.
  if constexpr (kPersist) {
    // every wave is done with this tile's last slot (the bands go there; the
    // next tile's loads into the other slots stay in flight)
    __builtin_amdgcn_s_barrier();
  } else {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // no DMA still writing the ring
    __syncthreads();                             // every wave is done with the ring
  }
  // The epilogue's lane-dependent addresses derive from an opaque copy of
  // the lane index, so that in the tile walk they are formed here, per tile,
  // instead of being hoisted out of it (they would stay live, and spill,
  // across the main loop).
  int lane_e = lane;
  if constexpr (kPersist)    // the lane index again, from the hardware
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
  const int fr_e = lane_e & 31, fh_e = lane_e >> 5;
  // kPersist: one output type, its bands in this tile's last slot
  uint8_t* const band_base = kPersist ? lds + slot(nk - 1) * kStageBytes : lds;
  // alpha_a alpha_b 2^8 per fragment column (one alpha_b per B row when B
  // concatenates several tensors, else the group's)
  // (alpha_a and a group's alpha_b are uniform: scalar loads, so that no
  // vector-memory wait drains the next tile's loads in flight)
  float scale[TN];
  const float alpha_a = load_uniform(p.alpha_a);
  const float alpha_g = p.alpha_b_rows ? 0.0f : load_uniform(p.alpha_b + tc.group);
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    float ab;
    if (p.alpha_b_rows) {
      const int64_t col = tc.n0 + wn + 32 * j + fr_e;
      ab = p.alpha_b_rows[col < p.N ? col : p.N - 1];
    } else {
      ab = alpha_g;
    }
    scale[j] = alpha_a * ab * 256.0f;
  }
  const int64_t row_lim = tc.m0 + BM < tc.m_end ? tc.m0 + BM : tc.m_end;
  const bool want32 = p.y_f32 != nullptr, want16 = p.y_bf16 != nullptr;
  constexpr int kBandRows = 16;
  constexpr int kPitch32 = WN * 4 + 32, kPitch16 = WN * 2 + 16;   // padded rows
  constexpr int kBandBytes = kBandRows * (kPitch32 + kPitch16);
  static_assert(4 * kBandBytes <= kRing * kStageBytes, "epilogue bands fit the ring");
  static_assert(!kPersist || 4 * kBandRows * kPitch32 <= kStageBytes, "bands fit one slot");
  uint8_t* band32 = band_base + wave * (kPersist ? kBandRows * kPitch32 : kBandBytes);
  uint8_t* band16 = kPersist ? band32 : band32 + kBandRows * kPitch32;
  const bool interior = tc.m0 + BM <= tc.m_end && tc.n0 + BN <= p.N;

  // Band (i, h): rows 16h .. 16h + 15 of fragment row i, i.e. accumulator
  // registers r = 8h .. 8h + 7 (row 8(r/4) + 4(lane/32) + r%4).  Each lane
  // writes at a fixed base plus compile-time offsets.
  uint8_t* w32 = band32 + (4 * fh_e) * kPitch32 + fr_e * 4;
  uint8_t* w16 = band16 + (4 * fh_e) * kPitch16 + fr_e * 2;
  auto band_write = [&](int i, int h, auto k32, auto k16) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 8 * h; r < 8 * h + 8; r += 2) {
        const int row = 8 * ((r >> 2) - 2 * h) + (r & 3);
        const float v0 = acc[i][j][r] * scale[j], v1 = acc[i][j][r + 1] * scale[j];
        if (decltype(k32)::value) {
          *reinterpret_cast<float*>(w32 + row * kPitch32 + 32 * j * 4) = v0;
          *reinterpret_cast<float*>(w32 + (row + 1) * kPitch32 + 32 * j * 4) = v1;
        }
        if (decltype(k16)::value) {
          const bf16x2_t b = __builtin_convertvector((float2_t){v0, v1}, bf16x2_t);
          *reinterpret_cast<__bf16*>(w16 + row * kPitch16 + 32 * j * 2) = b[0];
          *reinterpret_cast<__bf16*>(w16 + (row + 1) * kPitch16 + 32 * j * 2) = b[1];
        }
      }
  };
  // Stores band (i, h) of one output.  Chunk q of a lane covers row
  // q * kRowsPerQ + lane_row, columns lane_col .. lane_col + kPer - 1 of the
  // band.  Straight-line 16-byte stores when the tile is inside the output
  // and rows are 16-byte aligned (a uniform test), else element by element
  // with bounds checks.  The 16-byte stores are non-temporal: this kernel
  // never reads the output, so it need not sit dirty in L2 at the end.
  auto band_store = [&](auto* y, const uint8_t* band, int vec, int i, int h)
      __attribute__((always_inline)) {
    using T = typename std::remove_pointer<decltype(y)>::type;
    constexpr int kE = (int)sizeof(T), kPitch = kE == 4 ? kPitch32 : kPitch16;
    constexpr int kPer = 16 / kE;                    // elements per 16-byte chunk
    constexpr int kLanesPerRow = WN / kPer;
    constexpr int kRowsPerQ = 64 / kLanesPerRow;
    static_assert(64 % kLanesPerRow == 0, "a row is a whole number of lanes");
    constexpr int kQ = kBandRows / kRowsPerQ;
    const int lane_row = lane_e / kLanesPerRow, lane_col = (lane_e % kLanesPerRow) * kPer;
    const int64_t row0 = tc.m0 + wm + 32 * i + kBandRows * h;
    const uint8_t* src = band + lane_row * kPitch + lane_col * kE;
    T* dst = y + (row0 + lane_row) * p.ld_y + tc.n0 + wn + lane_col;
    const int64_t step = (int64_t)kRowsPerQ * p.ld_y;
    if (interior && vec) {
#pragma unroll
      for (int q = 0; q < kQ; ++q)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(src + q * kRowsPerQ * kPitch),
                                    reinterpret_cast<u32x4*>(dst + q * step));
    } else {
      const int64_t rows_left = row_lim - row0;
      const int64_t cols_left = p.N - (tc.n0 + wn);
#pragma unroll 1
      for (int q = 0; q < kQ; ++q) {
        const T* t = reinterpret_cast<const T*>(src + q * kRowsPerQ * kPitch);
        if (q * kRowsPerQ + lane_row < rows_left) {
#pragma unroll 1
          for (int k = 0; k < kPer; ++k)
            if (lane_col + k < cols_left) dst[q * step + k] = t[k];
        }
      }
    }
  };
  if constexpr (kSilu) {
    // ---- gated activation: H = SiLU(g) * u --------------------------------
    // Fragments 2jp and 2jp + 1 hold the gate and up outputs of the same 32
    // units (B rows 64b .. 64b + 31 and 64b + 32 .. 64b + 63), so a lane
    // finds g and u of an H value in its own registers.  H leaves through
    // LDS bands as the outputs do; the amax of |H| over the tile's real
    // rows and columns goes to h_partials[tile].
    static_assert(TN % 2 == 0, "gate/up fragment pairs");
    constexpr int HW = WN / 2;                       // H columns of the wave
    constexpr int kPitchH = HW * 2 + 16;
    static_assert(4 * kBandRows * kPitchH <= kRing * kStageBytes, "bands fit the ring");
    uint8_t* bandh = band_base + wave * (kBandRows * kPitchH);
    uint8_t* wh = bandh + (4 * fh_e) * kPitchH + fr_e * 2;
    const int64_t n_h = p.N / 2;
    const int64_t hcol0 = (tc.n0 + wn) / 2;
    constexpr int kPer = 8, kLanesPerRow = HW / kPer, kRowsPerQ = 64 / kLanesPerRow;
    static_assert(64 % kLanesPerRow == 0, "a row is a whole number of lanes");
    constexpr int kQ = kBandRows / kRowsPerQ;
    const int lane_row = lane_e / kLanesPerRow, lane_col = (lane_e % kLanesPerRow) * kPer;
    const bool interior_h = tc.m0 + BM <= tc.m_end && (tc.n0 + BN) / 2 <= n_h;
    // |H| maxima of the lane, as two BF16 magnitudes (rows r and r + 1)
    u16x2 hm2 = {0, 0};
    // interior tiles skip the row and column masks of the maxima and the
    // bounds-checked stores (a uniform choice, one copy of the code each)
    auto silu_epilogue = [&](auto k_in) __attribute__((always_inline)) {
      constexpr bool kIn = decltype(k_in)::value;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int64_t row0 = tc.m0 + wm + 32 * i + kBandRows * h;
          const int64_t lim = row_lim - row0 - 4 * fh_e;   // rows of the band this lane may count
#pragma unroll
          for (int jp = 0; jp < TN / 2; ++jp) {
            const bool col_ok = hcol0 + 32 * jp + fr_e < n_h;
#pragma unroll
            for (int r = 8 * h; r < 8 * h + 8; r += 2) {
              const int row = 8 * ((r >> 2) - 2 * h) + (r & 3);
              const float g0 = acc[i][2 * jp][r] * scale[2 * jp];
              const float g1 = acc[i][2 * jp][r + 1] * scale[2 * jp];
              const float u0 = acc[i][2 * jp + 1][r] * scale[2 * jp + 1];
              const float u1 = acc[i][2 * jp + 1][r + 1] * scale[2 * jp + 1];
              const bf16x2_t b = __builtin_convertvector(
                  (float2_t){silu_mul(g0, u0), silu_mul(g1, u1)}, bf16x2_t);
              *reinterpret_cast<__bf16*>(wh + row * kPitchH + 32 * jp * 2) = b[0];
              *reinterpret_cast<__bf16*>(wh + (row + 1) * kPitchH + 32 * jp * 2) = b[1];
              uint32_t bits = __builtin_bit_cast(uint32_t, b) & 0x7FFF7FFFu;
              if constexpr (!kIn)
                bits &= (col_ok && row < lim ? 0xFFFFu : 0u) |
                        (col_ok && row + 1 < lim ? 0xFFFF0000u : 0u);
              hm2 = __builtin_elementwise_max(hm2, __builtin_bit_cast(u16x2, bits));
            }
          }
          __builtin_amdgcn_wave_barrier();
          const uint8_t* src = bandh + lane_row * kPitchH + lane_col * 2;
          uint16_t* dst = p.h_bf16 + (row0 + lane_row) * p.ld_h + hcol0 + lane_col;
          const int64_t step = (int64_t)kRowsPerQ * p.ld_h;
          if (kIn && p.vec_h) {
#pragma unroll
            for (int q = 0; q < kQ; ++q)
              *reinterpret_cast<u32x4*>(dst + q * step) =
                  *reinterpret_cast<const u32x4*>(src + q * kRowsPerQ * kPitchH);
          } else {
            const int64_t rows_left = row_lim - row0;
            const int64_t cols_left = n_h - hcol0;
#pragma unroll 1
            for (int q = 0; q < kQ; ++q) {
              const uint16_t* t = reinterpret_cast<const uint16_t*>(src + q * kRowsPerQ * kPitchH);
              if (q * kRowsPerQ + lane_row < rows_left) {
#pragma unroll 1
                for (int k = 0; k < kPer; ++k)
                  if (lane_col + k < cols_left) dst[q * step + k] = t[k];
              }
            }
          }
          __builtin_amdgcn_wave_barrier();
        }
    };
    if (interior_h)
      silu_epilogue(std::true_type{});
    else
      silu_epilogue(std::false_type{});
    uint32_t hmax = max((uint32_t)hm2[0], (uint32_t)hm2[1]);
    hmax = wave_max_u32(hmax);
    // the four wave maxima meet in the ring, past the H bands (one LDS
    // array in the kernel: a second would make every fragment read of the
    // main loop wait for all DMA in flight); LDS-scoped workgroup fences
    // order the exchange (lgkmcnt(0) and the barrier) without waiting for
    // the output stores
    static_assert(4 * kBandRows * kPitchH + 16 <= (kPersist ? 1 : kRing) * kStageBytes,
                  "wave maxima fit past the bands");
    uint32_t* hred = reinterpret_cast<uint32_t*>(band_base + 4 * kBandRows * kPitchH);
    if (lane_e == 0) hred[wave] = hmax;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    if (tid == 0)
      p.h_partials[tile] =
          max(max(hred[0], hred[1]), max(hred[2], hred[3]));
  } else {
  auto epilogue = [&](auto k32, auto k16) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        band_write(i, h, k32, k16);
        __builtin_amdgcn_wave_barrier();
        if (decltype(k32)::value) band_store(p.y_f32, band32, p.vec_f32, i, h);
        if (decltype(k16)::value)
          band_store(reinterpret_cast<__bf16*>(p.y_bf16), band16, p.vec_bf16, i, h);
        __builtin_amdgcn_wave_barrier();
      }
  };
  using yes = std::true_type;
  using no = std::false_type;
  if (want32 && want16) epilogue(yes{}, yes{});
  else if (want32) epilogue(yes{}, no{});
  else epilogue(no{}, yes{});
  }

  if (!has_next) break;
  // the next tile: its stage 0 has landed (the last iteration waited for
  // it), its stages 1 and 2 are in flight.  Every wave's band reads end
  // before the first loads into the bands' slot.
  tile += (int)gridDim.x;
  tc = tl;
  ring0 = (ring0 + nk) % kRing;
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(63));   // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  }                                            // tiles
}

// Compute units of the current device (cached per device).
int cu_count() {
  static std::atomic<int> cached[64];         // 0: not yet known
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int BM, int BN, bool kFused, int kRing, int kOcc, bool kSilu = false>
hipError_t launch_tiles(const W4A4Args& a, hipStream_t stream) {
  int tiles_m = (int)((a.M + BM - 1) / BM);
  if (a.group_offsets != nullptr) tiles_m += a.num_groups;
  const int tiles_n = (int)((a.N + BN - 1) / BN);
  // persistent walk: the DMA path with a 4-deep ring, dense, one output type
  // (its bands fit one ring slot), an even number of at least 4 stages and
  // two tiles per CU; the NVFP4_PATH_GEMM_GRID flag turns it off (a
  // persistent walk over grouped tiles, built and measured, was no faster
  // than the grid launch in the same tile order)
  if constexpr (kRing == 4 && !kFused) {
    const bool allowed = (path_flags() & kPathGemmGrid) == 0;
    const int64_t n_tiles = (int64_t)tiles_m * tiles_n;
    const int cus = cu_count();
    if (allowed && a.K % (2 * kBK) == 0 && a.K / kBK >= 4 && a.group_offsets == nullptr &&
        a.a_row_index == nullptr && (kSilu || ((a.y_f32 != nullptr) != (a.y_bf16 != nullptr))) &&
        n_tiles >= 2 * (int64_t)cus) {
      hipLaunchKernelGGL((w4a4_gemm_kernel<BM, BN, true, false, kRing, kOcc, kSilu, true>),
                         dim3(cus), dim3(kThreads), 0, stream, a);
      return hipGetLastError();
    }
  }
  dim3 grid(tiles_m, tiles_n);
  if (a.K % kBK == 0)
    hipLaunchKernelGGL((w4a4_gemm_kernel<BM, BN, true, kFused, kRing, kOcc, kSilu>), grid,
                       dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((w4a4_gemm_kernel<BM, BN, false, kFused, kRing, kOcc, kSilu>), grid,
                       dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// Tile choice: 256x256 when that gives at least one tile per CU of the
// chip, else 128x256 when that does (fewer decodes per MFMA than 128x128:
// 8192x1024x4096 took 63-64 against 68-70 us), else 128x128.  0: 256x256,
// 1: 128x256, 2: 128x128.
int tile_choice(int64_t M, int64_t N) {
  const int64_t t0 = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t t1 = ((M + 127) / 128) * ((N + 255) / 256);
  return t0 >= 256 ? 0 : (t1 >= 256 ? 1 : 2);
}

template <bool kFused, bool kSilu = false>
hipError_t launch_any(const W4A4Args& args, hipStream_t stream) {
  if (args.M == 0 || args.N == 0) return hipSuccess;
  W4A4Args a = args;
  a.vec_f32 = (reinterpret_cast<uintptr_t>(a.y_f32) % 16 == 0) && (a.ld_y * 4) % 16 == 0;
  a.vec_bf16 = (reinterpret_cast<uintptr_t>(a.y_bf16) % 16 == 0) && (a.ld_y * 2) % 16 == 0;
  a.vec_h = (reinterpret_cast<uintptr_t>(a.h_bf16) % 16 == 0) && (a.ld_h * 2) % 16 == 0;
  const int choice = tile_choice(a.M, a.N);
  if (choice == 0) return launch_tiles<256, 256, kFused, kFused ? 3 : 4, 1, kSilu>(a, stream);
  if (choice == 1) return launch_tiles<128, 256, kFused, 3, 1, kSilu>(a, stream);
  return launch_tiles<128, 128, kFused, 3, 2, kSilu>(a, stream);
}

}  // namespace

hipError_t launch_w4a4(const W4A4Args& a, hipStream_t stream) {
  return launch_any<false>(a, stream);
}

hipError_t launch_w4a4_fused(const W4A4Args& a, hipStream_t stream) {
  return launch_any<true>(a, stream);
}

hipError_t launch_w4a4_silu(const W4A4Args& a, hipStream_t stream) {
  return launch_any<false, true>(a, stream);
}

int64_t w4a4_silu_tiles_max(int64_t M, int64_t N) {
  // the smallest tile gives the most workgroups
  return ((M + 127) / 128) * ((N + 127) / 128);
}

int64_t w4a4_tiles(int64_t M, int64_t N) {
  const int c = tile_choice(M, N);
  const int64_t bm = c == 0 ? 256 : 128, bn = c == 2 ? 128 : 256;
  return ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
}

}  // namespace nvfp4
