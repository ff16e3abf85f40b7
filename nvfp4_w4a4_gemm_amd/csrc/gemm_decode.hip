// Decode-shaped NVFP4 W4A4 GEMM for gfx950: a few token rows (M <= 64)
// against a whole weight matrix, the shape of the decode steps in the
// uniform-NVFP4 configuration that Mix-Quant is compared with
// ("Mix-Quant：面向智能体LLM的量化预填充与精确解码", paper.rainbus.top digest,
// 实验结果, Table 1 and the phase-wise ablation of Table 3).  The arithmetic
// is the W4A4 linear layer of the same digest (核心方法; 方法步骤详情 steps (3)
// and (4)):
//
//   Y[m][n] = alpha_a alpha_b sum_b sigma^a_{m,b} sigma^b_{n,b}
//             sum_{k in b} q^a_{m,k} q^b_{n,k}
//
// At this shape the work is a stream over the weight codes (0.5625 bytes a
// weight): the kernel is bound by HBM, not by the matrix cores.  One token
// row (with K % 32 == 0) takes a matrix-vector kernel: w4a4_gemv_kernel
// (K <= 8192, whole weight rows a wave) or w4a4_gemv_split_kernel
// (K <= 32768, each row's K split over the four waves of a workgroup), both
// described there; otherwise the layout is:
//
//  - A workgroup (4 waves) owns 16 output columns and all of K.  The K axis
//    is cut into 32-element chunks (16 code bytes and 2 scale bytes a row);
//    the 16 lane groups of the workgroup (wave w, lane group g = lane / 16)
//    take chunks 4w + g, 4w + g + 16, ... so that each row is read in runs
//    of 256 contiguous code bytes.  Lane l of a group reads chunk data of
//    weight row n0 + l % 16 and of token row l % 16 (+ 16 t for M-tile t).
//  - Both operands are decoded to float16 with the block scale folded in
//    (exact: every q * sigma has at most 6 significant bits) and multiplied
//    by v_mfma_f32_16x16x32_f16, whose operand lanes hold 8 K-elements of
//    one row (lane group g supplies K-slots 8g..8g+7).  A and B lanes of one
//    group supply the same chunk, so the contraction pairs the right
//    elements; which chunk lands in which K-slot does not matter to a sum.
//  - The four waves' float32 partial sums meet in LDS and are added in a
//    fixed order (wave 0 + 1 + 2 + 3), then scaled by alpha_a alpha_b 2^8.
#include "device_common.h"
#include "kernels.h"

#include <atomic>

#include <cstdlib>

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kCols = 16;                 // output columns per workgroup
constexpr int kGroups = kWaves * 4;       // lane groups sharing a row's chunks
constexpr int kDepth = 4;                 // chunks in flight per lane

// s_waitcnt immediate (gfx9 encoding): vector-memory count n, no expcnt
// wait, LDS/scalar count 0.
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// sigma (E4M3FN byte) -> float16 sigma * 2^-8 in both halves (the byte's
// exponent and mantissa fields land in the f16 fields; a subnormal E4M3
// byte becomes a subnormal f16).
__device__ __forceinline__ half2_t scale_pair(uint32_t sb) {
  return __builtin_bit_cast(half2_t, sb * 0x00800080u);
}

// 8 FP4 codes (one 32-bit word, element 2j in the low nibble of byte j) ->
// 8 float16 values q * sigma * 2^-4, exactly: the conversion multiplies by
// 16 (the exponent of its scale operand), the packed multiply by sigma 2^-8.
__device__ __forceinline__ half8_t decode8(uint32_t w, half2_t s) {
  half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 16.0f, 0) * s;
  half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 16.0f, 1) * s;
  half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 16.0f, 2) * s;
  half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 16.0f, 3) * s;
  half8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// The codes (16 bytes) and the two scale bytes of one row's 32-element chunk
// j, loaded from a clamped (always valid) chunk index: the loads are
// unconditional, so the compiler keeps them in flight across the pipeline.
// A chunk past the end of the row, or a token row that is not there, is
// removed where the data is used, by a zero A scale (a zero scale decodes
// to zero whatever the codes; B never needs it, since every B value meets an
// A value).  kFull: K % 32 == 0, so a chunk is whole and its scale pair is
// 2-byte aligned.  Otherwise the last chunk holds one block (16 elements),
// whose second half repeats the first and gets a zero A scale.  kStream:
// the data is read once (non-temporal loads).
struct ChunkData {
  u32x4 codes;
  uint32_t scales;     // byte 0: block 2j, byte 1: block 2j + 1
};

// Raw buffer resource (stride 0, plain 32-bit data format) over
// [base, base + bytes).  Buffer loads are intrinsics, not plain loads, so
// the compiler does not move them next to their use in a later iteration.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// codes_off / scales_off: byte offsets of the row in the two buffers.
template <bool kFull, bool kStream>
__device__ __forceinline__ ChunkData load_chunk(__amdgpu_buffer_rsrc_t rc, uint32_t codes_off,
                                                __amdgpu_buffer_rsrc_t rs, uint32_t scales_off,
                                                int j, int n_chunks, int n_blocks) {
  constexpr int kPolicy = kStream ? 2 : 0;          // nt: read once
  const uint32_t jc = (uint32_t)(j < n_chunks ? j : n_chunks - 1);
  ChunkData d;
  if (kFull) {
    d.codes = __builtin_amdgcn_raw_buffer_load_b128(rc, codes_off + 16u * jc, 0, kPolicy);
    d.scales = __builtin_amdgcn_raw_buffer_load_b16(rs, scales_off + 2u * jc, 0, 0);
  } else {
    const uint32_t second = 2 * jc + 1 < (uint32_t)n_blocks ? 1u : 0u;  // the chunk is whole
    const u32x2 lo = __builtin_amdgcn_raw_buffer_load_b64(rc, codes_off + 16u * jc, 0, kPolicy);
    const u32x2 hi =
        __builtin_amdgcn_raw_buffer_load_b64(rc, codes_off + 16u * jc + 8u * second, 0, kPolicy);
    d.codes = u32x4{lo.x, lo.y, hi.x, hi.y};
    d.scales = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, scales_off + 2u * jc, 0, 0) |
               ((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, scales_off + 2u * jc + second,
                                                              0, 0) << 8);
  }
  return d;
}

// Which scale bytes of chunk j are real (0xFFFF, 0x00FF for a half chunk,
// 0 past the end).
__device__ __forceinline__ uint32_t chunk_mask(int j, int n_chunks, int n_blocks) {
  if (j >= n_chunks) return 0u;
  return 2 * j + 1 < n_blocks ? 0xFFFFu : 0x00FFu;
}

template <int MT, bool kFull>
__global__ __launch_bounds__(kThreads) void w4a4_decode_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ alpha_a, const uint8_t* __restrict__ b_codes,
    const uint8_t* __restrict__ b_scales, const float* __restrict__ alpha_b,
    const float* __restrict__ alpha_b_rows, int M, int N, int K,
    float* __restrict__ y_f32, uint16_t* __restrict__ y_bf16, int64_t ld_y) {
  __shared__ float red[kWaves][MT][16][17];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int group = wave * 4 + (lane >> 4);
  const int n0 = blockIdx.x * kCols;
  const int n_chunks = (K + 31) / 32;
  const int n_blocks = K / 16;
  const int64_t row_codes = K / 2, row_scales = K / 16;

  const int nb = n0 + r16 < N ? n0 + r16 : N - 1;
  const __amdgpu_buffer_rsrc_t rbc = buffer_of(b_codes, (uint32_t)(N * row_codes));
  const __amdgpu_buffer_rsrc_t rbs = buffer_of(b_scales, (uint32_t)(N * row_scales));
  const __amdgpu_buffer_rsrc_t rac = buffer_of(a_codes, (uint32_t)(M * row_codes));
  const __amdgpu_buffer_rsrc_t ras = buffer_of(a_scales, (uint32_t)(M * row_scales));
  const uint32_t bc = (uint32_t)(nb * row_codes), bs = (uint32_t)(nb * row_scales);
  uint32_t ac[MT], as[MT];
  bool a_ok[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = 16 * t + r16;
    a_ok[t] = m < M;
    const int mc = a_ok[t] ? m : 0;
    ac[t] = (uint32_t)(mc * row_codes);
    as[t] = (uint32_t)(mc * row_scales);
  }

  float4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

  // chunks of this lane: group, group + 16, ...  The trip count is that of
  // the workgroup's first lane group rounded up to whole pipeline rounds, so
  // the loop body has no branch (which would make the compiler drain the
  // loads in flight) and all lanes of a wave run the MFMAs together; a lane
  // whose chunk is past the end supplies zeros.
  const int iters = (n_chunks + kGroups - 1) / kGroups;

  ChunkData b_buf[kDepth];
  ChunkData a_buf[kDepth][MT];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    const int j = group + kGroups * d;
    b_buf[d] = load_chunk<kFull, true>(rbc, bc, rbs, bs, j, n_chunks, n_blocks);
#pragma unroll
    for (int t = 0; t < MT; ++t)
      a_buf[d][t] = load_chunk<kFull, false>(rac, ac[t], ras, as[t], j, n_chunks, n_blocks);
  }

  for (int i0 = 0; i0 < iters; i0 += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      {
        // decode the chunk in hand first, so that its raw registers are free
        // for the refill; the refill is then in flight during the MFMAs
        const int jd = group + kGroups * (i0 + d);
        const uint32_t mask = chunk_mask(jd, n_chunks, n_blocks);
        const uint32_t bw[4] = {b_buf[d].codes.x, b_buf[d].codes.y, b_buf[d].codes.z,
                                b_buf[d].codes.w};
        half8_t bv[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
          bv[s] = decode8(bw[s], scale_pair((b_buf[d].scales >> (8 * (s >> 1))) & 0xFFu));
        half8_t av[MT][4];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const uint32_t aw[4] = {a_buf[d][t].codes.x, a_buf[d][t].codes.y,
                                  a_buf[d][t].codes.z, a_buf[d][t].codes.w};
          const uint32_t as_eff = a_ok[t] ? (a_buf[d][t].scales & mask) : 0u;
#pragma unroll
          for (int s = 0; s < 4; ++s)
            av[t][s] = decode8(aw[s], scale_pair((as_eff >> (8 * (s >> 1))) & 0xFFu));
        }
        // refill this slot with the chunk kDepth iterations ahead
        const int j = jd + kGroups * kDepth;
        b_buf[d] = load_chunk<kFull, true>(rbc, bc, rbs, bs, j, n_chunks, n_blocks);
#pragma unroll
        for (int t = 0; t < MT; ++t)
          a_buf[d][t] = load_chunk<kFull, false>(rac, ac[t], ras, as[t], j, n_chunks, n_blocks);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int t = 0; t < MT; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[t][s], bv[s], acc[t], 0, 0, 0);
      }
    }
  }

  // D layout of the 16x16 MFMA: lane l holds rows 4 (l / 16) + r, column l % 16
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][t][4 * (lane >> 4) + r][r16] = acc[t][r];
  __syncthreads();

  const int n = threadIdx.x & 15;
  const int col = n0 + n;
  if (col >= N) return;
  const float ab = alpha_b_rows != nullptr ? alpha_b_rows[col] : *alpha_b;
  const float scale = (*alpha_a) * ab * 256.0f;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int mr = threadIdx.x >> 4;          // 0..15
    const int m = 16 * t + mr;
    if (m >= M) continue;
    float v = red[0][t][mr][n];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += red[w][t][mr][n];
    v *= scale;
    if (y_f32 != nullptr) y_f32[m * ld_y + col] = v;
    if (y_bf16 != nullptr) y_bf16[m * ld_y + col] = (uint16_t)f32_to_bf16_bits(v);
  }
}

// ---- LDS-staged variant (K % 64 == 0) --------------------------------------
// The stream over B is what the kernel waits for, and HBM serves it best in
// long runs of one row.  Here each K-stage (512 elements: 256 code bytes and
// 32 scale bytes a row) of the workgroup's 16 B rows, and of the 16 * MT
// token rows, goes global -> LDS by buffer_load ... lds: one wave
// instruction moves 4 rows x 256 contiguous bytes.  Lane i of the
// instruction fetches chunk (i % 16) ^ (row & 15) of its row into slot
// i % 16, so that the MFMA-layout reads (16 rows, one chunk) hit 16 distinct
// bank groups.  A ring of S stages keeps S - 1 stages in flight; past the
// last stage the loads repeat the last stage into the slot being refilled,
// which nobody reads again, so the wait count stays constant.  Each lane
// then handles one 32-element chunk of a stage (chunk 4 * wave + lane / 16).
constexpr int kStageCodes = 256;                       // code bytes a row and stage
constexpr int kStageScales = 32;                       // scale bytes a row and stage
constexpr int kTileBytes = 16 * (kStageCodes + kStageScales);   // 4608

__device__ __forceinline__ void dma16_lds(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4_lds(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 4,
                                           voff, 0, 0, 0);
}

// A workgroup takes at most kMaxTiles column tiles (blockIdx.x,
// blockIdx.x + gridDim.x, ...), streams all of them through the ring without
// a break, and keeps one accumulator set per tile; the cross-wave sums come
// at the very end.  (An LDS write while loads into LDS are in flight makes
// the compiler wait for them, which would drain the ring at every tile.)
constexpr int kMaxTiles = 8;

// With kARes (one M-tile, and M x K small enough) the token rows are not
// staged with every weight stage: the whole quantised activation is loaded
// into LDS once, with the same 256-byte segments and XOR slot order, and
// the ring carries the weight alone (half the LDS a stage, so more
// workgroups fit on a CU).  20 KB takes up to 8 token rows at K = 4096
// (24576 x 4096 at 8 tokens: 16.4 us against 18.9 staged); 16 rows there
// (37 KB) ran no faster resident, and 6144 x 4096 slower.  With one stage
// group a workgroup (more than two column tiles a CU) up to 48 KB stays
// resident (51200 x 5120 at 8 tokens: 34.1 against 39.5 us, at 16 tokens
// 38.4 against 40.4 us); with two or four groups the larger activation
// lowers occupancy (7168 x 5120 at 16 tokens: 9.7 against 8.9 us).
constexpr int kAResMaxBytes = 20 * 1024;
constexpr int kAResWideMaxBytes = 48 * 1024;

__host__ __device__ constexpr int decode_stage_bytes(int MT, bool ares) {
  return (ares ? 1 : 1 + MT) * kTileBytes + 256;
}
// Resident activation: code segments rounded up to whole 1 KB DMAs, scale
// segments to whole 256-byte DMAs (the last DMA's surplus lanes land in
// the padding).
__host__ __device__ constexpr int decode_ares_code_bytes(int M, int n_stages) {
  return (M * n_stages + 3) / 4 * 4 * kStageCodes;
}
__host__ __device__ constexpr int decode_ares_bytes(int M, int n_stages) {
  return decode_ares_code_bytes(M, n_stages) + (M * n_stages + 7) / 8 * 8 * kStageScales;
}

// kG groups of 4 waves share a workgroup's column tiles: group k computes
// stages k, k + kG, ... of each tile (a tile's stages padded to a multiple
// of kG; a padding stage reloads a real one and contributes nothing, its A
// scales being masked to zero), each group with its own S / kG ring slots,
// loads and wait counts, exactly as one 4-wave workgroup would.  Every wave
// passes the same barriers.  For weights with few column tiles this runs kG
// stage chains per CU instead of one.
template <int MT, int S, bool kARes, int kG>
__global__ __launch_bounds__(kThreads * kG) void w4a4_decode_lds_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ alpha_a, const uint8_t* __restrict__ b_codes,
    const uint8_t* __restrict__ b_scales, const float* __restrict__ alpha_b,
    const float* __restrict__ alpha_b_rows, int M, int N, int K,
    float* __restrict__ y_f32, uint16_t* __restrict__ y_bf16, int64_t ld_y) {
  static_assert(!kARes || MT == 1, "resident activations take one M-tile");
  static_assert(S % kG == 0 && S / kG >= 2, "each group has its ring slots");
  constexpr int kSG = S / kG;                          // ring slots of one group
  constexpr int kAllWaves = kWaves * kG;
  constexpr int kTiles = kARes ? 1 : 1 + MT;           // B tile, then the A tiles
  // scale DMAs: 8 rows x 32 bytes of one tile each (all 64 lanes); wave w
  // takes halves w, w + 4, ...; a wave left without one reloads a valid
  // half into a slack area, so every wave counts the same loads
  constexpr int kScaleDmas = (2 * kTiles + kWaves - 1) / kWaves;
  constexpr int kStage = decode_stage_bytes(MT, kARes);
  constexpr int kRed = kAllWaves * MT * 16 * 17 * 4;   // one tile's partial sums
  static_assert(kRed <= S * kStage, "the reduction fits in the ring");
  // ring, then (kARes) the resident activation
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = wave_all & (kWaves - 1);            // wave within its group
  const int grp = wave_all / kWaves;                   // its group (uniform)
  const int r16 = lane & 15;
  const int n_chunks = K / 32;
  const int n_stages = (K / 2 + kStageCodes - 1) / kStageCodes;
  const int n_pad = (n_stages + kG - 1) / kG * kG;     // a tile's stages, padded
  const int64_t row_codes = K / 2, row_scales = K / 16;
  const int n_tiles = (N + kCols - 1) / kCols;
  const int my_tiles = (n_tiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int total = my_tiles * n_pad;                  // stages of this workgroup (padded)

  const __amdgpu_buffer_rsrc_t rbc = buffer_of(b_codes, (uint32_t)(N * row_codes));
  const __amdgpu_buffer_rsrc_t rbs = buffer_of(b_scales, (uint32_t)(N * row_scales));
  const __amdgpu_buffer_rsrc_t rac = buffer_of(a_codes, (uint32_t)(M * row_codes));
  const __amdgpu_buffer_rsrc_t ras = buffer_of(a_scales, (uint32_t)(M * row_scales));

  // DMA lane offsets at stage 0.  Codes, per tile: row 4 * wave + lane / 16,
  // slot lane % 16 (1 KB a wave).  Scales, per half h of a tile: row
  // 8 h + lane / 8, bytes 4 (lane % 8) .. + 3 (K % 64 == 0 keeps them 4-byte
  // aligned).  B rows past N repeat row N - 1 (their outputs are dropped);
  // token rows past M repeat row M - 1 (their A scales are zeroed).
  const int dma_row = 4 * wave + (lane >> 4);
  const int dma_chunk = r16 ^ dma_row;                 // dma_row < 16
  auto a_row = [&](int t, int r) { return 16 * t + r < M ? 16 * t + r : M - 1; };
  uint32_t a_code_off[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
    a_code_off[t] = (uint32_t)(a_row(t, dma_row) * row_codes) + 16u * dma_chunk;
  int sc_tile[kScaleDmas], sc_r[kScaleDmas];
  uint32_t a_scale_off[kScaleDmas];
#pragma unroll
  for (int d = 0; d < kScaleDmas; ++d) {
    const int half = d * kWaves + wave;                // uniform
    const int hh = half < 2 * kTiles ? half : 0;
    sc_tile[d] = hh >> 1;
    sc_r[d] = 8 * (hh & 1) + (lane >> 3);
    a_scale_off[d] = sc_tile[d] == 0 ? 0u
                     : (uint32_t)(a_row(sc_tile[d] - 1, sc_r[d]) * row_scales) + 4u * (lane & 7);
  }
  // global stage g -> (column tile, stage within the tile); a padding stage
  // and, past the end, the last stage load a real stage again (into a slot
  // whose data nobody uses)
  auto issue = [&](int g) __attribute__((always_inline)) {
    const int gc = g < total ? g : total - 1;
    const int tile = (int)blockIdx.x + (gc / n_pad) * (int)gridDim.x;
    const int sp = gc % n_pad;
    const uint32_t st = (uint32_t)(sp < n_stages ? sp : n_stages - 1);
    const int nb0 = tile * kCols;
    uint8_t* base = lds + (g % S) * kStage;
    const int rb = nb0 + dma_row < N ? nb0 + dma_row : N - 1;
    dma16_lds(rbc, base + wave * 1024,
              (uint32_t)(rb * row_codes) + 16u * dma_chunk + st * kStageCodes);
    if (!kARes) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
        dma16_lds(rac, base + (1 + t) * kTileBytes + wave * 1024,
                  a_code_off[t] + st * kStageCodes);
    }
#pragma unroll
    for (int d = 0; d < kScaleDmas; ++d) {
      const int half = d * kWaves + wave;
      uint8_t* dst = half < 2 * kTiles
                         ? base + (half >> 1) * kTileBytes + 16 * kStageCodes + (half & 1) * 256
                         : base + kTiles * kTileBytes;
      // branch-free (a branch here makes the compiler drain the loads)
      const bool is_b = sc_tile[d] == 0;
      const int rs = nb0 + sc_r[d] < N ? nb0 + sc_r[d] : N - 1;
      const uint32_t off = is_b ? (uint32_t)(rs * row_scales) + 4u * (lane & 7) : a_scale_off[d];
      dma4_lds(is_b ? rbs : ras, dst, off + st * kStageScales);
    }
  };
  constexpr int kDmaPerStage = kTiles + kScaleDmas;
  static_assert((kSG - 1) * kDmaPerStage <= 63, "a group's loads in flight fit the wait counter");

  // resident activation: codes [M][n_stages * 256] (slot order as in the
  // ring), then scales [M][n_stages * 32]; 256-byte code segments and
  // 32-byte scale segments in row-major order, so one wave DMA moves four
  // code segments (1 KB) or eight scale segments (256 bytes)
  uint8_t* ares = lds + S * kStage;
  const int ares_code_pitch = n_stages * kStageCodes;
  const int ares_scale_base = decode_ares_code_bytes(M, n_stages);
  const int ares_scale_pitch = n_stages * kStageScales;
  if (kARes) {
    const int code_dmas = (M * n_stages + 3) / 4;      // 4 segments each
    for (int i = wave_all; i < code_dmas; i += kAllWaves) {
      const int seg = 4 * i + (lane >> 4);
      const int m = seg / n_stages < M ? seg / n_stages : M - 1;
      const int st = seg / n_stages < M ? seg % n_stages : n_stages - 1;
      const int chunk = r16 ^ (m & 15);
      dma16_lds(rac, ares + i * 1024,
                (uint32_t)(m * row_codes) + (uint32_t)st * kStageCodes + 16u * chunk);
    }
    const int scale_dmas = (M * n_stages + 7) / 8;     // 8 segments each
    for (int i = wave_all; i < scale_dmas; i += kAllWaves) {
      const int seg = 8 * i + (lane >> 3);
      const int m = seg / n_stages < M ? seg / n_stages : M - 1;
      const int st = seg / n_stages < M ? seg % n_stages : n_stages - 1;
      dma4_lds(ras, ares + ares_scale_base + i * 256,
               (uint32_t)(m * row_scales) + (uint32_t)st * kStageScales + 4u * (lane & 7));
    }
  }

  float4_t acc[kMaxTiles][MT];
#pragma unroll
  for (int tt = 0; tt < kMaxTiles; ++tt)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[tt][t] = float4_t{0.f, 0.f, 0.f, 0.f};
  bool a_ok[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) a_ok[t] = 16 * t + r16 < M;
  const int q = 4 * wave + (lane >> 4);                 // this lane's chunk of a stage
  const int rd_code = r16 * kStageCodes + ((q ^ r16) << 4);
  const int rd_scale = 16 * kStageCodes + r16 * kStageScales + 2 * q;
  // resident activation: this lane's token row (rows past M read row M - 1,
  // whose scales are zeroed)
  const int am = r16 < M ? r16 : M - 1;
  const int ares_code = am * ares_code_pitch + (((q ^ am) & 15) << 4);
  const int ares_scale = ares_scale_base + am * ares_scale_pitch + 2 * q;

  // the group's first kSG - 1 stages
#pragma unroll
  for (int j = 0; j < kSG - 1; ++j) issue(grp + kG * j);
  if (kARes) {
    // the resident activation is older than the group's first kSG - 1 stages
    __builtin_amdgcn_s_waitcnt(vm_wait((kSG - 1) * kDmaPerStage));
  }

  int g = grp;                                         // the group's next stage
#pragma unroll
  for (int tt = 0; tt < kMaxTiles; ++tt) {
    if (tt < my_tiles) {
      for (int st = grp; st < n_pad; st += kG, g += kG) {
        // this wave's loads of stage g are done when at most kSG - 2 of the
        // group's stages of loads are younger; the barrier makes every
        // wave's part visible and frees the slot of the group's stage
        // g - kG for the refill (a bare s_barrier: __syncthreads would also
        // wait for every load in flight; the stage's LDS reads cannot move
        // above it, since the refill loads, which write LDS, are issued
        // between the two)
        __builtin_amdgcn_s_waitcnt(vm_wait((kSG - 2) * kDmaPerStage));
        __builtin_amdgcn_s_barrier();
        issue(g + S - kG);
        const uint8_t* base = lds + (g % S) * kStage;
        // a padding stage (st >= n_stages) masks every A scale to zero
        const uint32_t mask = st * 16 + q < n_chunks ? 0xFFFFu : 0u;
        const int st_r = st < n_stages ? st : n_stages - 1;   // resident-activation stage
        const u32x4 bc = *reinterpret_cast<const u32x4*>(base + rd_code);
        const uint32_t bs = *reinterpret_cast<const uint16_t*>(base + rd_scale);
        u32x4 ac[MT];
        uint32_t as[MT];
        if (kARes) {
          ac[0] = *reinterpret_cast<const u32x4*>(ares + ares_code + st_r * kStageCodes);
          as[0] = *reinterpret_cast<const uint16_t*>(ares + ares_scale + st_r * kStageScales) &
                  (a_ok[0] ? mask : 0u);
        } else {
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const uint8_t* tl = base + (1 + t) * kTileBytes;
            ac[t] = *reinterpret_cast<const u32x4*>(tl + rd_code);
            as[t] = *reinterpret_cast<const uint16_t*>(tl + rd_scale) & (a_ok[t] ? mask : 0u);
          }
        }
        const uint32_t bw[4] = {bc.x, bc.y, bc.z, bc.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const half8_t bv = decode8(bw[s], scale_pair((bs >> (8 * (s >> 1))) & 0xFFu));
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const uint32_t aw = s == 0 ? ac[t].x : s == 1 ? ac[t].y : s == 2 ? ac[t].z : ac[t].w;
            const half8_t av = decode8(aw, scale_pair((as[t] >> (8 * (s >> 1))) & 0xFFu));
            acc[tt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc[tt][t], 0, 0, 0);
          }
        }
      }
    }
  }

  // every tile's four wave partials meet in LDS (the ring, once no load is
  // still writing it); D layout of the 16x16 MFMA: lane l holds rows
  // 4 (l / 16) + r, column l % 16
  __builtin_amdgcn_s_waitcnt(vm_wait(0));
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);          // [wave][t][16][17]
  const float alpha_x = *alpha_a;
  const int n = threadIdx.x & 15, mr = threadIdx.x >> 4;
#pragma unroll
  for (int tt = 0; tt < kMaxTiles; ++tt) {
    if (tt < my_tiles) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          red[((wave_all * MT + t) * 16 + 4 * (lane >> 4) + r) * 17 + r16] = acc[tt][t][r];
      __syncthreads();
      const int col = ((int)blockIdx.x + tt * (int)gridDim.x) * kCols + n;
      if (col < N && threadIdx.x < kThreads) {
        const float ab = alpha_b_rows != nullptr ? alpha_b_rows[col] : *alpha_b;
        const float scale = alpha_x * ab * 256.0f;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const int m = 16 * t + mr;
          if (m < M) {
            float v = red[((0 * MT + t) * 16 + mr) * 17 + n];
#pragma unroll
            for (int w = 1; w < kAllWaves; ++w) v += red[((w * MT + t) * 16 + mr) * 17 + n];
            v *= scale;
            if (y_f32 != nullptr) y_f32[m * ld_y + col] = v;
            if (y_bf16 != nullptr) y_bf16[m * ld_y + col] = (uint16_t)f32_to_bf16_bits(v);
          }
        }
      }
      __syncthreads();
    }
  }
}

// ---- one token row: a streamed matrix-vector product (K % 32 == 0) -------
// With one token row a 16 x 16 MFMA would use one of its 16 A rows, and
// staging K-slices of 16 weight rows breaks each row into 256-byte pieces.
// Here a wave takes whole weight rows, one at a time, its lanes across K:
// lane l owns the 32-element chunks c = l + 64 j (j < CH), reads the row's
// 16 code bytes and 2 scale bytes of each, and keeps the token's values of
// those chunks in registers, decoded once (q sigma 2^-4, exact in float16).
// A weight block (16 values) contributes sigma_w times an exact sum: the
// codes (exact float16) against the token values by two-term dot products
// accumulating in float32 (every product and partial sum is a multiple of
// sigma_a 2^-6 of at most 12 bits, so the sum is exact), then one multiply
// by sigma_w 2^-8 (the E4M3 byte as a float16, exact) into the lane's
// float32 sum.  The 64 lane sums of a row are added in a fixed DPP order
// (lane 63 ends with the total) and scaled by alpha_a alpha_b 2^12.  The
// row DEPTH rounds ahead is loaded while a row is reduced.
// The 8 FP4 codes of w as 4 float16 pairs, times 2^e (e = exponent of f).
struct Half2x4 {
  half2_t h[4];
};
__device__ __forceinline__ Half2x4 cvt8(uint32_t w, float f) {
  Half2x4 r;
  r.h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, f, 0);
  r.h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, f, 1);
  r.h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, f, 2);
  r.h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, f, 3);
  return r;
}

template <int CH, int DEPTH>
__global__ __launch_bounds__(kThreads) void w4a4_gemv_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ alpha_a, const uint8_t* __restrict__ b_codes,
    const uint8_t* __restrict__ b_scales, const float* __restrict__ alpha_b,
    const float* __restrict__ alpha_b_rows, int N, int K, float* __restrict__ y_f32,
    uint16_t* __restrict__ y_bf16) {
  const int lane = threadIdx.x & 63;
  const int nc = K / 32;                              // chunks a row
  const uint32_t row_codes = (uint32_t)(K / 2), row_scales = (uint32_t)(K / 16);
  const __amdgpu_buffer_rsrc_t rbc = buffer_of(b_codes, (uint32_t)N * row_codes);
  const __amdgpu_buffer_rsrc_t rbs = buffer_of(b_scales, (uint32_t)N * row_scales);

  // the token's values of this lane's chunks (zero past the row end)
  half2_t av[CH][16];
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = lane + 64 * j;
    const bool ok = c < nc;
    const u32x4 w = ok ? reinterpret_cast<const u32x4*>(a_codes)[c] : u32x4{0u, 0u, 0u, 0u};
    const uint32_t sb = ok ? (uint32_t)reinterpret_cast<const uint16_t*>(a_scales)[c] : 0u;
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const half2_t s = scale_pair((sb >> (8 * (q >> 1))) & 0xFFu);
      const Half2x4 v = cvt8(ww[q], 16.0f);
#pragma unroll
      for (int h = 0; h < 4; ++h) av[j][4 * q + h] = v.h[h] * s;
    }
  }

  struct RowData {
    u32x4 codes[CH];
    uint32_t scales[CH];
  };
  auto load_row = [&](int n, RowData& d) __attribute__((always_inline)) {
    const uint32_t rn = (uint32_t)(n < N ? n : N - 1);          // clamped: loads always valid
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = lane + 64 * j;
      const uint32_t cc = (uint32_t)(c < nc ? c : nc - 1);
      d.codes[j] = __builtin_amdgcn_raw_buffer_load_b128(rbc, rn * row_codes + 16u * cc, 0, 2);
      d.scales[j] = __builtin_amdgcn_raw_buffer_load_b16(rbs, rn * row_scales + 2u * cc, 0, 0);
    }
  };
  const int wstride = (int)gridDim.x * kWaves;
  const int n0 = (int)blockIdx.x * kWaves + (threadIdx.x >> 6);
  RowData ring[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) load_row(n0 + d * wstride, ring[d]);
  const float scale_a = (*alpha_a) * 4096.0f;

  for (int n = n0; n < N; n += DEPTH * wstride) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int nd = n + d * wstride;
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int c = lane + 64 * j;
        const uint32_t ww[4] = {ring[d].codes[j].x, ring[d].codes[j].y, ring[d].codes[j].z,
                                ring[d].codes[j].w};
#pragma unroll
        for (int b = 0; b < 2; ++b) {                  // the chunk's two blocks
          float p = 0.0f;
#pragma unroll
          for (int q = 2 * b; q < 2 * b + 2; ++q) {
            const Half2x4 wq = cvt8(ww[q], 1.0f);
#pragma unroll
            for (int h = 0; h < 4; ++h) p = __builtin_amdgcn_fdot2(wq.h[h], av[j][4 * q + h], p, false);
          }
          // sigma_w 2^-8: the E4M3 byte's fields in a float16's (a zero
          // byte past the row end)
          const uint32_t sb = c < nc ? (ring[d].scales[j] >> (8 * b)) & 0xFFu : 0u;
          const float sw = (float)__builtin_bit_cast(_Float16, (uint16_t)(sb << 7));
          acc = __builtin_fmaf(p, sw, acc);
        }
      }
      // refill the slot with the row DEPTH rounds ahead
      load_row(nd + DEPTH * wstride, ring[d]);
      // lane 63 ends with the sum of the 64 lanes (gfx9 DPP reduction)
      acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc), 0xB1, 0xF, 0xF, false));
      acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc), 0x4E, 0xF, 0xF, false));
      acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc), 0x141, 0xF, 0xF, false));
      acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc), 0x140, 0xF, 0xF, false));
      acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc), 0x142, 0xA, 0xF, false));
      acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc), 0x143, 0xC, 0xF, false));
      if (lane == 63 && nd < N) {
        const float ab = alpha_b_rows != nullptr ? alpha_b_rows[nd] : *alpha_b;
        const float v = acc * (scale_a * ab);
        if (y_f32 != nullptr) y_f32[nd] = v;
        if (y_bf16 != nullptr) y_bf16[nd] = (uint16_t)f32_to_bf16_bits(v);
      }
    }
  }
}

// The same product for long rows (8192 < K <= 32768) with the token in
// registers: the four waves of a workgroup split each row's chunks into four
// contiguous parts (wave w the w-th, up to 64 CH chunks), and each wave keeps
// the token's values of its part decoded in registers, as w4a4_gemv_kernel
// does for a whole row.  A workgroup walks rows b, b + gridDim.x, ...; each
// wave sums its part of a row as w4a4_gemv_kernel sums a row (exact block
// sums times sigma_w, a fixed-order DPP reduction) and leaves the partial
// in LDS; after every kSplitRows rows (and the last) one barrier, then the
// four partials of each row are added in a fixed order (part 0 + 1 + 2 + 3)
// and scaled.  The partials alternate between two LDS buffers, so one
// barrier a batch suffices.
constexpr int kSplitRows = 8;
constexpr int kGemvSplitMaxK = 4 * 64 * 32 * 4;     // 32768
template <int CH>
__global__ __launch_bounds__(kThreads) void w4a4_gemv_split_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ alpha_a, const uint8_t* __restrict__ b_codes,
    const uint8_t* __restrict__ b_scales, const float* __restrict__ alpha_b,
    const float* __restrict__ alpha_b_rows, int N, int K, float* __restrict__ y_f32,
    uint16_t* __restrict__ y_bf16) {
  __shared__ float part[2][kSplitRows][kWaves];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nc = K / 32;                              // chunks a row
  const int per = (nc + kWaves - 1) / kWaves;         // chunks a part (<= 64 CH)
  const int c0 = wave * per;
  const int c_end = c0 + per < nc ? c0 + per : nc;    // c0 < c_end: nc >= 4
  const uint32_t row_codes = (uint32_t)(K / 2), row_scales = (uint32_t)(K / 16);
  const __amdgpu_buffer_rsrc_t rbc = buffer_of(b_codes, (uint32_t)N * row_codes);
  const __amdgpu_buffer_rsrc_t rbs = buffer_of(b_scales, (uint32_t)N * row_scales);

  // the token's values of this lane's chunks of the part (zero past its end)
  half2_t av[CH][16];
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = c0 + lane + 64 * j;
    const bool ok = c < c_end;
    const u32x4 w = ok ? reinterpret_cast<const u32x4*>(a_codes)[c] : u32x4{0u, 0u, 0u, 0u};
    const uint32_t sb = ok ? (uint32_t)reinterpret_cast<const uint16_t*>(a_scales)[c] : 0u;
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const half2_t s = scale_pair((sb >> (8 * (q >> 1))) & 0xFFu);
      const Half2x4 v = cvt8(ww[q], 16.0f);
#pragma unroll
      for (int h = 0; h < 4; ++h) av[j][4 * q + h] = v.h[h] * s;
    }
  }

  struct RowData {
    u32x4 codes[CH];
    uint32_t scales[CH];
  };
  auto load_row = [&](int n, RowData& d) __attribute__((always_inline)) {
    const uint32_t rn = (uint32_t)(n < N ? n : N - 1);          // clamped: loads always valid
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = c0 + lane + 64 * j;
      const uint32_t cc = (uint32_t)(c < c_end ? c : c_end - 1);
      d.codes[j] = __builtin_amdgcn_raw_buffer_load_b128(rbc, rn * row_codes + 16u * cc, 0, 2);
      d.scales[j] = __builtin_amdgcn_raw_buffer_load_b16(rbs, rn * row_scales + 2u * cc, 0, 0);
    }
  };
  const int step = (int)gridDim.x;
  const int n0 = (int)blockIdx.x;
  const int rows = n0 < N ? (N - n0 + step - 1) / step : 0;     // rows of this workgroup
  RowData cur;
  load_row(n0, cur);
  const float scale_a = (*alpha_a) * 4096.0f;
  for (int t = 0; t < rows; ++t) {
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = c0 + lane + 64 * j;
      const uint32_t ww[4] = {cur.codes[j].x, cur.codes[j].y, cur.codes[j].z, cur.codes[j].w};
#pragma unroll
      for (int b = 0; b < 2; ++b) {                    // the chunk's two blocks
        float p = 0.0f;
#pragma unroll
        for (int q = 2 * b; q < 2 * b + 2; ++q) {
          const Half2x4 wq = cvt8(ww[q], 1.0f);
#pragma unroll
          for (int h = 0; h < 4; ++h) p = __builtin_amdgcn_fdot2(wq.h[h], av[j][4 * q + h], p, false);
        }
        const uint32_t sb = c < c_end ? (cur.scales[j] >> (8 * b)) & 0xFFu : 0u;
        const float sw = (float)__builtin_bit_cast(_Float16, (uint16_t)(sb << 7));
        acc = __builtin_fmaf(p, sw, acc);
      }
    }
    // the next row's loads while this row is reduced
    load_row(n0 + (t + 1) * step, cur);
    acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc), 0xB1, 0xF, 0xF, false));
    acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc), 0x4E, 0xF, 0xF, false));
    acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc), 0x141, 0xF, 0xF, false));
    acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc), 0x140, 0xF, 0xF, false));
    acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc), 0x142, 0xA, 0xF, false));
    acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc), 0x143, 0xC, 0xF, false));
    const int slot = t % kSplitRows, buf = (t / kSplitRows) & 1;
    if (lane == 63) part[buf][slot][wave] = acc;
    if (slot == kSplitRows - 1 || t == rows - 1) {
      __syncthreads();
      if (wave == 0 && lane <= slot) {
        const int n = n0 + (t - slot + lane) * step;
        const float* q = part[buf][lane];
        const float v = (((q[0] + q[1]) + q[2]) + q[3]) *
                        (scale_a * (alpha_b_rows != nullptr ? alpha_b_rows[n] : *alpha_b));
        if (y_f32 != nullptr) y_f32[n] = v;
        if (y_bf16 != nullptr) y_bf16[n] = (uint16_t)f32_to_bf16_bits(v);
      }
    }
  }
}

int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  (void)hipGetDevice(&dev);
  int c = cached[dev & 63].load(std::memory_order_relaxed);
  if (c <= 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        c < 1)
      c = 256;
    cached[dev & 63].store(c, std::memory_order_relaxed);
  }
  return c;
}

// Launches the LDS-staged kernel with the ring (and resident activation)
// in dynamic LDS, on as many workgroups as fit at once (at most one per
// column tile, and enough that none takes more than kMaxTiles tiles).
template <int MT, int S, bool kARes, int kG>
hipError_t launch_lds(const DecodeArgs& p, int lds_bytes, hipStream_t stream) {
  // per device: the LDS size the attribute was set for, and the workgroups
  // that fit (host threads may race here: wgs is published before bytes)
  static std::atomic<int> cache_bytes[64], cache_wgs[64];
  const auto kernel = w4a4_decode_lds_kernel<MT, S, kARes, kG>;
  int dev = 0;
  (void)hipGetDevice(&dev);
  const int slot = dev & 63;
  int fit;
  if (cache_bytes[slot].load(std::memory_order_acquire) != lds_bytes) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes) != hipSuccess)
      return hipErrorInvalidValue;
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kThreads * kG, lds_bytes) !=
            hipSuccess ||
        occ < 1)
      occ = 1;
    fit = occ * device_cus();
    cache_wgs[slot].store(fit, std::memory_order_relaxed);
    cache_bytes[slot].store(lds_bytes, std::memory_order_release);
  } else {
    fit = cache_wgs[slot].load(std::memory_order_relaxed);
  }
  const int tiles = (int)((p.N + kCols - 1) / kCols);
  int wgs = tiles < fit ? tiles : fit;
  const int need = (tiles + kMaxTiles - 1) / kMaxTiles;
  if (wgs < need) wgs = need;
  hipLaunchKernelGGL(kernel, dim3((unsigned)wgs), dim3(kThreads * kG), lds_bytes, stream,
                     p.a_codes, p.a_scales, p.alpha_a, p.b_codes, p.b_scales, p.alpha_b,
                     p.alpha_b_rows, (int)p.M, (int)p.N, (int)p.K, p.y_f32, p.y_bf16, p.ld_y);
  return hipGetLastError();
}

// One M-tile: kG stage groups a workgroup when the weight has too few column
// tiles to give every CU several workgroups (4 groups up to one tile a CU,
// 2 up to two), else one.
template <bool kARes>
hipError_t launch_one_mtile(const DecodeArgs& p, int n_stages, hipStream_t stream) {
  const int tiles = (int)((p.N + kCols - 1) / kCols);
  const int cus = device_cus();
  const int kg = tiles <= cus ? 4 : tiles <= 2 * cus ? 2 : 1;
  // ring stages: 4 a group with the resident activation, else 6 (one group)
  // or 4 a group (several; 16 stages fill most of the LDS)
  const int ares = kARes ? decode_ares_bytes((int)p.M, n_stages) : 0;
  constexpr int kStage = decode_stage_bytes(1, kARes);
  if (kARes) {
    if (kg == 4) return launch_lds<1, 16, true, 4>(p, 16 * kStage + ares, stream);
    if (kg == 2) return launch_lds<1, 8, true, 2>(p, 8 * kStage + ares, stream);
    return launch_lds<1, 4, true, 1>(p, 4 * kStage + ares, stream);
  }
  if (kg == 4) return launch_lds<1, 16, false, 4>(p, 16 * kStage, stream);
  if (kg == 2) return launch_lds<1, 8, false, 2>(p, 8 * kStage, stream);
  return launch_lds<1, 6, false, 1>(p, 6 * kStage, stream);
}

template <int CH>
hipError_t launch_gemv(const DecodeArgs& p, hipStream_t stream) {
  // one row in flight a wave and four rows a wave (measured best at
  // 24576 x 4096 and 51200 x 5120 against 2-8 rows in flight and 2-16 rows
  // a wave: fewer registers, more waves), at most 8 workgroups a CU; weights
  // of up to 8192 rows take two rows a wave, so that enough waves have rows
  // in flight (5120 x 5120: 6.9 -> 6.1 us, 6144 x 4096: 6.7 -> 5.8 us;
  // one row a wave overran the resident workgroups at 7168 rows)
  constexpr int kDepth = 1;
  const int64_t rows_per_wave = p.N <= 8192 ? 2 : 4;
  const int64_t waves = (p.N + rows_per_wave - 1) / rows_per_wave;
  int64_t wgs = (waves + kWaves - 1) / kWaves;
  const int64_t cap = (int64_t)device_cus() * 8;
  if (wgs > cap) wgs = cap;
  hipLaunchKernelGGL((w4a4_gemv_kernel<CH, kDepth>), dim3((unsigned)wgs), dim3(kThreads), 0, stream,
                     p.a_codes, p.a_scales, p.alpha_a, p.b_codes, p.b_scales, p.alpha_b,
                     p.alpha_b_rows, (int)p.N, (int)p.K, p.y_f32, p.y_bf16);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_mt(const DecodeArgs& p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.N + kCols - 1) / kCols));
  // ring depths (stages) measured best at these LDS footprints
  constexpr int kS = MT == 2 ? 5 : 3;
  if (p.K % 64 == 0 && (path_flags() & kPathDecodeDirect) == 0) {
    const int n_stages = (int)((p.K / 2 + kStageCodes - 1) / kStageCodes);
    if constexpr (MT == 1) {
      const int64_t ares_bytes = (p.M * n_stages + 7) / 8 * 8 * (int64_t)(kStageCodes + kStageScales);
      const int64_t tiles = (p.N + kCols - 1) / kCols;
      if (ares_bytes <= kAResMaxBytes ||
          (ares_bytes <= kAResWideMaxBytes && tiles > 2 * (int64_t)device_cus()))
        return launch_one_mtile<true>(p, n_stages, stream);
      return launch_one_mtile<false>(p, n_stages, stream);
    } else {
      return launch_lds<MT, kS, false, 1>(p, kS * decode_stage_bytes(MT, false), stream);
    }
  } else if (p.K % 32 == 0)
    hipLaunchKernelGGL((w4a4_decode_kernel<MT, true>), grid, dim3(kThreads), 0, stream,
                       p.a_codes, p.a_scales, p.alpha_a, p.b_codes, p.b_scales, p.alpha_b,
                       p.alpha_b_rows, (int)p.M, (int)p.N, (int)p.K, p.y_f32, p.y_bf16, p.ld_y);
  else
    hipLaunchKernelGGL((w4a4_decode_kernel<MT, false>), grid, dim3(kThreads), 0, stream,
                       p.a_codes, p.a_scales, p.alpha_a, p.b_codes, p.b_scales, p.alpha_b,
                       p.alpha_b_rows, (int)p.M, (int)p.N, (int)p.K, p.y_f32, p.y_bf16, p.ld_y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w4a4_decode(const DecodeArgs& p, hipStream_t stream) {
  // one token row, whole 32-element chunks: whole weight rows a wave
  // (written to column n of row 0; ld_y unused), the token's values in
  // registers (at most 4 chunks a lane) or in LDS
  if (p.M == 1 && p.K % 32 == 0 && p.K <= 64 * 32 * 4 && (path_flags() & kPathDecodeDirect) == 0) {
    const int64_t ch = (p.K / 32 + 63) / 64;
    if (ch <= 1) return launch_gemv<1>(p, stream);
    if (ch <= 2) return launch_gemv<2>(p, stream);
    if (ch <= 3) return launch_gemv<3>(p, stream);
    return launch_gemv<4>(p, stream);
  }
  if (p.M == 1 && p.K % 32 == 0 && p.K <= kGemvSplitMaxK && (path_flags() & kPathDecodeDirect) == 0) {
    // four parts of at most 4 chunks a lane each; every workgroup resident
    // (measured 21.8 -> 17.3 us at 5120 x 25600 and 10.5 -> 8.1 us at
    // 4096 x 12288 against the token held in LDS; for rows up to 8192 the
    // whole-row kernel above stays faster: 24576 x 4096 12.7 against 17.2 us)
    const int64_t ch = (p.K / 32 + 4 * 64 - 1) / (4 * 64);
    auto go = [&](auto kernel) {
      static std::atomic<int> fit_cache[64];
      int dev = 0;
      (void)hipGetDevice(&dev);
      int fit = fit_cache[dev & 63].load(std::memory_order_relaxed);
      if (fit == 0) {
        int occ = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kThreads, 0) != hipSuccess ||
            occ < 1)
          occ = 1;
        fit = occ * device_cus();
        fit_cache[dev & 63].store(fit, std::memory_order_relaxed);
      }
      const int64_t wgs = p.N < fit ? p.N : fit;
      hipLaunchKernelGGL(kernel, dim3((unsigned)wgs), dim3(kThreads), 0, stream, p.a_codes,
                         p.a_scales, p.alpha_a, p.b_codes, p.b_scales, p.alpha_b, p.alpha_b_rows,
                         (int)p.N, (int)p.K, p.y_f32, p.y_bf16);
      return hipGetLastError();
    };
    if (ch <= 2) return go(w4a4_gemv_split_kernel<2>);
    if (ch <= 3) return go(w4a4_gemv_split_kernel<3>);
    return go(w4a4_gemv_split_kernel<4>);
  }
  if (p.M <= 16) return launch_mt<1>(p, stream);
  if (p.M <= 32) return launch_mt<2>(p, stream);
  return launch_mt<4>(p, stream);
}

}  // namespace nvfp4
