// BF16 comparison GEMM for gfx950: Y = X . W^T with BF16 operands and float32
// accumulation.  The pages measure NVFP4 prefill against a BF16 baseline
// ("Mix-Quant：面向智能体LLM的量化预填充与精确解码", paper.rainbus.top
// digest, 实验结果 (3), Figure 4); this kernel is a plain BF16 GEMM for the
// same layer shapes: 256-thread workgroups of 2 x 2 waves and 32x32x16 MFMAs
// like the W4A4 kernel, but global -> registers -> LDS double buffering with a
// full barrier a stage, none of the W4A4 kernel's LDS DMA ring, swizzle or
// banded epilogue.  It runs well below hipBLASLt, which is the BF16 figure the
// W4A4 layer is compared with.  Each stage covers BK K-elements: lanes 0-31 of a fragment
// read K-elements [0, BK/2) of the stage and lanes 32-63 read [BK/2, BK),
// eight per MFMA step.
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;

template <int BM>
__device__ __forceinline__ bool bf16_tile_coord(int tile_m, const int64_t* offsets,
                                                int num_groups, int64_t M,
                                                int64_t& m0, int64_t& m_end,
                                                int& group) {
  if (offsets == nullptr) {
    group = 0;
    m0 = (int64_t)tile_m * BM;
    m_end = M;
    return m0 < M;
  }
  int64_t before = 0;
  for (int g = 0; g < num_groups; ++g) {
    int64_t lo = offsets[g], hi = offsets[g + 1];
    int64_t nt = (hi - lo + BM - 1) / BM;
    if (tile_m < before + nt) {
      group = g;
      m0 = lo + (tile_m - before) * BM;
      m_end = hi;
      return true;
    }
    before += nt;
  }
  return false;
}

// BK K-elements a stage; rows of 2*BK bytes padded by 16 in LDS.
template <int BM, int BN, int BK>
__global__ __launch_bounds__(kThreads, 1) void bf16_gemm_kernel(Bf16Args p) {
  constexpr int kBK = BK;
  constexpr int kPitch = 2 * BK + 16;
  constexpr int kChunks = BK / 8;              // 16-byte chunks a row
  constexpr int kSteps = BK / 16;              // MFMA steps a stage
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int kStageBytes = (BM + BN) * kPitch;
  __shared__ __align__(16) uint8_t lds[2 * kStageBytes];

  int64_t m0, m_end;
  int group;
  if (!bf16_tile_coord<BM>(blockIdx.x, p.group_offsets, p.num_groups, p.M, m0, m_end, group))
    return;
  const int64_t n0 = (int64_t)blockIdx.y * BN;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;
  const int64_t K = p.K;
  const uint16_t* w = p.w + (int64_t)group * p.N * K;

  // loader: 16-byte chunk c = tid % kChunks (8 elements) of row
  // i * (256 / kChunks) + tid / kChunks
  constexpr int kRowsPer = kThreads / kChunks;
  constexpr int kAIters = BM / kRowsPer, kBIters = BN / kRowsPer;
  const int chunk = tid % kChunks;
  const uint16_t* a_ptr[kAIters];
  const uint16_t* b_ptr[kBIters];
#pragma unroll
  for (int i = 0; i < kAIters; ++i) {
    int64_t r = m0 + i * kRowsPer + tid / kChunks;
    r = r < m_end ? r : m_end - 1;
    a_ptr[i] = p.x + r * K + chunk * 8;
  }
#pragma unroll
  for (int i = 0; i < kBIters; ++i) {
    int64_t r = n0 + i * kRowsPer + tid / kChunks;
    r = r < p.N ? r : p.N - 1;
    b_ptr[i] = w + r * K + chunk * 8;
  }
  u32x4 ra[kAIters], rb[kBIters];

  auto load_stage = [&](int kt) __attribute__((always_inline)) {
    const int64_t k0 = (int64_t)kt * kBK;
    const bool ok = k0 + chunk * 8 < K;
#pragma unroll
    for (int i = 0; i < kAIters; ++i)
      ra[i] = ok ? *reinterpret_cast<const u32x4*>(a_ptr[i] + k0) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kBIters; ++i)
      rb[i] = ok ? *reinterpret_cast<const u32x4*>(b_ptr[i] + k0) : u32x4{0u, 0u, 0u, 0u};
  };
  auto store_stage = [&](int buf) __attribute__((always_inline)) {
    uint8_t* a_lds = lds + buf * kStageBytes;
    uint8_t* b_lds = a_lds + BM * kPitch;
#pragma unroll
    for (int i = 0; i < kAIters; ++i)
      *reinterpret_cast<u32x4*>(a_lds + (i * kRowsPer + tid / kChunks) * kPitch + chunk * 16) = ra[i];
#pragma unroll
    for (int i = 0; i < kBIters; ++i)
      *reinterpret_cast<u32x4*>(b_lds + (i * kRowsPer + tid / kChunks) * kPitch + chunk * 16) = rb[i];
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
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_stage(kt + 1);
    const uint8_t* a_lds = lds + buf * kStageBytes;
    const uint8_t* b_lds = a_lds + BM * kPitch;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      bf16x8_t af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(a_lds + (wm + i * 32 + fr) * kPitch + fh * (BK) + s * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bf[j] = *reinterpret_cast<const bf16x8_t*>(b_lds + (wn + j * 32 + fr) * kPitch + fh * (BK) + s * 16);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_stage(buf ^ 1);
    __syncthreads();
  }

  const int64_t row_lim = m0 + BM < m_end ? m0 + BM : m_end;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = n0 + wn + j * 32 + fr;
      if (col >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm + i * 32 + 8 * (r >> 2) + 4 * fh + (r & 3);
        if (row < row_lim) {
          const float v = acc[i][j][r];
          if (p.y_f32) p.y_f32[row * p.ld_y + col] = v;
          if (p.y_bf16) p.y_bf16[row * p.ld_y + col] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
    }
  }
}

template <int BM, int BN, int BK>
hipError_t launch_bf16_tiles(const Bf16Args& a, hipStream_t stream) {
  int tiles_m = (int)((a.M + BM - 1) / BM);
  if (a.group_offsets != nullptr) tiles_m += a.num_groups;
  const int tiles_n = (int)((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((bf16_gemm_kernel<BM, BN, BK>), dim3(tiles_m, tiles_n), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bf16(const Bf16Args& a, hipStream_t stream) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  const int64_t big = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  if (big >= 256) return launch_bf16_tiles<256, 256, 32>(a, stream);
  return launch_bf16_tiles<128, 128, 64>(a, stream);
}

}  // namespace nvfp4
