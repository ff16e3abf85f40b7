// Quantisation of one 16-element NVFP4 block with the exact decision tables
// built by the prepare kernel (see quantize.hip).  Used by the streaming
// quantiser and by the GEMM that quantises its activation tile on load, so
// both produce the same bytes.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

// Tables (in LDS) and offsets for one tensor scale alpha.
struct BlockTables {
  const uint8_t* sig;    // kSigLutN entries
  const uint8_t* code;   // kCodeLutN entries
  int sig_off;
  int code_off;
  int shift;
  int slow;
};

// Exponent e and mantissa class k (sigma = (1 + k/8) 2^e) of a nonzero
// E4M3FN byte.
__device__ __forceinline__ void scale_class(uint32_t sb, int& e, int& k) {
  if (sb >= 8) {
    e = (int)(sb >> 3) - 7;
    k = (int)(sb & 7);
  } else {                                  // subnormal m 2^-9, m = 1..7
    int p = 31 - __clz((int)sb);            // floor(log2 m)
    e = p - 9;
    k = (int)((sb << (3 - p)) & 7);
  }
}

// Magnitude bits (BF16 without the sign) of the 2n values packed in w[n]
// (element 2i in the low half of w[i]); on the slow path (alpha's exponent
// beyond +-100) the magnitudes are first multiplied by 2^shift.
template <int n>
__device__ __forceinline__ void magnitudes(const uint32_t* w, const BlockTables& t,
                                           uint32_t* mag) {
#pragma unroll
  for (int i = 0; i < n; ++i) {
    mag[2 * i] = w[i] & 0x7FFFu;
    mag[2 * i + 1] = (w[i] >> 16) & 0x7FFFu;
  }
  if (t.slow) {
#pragma unroll
    for (int i = 0; i < 2 * n; ++i) {
      float f = ldexpf(bf16_bits_to_f32(mag[i]), t.shift);
      mag[i] = __float_as_uint(f) >> 16;    // inf -> 0x7F80: clamps high
    }
  }
}

// Where a block's codes are found in the code table: the row of the scale's
// mantissa class [lo, hi] and the offset added to an element's bits.
struct CodeRow {
  int lo, hi, off;
};

// Scale byte of a block whose largest magnitude has bits amax.
__device__ __forceinline__ uint32_t block_scale(uint32_t amax, const BlockTables& t,
                                                CodeRow& row) {
  const int sidx = min(max((int)amax + t.sig_off, 0), kSigLutN - 1);
  const uint32_t sb = t.sig[sidx];
  row.lo = row.hi = row.off = 0;            // sigma = 0: every index hits entry 0 (code 0)
  if (sb != 0) {
    int e, k;
    scale_class(sb, e, k);
    row.lo = k * kCodeLutRow;
    row.hi = row.lo + kCodeLutRow - 1;
    row.off = t.code_off + row.lo - 128 * e;
  }
  return sb;
}

// Codes of 8 consecutive elements (magnitudes mag[8], packed values w[4]):
// element i in nibble i, sign bit in bit 3 of the nibble.
__device__ __forceinline__ uint32_t codes8(const uint32_t* mag, const uint32_t* w,
                                           const CodeRow& row, const BlockTables& t) {
  uint32_t o = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = min(max((int)mag[i] + row.off, row.lo), row.hi);
    uint32_t c = t.code[idx];
    c |= (w[i >> 1] >> ((i & 1) ? 28 : 12)) & 8u;    // sign bit -> bit 3
    o |= c << (4 * i);
  }
  return o;
}

// w[8]: the 16 BF16 values of the block, two per word (element 2i in the low
// half of w[i]).  Produces the 8 code bytes (out0: elements 0-7, out1: 8-15,
// element 2j in the low nibble of byte j) and the scale byte.
__device__ __forceinline__ void quantize16(const uint32_t w[8], const BlockTables& t,
                                           uint32_t& out0, uint32_t& out1,
                                           uint32_t& scale_byte) {
  uint32_t mag[16];
  magnitudes<8>(w, t, mag);
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = max(amax, mag[i]);
  CodeRow row;
  scale_byte = block_scale(amax, t, row);
  out0 = codes8(mag, w, row, t);
  out1 = codes8(mag + 8, w + 4, row, t);
}

// Copies the two tables from the workspace into LDS (all threads of the
// workgroup take part; the caller synchronises before use).
__device__ __forceinline__ void load_tables_to_lds(const uint8_t* ws, uint8_t* lds_sig,
                                                   uint8_t* lds_code, int tid, int nthreads) {
  const u32x4* src = reinterpret_cast<const u32x4*>(ws + kWsSigLut);
  u32x4* dst = reinterpret_cast<u32x4*>(lds_sig);
  for (int i = tid; i < kSigLutN / 16; i += nthreads) dst[i] = src[i];
  src = reinterpret_cast<const u32x4*>(ws + kWsCodeLut);
  dst = reinterpret_cast<u32x4*>(lds_code);
  for (int i = tid; i < kCodeLutN / 16; i += nthreads) dst[i] = src[i];
}

__device__ __forceinline__ BlockTables tables_from(const uint8_t* ws, const uint8_t* lds_sig,
                                                   const uint8_t* lds_code) {
  const QuantParams P = *reinterpret_cast<const QuantParams*>(ws + kWsParams);
  BlockTables t;
  t.sig = lds_sig;
  t.code = lds_code;
  t.sig_off = P.sig_off;
  t.code_off = P.code_off;
  t.shift = P.shift;
  t.slow = P.slow;
  return t;
}

}  // namespace nvfp4
