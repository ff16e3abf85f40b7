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

// Per E4M3 scale byte sb, where its blocks find their codes in the code
// table: the row of its mantissa class starts at lo = 1024 k and an
// element's index is its magnitude bits plus code_off + delta, delta = lo -
// 128 e (sigma = (1 + k/8) 2^e).  Both as 16-bit pairs, for packed
// arithmetic on two elements at once.  Byte 0 (sigma = 0) sends every index
// below the table, i.e. to code 0.
struct RowDesc {
  uint32_t lo2;      // lo in both halves
  uint32_t delta2;   // delta in both halves (int16)
};

__device__ __forceinline__ RowDesc row_desc(uint32_t sb) {
  RowDesc d;
  if (sb == 0) {
    d.lo2 = 0;
    d.delta2 = 0x80008000u;                 // -32768: saturates below lo
  } else {
    int e, k;
    scale_class(sb, e, k);
    const int lo = k * kCodeLutRow;
    const int delta = lo - 128 * e;
    d.lo2 = (uint32_t)lo * 0x10001u;
    d.delta2 = ((uint32_t)delta & 0xFFFFu) * 0x10001u;
  }
  return d;
}

// Signs of the 8 BF16 values of w[4] at bit 3 of their code nibbles.
__device__ __forceinline__ uint32_t sign_nibbles(const uint32_t (&w)[4]) {
  // bytes 1 and 3 of each word hold the signs (bit 7) of its two values
  const uint32_t a = __builtin_amdgcn_perm(w[1], w[0], 0x07050301u);   // e0 e1 e2 e3
  const uint32_t b = __builtin_amdgcn_perm(w[3], w[2], 0x07050301u);   // e4 e5 e6 e7
  const uint32_t even = __builtin_amdgcn_perm(b, a, 0x06040200u);      // e0 e2 e4 e6
  const uint32_t odd = __builtin_amdgcn_perm(b, a, 0x07050301u);       // e1 e3 e5 e7
  return ((even >> 4) & 0x08080808u) | (odd & 0x80808080u);
}

typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2v __attribute__((ext_vector_type(2)));

// The tables of the fast path (alpha's exponent within +-100) in LDS, and
// the offsets of QuantParams in the form it uses.
struct FastTables {
  const uint8_t* sig;
  const uint8_t* code;
  const RowDesc* desc;
  int sig_off;
  uint32_t code_off2;   // code_off in both halves (int16)
};

// The LDS of a workgroup's tables (kThreads = 256 threads copy them).
struct TableLds {
  __align__(16) uint8_t sig[kSigLutN];
  __align__(16) uint8_t code[kCodeLutN];
  RowDesc desc[128];
};

// Copies the tables of the workspace into LDS with every thread of a
// 256-thread workgroup (one or two 16-byte pieces each) and fills the row
// descriptors.  The loads are issued before first() (which issues the
// workgroup's first data loads): loads return in order, so the copy can
// proceed while the data is still in flight.  The caller synchronises.
template <typename First>
__device__ __forceinline__ void copy_tables_first(const uint8_t* ws, TableLds& t, int tid,
                                                  First first) {
  static_assert(kSigLutN / 16 <= 256 && kCodeLutN / 16 == 512, "table copy shape");
  const u32x4* sig = reinterpret_cast<const u32x4*>(ws + kWsSigLut);
  const u32x4* code = reinterpret_cast<const u32x4*>(ws + kWsCodeLut);
  const u32x4 t0 = tid < kSigLutN / 16 ? sig[tid] : u32x4{0u, 0u, 0u, 0u};
  const u32x4 t1 = code[tid], t2 = code[tid + 256];
  first();
  if (tid < kSigLutN / 16) reinterpret_cast<u32x4*>(t.sig)[tid] = t0;
  reinterpret_cast<u32x4*>(t.code)[tid] = t1;
  reinterpret_cast<u32x4*>(t.code)[tid + 256] = t2;
  if (tid < 128) t.desc[tid] = row_desc(tid);
}

__device__ __forceinline__ FastTables fast_tables(const TableLds& t, const QuantParams& P) {
  FastTables f;
  f.sig = t.sig;
  f.code = t.code;
  f.desc = t.desc;
  f.sig_off = P.sig_off;
  f.code_off2 = ((uint32_t)P.code_off & 0xFFFFu) * 0x10001u;
  return f;
}

// Codes of the 8 BF16 values w[4] (half a block; the other half is in lane
// l ^ 1, which must run this too) and the block's scale byte: the fast-path
// equivalent of magnitudes + block_scale + codes8.  Magnitudes, indices and
// clamps are formed two values at a time in 16-bit halves (the sum
// saturates; off and lo fit 16 bits when alpha's exponent is within +-100).
__device__ __forceinline__ uint32_t quantize_half_block(const uint32_t (&w)[4], const FastTables& t,
                                                        uint32_t& scale_byte) {
  uint32_t mw[4];                          // magnitudes, two a word
#pragma unroll
  for (int i = 0; i < 4; ++i) mw[i] = w[i] & 0x7FFF7FFFu;
  const u16x2v mx = __builtin_elementwise_max(
      __builtin_elementwise_max(__builtin_bit_cast(u16x2v, mw[0]), __builtin_bit_cast(u16x2v, mw[1])),
      __builtin_elementwise_max(__builtin_bit_cast(u16x2v, mw[2]), __builtin_bit_cast(u16x2v, mw[3])));
  uint32_t amax = max((uint32_t)mx.x, (uint32_t)mx.y);
  amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0xB1, 0xF, 0xF, false));
  const int sidx = min(max((int)amax + t.sig_off, 0), kSigLutN - 1);
  const uint32_t sb = t.sig[sidx];
  const RowDesc d = t.desc[sb];
  // index = clamp(magnitude + off, lo, lo + 1023)
  const i16x2 off2 = __builtin_elementwise_add_sat(__builtin_bit_cast(i16x2, t.code_off2),
                                                   __builtin_bit_cast(i16x2, d.delta2));
  const i16x2 lo2 = __builtin_bit_cast(i16x2, d.lo2);
  const i16x2 hi2 = lo2 + (i16x2){(short)(kCodeLutRow - 1), (short)(kCodeLutRow - 1)};
  uint32_t o = sign_nibbles(w);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    i16x2 idx = __builtin_elementwise_add_sat(__builtin_bit_cast(i16x2, mw[i]), off2);
    idx = __builtin_elementwise_min(__builtin_elementwise_max(idx, lo2), hi2);
    const uint32_t p = __builtin_bit_cast(uint32_t, idx);
    const uint32_t c_lo = t.code[p & 0xFFFFu];
    const uint32_t c_hi = t.code[p >> 16];
    o |= (c_lo << (8 * i)) | (c_hi << (8 * i + 4));
  }
  scale_byte = sb;
  return o;
}

}  // namespace nvfp4
