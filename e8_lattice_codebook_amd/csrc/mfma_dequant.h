// Codeword fragments for fp16 MFMA operands: the eight signed 4-bit lanes 2c of a
// slot word (or its complement) as exact fp16 values, and the byte addresses of the
// fp16 residual table.  Shared by the prefill kernels.
#pragma once
#include "lds_codebook.h"

namespace glq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// fp16 (2c_0 .. 2c_7) of a slot word w, negated (complement) when m = ~0
__device__ __forceinline__ half8 word_to_half8(uint32_t w, uint32_t m) {
  const uint32_t t = w ^ m ^ 0x88888888u;                   // nibble = lane + 8, or 7 - lane
  const uint32_t nb = 0xE408E408u ^ (m & 0x000F000Fu);      // -(1024 + 8), or -(1024 + 7)
  const half2v bias = __builtin_bit_cast(half2v, nb);
  half2v p[4];
  p[0] = __builtin_bit_cast(half2v, (t & 0x000F000Fu) | 0x64006400u) + bias;
  p[1] = __builtin_bit_cast(half2v, ((t >> 4) & 0x000F000Fu) | 0x64006400u) + bias;
  p[2] = __builtin_bit_cast(half2v, ((t >> 8) & 0x000F000Fu) | 0x64006400u) + bias;
  p[3] = __builtin_bit_cast(half2v, ((t >> 12) & 0x000F000Fu) | 0x64006400u) + bias;
  return half8{p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
}

// the codeword of the 16-bit index (page image) or slot code (slot image) in half HI of w
template <int HI, bool CODES>
__device__ __forceinline__ half8 primary_half8(const uint32_t* lds, uint32_t w, uint32_t two, uint32_t delta) {
  uint32_t m, word;
  if constexpr (CODES) {
    word = code_word<HI>(lds, w, delta, m);
  } else {
    const uint32_t desc = page_desc<HI>(lds, w, two);
    m = page_mask(desc);
    word = slot_word<HI>(lds, w, desc, m, two);
  }
  return word_to_half8(word, m);
}

// 16 * byte SEL of w (a byte address into the fp16 residual table)
template <int SEL>
__device__ __forceinline__ uint32_t byte_x16(uint32_t w) {
  uint32_t r;
  const uint32_t four = 4;
  if (SEL == 0) asm volatile("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(four), "v"(w));
  else if (SEL == 1) asm volatile("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(four), "v"(w));
  else if (SEL == 2) asm volatile("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(four), "v"(w));
  else asm volatile("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(four), "v"(w));
  return r;
}

}  // namespace
}  // namespace glq
