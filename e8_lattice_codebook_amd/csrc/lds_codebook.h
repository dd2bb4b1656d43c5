// Device helpers shared by the decode kernels that keep the E8 codebook image
// in LDS (the page table + 4-byte slot words of a codebook pack, built on the
// host): index-vector loads, SDWA byte selects, the two-level lookup, DPP lane
// reductions.
#pragma once

#include "internal.h"

namespace glq {
namespace {

// ---- DPP reduction over LPR consecutive lanes; the sum lands in lane LPR - 1 ---------
__device__ __forceinline__ float dpp_add(float v, int ctrl_sel) {
  int r;
  const int x = __float_as_int(v);
  switch (ctrl_sel) {
    case 0: r = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false); break;   // quad_perm [1,0,3,2]
    case 1: r = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false); break;   // quad_perm [2,3,0,1]
    case 2: r = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    case 3: r = __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false); break;  // row_mirror
    case 4: r = __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false); break;  // row_bcast15 -> rows 1,3
    default: r = __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false); break; // row_bcast31 -> rows 2,3
  }
  return v + __int_as_float(r);
}

__device__ __forceinline__ float lane_reduce(float v, int lpr_log2) {
  if (lpr_log2 >= 1) v = dpp_add(v, 0);
  if (lpr_log2 >= 2) v = dpp_add(v, 1);
  if (lpr_log2 >= 3) v = dpp_add(v, 2);
  if (lpr_log2 >= 4) v = dpp_add(v, 3);
  if (lpr_log2 >= 5) v = dpp_add(v, 4);
  if (lpr_log2 >= 6) v = dpp_add(v, 5);
  return v;
}

template <int GL>
struct IdxRow {
  uint32_t w[GL >= 2 ? GL / 2 : 1];
};

template <int GL>
__device__ __forceinline__ void load_idx16(const uint16_t* p, IdxRow<GL>& r) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  if constexpr (GL == 8) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else if constexpr (GL == 4) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    r.w[0] = v.x; r.w[1] = v.y;
  } else if constexpr (GL == 2) {
    r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const unsigned int*>(p));
  } else {
    r.w[0] = __builtin_nontemporal_load(p);
  }
}

template <int GL>
__device__ __forceinline__ uint32_t idx16_at(const IdxRow<GL>& r, int q) {
  if constexpr (GL == 1) return r.w[0] & 0xFFFFu;
  return (r.w[q >> 1] >> (16 * (q & 1))) & 0xFFFFu;
}

template <int GL>
struct Idx8Row {
  uint32_t w[GL >= 4 ? GL / 4 : 1];
};

template <int GL>
__device__ __forceinline__ void load_idx8(const uint8_t* p, Idx8Row<GL>& r) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  if constexpr (GL == 8) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    r.w[0] = v.x; r.w[1] = v.y;
  } else if constexpr (GL == 4) {
    r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const unsigned int*>(p));
  } else if constexpr (GL == 2) {
    r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const unsigned short*>(p));
  } else {
    r.w[0] = __builtin_nontemporal_load(p);
  }
}

template <int GL>
__device__ __forceinline__ uint32_t idx8_at(const Idx8Row<GL>& r, int q) {
  if constexpr (GL < 4) return (r.w[0] >> (8 * q)) & 0xFFu;
  return (r.w[q >> 2] >> (8 * (q & 3))) & 0xFFu;
}

// ---- VALU byte selects (SDWA) ----------------------------------------------------
// The index words hold two 16-bit indices (bytes 0-1 and 2-3) or four 8-bit ones.
// 4 * byte SEL of w, and (byte SEL of w) ^ (byte 0 of d), in one instruction each.
template <int SEL>
__device__ __forceinline__ uint32_t byte_x4(uint32_t w, uint32_t two) {
  uint32_t r;
  if constexpr (SEL == 0)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
        : "=v"(r) : "v"(two), "v"(w));
  else if constexpr (SEL == 1)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
        : "=v"(r) : "v"(two), "v"(w));
  else if constexpr (SEL == 2)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
        : "=v"(r) : "v"(two), "v"(w));
  else
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
        : "=v"(r) : "v"(two), "v"(w));
  return r;
}
template <int SEL>
__device__ __forceinline__ uint32_t xor_byte(uint32_t w, uint32_t d) {
  uint32_t r;
  if constexpr (SEL == 0)
    asm("v_xor_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0 src1_sel:BYTE_0"
        : "=v"(r) : "v"(w), "v"(d));
  else
    asm("v_xor_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2 src1_sel:BYTE_0"
        : "=v"(r) : "v"(w), "v"(d));
  return r;
}

// LDS layout of the decode kernel (dwords): [0, 256) the 8-bit residual slots,
// [256, 256 + image) the primary image (page table, then slots).
constexpr int kResOff = 0;
constexpr int kImgOff = kResidDwords;
constexpr int kLdsDwords = kResidDwords + kImageMaxDwords;

__device__ __forceinline__ uint32_t lds_at(const uint32_t* lds, uint32_t byte_addr) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(lds) + byte_addr);
}

// Primary-codebook lookup of the 16-bit index in half HI of word w: the page
// descriptor (image word idx >> 8), then the slot at image byte offset
// 4 * ((idx ^ desc) & 255) + (desc >> 8), complemented (m = ~0) on descending pages.
template <int HI>
__device__ __forceinline__ uint32_t page_desc(const uint32_t* lds, uint32_t w, uint32_t two) {
  return lds_at(lds + kImgOff, byte_x4<HI ? 3 : 1>(w, two));
}
template <int HI>
__device__ __forceinline__ uint32_t slot_word(const uint32_t* lds, uint32_t w, uint32_t desc) {
  const uint32_t x = xor_byte<HI ? 2 : 0>(w, desc);
  return lds_at(lds + kImgOff, (x << 2) + (desc >> 8));
}

}  // namespace
}  // namespace glq
