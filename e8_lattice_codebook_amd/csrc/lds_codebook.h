// Device helpers shared by the decode kernels that keep the E8 codebook image
// in LDS (the page table + 4-byte slot words of a codebook pack, built on the
// host): index-vector loads, SDWA byte selects, the two-level lookup, DPP lane
// reductions, the image load, the per-row integer dot products and the
// fixed-point digit planes of the activations.
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
// 4 * byte SEL of w in one instruction.
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

// 4 * the 16-bit half HI of w in one instruction
template <int HI>
__device__ __forceinline__ uint32_t word_x4(uint32_t w, uint32_t two) {
  uint32_t r;
  if constexpr (HI == 0)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_0"
        : "=v"(r) : "v"(two), "v"(w));
  else
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
        : "=v"(r) : "v"(two), "v"(w));
  return r;
}

// n ^ m for the 16-bit mask (0 or 0xFFFF) in half HI of mm, sign-extended to 32 bits
template <int HI>
__device__ __forceinline__ uint32_t xor_half_mask(uint32_t n, uint32_t mm) {
  uint32_t r;
  if constexpr (HI == 0)
    asm("v_xor_b32_sdwa %0, sext(%1), %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_0 src1_sel:DWORD"
        : "=v"(r) : "v"(mm), "v"(n));
  else
    asm("v_xor_b32_sdwa %0, sext(%1), %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1 src1_sel:DWORD"
        : "=v"(r) : "v"(mm), "v"(n));
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
// a word of the codebook image (byte offset from kImgOff) / of the residual slots
__device__ __forceinline__ uint32_t lds_img(const uint32_t* lds, uint32_t byte_addr) {
  GLQ_DCHECK(byte_addr < uint32_t(kImageMaxDwords) * 4u);
  return lds_at(lds + kImgOff, byte_addr);
}
__device__ __forceinline__ uint32_t lds_res(const uint32_t* lds, uint32_t byte_addr) {
  GLQ_DCHECK(byte_addr < uint32_t(kResidDwords) * 4u);
  return lds_at(lds + kResOff, byte_addr);
}

// Primary-codebook lookup of the 16-bit index in half HI of word w: the page
// descriptor (image word idx >> 8), then the slot at image byte offset
// ((4 (idx & 255)) ^ m) + desc with m = -(desc & 1), all ones on descending pages,
// whose words are read complemented (m again).
template <int HI>
__device__ __forceinline__ uint32_t page_desc(const uint32_t* lds, uint32_t w, uint32_t two) {
  return lds_img(lds, byte_x4<HI ? 3 : 1>(w, two));
}
__device__ __forceinline__ uint32_t page_mask(uint32_t desc) { return uint32_t(__builtin_amdgcn_sbfe(desc, 0, 1)); }
template <int HI>
__device__ __forceinline__ uint32_t slot_word(const uint32_t* lds, uint32_t w, uint32_t desc, uint32_t m,
                                              uint32_t two) {
  return lds_img(lds, (byte_x4<HI ? 2 : 0>(w, two) ^ m) + desc);
}

// Slot-code lookup of the code in half HI of w (the slot image in LDS at kImgOff):
// m = all ones when the code is negative as int16, slot (code ^ m) + (m & delta),
// the word to be read complemented when m is all ones.  delta <= kImageMaxDwords -
// 32768 keeps every slot inside the image.
template <int HI>
__device__ __forceinline__ uint32_t code_word(const uint32_t* lds, uint32_t w, uint32_t delta, uint32_t& m) {
  uint32_t x;
  if (HI) {
    m = uint32_t(int32_t(w) >> 31);
    asm("v_xor_b32_sdwa %0, sext(%1), %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1 src1_sel:DWORD"
        : "=v"(x) : "v"(w), "v"(m));
  } else {
    m = uint32_t(__builtin_amdgcn_sbfe(w, 15, 1));
    asm("v_xor_b32_sdwa %0, sext(%1), %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_0 src1_sel:DWORD"
        : "=v"(x) : "v"(w), "v"(m));
  }
  return lds_img(lds, (x + (m & delta)) << 2);
}

// The slot-code lookups of both codes of w, on 16-bit halves: mm gets the two masks
// (0 or 0xFFFF per half), each half's slot is (code ^ m) + (m & delta), formed as
// (code ^ m) + m * ndelta2 modulo 2^16 with ndelta2 = -delta in both halves (m = -1
// as int16).  No half can carry into the other: every slot is below 2^16.
__device__ __forceinline__ void code_pair(const uint32_t* lds, uint32_t w, uint32_t ndelta2, uint32_t& mm,
                                          uint32_t& n_lo, uint32_t& n_hi) {
  const uint32_t fifteen = 0x000F000Fu, two = 2;
  uint32_t slot;
  asm("v_pk_ashrrev_i16 %0, %1, %2" : "=v"(mm) : "v"(fifteen), "v"(w));
  const uint32_t x = w ^ mm;
  asm("v_pk_mad_u16 %0, %1, %2, %3" : "=v"(slot) : "v"(mm), "v"(ndelta2), "v"(x));
  n_lo = lds_img(lds, word_x4<0>(slot, two));
  n_hi = lds_img(lds, word_x4<1>(slot, two));
}
__device__ __forceinline__ uint32_t pair_ndelta(uint32_t delta) { return ((0u - delta) & 0xFFFFu) * 0x10001u; }

// delta of a pack's slot-code format, clamped so that no slot leaves the image
__device__ __forceinline__ uint32_t slot_delta(const uint32_t* pack_hdr) {
  const uint32_t d = pack_hdr[kHdrSlotDelta];
  return d < uint32_t(kImageMaxDwords - kSlotShared) ? d : uint32_t(kImageMaxDwords - kSlotShared);
}


// ---- activations in 16-bit fixed point ----------------------------------------------
// Per 64 columns, U = rint(u * kUqMax / max|u|); U is written as four balanced
// base-16 digits d_p in [-8, 7] (U = sum_p 16^p d_p), one 4-bit lane per column
// of the 8-column group in each of four digit-plane words.
constexpr int kUqMax = 30583;  // 7 * (16^3 + 16^2 + 16 + 1): four balanced base-16 digits

__device__ __forceinline__ void quantize_group(const float (&v)[8], float inv, uint32_t (&planes)[4], int32_t& sum) {
  planes[0] = planes[1] = planes[2] = planes[3] = 0u;
  sum = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int U = int(rintf(v[j] * inv));
    U = U > kUqMax ? kUqMax : (U < -kUqMax ? -kUqMax : U);
    sum += U;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int d = ((U + 8) & 15) - 8;  // balanced digit in [-8, 7]
      planes[p] |= uint32_t(d & 15) << (4 * lane_nibble(j));
      U = (U - d) >> 4;
    }
  }
}

// ---- the codebook image into LDS (1024 threads) ---------------------------------------
// The primary image (its dword count is word 3 of the pack header, clamped to
// the budget) goes to kImgOff, the 8-bit residual slots (RESID == 8) to kResOff.
// image_issue puts every global load in flight (clamped, unconditional loads);
// image_store<K0, K1> writes parts K0 .. K1-1 (part k: uint4 k * 1024 + tid of
// the image, i.e. LDS dwords below kImgOff + 4 * 1024 * (k + 1)), and with
// TAIL the last nd % 4 dwords and the residual slots.
typedef uint32_t img_x4 __attribute__((ext_vector_type(4)));  // native vector: stays in registers

struct ImageRegs {
  img_x4 t0, t1, t2, t3, t4, t5, t6, t7, t8, t9;
  uint32_t tail, res, nd, nd4;
};

template <int RESID>
__device__ __forceinline__ void image_issue(ImageRegs& r, const uint32_t* __restrict__ pack0_hdr,
                                            const uint32_t* __restrict__ img0,
                                            const uint32_t* __restrict__ res_slots, int tid, int nd_word) {
  constexpr int kT = 1024;
  static_assert((kImageMaxDwords / 4 + kT - 1) / kT == 10, "image load unrolled for 10 parts");
  uint32_t nd = pack0_hdr[nd_word];
  nd = nd > uint32_t(kImageMaxDwords) ? uint32_t(kImageMaxDwords) : nd;
  r.nd = nd;
  r.nd4 = nd >> 2;
  const img_x4* src4 = reinterpret_cast<const img_x4*>(img0);
  const uint32_t last4 = r.nd4 > 0 ? r.nd4 - 1 : 0;
  r.t0 = src4[min(uint32_t(tid), last4)];
  r.t1 = src4[min(uint32_t(tid) + 1 * kT, last4)];
  r.t2 = src4[min(uint32_t(tid) + 2 * kT, last4)];
  r.t3 = src4[min(uint32_t(tid) + 3 * kT, last4)];
  r.t4 = src4[min(uint32_t(tid) + 4 * kT, last4)];
  r.t5 = src4[min(uint32_t(tid) + 5 * kT, last4)];
  r.t6 = src4[min(uint32_t(tid) + 6 * kT, last4)];
  r.t7 = src4[min(uint32_t(tid) + 7 * kT, last4)];
  r.t8 = src4[min(uint32_t(tid) + 8 * kT, last4)];
  r.t9 = src4[min(uint32_t(tid) + 9 * kT, last4)];
  r.tail = 0;
  r.res = 0;
  const uint32_t ti = (r.nd4 << 2) + tid;
  if (ti < nd) r.tail = img0[ti];
  if (RESID == 8 && tid < kResidDwords) r.res = res_slots[tid];
}

template <int K0, int K1, bool TAIL, int RESID>
__device__ __forceinline__ void image_store(const ImageRegs& r, uint32_t* lds, int tid) {
  constexpr int kT = 1024;
  img_x4* dst4 = reinterpret_cast<img_x4*>(lds + kImgOff);
  // clamped like the loads: a thread past the end writes the last uint4 with
  // the value it loaded from there, the same value its owner writes
  const uint32_t last4 = r.nd4 > 0 ? r.nd4 - 1 : 0;
#define GLQ_IMAGE_PART(k, v) \
  if (K0 <= k && k < K1) dst4[min(uint32_t(tid) + k * kT, last4)] = r.v;
  GLQ_IMAGE_PART(0, t0)
  GLQ_IMAGE_PART(1, t1)
  GLQ_IMAGE_PART(2, t2)
  GLQ_IMAGE_PART(3, t3)
  GLQ_IMAGE_PART(4, t4)
  GLQ_IMAGE_PART(5, t5)
  GLQ_IMAGE_PART(6, t6)
  GLQ_IMAGE_PART(7, t7)
  GLQ_IMAGE_PART(8, t8)
  GLQ_IMAGE_PART(9, t9)
#undef GLQ_IMAGE_PART
  if (TAIL) {
    const uint32_t ti = (r.nd4 << 2) + tid;
    if (ti < r.nd) lds[kImgOff + ti] = r.tail;
    if (RESID == 8 && tid < kResidDwords) lds[kResOff + tid] = r.res;
  }
}

template <int RESID>
__device__ __forceinline__ void load_image_1024(uint32_t* lds, const uint32_t* __restrict__ pack0_hdr,
                                                const uint32_t* __restrict__ img0,
                                                const uint32_t* __restrict__ res_slots, int tid, int nd_word) {
  ImageRegs r;
  image_issue<RESID>(r, pack0_hdr, img0, res_slots, tid, nd_word);
  image_store<0, 10, true, RESID>(r, lds, tid);
}

// sum of the eight signed 4-bit products of a and b, starting from zero: the VOP3P
// form with an inline-constant accumulator (the compiler otherwise zeroes a register
// for the accumulating VOP2 form)
__device__ __forceinline__ int sdot8_zero(uint32_t a, uint32_t b) {
  int r;
  asm("v_dot8_i32_i4 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ int sdot8_acc(uint32_t a, uint32_t b, int c, bool first) {
  return first ? sdot8_zero(a, b) : __builtin_amdgcn_sdot8(int(a), int(b), c, false);
}

// ---- the groups' activation sums -------------------------------------------------------
// gs = -sum_j U_j of a group (|gs| < 2^18), added once per complemented read to undo
// its -1s.  With codebook indices every lookup has a 32-bit mask m and gs is added as
// m * gs.  With slot codes (GL >= 2) the masks of a word's two lookups are 16-bit
// halves (0 or -1), so the sums of groups 2k and 2k + 1 are kept as two int16 pairs,
// gs = 256 gh + gl with gl in [0, 256), and m * gs is added to the 1s and 256s digit
// planes by two 16-bit dot products per pair.
template <int NB, int GL, bool PAIRS>
struct GroupSums {
  int32_t g[NB][GL];
  __device__ __forceinline__ void set(int b, int q, int32_t v) { g[b][q] = v; }
};
template <int NB, int GL>
struct GroupSums<NB, GL, true> {
  static_assert(GL % 2 == 0, "group sums in pairs need an even group count");
  uint32_t lo[NB][GL / 2], hi[NB][GL / 2];
  // groups are set in increasing q, the even one of a pair first
  __device__ __forceinline__ void set(int b, int q, int32_t v) {
    const uint32_t l = uint32_t(v) & 0xFFu, h = uint32_t(v >> 8) & 0xFFFFu;
    if (q & 1) {
      lo[b][q >> 1] |= l << 16;
      hi[b][q >> 1] |= h << 16;
    } else {
      lo[b][q >> 1] = l;
      hi[b][q >> 1] = h;
    }
  }
};
template <int NB, int GL, bool CODES>
using GroupSumsFor = GroupSums<NB, GL, CODES && GL >= 2>;

typedef short glq_short2 __attribute__((ext_vector_type(2)));
// acc + the int16 dot product of the halves of a and b; the first one of a sum in the
// VOP3P form with a zero accumulator (as sdot8_zero)
__device__ __forceinline__ int sdot2_acc(uint32_t a, uint32_t b, int acc, bool first) {
  if (first) {
    int r;
    asm("v_dot2_i32_i16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
  }
  return __builtin_amdgcn_sdot2(__builtin_bit_cast(glq_short2, a), __builtin_bit_cast(glq_short2, b), acc, false);
}

// ---- one row-step: the lane's GL groups against NB activation rows -------------------
// v[b] = T0 + sr * T1 with T_k = sum over the lane's columns of 2 c_k U (exact
// integers, converted once to fp32): stage-0 codewords from the primary image,
// stage-1 codewords from the primary image (16-bit residual) or the residual
// slots (8-bit residual).  Reads go in three phases (every page descriptor,
// every slot word, then the dot products) so the LDS latencies overlap.  On a
// descending page (or a negative slot code) the complemented word n ^ ~0 has
// lanes -2c - 1, and the group's -sum_j U_j is added to undo the -1s.
template <int NB, int GL, int RESID, bool CODES>
__device__ __forceinline__ void row_dots(const uint32_t* lds, const IdxRow<GL>& i0, const IdxRow<GL>& i1w,
                                         const Idx8Row<GL>& i1b, const uint32_t (&dig)[NB][GL][4],
                                         const GroupSumsFor<NB, GL, CODES>& gs, float sr, float (&v)[NB],
                                         uint32_t delta) {
  constexpr bool PAIRS = CODES && GL >= 2;
  const uint32_t two = 2;
  int acc0[NB][4], acc1[NB][4];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int p = 0; p < 4; ++p) acc1[b][p] = 0;
  }
  // m0/m1: per-lookup 32-bit masks, or (PAIRS) the 16-bit mask pair of index word k
  uint32_t d0[GL], d1[GL], m0[GL], m1[GL], n0w[GL], n1w_[GL];
  if constexpr (PAIRS) {
    const uint32_t nd = pair_ndelta(delta);
#pragma unroll
    for (int k = 0; k < GL / 2; ++k) {
      code_pair(lds, i0.w[k], nd, m0[k], n0w[2 * k], n0w[2 * k + 1]);
      if (RESID == 16) code_pair(lds, i1w.w[k], nd, m1[k], n1w_[2 * k], n1w_[2 * k + 1]);
    }
  } else if constexpr (CODES) {
#pragma unroll
    for (int q = 0; q < GL; ++q) {
      n0w[q] = (q & 1) ? code_word<1>(lds, i0.w[q >> 1], delta, m0[q]) : code_word<0>(lds, i0.w[q >> 1], delta, m0[q]);
      if (RESID == 16)
        n1w_[q] = (q & 1) ? code_word<1>(lds, i1w.w[q >> 1], delta, m1[q])
                          : code_word<0>(lds, i1w.w[q >> 1], delta, m1[q]);
    }
  } else {
#pragma unroll
    for (int q = 0; q < GL; ++q) {
      d0[q] = (q & 1) ? page_desc<1>(lds, i0.w[q >> 1], two) : page_desc<0>(lds, i0.w[q >> 1], two);
      if (RESID == 16)
        d1[q] = (q & 1) ? page_desc<1>(lds, i1w.w[q >> 1], two) : page_desc<0>(lds, i1w.w[q >> 1], two);
    }
#pragma unroll
    for (int q = 0; q < GL; ++q) {
      m0[q] = page_mask(d0[q]);
      n0w[q] = (q & 1) ? slot_word<1>(lds, i0.w[q >> 1], d0[q], m0[q], two)
                       : slot_word<0>(lds, i0.w[q >> 1], d0[q], m0[q], two);
      if (RESID == 16) {
        m1[q] = page_mask(d1[q]);
        n1w_[q] = (q & 1) ? slot_word<1>(lds, i1w.w[q >> 1], d1[q], m1[q], two)
                          : slot_word<0>(lds, i1w.w[q >> 1], d1[q], m1[q], two);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < GL; ++q) {
    if (RESID == 8) {
      const uint32_t w1 = i1b.w[q >> 2];
      uint32_t a1;
      switch (q & 3) {
        case 0: a1 = byte_x4<0>(w1, two); break;
        case 1: a1 = byte_x4<1>(w1, two); break;
        case 2: a1 = byte_x4<2>(w1, two); break;
        default: a1 = byte_x4<3>(w1, two); break;
      }
      n1w_[q] = lds_res(lds, a1);
    }
  }
  // the stage's complement corrections and dot products for group q into acc
  auto stage_q = [&](int (&acc)[NB][4], const uint32_t (&nw)[GL], const uint32_t (&mk)[GL], int q) {
    uint32_t n;
    if constexpr (PAIRS) {
      n = (q & 1) ? xor_half_mask<1>(nw[q], mk[q >> 1]) : xor_half_mask<0>(nw[q], mk[q >> 1]);
      if ((q & 1) == 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          acc[b][0] = sdot2_acc(mk[q >> 1], gs.lo[b][q >> 1], acc[b][0], q == 0);
          acc[b][2] = sdot2_acc(mk[q >> 1], gs.hi[b][q >> 1], acc[b][2], q == 0);
        }
      }
    } else {
      n = nw[q] ^ mk[q];
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b][0] = __mul24(int32_t(mk[q]), gs.g[b][q]) + (q == 0 ? 0 : acc[b][0]);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const bool seeded = p == 0 || (PAIRS && p == 2);  // started by a correction above
        acc[b][p] = sdot8_acc(n, dig[b][q][p], acc[b][p], q == 0 && !seeded);
      }
    }
  };
#pragma unroll
  for (int q = 0; q < GL; ++q) {
    stage_q(acc0, n0w, m0, q);
    if (RESID == 16) stage_q(acc1, n1w_, m1, q);
    if (RESID == 8) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int p = 0; p < 4; ++p) acc1[b][p] = sdot8_acc(n1w_[q], dig[b][q][p], acc1[b][p], q == 0);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int t0 = ((acc0[b][3] * 16 + acc0[b][2]) * 16 + acc0[b][1]) * 16 + acc0[b][0];
    float r = float(t0);
    if (RESID != 0) {
      const int t1 = ((acc1[b][3] * 16 + acc1[b][2]) * 16 + acc1[b][1]) * 16 + acc1[b][0];
      r = fmaf(sr, float(t1), r);
    }
    v[b] = r;
  }
}

// ---- one further stage of a 5-8 bpw layer (one activation row) ---------------------
// The exact integer total sum_j 2c_j U_j over the lane's GL groups of a 16-bit stage
// (primary image, the same lookup and complement correction as the primary stage of
// row_dots) or of an 8-bit stage (the 256-entry residual slots, no complement).
template <int GL, bool CODES>
__device__ __forceinline__ int stage16_total(const uint32_t* lds, const IdxRow<GL>& ix,
                                             const uint32_t (&dig)[1][GL][4], const GroupSumsFor<1, GL, CODES>& gs,
                                             uint32_t delta) {
  constexpr bool PAIRS = CODES && GL >= 2;
  const uint32_t two = 2;
  uint32_t nw[GL], mm[GL];
  if constexpr (PAIRS) {
    const uint32_t nd = pair_ndelta(delta);
#pragma unroll
    for (int k = 0; k < GL / 2; ++k) code_pair(lds, ix.w[k], nd, mm[k], nw[2 * k], nw[2 * k + 1]);
  } else if constexpr (CODES) {
#pragma unroll
    for (int q = 0; q < GL; ++q)
      nw[q] = (q & 1) ? code_word<1>(lds, ix.w[q >> 1], delta, mm[q]) : code_word<0>(lds, ix.w[q >> 1], delta, mm[q]);
  } else {
    uint32_t d[GL];
#pragma unroll
    for (int q = 0; q < GL; ++q) d[q] = (q & 1) ? page_desc<1>(lds, ix.w[q >> 1], two) : page_desc<0>(lds, ix.w[q >> 1], two);
#pragma unroll
    for (int q = 0; q < GL; ++q) {
      mm[q] = page_mask(d[q]);
      nw[q] = (q & 1) ? slot_word<1>(lds, ix.w[q >> 1], d[q], mm[q], two)
                      : slot_word<0>(lds, ix.w[q >> 1], d[q], mm[q], two);
    }
  }
  int acc[4];
#pragma unroll
  for (int q = 0; q < GL; ++q) {
    uint32_t n;
    if constexpr (PAIRS) {
      n = (q & 1) ? xor_half_mask<1>(nw[q], mm[q >> 1]) : xor_half_mask<0>(nw[q], mm[q >> 1]);
      if ((q & 1) == 0) {
        acc[0] = sdot2_acc(mm[q >> 1], gs.lo[0][q >> 1], acc[0], q == 0);
        acc[2] = sdot2_acc(mm[q >> 1], gs.hi[0][q >> 1], acc[2], q == 0);
      }
    } else {
      n = nw[q] ^ mm[q];
      acc[0] = __mul24(int32_t(mm[q]), gs.g[0][q]) + (q == 0 ? 0 : acc[0]);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const bool seeded = p == 0 || (PAIRS && p == 2);
      acc[p] = sdot8_acc(n, dig[0][q][p], acc[p], q == 0 && !seeded);
    }
  }
  return ((acc[3] * 16 + acc[2]) * 16 + acc[1]) * 16 + acc[0];
}

template <int GL>
__device__ __forceinline__ int stage8_total(const uint32_t* lds, const Idx8Row<GL>& ix,
                                            const uint32_t (&dig)[1][GL][4]) {
  const uint32_t two = 2;
  uint32_t nw[GL];
#pragma unroll
  for (int q = 0; q < GL; ++q) {
    const uint32_t w1 = ix.w[q >> 2];
    uint32_t a1;
    switch (q & 3) {
      case 0: a1 = byte_x4<0>(w1, two); break;
      case 1: a1 = byte_x4<1>(w1, two); break;
      case 2: a1 = byte_x4<2>(w1, two); break;
      default: a1 = byte_x4<3>(w1, two); break;
    }
    nw[q] = lds_res(lds, a1);
  }
  int acc[4];
#pragma unroll
  for (int q = 0; q < GL; ++q)
#pragma unroll
    for (int p = 0; p < 4; ++p) acc[p] = sdot8_acc(nw[q], dig[0][q][p], acc[p], q == 0);
  return ((acc[3] * 16 + acc[2]) * 16 + acc[1]) * 16 + acc[0];
}

}  // namespace
}  // namespace glq
