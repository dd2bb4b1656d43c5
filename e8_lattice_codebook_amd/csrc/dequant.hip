// Codebook packing and explicit dequantization on gfx950.
//
// glq 0.5.1 (PyPI project page), "How it works", item 1: an 8-weight group is a
// 16-bit index into the 65,536-entry E8 codebook, refined by an 8-bit (256-entry)
// or 16-bit residual stage; table "Bit widths": one global scale per layer;
// "Inference kernels": the kernels gather 8-D codewords from a compact cached
// codebook.
//
// The codebook pack holds 2c as an int8 table [entries][8] (exact: every E8
// coordinate of norm^2 <= 12 is a multiple of 1/2 with |c| <= 3).
//
// Dequant: e = c0 + s_r * c1 (exact in fp32 for the codebook values and
// s_r = 2^-k; in general one rounding), w = RN(s * e); fp16 / bf16 outputs are
// RN(w).  One thread per 8-weight group, one 16- or 32-byte store per group.
#include "internal.h"

namespace glq {
namespace {

__device__ __forceinline__ float i8_at(uint32_t w, int j) { return float(int8_t(uint8_t(w >> (8 * j)))); }

template <class WT>
__device__ __forceinline__ void store8(WT* p, const float* v);
template <>
__device__ __forceinline__ void store8<float>(float* p, const float* v) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
template <>
__device__ __forceinline__ void store8<half_t>(half_t* p, const float* v) {
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = __builtin_bit_cast(uint16_t, (half_t)v[2 * k]);
    const uint32_t hi = __builtin_bit_cast(uint16_t, (half_t)v[2 * k + 1]);
    w[k] = lo | (hi << 16);
  }
  *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}
template <>
__device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float* v) {
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = from_f32<bf16_t>(v[2 * k]).bits;
    const uint32_t hi = from_f32<bf16_t>(v[2 * k + 1]).bits;
    w[k] = lo | (hi << 16);
  }
  *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

// Further residual stages (5-8 bpw): added in order, e = RN32(e + s_k c_k).
struct ExtraStages {
  int n;
  const void* idx[2];
  int bits[2];
  float scale[2];
  const int8_t* tab[2];   // int8 table of the stage's pack
  const uint16_t* map;    // code -> index of 16-bit stages with slot codes, else null
};

// map0 / map1: the pack's code -> index tables when the 16-bit stages hold slot
// codes, else null
template <class WT, int RESID>
__global__ __launch_bounds__(256) void dequant_kernel(const uint16_t* __restrict__ idx0, const void* __restrict__ idx1,
                                                      const int8_t* __restrict__ cb0, const int8_t* __restrict__ cb1,
                                                      const uint16_t* __restrict__ map0,
                                                      const uint16_t* __restrict__ map1, float s, float sr,
                                                      int64_t groups, WT* __restrict__ w, ExtraStages x) {
  const int64_t g = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= groups) return;
  const uint32_t i0 = map0 ? uint32_t(map0[idx0[g]]) : uint32_t(idx0[g]);
  const uint2 c0 = *reinterpret_cast<const uint2*>(cb0 + size_t(i0) * 8);
  float e[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    e[j] = 0.5f * i8_at(c0.x, j);
    e[j + 4] = 0.5f * i8_at(c0.y, j);
  }
  if (RESID != 0) {
    uint32_t i1 = RESID == 8 ? uint32_t(static_cast<const uint8_t*>(idx1)[g])
                             : uint32_t(static_cast<const uint16_t*>(idx1)[g]);
    if (RESID == 16 && map1) i1 = map1[i1];
    const uint2 c1 = *reinterpret_cast<const uint2*>(cb1 + size_t(i1) * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      e[j] = fmaf(sr, 0.5f * i8_at(c1.x, j), e[j]);
      e[j + 4] = fmaf(sr, 0.5f * i8_at(c1.y, j), e[j + 4]);
    }
  }
  for (int k = 0; k < x.n; ++k) {
    uint32_t ik = x.bits[k] == 8 ? uint32_t(static_cast<const uint8_t*>(x.idx[k])[g])
                                 : uint32_t(static_cast<const uint16_t*>(x.idx[k])[g]);
    if (x.bits[k] == 16 && x.map) ik = x.map[ik];
    const uint2 ck = *reinterpret_cast<const uint2*>(x.tab[k] + size_t(ik) * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      e[j] = fmaf(x.scale[k], 0.5f * i8_at(ck.x, j), e[j]);
      e[j + 4] = fmaf(x.scale[k], 0.5f * i8_at(ck.y, j), e[j + 4]);
    }
  }
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = s * e[j];
  store8<WT>(w + g * 8, v);
}

template <class WT>
hipError_t dequant_typed(const glq_layer& L, void* w, hipStream_t stream) {
  const int64_t groups = L.m_pad * (L.n_pad / 8);
  const dim3 grid(unsigned((groups + 255) / 256)), block(256);
  const int8_t* cb0 = static_cast<const int8_t*>(L.cb_pack) + pack_i8_offset();
  const int8_t* cb1 = L.cb2_pack ? static_cast<const int8_t*>(L.cb2_pack) + pack_i8_offset() : nullptr;
  WT* out = static_cast<WT*>(w);
  const uint16_t* map0 = nullptr;
  const uint16_t* map1 = nullptr;
  if (L.index_format == GLQ_INDEX_SLOT) {
    map0 = reinterpret_cast<const uint16_t*>(static_cast<const char*>(L.cb_pack) +
                                             pack_index_of_offset(GLQ_CODEBOOK_ENTRIES));
    if (L.resid_bits == 16)
      map1 = reinterpret_cast<const uint16_t*>(static_cast<const char*>(L.cb2_pack) +
                                               pack_index_of_offset(GLQ_CODEBOOK_ENTRIES));
  }
  ExtraStages x{};
  x.n = L.n_extra;
  x.map = map0;
  for (int k = 0; k < L.n_extra && k < 2; ++k) {
    x.idx[k] = L.extra_idx[k];
    x.bits[k] = L.extra_bits[k];
    x.scale[k] = L.extra_scale[k];
    x.tab[k] = static_cast<const int8_t*>(L.extra_bits[k] == 8 ? L.cb8_pack : L.cb_pack) + pack_i8_offset();
  }
  switch (L.resid_bits) {
    case 0:
      hipLaunchKernelGGL((dequant_kernel<WT, 0>), grid, block, 0, stream, L.idx0, L.idx1, cb0, cb1, map0, map1,
                         L.wscale, L.resid_scale, groups, out, x);
      break;
    case 8:
      hipLaunchKernelGGL((dequant_kernel<WT, 8>), grid, block, 0, stream, L.idx0, L.idx1, cb0, cb1, map0, map1,
                         L.wscale, L.resid_scale, groups, out, x);
      break;
    default:
      hipLaunchKernelGGL((dequant_kernel<WT, 16>), grid, block, 0, stream, L.idx0, L.idx1, cb0, cb1, map0, map1,
                         L.wscale, L.resid_scale, groups, out, x);
      break;
  }
  return hipGetLastError();
}

// codes[i] = code_of[idx[i]], eight values per thread where the buffers allow
__global__ __launch_bounds__(256) void slot_codes_kernel(const uint16_t* __restrict__ code_of, const uint16_t* idx,
                                                         int64_t count, uint16_t* codes, int vec) {
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (vec) {
    if (t * 8 + 8 > count) return;
    const uint4 v = reinterpret_cast<const uint4*>(idx)[t];
    uint4 r;
    r.x = uint32_t(code_of[v.x & 0xFFFFu]) | (uint32_t(code_of[v.x >> 16]) << 16);
    r.y = uint32_t(code_of[v.y & 0xFFFFu]) | (uint32_t(code_of[v.y >> 16]) << 16);
    r.z = uint32_t(code_of[v.z & 0xFFFFu]) | (uint32_t(code_of[v.z >> 16]) << 16);
    r.w = uint32_t(code_of[v.w & 0xFFFFu]) | (uint32_t(code_of[v.w >> 16]) << 16);
    reinterpret_cast<uint4*>(codes)[t] = r;
  } else {
    if (t >= count) return;
    codes[t] = code_of[idx[t]];
  }
}

}  // namespace

hipError_t launch_slot_codes(const void* cb_pack, const uint16_t* idx, int64_t count, uint16_t* codes,
                             hipStream_t stream) {
  if (count == 0) return hipSuccess;
  const uint16_t* code_of = reinterpret_cast<const uint16_t*>(static_cast<const char*>(cb_pack) +
                                                              pack_code_of_offset(GLQ_CODEBOOK_ENTRIES));
  const bool vec = (reinterpret_cast<uintptr_t>(idx) % 16 == 0) && (reinterpret_cast<uintptr_t>(codes) % 16 == 0);
  const int64_t vcount = vec ? count / 8 : 0;
  if (vcount > 0)
    hipLaunchKernelGGL(slot_codes_kernel, dim3(unsigned((vcount + 255) / 256)), dim3(256), 0, stream, code_of, idx,
                       vcount * 8, codes, 1);
  const int64_t rest = count - vcount * 8;
  if (rest > 0)
    hipLaunchKernelGGL(slot_codes_kernel, dim3(unsigned((rest + 255) / 256)), dim3(256), 0, stream, code_of,
                       idx + vcount * 8, rest, codes + vcount * 8, 0);
  return hipGetLastError();
}

hipError_t launch_dequant(const glq_layer& layer, void* w, glq_dtype w_dt, hipStream_t stream) {
  switch (w_dt) {
    case GLQ_F32: return dequant_typed<float>(layer, w, stream);
    case GLQ_F16: return dequant_typed<half_t>(layer, w, stream);
    case GLQ_BF16: return dequant_typed<bf16_t>(layer, w, stream);
  }
  return hipErrorInvalidValue;
}

GLQ_DEBUG_COUNTER(debug_violations_dequant)

}  // namespace glq
