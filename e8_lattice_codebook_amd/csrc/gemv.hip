// Decode matmul (B <= 16) on gfx950: z = u W~^T taken directly against the
// 16-bit E8 indices, W~ never formed.
//
// glq 0.5.1 (PyPI project page), "Inference kernels": the kernel walks the N/8
// codebook blocks of each output row, gathers each 8-D codeword from the cached
// codebook and accumulates the matmul; split-K partial sums go to a scratch
// buffer and are reduced in a fixed order instead of with atomics.  "How it
// works", items 1 and 4; table "Bit widths" (2/3/4 bpw stage layouts).
//
// Mapping: a wave owns a K-chunk of LPR * GL groups; lane l of a row holds GL
// groups (8 * GL columns) of u for every batch row in registers.  The wave walks
// `steps` row-steps of 64 / LPR rows each: per row, a lane loads its GL primary
// indices with one vector load, gathers the int8 (2x) codewords from the packed
// table, converts and accumulates in fp32; the 256-entry residual table sits in
// LDS, a 16-bit residual is gathered like the primary.  The LPR lanes of a row
// are reduced with cross-lane adds and one lane writes the split's partial sum,
// scaled by s / 2, to z_parts[split][b][o].
#include "internal.h"

namespace glq {
namespace {

template <int GL>
struct IdxVec;
template <>
struct IdxVec<1> {
  __device__ static void load(const uint16_t* p, uint32_t* out) { out[0] = p[0]; }
};
template <>
struct IdxVec<2> {
  __device__ static void load(const uint16_t* p, uint32_t* out) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    out[0] = w & 0xFFFFu;
    out[1] = w >> 16;
  }
};
template <>
struct IdxVec<4> {
  __device__ static void load(const uint16_t* p, uint32_t* out) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    out[0] = w.x & 0xFFFFu;
    out[1] = w.x >> 16;
    out[2] = w.y & 0xFFFFu;
    out[3] = w.y >> 16;
  }
};
template <>
struct IdxVec<8> {
  __device__ static void load(const uint16_t* p, uint32_t* out) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    out[0] = w.x & 0xFFFFu;
    out[1] = w.x >> 16;
    out[2] = w.y & 0xFFFFu;
    out[3] = w.y >> 16;
    out[4] = w.z & 0xFFFFu;
    out[5] = w.z >> 16;
    out[6] = w.w & 0xFFFFu;
    out[7] = w.w >> 16;
  }
};

__device__ __forceinline__ float i8_at(uint32_t w, int j) { return float(int8_t(uint8_t(w >> (8 * j)))); }

template <int NB, int GL, int RESID>
__global__ __launch_bounds__(256) void gemv_kernel(const uint16_t* __restrict__ idx0, const void* __restrict__ idx1v,
                                                   const int8_t* __restrict__ cb0, const int8_t* __restrict__ cb1,
                                                   const float* __restrict__ u, int B, int64_t n_pad, int64_t m_pad,
                                                   int lpr_log2, int steps, float out_scale, float sr,
                                                   float* __restrict__ z_parts) {
  __shared__ uint2 res_tab[RESID == 8 ? 256 : 1];
  if (RESID == 8) {
    for (int k = threadIdx.x; k < 256; k += blockDim.x) res_tab[k] = reinterpret_cast<const uint2*>(cb1)[k];
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int LPR = 1 << lpr_log2;
  const int RPS = 64 >> lpr_log2;  // rows per step
  const int lane_in_row = lane & (LPR - 1);
  const int row_in_step = lane >> lpr_log2;
  const int64_t gpr = n_pad >> 3;
  const int split = blockIdx.y;
  const int64_t g0 = int64_t(split) * (LPR * GL) + int64_t(lane_in_row) * GL;

  float ur[NB][GL * 8];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int q = 0; q < GL * 8; ++q) ur[b][q] = (b < B) ? u[int64_t(b) * n_pad + g0 * 8 + q] : 0.0f;
  }

  const int64_t wave_id = int64_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t row0 = wave_id * steps * RPS;
  const uint8_t* idx1_8 = static_cast<const uint8_t*>(idx1v);
  const uint16_t* idx1_16 = static_cast<const uint16_t*>(idx1v);

  for (int st = 0; st < steps; ++st) {
    const int64_t o = row0 + int64_t(st) * RPS + row_in_step;
    const bool valid = o < m_pad;
    float acc0[NB], acc1[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc0[b] = acc1[b] = 0.0f;
    if (valid) {
      uint32_t i0[GL];
      IdxVec<GL>::load(idx0 + o * gpr + g0, i0);
#pragma unroll
      for (int q = 0; q < GL; ++q) {
        const uint2 c0 = *reinterpret_cast<const uint2*>(cb0 + size_t(i0[q]) * 8);
        float cf[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          cf[j] = i8_at(c0.x, j);
          cf[j + 4] = i8_at(c0.y, j);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
          for (int j = 0; j < 8; ++j) acc0[b] = fmaf(cf[j], ur[b][q * 8 + j], acc0[b]);
        }
        if (RESID != 0) {
          uint2 c1;
          if (RESID == 8) {
            c1 = res_tab[idx1_8[o * gpr + g0 + q]];
          } else {
            c1 = *reinterpret_cast<const uint2*>(cb1 + size_t(idx1_16[o * gpr + g0 + q]) * 8);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            cf[j] = i8_at(c1.x, j);
            cf[j + 4] = i8_at(c1.y, j);
          }
#pragma unroll
          for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int j = 0; j < 8; ++j) acc1[b] = fmaf(cf[j], ur[b][q * 8 + j], acc1[b]);
          }
        }
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float v = RESID != 0 ? fmaf(sr, acc1[b], acc0[b]) : acc0[b];
      for (int off = LPR >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
      if (valid && lane_in_row == 0 && b < B) z_parts[(int64_t(split) * B + b) * m_pad + o] = v * out_scale;
    }
  }
}

// Groups per lane per row for a batch tile of NB rows (u held in registers:
// 8 * GL * NB floats per lane).
constexpr int gl_for(int nb) { return nb <= 1 ? 8 : nb == 2 ? 4 : nb <= 4 ? 2 : 1; }

int nb_tile(int64_t B) { return B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : B <= 8 ? 8 : 16; }

struct Plan {
  int nb, gl, lpr_log2, splits;
};

Plan make_plan(int64_t n_pad, int64_t B) {
  Plan p;
  p.nb = nb_tile(B);
  const int64_t gpr = n_pad / 8;
  int gl = gl_for(p.nb);
  while (gl > gpr || gpr % gl != 0) gl >>= 1;
  p.gl = gl;
  int64_t lanes = gpr / gl;  // lanes needed to cover a row once
  int lpr_log2 = 0;
  while ((int64_t(1) << lpr_log2) < lanes && lpr_log2 < 6) ++lpr_log2;
  // the splits must tile the row (a block-diagonal n_pad is not a power of two)
  while (lpr_log2 > 0 && gpr % (int64_t(gl) << lpr_log2) != 0) --lpr_log2;
  p.lpr_log2 = lpr_log2;
  p.splits = int(gpr / (int64_t(gl) << lpr_log2));
  return p;
}

template <int NB, int GL>
hipError_t launch_nb_gl(const glq_layer& L, const float* u, int64_t B, float* z, const Plan& p,
                        hipStream_t stream) {
  const int rps = 64 >> p.lpr_log2;
  const int64_t row_steps = (L.m_pad + rps - 1) / rps;
  // aim for ~4096 waves over the whole launch
  const int64_t total_waves_target = 4096;
  int64_t waves_per_split = total_waves_target / p.splits;
  if (waves_per_split < 1) waves_per_split = 1;
  int steps = int((row_steps + waves_per_split - 1) / waves_per_split);
  if (steps < 1) steps = 1;
  const int64_t waves = (row_steps + steps - 1) / steps;
  const int64_t blocks = (waves + 3) / 4;
  const dim3 grid(unsigned(blocks), unsigned(p.splits)), block(256);
  const int8_t* cb0 = static_cast<const int8_t*>(L.cb_pack) + pack_i8_offset();
  const int8_t* cb1 = L.cb2_pack ? static_cast<const int8_t*>(L.cb2_pack) + pack_i8_offset() : nullptr;
  const float out_scale = 0.5f * L.wscale;
  switch (L.resid_bits) {
    case 0:
      hipLaunchKernelGGL((gemv_kernel<NB, GL, 0>), grid, block, 0, stream, L.idx0, L.idx1, cb0, cb1, u, int(B),
                         L.n_pad, L.m_pad, p.lpr_log2, steps, out_scale, L.resid_scale, z);
      break;
    case 8:
      hipLaunchKernelGGL((gemv_kernel<NB, GL, 8>), grid, block, 0, stream, L.idx0, L.idx1, cb0, cb1, u, int(B),
                         L.n_pad, L.m_pad, p.lpr_log2, steps, out_scale, L.resid_scale, z);
      break;
    default:
      hipLaunchKernelGGL((gemv_kernel<NB, GL, 16>), grid, block, 0, stream, L.idx0, L.idx1, cb0, cb1, u, int(B),
                         L.n_pad, L.m_pad, p.lpr_log2, steps, out_scale, L.resid_scale, z);
      break;
  }
  return hipGetLastError();
}

template <int NB>
hipError_t launch_nb(const glq_layer& L, const float* u, int64_t B, float* z, const Plan& p, hipStream_t stream) {
  switch (p.gl) {
    case 8:
      if constexpr (gl_for(NB) >= 8) return launch_nb_gl<NB, 8>(L, u, B, z, p, stream);
      break;
    case 4:
      if constexpr (gl_for(NB) >= 4) return launch_nb_gl<NB, 4>(L, u, B, z, p, stream);
      break;
    case 2:
      if constexpr (gl_for(NB) >= 2) return launch_nb_gl<NB, 2>(L, u, B, z, p, stream);
      break;
    case 1:
      return launch_nb_gl<NB, 1>(L, u, B, z, p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int gemv_splits(int64_t n_pad, int64_t B) { return make_plan(n_pad, B).splits; }

hipError_t launch_gemv(const glq_layer& L, const float* u, int64_t B, float* z_parts, hipStream_t stream) {
  const Plan p = make_plan(L.n_pad, B);
  switch (p.nb) {
    case 1: return launch_nb<1>(L, u, B, z_parts, p, stream);
    case 2: return launch_nb<2>(L, u, B, z_parts, p, stream);
    case 4: return launch_nb<4>(L, u, B, z_parts, p, stream);
    case 8: return launch_nb<8>(L, u, B, z_parts, p, stream);
    default: return launch_nb<16>(L, u, B, z_parts, p, stream);
  }
}

GLQ_DEBUG_COUNTER(debug_violations_gemv)

}  // namespace glq
