// Prefill matmul (B > 16) on gfx950: z = u W~^T with W~ dequantized tile by
// tile into LDS and fed to fp16 MFMA (v_mfma_f32_16x16x32_f16), fp32 accumulate.
//
// glq 0.5.1 (PyPI project page), "Inference kernels": for B >= 2 the matmul runs
// on the matrix units against codebook-loaded operands, without forming W.
// "How it works", items 1 and 4; table "Bit widths".
//
// The B operand of a 16x16x32 MFMA holds, per lane, 8 consecutive k of one
// column, which is exactly one E8 group of one output row: the dequantized tile
// is stored row-major [o][k] in LDS so each lane reads one group as 16 bytes.
// e = c0 + s_r c1 is exact in fp16 for the E8 codebook and s_r = 1/4 (8e is an
// integer in [-30, 30]), so the only roundings are u -> fp16 and the fp32
// accumulation; s is applied in the epilogue.
//
// Tile: 128 tokens x 128 output rows per workgroup, 4 waves of 64 x 64, K step 64.
#include "internal.h"

namespace glq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int LDK = BK + 8;  // LDS row stride in halves (144 bytes)

__device__ __forceinline__ float i8_at(uint32_t w, int j) { return float(int8_t(uint8_t(w >> (8 * j)))); }

template <int RESID>
__global__ __launch_bounds__(256) void gemm_kernel(const half_t* __restrict__ A, int64_t M, int64_t n_pad,
                                                   int64_t m_pad, const uint16_t* __restrict__ idx0,
                                                   const void* __restrict__ idx1v, const int8_t* __restrict__ cb0,
                                                   const int8_t* __restrict__ cb1,
                                                   const uint16_t* __restrict__ map, float s, float sr,
                                                   const int32_t* __restrict__ rexp, float* __restrict__ z,
                                                   int accumulate) {
  __shared__ __attribute__((aligned(16))) half_t As[BM * LDK];
  __shared__ __attribute__((aligned(16))) half_t Bs[BN * LDK];
  __shared__ uint2 res_tab[RESID == 8 ? 256 : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t m0 = int64_t(blockIdx.y) * BM;
  const int64_t o0 = int64_t(blockIdx.x) * BN;
  const int64_t gpr = n_pad >> 3;
  const uint8_t* idx1_8 = static_cast<const uint8_t*>(idx1v);
  const uint16_t* idx1_16 = static_cast<const uint16_t*>(idx1v);
  if (RESID == 8) {
    res_tab[tid] = reinterpret_cast<const uint2*>(cb1)[tid];  // 256 threads, 256 entries
    __syncthreads();
  }

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = 0; k0 < n_pad; k0 += BK) {
    // activations: BM rows x BK halves, 16 bytes per thread per step
    for (int c = tid; c < BM * (BK / 8); c += 256) {
      const int r = c >> 3, kc = (c & 7) * 8;
      const int64_t gm = m0 + r, gk = k0 + kc;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (gm < M && gk < n_pad) v = *reinterpret_cast<const uint4*>(A + gm * n_pad + gk);
      *reinterpret_cast<uint4*>(As + r * LDK + kc) = v;
    }
    // weights: BN rows x BK / 8 groups, dequantized to fp16
    for (int c = tid; c < BN * (BK / 8); c += 256) {
      const int r = c >> 3, gq = c & 7;
      const int64_t o = o0 + r, g = (k0 >> 3) + gq;
      half8 w = half8{0, 0, 0, 0, 0, 0, 0, 0};
      if (o < m_pad && g < gpr) {
        const uint32_t i0 = map ? uint32_t(map[idx0[o * gpr + g]]) : uint32_t(idx0[o * gpr + g]);
        const uint2 c0 = *reinterpret_cast<const uint2*>(cb0 + size_t(i0) * 8);
        float e[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          e[j] = 0.5f * i8_at(c0.x, j);
          e[j + 4] = 0.5f * i8_at(c0.y, j);
        }
        if (RESID != 0) {
          uint2 c1;
          if (RESID == 8) {
            c1 = res_tab[idx1_8[o * gpr + g]];
          } else {
            const uint32_t i1 = map ? uint32_t(map[idx1_16[o * gpr + g]]) : uint32_t(idx1_16[o * gpr + g]);
            c1 = *reinterpret_cast<const uint2*>(cb1 + size_t(i1) * 8);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            e[j] = fmaf(sr, 0.5f * i8_at(c1.x, j), e[j]);
            e[j + 4] = fmaf(sr, 0.5f * i8_at(c1.y, j), e[j + 4]);
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = (half_t)e[j];
      }
      *reinterpret_cast<half8*>(Bs + r * LDK + gq * 8) = w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      half8 a[4], b[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        a[mi] = *reinterpret_cast<const half8*>(As + (wm * 64 + mi * 16 + (lane & 15)) * LDK + kk + (lane >> 4) * 8);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        b[ni] = *reinterpret_cast<const half8*>(Bs + (wn * 64 + ni * 16 + (lane & 15)) * LDK + kk + (lane >> 4) * 8);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
    __syncthreads();
  }

#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int64_t col = o0 + wn * 64 + ni * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + wm * 64 + mi * 16 + (lane >> 4) * 4 + i;
        if (row < M && col < m_pad) {
          float* zo = z + row * m_pad + col;
          const float v = row_scaled(acc[mi][ni][i] * s, rexp ? rexp[row] : 0);
          *zo = accumulate ? *zo + v : v;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const glq_layer& L, const half_t* u16, const int32_t* rexp, int64_t M, float* z,
                       hipStream_t stream, bool accumulate) {
  if (gemm_lds_supported(L)) return launch_gemm_lds(L, u16, rexp, M, false, z, stream, accumulate);
  const dim3 grid(unsigned((L.m_pad + BN - 1) / BN), unsigned((M + BM - 1) / BM)), block(256);
  const int8_t* cb0 = static_cast<const int8_t*>(L.cb_pack) + pack_i8_offset();
  const int8_t* cb1 = L.cb2_pack ? static_cast<const int8_t*>(L.cb2_pack) + pack_i8_offset() : nullptr;
  // slot codes (16-bit stages, one pack): back to indices through the pack's table
  const uint16_t* map = L.index_format == GLQ_INDEX_SLOT
                            ? reinterpret_cast<const uint16_t*>(static_cast<const char*>(L.cb_pack) +
                                                                pack_index_of_offset(GLQ_CODEBOOK_ENTRIES))
                            : nullptr;
  switch (L.resid_bits) {
    case 0:
      hipLaunchKernelGGL((gemm_kernel<0>), grid, block, 0, stream, u16, M, L.n_pad, L.m_pad, L.idx0, L.idx1, cb0,
                         cb1, map, L.wscale, L.resid_scale, rexp, z, int(accumulate));
      break;
    case 8:
      hipLaunchKernelGGL((gemm_kernel<8>), grid, block, 0, stream, u16, M, L.n_pad, L.m_pad, L.idx0, L.idx1, cb0,
                         cb1, map, L.wscale, L.resid_scale, rexp, z, int(accumulate));
      break;
    default:
      hipLaunchKernelGGL((gemm_kernel<16>), grid, block, 0, stream, u16, M, L.n_pad, L.m_pad, L.idx0, L.idx1, cb0,
                         cb1, map, L.wscale, L.resid_scale, rexp, z, int(accumulate));
      break;
  }
  return hipGetLastError();
}

GLQ_DEBUG_COUNTER(debug_violations_gemm)

}  // namespace glq
