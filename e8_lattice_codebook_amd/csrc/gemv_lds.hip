// Decode matmul (B <= 16) with the E8 codebook resident in LDS, on gfx950.
//
// glq 0.5.1 (PyPI project page), "Inference kernels": for each output row the
// kernel walks the N/8 codebook blocks, gathers each 8-D codeword and accumulates
// the matmul against the indices without forming W; split-K partial sums go to a
// scratch buffer and are reduced in a fixed order.  "How it works", items 1 and
// 4; table "Bit widths" (16-bit primary; 8-bit or 16-bit residual stage).
//
// Gathers: the pack's LDS image (page table + 4-byte codeword slots, each
// negation-symmetric shell stored once) is copied into LDS by every workgroup;
// a codeword costs two LDS reads (descriptor, slot).  A negated shell entry is
// read as its bitwise complement n ^ ~0, whose signed 4-bit lanes are -2c - 1.
// The image takes ~155 KiB of the CU's 160 KiB.
//
// Arithmetic: u is quantized per 64 columns to integers U (|U| <= 30583) written
// as four signed base-16 digit planes d_p (U = sum_p 16^p d_p).  For one group,
// v_dot8_i32_i4(n, d_p) gives sum_j 2c_j d_pj exactly, so four of them give
// sum_j 2c_j U_j; for a complemented codeword the result is -sum 2c U - sum U,
// and sum_j U_j of the group (precomputed) is added back into plane 0.  Per row and lane the
// integer total is exact (< 2^24), converted to fp32, scaled by the lane's 64-
// column scale, reduced over the lanes of the row with DPP adds in a fixed order,
// and one lane writes (s / 2) * total to z_parts[split][b][o].
//
// Mapping: 1024-thread persistent workgroups (one per CU, the image takes ~151
// KiB).  A wave owns a K-chunk of LPR * GL groups (lane: GL groups, digits for
// every batch row in registers) and walks contiguous row-steps of 64 / LPR rows,
// prefetching the next row-step's index vectors with non-temporal loads.
#include "lds_codebook.h"

namespace glq {
namespace {

constexpr int kThreads = 1024;
constexpr int kNoExp = -1024;  // the common exponent of all-zero blocks

// quantized u: digits [B][G][4] u32 | gsum [B][G] i32 | scale [B][nblk] f32
struct UqLayout {
  size_t dig_off, sum_off, scale_off, total;
  int64_t nblk, bg;
};

UqLayout uq_layout(int64_t B, int64_t n_pad) {
  UqLayout L;
  const int64_t G = n_pad / 8;
  L.bg = G < 8 ? G : 8;
  L.nblk = G / L.bg;
  L.dig_off = 0;
  L.sum_off = align256(size_t(B * G) * 16);
  L.scale_off = L.sum_off + align256(size_t(B * G) * 4);
  L.total = L.scale_off + align256(size_t(B * L.nblk) * 4);
  return L;
}

// ---- u -> digit planes -----------------------------------------------------------
__global__ __launch_bounds__(256) void quant_u_kernel(const float* __restrict__ u, int64_t B, int64_t G, int bg_log2,
                                                      uint32_t* __restrict__ dig, int32_t* __restrict__ gsum,
                                                      float* __restrict__ scale) {
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const bool live = t < B * G;
  const int64_t tt = live ? t : 0;
  const float4 a = reinterpret_cast<const float4*>(u)[tt * 2];
  const float4 b = reinterpret_cast<const float4*>(u)[tt * 2 + 1];
  float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float mx = 0.0f, poison = 0.0f;  // poison: 0, or NaN when a value is not finite
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    mx = fmaxf(mx, fabsf(v[j]));
    poison += v[j] - v[j];
  }
  // a block is 2^bg_log2 consecutive groups = consecutive threads
  for (int off = 1; off < (1 << bg_log2); off <<= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    poison += __shfl_xor(poison, off, 64);
  }
  // normalized by a power of two (max = f 2^fe, f in [1/2, 1)): U = rint(v 2^-fe
  // kUqMax / f) never overflows for a tiny max
  const bool nz = mx > 0.0f && poison == 0.0f;
  const int fe = nz ? __builtin_amdgcn_frexp_expf(mx) : 0;
  const float inv = nz ? float(kUqMax) / __builtin_amdgcn_frexp_mantf(mx) : 0.0f;
  float vn[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) vn[j] = __builtin_amdgcn_ldexpf(v[j], -fe);
  uint32_t planes[4];
  int32_t s;
  quantize_group(vn, inv, planes, s);
  if (!live) return;
  reinterpret_cast<uint4*>(dig)[t] = make_uint4(planes[0], planes[1], planes[2], planes[3]);
  gsum[t] = s;
  // the block's max itself (NaN for a non-finite block): the matmul forms the scale
  // max / kUqMax relative to a common power of two, so it stays in the normal range
  if ((t & ((int64_t(1) << bg_log2) - 1)) == 0) scale[t >> bg_log2] = (nz ? mx : 0.0f) + poison;
}

template <int NB, int GL, int RESID, bool FULL, bool CODES>
__global__ __launch_bounds__(kThreads) void gemv_lds_kernel(
    const uint16_t* __restrict__ idx0, const void* __restrict__ idx1v, const uint32_t* __restrict__ pack0_hdr,
    const uint32_t* __restrict__ img0, const uint32_t* __restrict__ res_slots, const uint32_t* __restrict__ uq_dig,
    const int32_t* __restrict__ uq_sum, const float* __restrict__ uq_scale, int B, int G, int m_pad, int lpr_log2,
    int bg_log2, int nblk, int units_per_wave, int row_steps, int splits, float out_scale, float sr,
    float* __restrict__ z_parts, int accumulate) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsDwords];
  const int tid = threadIdx.x;
  load_image_1024<RESID>(lds, pack0_hdr, img0, res_slots, tid, CODES ? kHdrSlotDwords : 3);
  const uint32_t delta = CODES ? slot_delta(pack0_hdr) : 0u;

  const int lane = tid & 63;
  const int lpr = FULL ? 6 : lpr_log2;
  const int LPR = 1 << lpr;
  const int RPS = 64 >> lpr;
  const int lane_in_row = lane & (LPR - 1);
  const int row_in_step = lane >> lpr;
  const int total_units = row_steps * splits;
  const int wave_global = int(blockIdx.x) * (kThreads / 64) + (tid >> 6);
  const int u_begin = wave_global * units_per_wave;
  const int u_end = min(u_begin + units_per_wave, total_units);
  const uint8_t* idx1_8 = static_cast<const uint8_t*>(idx1v);
  const uint16_t* idx1_16 = static_cast<const uint16_t*>(idx1v);

  uint32_t dig[NB][GL][4];
  GroupSumsFor<NB, GL, CODES> gs;
  float sc[NB];
  int wexp[NB];

  // (split, row-step) of the wave's current unit, advanced without divisions
  int split = u_begin / row_steps;
  int rs = u_begin - split * row_steps;
  int nsplit = split, nrs = rs;
  auto lane_g0 = [&](int sp) { return sp * (LPR * GL) + lane_in_row * GL; };
  auto row_off = [&](int sp, int r) {
    const int o = r * RPS + row_in_step;
    return (o < m_pad ? o : 0) * G + lane_g0(sp);
  };

  IdxRow<GL> n0, n1w;
  Idx8Row<GL> n1b;
  if (u_begin < u_end) {
    const int off = row_off(split, rs);
    load_idx16<GL>(idx0 + off, n0);
    if (RESID == 16) load_idx16<GL>(idx1_16 + off, n1w);
    if (RESID == 8) load_idx8<GL>(idx1_8 + off, n1b);
  }
  __syncthreads();

  int cur_split = -1;
  for (int unit = u_begin; unit < u_end; ++unit) {
    split = nsplit;
    rs = nrs;
    if (++nrs == row_steps) {
      nrs = 0;
      ++nsplit;
    }
    const int o = rs * RPS + row_in_step;
    const bool valid = o < m_pad;
    const IdxRow<GL> i0 = n0;
    const IdxRow<GL> i1w = n1w;
    const Idx8Row<GL> i1b = n1b;
    if (split != cur_split) {
      cur_split = split;
      const int g0 = lane_g0(split);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int bb = b < B ? b : 0;
#pragma unroll
        for (int q = 0; q < GL; ++q) {
          const uint4 v = reinterpret_cast<const uint4*>(uq_dig)[bb * G + g0 + q];
          dig[b][q][0] = v.x; dig[b][q][1] = v.y; dig[b][q][2] = v.z; dig[b][q][3] = v.w;
          gs.set(b, q, -uq_sum[bb * G + g0 + q]);  // negated: added on complemented reads
        }
        sc[b] = b < B ? uq_scale[bb * nblk + (g0 >> bg_log2)] : 0.0f;
      }
      // the block maxima relative to the wave's largest binary exponent E[b]: the
      // lanes' scales max 2^-E / kUqMax stay normal, and 2^E is applied to the
      // reduced row value
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        int e = sc[b] > 0.0f && sc[b] <= 3.4028235e38f ? __builtin_amdgcn_frexp_expf(sc[b]) : kNoExp;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) e = max(e, __shfl_xor(e, off, 64));
        wexp[b] = e;
        sc[b] = __builtin_amdgcn_ldexpf(sc[b], -e) / float(kUqMax);
      }
    }

    if (unit + 1 < u_end) {
      const int off = row_off(nsplit, nrs);
      load_idx16<GL>(idx0 + off, n0);
      if (RESID == 16) load_idx16<GL>(idx1_16 + off, n1w);
      if (RESID == 8) load_idx8<GL>(idx1_8 + off, n1b);
    }

    float vv[NB];
    row_dots<NB, GL, RESID, CODES>(lds, i0, i1w, i1b, dig, gs, sr, vv, delta);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float v = vv[b] * sc[b];
      if (FULL) {
        v = dpp_add(v, 0);
        v = dpp_add(v, 1);
        v = dpp_add(v, 2);
        v = dpp_add(v, 3);
        v = dpp_add(v, 4);
        v = dpp_add(v, 5);
      } else {
        v = lane_reduce(v, lpr);
      }
      if (valid && lane_in_row == LPR - 1 && b < B) {
        float* zo = z_parts + (split * B + b) * m_pad + o;
        const float zv = __builtin_amdgcn_ldexpf(v * out_scale, wexp[b]);
        *zo = accumulate ? *zo + zv : zv;
      }
    }
  }
}

constexpr int gl_for(int nb) { return nb <= 1 ? 8 : nb <= 2 ? 4 : nb <= 8 ? 2 : 1; }

int nb_tile(int64_t B) { return B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : B <= 8 ? 8 : 16; }

struct Plan {
  int nb, gl, lpr_log2, splits;
};

Plan make_plan(int64_t n_pad, int64_t B) {
  Plan p;
  p.nb = nb_tile(B);
  const int64_t G = n_pad / 8;
  int gl = gl_for(p.nb);
  while (gl > G || G % gl != 0) gl >>= 1;
  p.gl = gl;
  const int64_t lanes = G / gl;
  int l = 0;
  while ((int64_t(1) << l) < lanes && l < 6) ++l;
  // a split's columns (gl groups on each of 2^l lanes) must tile the row: with a
  // block-diagonal n_pad, G is a multiple of only its smallest block's groups
  while (l > 0 && G % (int64_t(gl) << l) != 0) --l;
  p.lpr_log2 = l;
  p.splits = int(G / (int64_t(gl) << l));
  return p;
}


template <int NB, int GL, int RESID, bool FULL, bool CODES>
hipError_t launch_t(const glq_layer& L, const void* uq, int64_t B, float* z, const Plan& p, hipStream_t stream,
                    bool accumulate) {
  auto kern = gemv_lds_kernel<NB, GL, RESID, FULL, CODES>;
  const int rps = 64 >> p.lpr_log2;
  const int64_t row_steps = (L.m_pad + rps - 1) / rps;
  const int64_t units = row_steps * p.splits;
  const int64_t max_waves = int64_t(device_cus()) * (kThreads / 64);
  const int64_t upw = (units + max_waves - 1) / max_waves;
  const int64_t waves = (units + upw - 1) / upw;
  const int64_t blocks = (waves + (kThreads / 64) - 1) / (kThreads / 64);
  const UqLayout U = uq_layout(B, L.n_pad);
  const char* uqc = static_cast<const char*>(uq);
  const char* p0 = static_cast<const char*>(L.cb_pack);
  const uint32_t* img0 = reinterpret_cast<const uint32_t*>(
      p0 + (CODES ? pack_slot_image_offset(GLQ_CODEBOOK_ENTRIES) : pack_image_offset(GLQ_CODEBOOK_ENTRIES)));
  const uint32_t* res = nullptr;
  if (RESID == 8)
    res = reinterpret_cast<const uint32_t*>(static_cast<const char*>(L.cb2_pack) +
                                            pack_image_offset(GLQ_RESID8_ENTRIES)) + kPageCount;
  int bg_log2 = 0;
  while ((int64_t(1) << bg_log2) < U.bg) ++bg_log2;
  hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, L.idx0, L.idx1,
                     reinterpret_cast<const uint32_t*>(p0), img0, res,
                     reinterpret_cast<const uint32_t*>(uqc + U.dig_off), reinterpret_cast<const int32_t*>(uqc + U.sum_off),
                     reinterpret_cast<const float*>(uqc + U.scale_off), int(B), int(L.n_pad / 8), int(L.m_pad),
                     p.lpr_log2, bg_log2, int(U.nblk), int(upw), int(row_steps), p.splits, 0.5f * L.wscale,
                     L.resid_scale, z, int(accumulate));
  return hipGetLastError();
}

template <int NB, int GL, int RESID>
hipError_t launch_f(const glq_layer& L, const void* uq, int64_t B, float* z, const Plan& p, hipStream_t stream,
                    bool acc) {
  const bool codes = L.index_format == GLQ_INDEX_SLOT;
  if (p.lpr_log2 == 6)
    return codes ? launch_t<NB, GL, RESID, true, true>(L, uq, B, z, p, stream, acc)
                 : launch_t<NB, GL, RESID, true, false>(L, uq, B, z, p, stream, acc);
  return codes ? launch_t<NB, GL, RESID, false, true>(L, uq, B, z, p, stream, acc)
               : launch_t<NB, GL, RESID, false, false>(L, uq, B, z, p, stream, acc);
}

template <int NB, int GL>
hipError_t launch_r(const glq_layer& L, const void* uq, int64_t B, float* z, const Plan& p, hipStream_t stream,
                    bool acc) {
  switch (L.resid_bits) {
    case 0: return launch_f<NB, GL, 0>(L, uq, B, z, p, stream, acc);
    case 8: return launch_f<NB, GL, 8>(L, uq, B, z, p, stream, acc);
    default: return launch_f<NB, GL, 16>(L, uq, B, z, p, stream, acc);
  }
}

template <int NB>
hipError_t launch_nb(const glq_layer& L, const void* uq, int64_t B, float* z, const Plan& p, hipStream_t stream,
                     bool acc) {
  switch (p.gl) {
    case 8:
      if constexpr (gl_for(NB) >= 8) return launch_r<NB, 8>(L, uq, B, z, p, stream, acc);
      break;
    case 4:
      if constexpr (gl_for(NB) >= 4) return launch_r<NB, 4>(L, uq, B, z, p, stream, acc);
      break;
    case 2:
      if constexpr (gl_for(NB) >= 2) return launch_r<NB, 2>(L, uq, B, z, p, stream, acc);
      break;
    default:
      return launch_r<NB, 1>(L, uq, B, z, p, stream, acc);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t uq_bytes(int64_t B, int64_t n_pad) { return uq_layout(B, n_pad).total; }

int gemv_lds_splits(int64_t n_pad, int64_t B) { return make_plan(n_pad, B).splits; }

hipError_t launch_quant_u(const float* u, int64_t B, int64_t n_pad, void* uq, hipStream_t stream) {
  const UqLayout U = uq_layout(B, n_pad);
  const int64_t G = n_pad / 8;
  int bg_log2 = 0;
  while ((int64_t(1) << bg_log2) < U.bg) ++bg_log2;
  char* q = static_cast<char*>(uq);
  const int64_t threads = B * G;
  hipLaunchKernelGGL(quant_u_kernel, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, stream, u, B, G, bg_log2,
                     reinterpret_cast<uint32_t*>(q + U.dig_off), reinterpret_cast<int32_t*>(q + U.sum_off),
                     reinterpret_cast<float*>(q + U.scale_off));
  return hipGetLastError();
}

hipError_t launch_gemv_lds(const glq_layer& L, const void* uq, int64_t B, float* z_parts, hipStream_t stream,
                           bool accumulate) {
  const Plan p = make_plan(L.n_pad, B);
  switch (p.nb) {
    case 1: return launch_nb<1>(L, uq, B, z_parts, p, stream, accumulate);
    case 2: return launch_nb<2>(L, uq, B, z_parts, p, stream, accumulate);
    case 4: return launch_nb<4>(L, uq, B, z_parts, p, stream, accumulate);
    case 8: return launch_nb<8>(L, uq, B, z_parts, p, stream, accumulate);
    default: return launch_nb<16>(L, uq, B, z_parts, p, stream, accumulate);
  }
}

GLQ_DEBUG_COUNTER(debug_violations_gemv_lds)

}  // namespace glq
