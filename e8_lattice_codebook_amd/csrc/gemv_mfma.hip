// Decode matmul for a few activation rows (4 <= B <= 16) on gfx950: z = u W~^T on
// the matrix units, one fp16 MFMA (v_mfma_f32_16x16x32_f16) per 16 output rows and
// 32 columns, with each lane dequantizing one codeword per k-step from the LDS codebook
// straight into the MFMA's codeword operand.
//
// glq 0.5.1 (PyPI project page), "Inference kernels": the matmul reads the indices
// and the cached codebook and never forms W; for more than one activation row the
// product runs on the matrix units; split-K partial sums are reduced in a fixed order.
// "How it works", items 1 and 4; table "Bit widths".
//
// At B activation rows the work per 8-weight group is 8 B multiply-adds per stage.
// The integer GEMV of the B = 1 path spends four dot8 instructions per row and group
// on top of the codeword lookup, so at B = 16 it issues about 70 vector instructions
// per lookup; here the lookup and the fp16 conversion of the codeword (about 17
// instructions) are paid once and the B rows ride in one MFMA.  The activations are
// fp16 with a power-of-two scale per row (the prefill operand format, fragment order,
// one 16-token block whose rows past B are zero), which keeps the relative error near
// 3e-4, inside the decode bound.
//
// A wave owns a unit: 16 output rows and one split of the k-steps.  Lane l takes
// output row 16 rb + l % 16 and, at k-step ks, group 16 (ks / 4) + 4 q + ks % 4 of its
// row (q = l / 16), i.e. four consecutive groups per index block of four k-steps: one
// 8-byte load of the primary indices per block.  The u fragment of k-step ks is 1 KiB,
// 16 bytes per lane.  D holds, per lane, output l % 16 for tokens 4 q .. 4 q + 3.
// Workgroups of 16 waves are persistent, one per compute unit (the codebook image fills
// the LDS), and take units in turn; a unit's partial sums go to z_parts[split].
#include "mfma_dequant.h"

namespace glq {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kSkThreads = 1024;
constexpr int kSkWaves = kSkThreads / 64;

struct SkinnyArgs {
  const half_t* u;            // fragment order, one 16-token block: [KS][4][16][8] fp16
  const int32_t* rexp;        // the rows' power-of-two exponents [16]
  const uint16_t* idx0;       // [m_pad][G]
  const void* idx1;           // [m_pad][G] u8 or u16
  const uint32_t* pack0_hdr;
  const uint32_t* img0;       // page image (codebook indices) or slot image (slot codes)
  const int8_t* res_i8;       // 8-bit residual: int8 table [256][8] = 2c
  float* z;                   // [splits][B][m_pad]
  int B, m_pad, G, KS;
  int kss;                    // k-steps per split, a multiple of 4
  int row_blocks, units;
  float scale;                // s / 2
  float sr;
  int accumulate;             // add to z (second pass of a 5-8 bpw layer)
};

template <int RESID, bool CODES>
__global__ __launch_bounds__(kSkThreads, 1) void gemv_mfma_kernel(SkinnyArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsDwords];
  __shared__ __attribute__((aligned(16))) uint32_t res16[RESID == 8 ? 256 * 4 : 4];  // fp16 2c1, natural order
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const uint32_t two = 2;
  const uint32_t delta = CODES ? slot_delta(a.pack0_hdr) : 0u;

  // ---- the image (and the fp16 residual table) into LDS, once per workgroup
  {
    uint32_t nd = a.pack0_hdr[CODES ? kHdrSlotDwords : 3];
    nd = nd > uint32_t(kImageMaxDwords) ? uint32_t(kImageMaxDwords) : nd;
    const uint32_t nd4 = nd >> 2;
    const u32x4* src4 = reinterpret_cast<const u32x4*>(a.img0);
    u32x4* dst4 = reinterpret_cast<u32x4*>(lds + kImgOff);
    const uint32_t last4 = nd4 > 0 ? nd4 - 1 : 0;
    for (uint32_t base = 0; base < nd4; base += 4 * kSkThreads) {
      u32x4 t[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) t[k] = src4[min(base + k * kSkThreads + tid, last4)];
#pragma unroll
      for (int k = 0; k < 4; ++k) dst4[min(base + k * kSkThreads + tid, last4)] = t[k];
    }
    for (uint32_t i = (nd4 << 2) + tid; i < nd; i += kSkThreads) lds[kImgOff + i] = a.img0[i];
    if (RESID == 8 && tid < 256) {
      const u32x2 c = reinterpret_cast<const u32x2*>(a.res_i8)[tid];  // one entry per thread
      u32x4 h;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w = k < 2 ? c.x : c.y;
        const int lo = int8_t(uint8_t(w >> (16 * (k & 1))));
        const int hi = int8_t(uint8_t(w >> (16 * (k & 1) + 8)));
        const half2v v = half2v{_Float16(float(lo)), _Float16(float(hi))};
        h[k] = __builtin_bit_cast(uint32_t, v);
      }
      reinterpret_cast<u32x4*>(res16)[tid] = h;
    }
  }
  __syncthreads();

  const int q = lane >> 4;    // lane quarter: its groups of each k-step
  const int r16 = lane & 15;  // the lane's output row within the unit
  const int G = a.G;
  const half2v sr2 = half2v{_Float16(a.sr), _Float16(a.sr)};
  const uint8_t* idx1_8 = static_cast<const uint8_t*>(a.idx1);
  const uint16_t* idx1_16 = static_cast<const uint16_t*>(a.idx1);
  const half_t* ubase = a.u + 8 * lane;

  // the codeword fragment of k-step kk of an index block (fp16 2e = 2c0 + s_r 2c1)
  auto dequant = [&](const u32x2& i0, uint32_t i1b, const u32x2& i1w, int kk) -> half8 {
    const uint32_t w0 = (kk < 2) ? i0.x : i0.y;
    half8 b = (kk & 1) ? primary_half8<1, CODES>(lds, w0, two, delta) : primary_half8<0, CODES>(lds, w0, two, delta);
    if (RESID != 0) {
      half8 r;
      if (RESID == 8) {
        uint32_t ra;
        switch (kk) {
          case 0: ra = byte_x16<0>(i1b); break;
          case 1: ra = byte_x16<1>(i1b); break;
          case 2: ra = byte_x16<2>(i1b); break;
          default: ra = byte_x16<3>(i1b); break;
        }
        r = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(res16) + ra));
      } else {
        const uint32_t w1 = (kk < 2) ? i1w.x : i1w.y;
        r = (kk & 1) ? primary_half8<1, CODES>(lds, w1, two, delta) : primary_half8<0, CODES>(lds, w1, two, delta);
      }
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const half2v f = half2v{r[j], r[j + 1]} * sr2 + half2v{b[j], b[j + 1]};
        b[j] = f.x;
        b[j + 1] = f.y;
      }
    }
    return b;
  };

  const int nwaves = int(gridDim.x) * kSkWaves;
  for (int unit = int(blockIdx.x) * kSkWaves + (tid >> 6); unit < a.units; unit += nwaves) {
    // split-major: the waves running together share one range of k-steps (of u)
    const int split = unit / a.row_blocks;
    const int rb = unit - split * a.row_blocks;
    const int o = rb * 16 + r16;
    const int kb0 = (split * a.kss) >> 2;
    const int kb1 = min(split * a.kss + a.kss, a.KS) >> 2;  // index blocks [kb0, kb1)
    const int64_t ibase = int64_t(o) * G + 4 * q;
    auto load_idx = [&](int kb, u32x2& i0, uint32_t& i1b, u32x2& i1w) {
      const int kc = kb < kb1 ? kb : kb1 - 1;  // past the split's end: its last block again (never used)
      const int64_t off = ibase + 16 * int64_t(kc);
      i0 = *reinterpret_cast<const u32x2*>(a.idx0 + off);
      if (RESID == 8) i1b = *reinterpret_cast<const uint32_t*>(idx1_8 + off);
      if (RESID == 16) i1w = *reinterpret_cast<const u32x2*>(idx1_16 + off);
    };
    auto load_u = [&](int kb, half8 (&f)[4]) {
      const int kc = kb < kb1 ? kb : kb1 - 1;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) f[kk] = *reinterpret_cast<const half8*>(ubase + (int64_t(4 * kc + kk) << 9));
    };

    // Indices stream from HBM: three index blocks in flight per wave (a ring of three
    // register sets, each reloaded two blocks ahead as soon as it is consumed), so
    // that a wave keeps about 2 KiB of index loads outstanding.  u (L2-resident) is
    // loaded one block ahead.
    floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
    u32x2 i0[3], i1w[3];
    uint32_t i1b[3] = {0, 0, 0};
    half8 ua[4], un[4];
    load_idx(kb0, i0[0], i1b[0], i1w[0]);
    load_idx(kb0 + 1, i0[1], i1b[1], i1w[1]);
    load_idx(kb0 + 2, i0[2], i1b[2], i1w[2]);
    load_u(kb0, ua);
    auto block = [&](int kb, int s) {
      load_u(kb + 1, un);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const half8 b = dequant(i0[s], i1b[s], i1w[s], kk);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ua[kk], b, acc, 0, 0, 0);
      }
      load_idx(kb + 3, i0[s], i1b[s], i1w[s]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) ua[kk] = un[kk];
    };
    // three blocks per iteration, one per register set; loads past the split's end
    // read its last block again (in bounds, never used), so every path keeps the same
    // loads in flight
    for (int kb = kb0; kb < kb1; kb += 3) {
      block(kb, 0);
      if (kb + 1 < kb1) block(kb + 1, 1);
      if (kb + 2 < kb1) block(kb + 2, 2);
    }

    // ---- z_parts[split][b][o] = acc * s / 2 * 2^rexp[b] for the lane's tokens b < B
    if (o < a.m_pad) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = 4 * q + i;
        if (b < a.B) {
          float* zo = a.z + (int64_t(split) * a.B + b) * a.m_pad + o;
          const float v = row_scaled(acc[i] * a.scale, a.rexp[b]);
          *zo = a.accumulate ? *zo + v : v;
        }
      }
    }
  }
}

struct SkinnyPlan {
  int splits, kss, row_blocks, units;
};

SkinnyPlan skinny_plan(int64_t n_pad, int64_t m_pad) {
  SkinnyPlan p;
  const int KS = int(n_pad / 32);
  p.row_blocks = int((m_pad + 15) / 16);
  // enough units for every wave slot twice over, with at least 16 k-steps per unit and
  // at most 16 splits (the output transform sums them per element)
  const int64_t want = int64_t(device_cus()) * kSkWaves * 2;
  int s = 1;
  while (int64_t(p.row_blocks) * s < want && KS / (2 * s) >= 16 && s < 16) s *= 2;
  p.kss = ((KS + s - 1) / s + 3) & ~3;
  p.splits = (KS + p.kss - 1) / p.kss;
  p.units = p.row_blocks * p.splits;
  return p;
}

template <int RESID, bool CODES>
hipError_t launch_t(const SkinnyArgs& a, hipStream_t stream) {
  const int cus = device_cus();
  const int need = (a.units + kSkWaves - 1) / kSkWaves;
  const dim3 grid(unsigned(need < cus ? need : cus)), block(kSkThreads);
  hipLaunchKernelGGL((gemv_mfma_kernel<RESID, CODES>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

bool gemv_mfma_supported(const glq_layer& L) {
  // fragment-order u (n_pad a multiple of 128, at least 256), whole 16-row units,
  // residual from the primary image or an 8-bit table
  return L.n_pad >= 256 && L.n_pad % 128 == 0 && L.m_pad % 16 == 0 &&
         (L.resid_bits != 16 || L.cb2_pack == L.cb_pack);
}

int gemv_mfma_splits(int64_t n_pad, int64_t m_pad) { return skinny_plan(n_pad, m_pad).splits; }

hipError_t launch_gemv_mfma(const glq_layer& L, const half_t* u16, const int32_t* rexp, int64_t B, float* z_parts,
                            hipStream_t stream, bool accumulate) {
  const SkinnyPlan p = skinny_plan(L.n_pad, L.m_pad);
  SkinnyArgs a;
  a.u = u16;
  a.rexp = rexp;
  a.idx0 = L.idx0;
  a.idx1 = L.idx1;
  const char* p0 = static_cast<const char*>(L.cb_pack);
  a.pack0_hdr = reinterpret_cast<const uint32_t*>(p0);
  const bool codes = L.index_format == GLQ_INDEX_SLOT;
  a.img0 = reinterpret_cast<const uint32_t*>(
      p0 + (codes ? pack_slot_image_offset(GLQ_CODEBOOK_ENTRIES) : pack_image_offset(GLQ_CODEBOOK_ENTRIES)));
  a.res_i8 = L.resid_bits == 8 ? static_cast<const int8_t*>(L.cb2_pack) + pack_i8_offset() : nullptr;
  a.z = z_parts;
  a.B = int(B);
  a.m_pad = int(L.m_pad);
  a.G = int(L.n_pad / 8);
  a.KS = int(L.n_pad / 32);
  a.kss = p.kss;
  a.row_blocks = p.row_blocks;
  a.units = p.units;
  a.scale = 0.5f * L.wscale;
  a.sr = L.resid_scale;
  a.accumulate = int(accumulate);
  switch (L.resid_bits) {
    case 0: return codes ? launch_t<0, true>(a, stream) : launch_t<0, false>(a, stream);
    case 8: return codes ? launch_t<8, true>(a, stream) : launch_t<8, false>(a, stream);
    default: return codes ? launch_t<16, true>(a, stream) : launch_t<16, false>(a, stream);
  }
}

GLQ_DEBUG_COUNTER(debug_violations_gemv_mfma)

}  // namespace glq
