// Prefill matmul (B > 16) on gfx950 with the E8 codebook resident in LDS:
// z = u W~^T, codeword fragments dequantized straight into registers and fed to
// fp16 MFMA (v_mfma_f32_16x16x32_f16), fp32 accumulation.
//
// glq 0.5.1 (PyPI project page), "Inference kernels": for B >= 2 the matmul runs
// on the matrix units against codebook-loaded operands, without forming W.
// "How it works", items 1 and 4; table "Bit widths".
//
// The B operand of a 16x16x32 MFMA holds, per lane, 8 consecutive k of one
// column: exactly one E8 group of one output row.  Each lane therefore looks its
// codeword up in the LDS image (page descriptor, slot word; a descending page
// reads the complement) and turns the eight signed 4-bit lanes 2c into fp16
// without a table: nibbles j and j + 4 of the (offset-binary) word are masked
// into the mantissas of two fp16 1024 + nibble and the bias is subtracted with a
// packed add, giving (2c_{2j}, 2c_{2j+1}) exactly.  The 8-bit residual table sits
// in LDS as fp16; a 16-bit residual stage uses the image again.  2e = 2c0 + s_r 2c1
// is exact in fp16 (s_r = 1/4: multiples of 1/4 below 8); s / 2 is applied in the
// epilogue.  The A operand (u, fp16) is read from global memory by every wave;
// the four waves of a workgroup share it through L1.  The linear takes this
// kernel for layers with codebook indices (their page image leaves no LDS for
// the shared codeword tiles of the slot-code kernel), and the matmul on row-order
// u for every format.
//
// K order: at k-step ks, lane quarter q = lane / 16 of every MFMA takes group
// 16 (ks / 4) + 4 q + ks % 4 (G = n_pad / 8 groups, KS = G / 4 k-steps), so over
// a block of 4 k-steps a lane's indices are 4 consecutive groups and the four
// quarters of a row read 16 consecutive groups (one 32-byte piece per row per
// index load); A uses the same order.  The linear's input transform writes u in
// fragment order (each 16-token x 32-k fragment 1 KiB contiguous, tiled_u_bytes) so
// that every A load is one coalesced 1 KiB read; u in plain row order is also
// accepted.
//
// Tile: 16 kMB tokens x kWaves * 16 kNB outputs per workgroup (kMB x kNB MFMA
// blocks per wave); persistent workgroups, one per CU, load the image once.
#include "mfma_dequant.h"

namespace glq {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;       // one per SIMD (the accumulators take the AGPRs)
constexpr int kPThreads = 64 * kWaves;
constexpr int kMB = 8;          // 16-token blocks per wave (all waves share them)
constexpr int kNB = 4;          // 16-output blocks per wave
constexpr int kTM = 16 * kMB;   // tokens per tile
constexpr int kTNW = 16 * kNB;  // outputs per wave
constexpr int kTN = kWaves * kTNW;  // outputs per tile
constexpr int kKB = 4;          // k-steps per index load

struct GemmArgs {
  const half_t* u;            // [M][n_pad] fp16
  const uint16_t* idx0;       // [m_pad][G]
  const void* idx1;           // [m_pad][G] u8 or u16
  const uint32_t* pack0_hdr;
  const uint32_t* img0;       // primary LDS image
  const int8_t* res_i8;       // 8-bit residual: int8 table [256][8] = 2c
  const int32_t* rexp;        // the rows' power-of-two exponents (NULL: none)
  float* z;                   // [M][m_pad] fp32
  int64_t M;
  int n_pad, m_pad, G;
  int out_tiles, tok_tiles, tiles;
  float scale;                // s / 2
  float sr;
  int accumulate;             // add to z (second pass of a 5-8 bpw layer)
};

template <int RESID, bool TILED, bool CODES>
__global__ __launch_bounds__(kPThreads, 1) void gemm_lds_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsDwords];
  __shared__ __attribute__((aligned(16))) uint32_t res16[RESID == 8 ? 256 * 4 : 4];  // fp16 2c1, natural order
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
    for (uint32_t base = 0; base < nd4; base += 8 * kPThreads) {
      u32x4 t[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) t[k] = src4[min(base + k * kPThreads + tid, last4)];
#pragma unroll
      for (int k = 0; k < 8; ++k) dst4[min(base + k * kPThreads + tid, last4)] = t[k];
    }
    for (uint32_t i = (nd4 << 2) + tid; i < nd; i += kPThreads) lds[kImgOff + i] = a.img0[i];
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

  const int q = lane >> 4;       // lane quarter: its K range
  const int r16 = lane & 15;     // row / column of the lane in a 16 x 16 block
  const int G = a.G;
  const int KS = G >> 2;         // k-steps (groups per quarter)
  const half2v sr2 = half2v{_Float16(a.sr), _Float16(a.sr)};
  const uint8_t* idx1_8 = static_cast<const uint8_t*>(a.idx1);
  const uint16_t* idx1_16 = static_cast<const uint16_t*>(a.idx1);

  for (int tile = blockIdx.x; tile < a.tiles; tile += gridDim.x) {
    // workgroup ids are dealt to the 8 XCDs in turn: XCD x takes the output tiles
    // x, x + 8, ..., token-tile major, so the workgroups running at once on an XCD
    // share a few token tiles (A) and eight output tiles (index rows) in its L2
    int out_tile, tok_tile;
    if ((a.out_tiles & 7) == 0) {
      const int per = a.out_tiles >> 3;  // output tiles of one XCD
      const int i = tile >> 3;           // the tile's place in its XCD's order
      tok_tile = i / per;
      out_tile = (tile & 7) + 8 * (i - tok_tile * per);
    } else {
      out_tile = tile % a.out_tiles;
      tok_tile = tile / a.out_tiles;
    }
    const int64_t t0 = int64_t(tok_tile) * kTM;
    const int o_w = out_tile * kTN + wave * kTNW;

    floatx4 acc[kMB][kNB];
#pragma unroll
    for (int mi = 0; mi < kMB; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNB; ++ni) acc[mi][ni] = floatx4{0.f, 0.f, 0.f, 0.f};

    // A fragments.  TILED: u in fragment order [ceil(M/16)][KS][4][16][8] (the
    // fragment of token block tb at k-step ks is 1 KiB at (tb KS + ks) 512 + 8 lane
    // halves).  Natural: u [M][n_pad], the lane's row at group 16 (ks / 4) + 4 q + ks % 4.
    const half_t* abase = TILED ? a.u + (t0 >> 4) * int64_t(KS) * 512 + 8 * lane : a.u + t0 * a.n_pad + 32 * q;
    auto akoff = [&](int ks) { return TILED ? uint32_t(ks) * 512 : uint32_t(128 * (ks >> 2) + 8 * (ks & 3)); };
    // Token blocks past ceil(M / 16) (TILED) or rows past M read the tile's first
    // block or row instead: the buffer holds no more, and those rows are masked.
    auto arow_off = [&](int mi) {
      if (TILED) return uint32_t((t0 / 16 + mi < (a.M + 15) / 16 ? mi : 0) * KS * 512);
      const int64_t t = t0 + mi * 16 + r16;
      return uint32_t(t < a.M ? (mi * 16 + r16) * a.n_pad : 0);
    };
    // index rows of the lane: output o = o_w + 16 ni + r16, groups 4 kb + 4 q ..
    const int64_t ibase = int64_t(o_w + r16) * G + 4 * q;

    // codeword fragment of out-block ni at k-step kk of the current index block
    auto dequant = [&](const u32x2 (&i0)[kNB], const uint32_t (&i1b)[kNB], const u32x2 (&i1w)[kNB], int ni,
                       int kk) -> half8 {
      const uint32_t w0 = (kk < 2) ? i0[ni].x : i0[ni].y;
      half8 b = (kk & 1) ? primary_half8<1, CODES>(lds, w0, two, delta) : primary_half8<0, CODES>(lds, w0, two, delta);
      if (RESID != 0) {
        half8 r;
        if (RESID == 8) {
          uint32_t ra;
          switch (kk) {
            case 0: ra = byte_x16<0>(i1b[ni]); break;
            case 1: ra = byte_x16<1>(i1b[ni]); break;
            case 2: ra = byte_x16<2>(i1b[ni]); break;
            default: ra = byte_x16<3>(i1b[ni]); break;
          }
          r = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(res16) + ra));
        } else {
          const uint32_t w1 = (kk < 2) ? i1w[ni].x : i1w[ni].y;
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
    auto load_idx = [&](int kb, u32x2 (&i0)[kNB], uint32_t (&i1b)[kNB], u32x2 (&i1w)[kNB]) {
      const int kc = kb < KS ? kb : KS - kKB;  // past the end: reload the last block
#pragma unroll
      for (int ni = 0; ni < kNB; ++ni) {
        const int64_t off = ibase + int64_t(16 * ni) * G + 4 * kc;
        i0[ni] = *reinterpret_cast<const u32x2*>(a.idx0 + off);
        if (RESID == 8) i1b[ni] = *reinterpret_cast<const uint32_t*>(idx1_8 + off);
        if (RESID == 16) i1w[ni] = *reinterpret_cast<const u32x2*>(idx1_16 + off);
      }
    };

    // software pipeline: the fragments of k-step ks + 1 are dequantized while the
    // MFMAs of ks run; A is loaded two k-steps ahead (ping-pong av / aw)
    half8 av[kMB], aw[kMB];
#pragma unroll
    for (int mi = 0; mi < kMB; ++mi) {
      av[mi] = *reinterpret_cast<const half8*>(abase + arow_off(mi));
      aw[mi] = *reinterpret_cast<const half8*>(abase + arow_off(mi) + akoff(KS > 1 ? 1 : 0));
    }
    u32x2 i0[kNB], i0n[kNB];
    uint32_t i1b[kNB], i1bn[kNB];
    u32x2 i1w[kNB], i1wn[kNB];
    load_idx(0, i0, i1b, i1w);
    half8 b0[kNB], b1[kNB];
#pragma unroll
    for (int ni = 0; ni < kNB; ++ni) b0[ni] = dequant(i0, i1b, i1w, ni, 0);

    for (int kb = 0; kb < KS; kb += kKB) {
      load_idx(kb + kKB, i0n, i1bn, i1wn);
#pragma unroll
      for (int kk = 0; kk < kKB; ++kk) {
        // one basic block per k-step (no runtime branches), so the fragments of
        // ks + 1 and the A loads of ks + 2 can interleave with the MFMAs of ks; past
        // the end they read clamped, in-bounds data that is never used
        const int ks = kb + kk;
        half8* bc = (kk & 1) ? b1 : b0;
        half8* bn = (kk & 1) ? b0 : b1;
        half8* ac = (kk & 1) ? aw : av;  // A of ks; refilled with ks + 2
#pragma unroll
        for (int ni = 0; ni < kNB; ++ni)
          bn[ni] = (kk + 1 < kKB) ? dequant(i0, i1b, i1w, ni, kk + 1) : dequant(i0n, i1bn, i1wn, ni, 0);
        const uint32_t ka = akoff(ks + 2 < KS ? ks + 2 : KS - 1);
#pragma unroll
        for (int mi = 0; mi < kMB; ++mi) {
#pragma unroll
          for (int ni = 0; ni < kNB; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ac[mi], bc[ni], acc[mi][ni], 0, 0, 0);
        }
        // the A loads of ks + 2 after every MFMA of ks: with these loads (or
        // scheduling barriers) among the MFMAs the register allocator rotates the
        // accumulators through copies in every iteration
#pragma unroll
        for (int mi = 0; mi < kMB; ++mi) ac[mi] = *reinterpret_cast<const half8*>(abase + arow_off(mi) + ka);
      }
#pragma unroll
      for (int ni = 0; ni < kNB; ++ni) {
        i0[ni] = i0n[ni];
        i1b[ni] = i1bn[ni];
        i1w[ni] = i1wn[ni];
      }
    }

    // ---- z = acc * s / 2: D holds, per lane, output column r16 of each block and
    // tokens 4 q .. 4 q + 3
#pragma unroll
    for (int mi = 0; mi < kMB; ++mi) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + mi * 16 + q * 4 + i;
        if (t < a.M) {
          const int32_t e = a.rexp ? a.rexp[t] : 0;
          float* zr = a.z + t * a.m_pad + o_w + r16;
#pragma unroll
          for (int ni = 0; ni < kNB; ++ni) {
            const float v = row_scaled(acc[mi][ni][i] * a.scale, e);
            zr[16 * ni] = a.accumulate ? zr[16 * ni] + v : v;
          }
        }
      }
    }
  }
}

}  // namespace

bool gemm_lds_supported(const glq_layer& L) {
  // K split in 4 lane quarters of whole index loads (G / 4 a multiple of kKB and of 4
  // groups for 8-byte index loads), whole 256-output tiles, residual from the image
  // or an 8-bit table
  const int64_t G = L.n_pad / 8;
  return L.n_pad >= 256 && (G / 4) % kKB == 0 && L.m_pad % kTN == 0 &&
         (L.resid_bits != 16 || L.cb2_pack == L.cb_pack);
}

hipError_t launch_gemm_lds(const glq_layer& L, const half_t* u16, const int32_t* rexp, int64_t M, bool tiled,
                           float* z, hipStream_t stream, bool accumulate) {
  GemmArgs a;
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
  a.z = z;
  a.M = M;
  a.n_pad = int(L.n_pad);
  a.m_pad = int(L.m_pad);
  a.G = int(L.n_pad / 8);
  a.out_tiles = int(L.m_pad / kTN);
  a.tok_tiles = int((M + kTM - 1) / kTM);
  a.tiles = a.out_tiles * a.tok_tiles;
  a.scale = 0.5f * L.wscale;
  a.sr = L.resid_scale;
  a.accumulate = int(accumulate);
  const int cus = device_cus();
  const int grid = a.tiles < cus ? a.tiles : cus;
#define GLQ_LAUNCH(R, T)                                                                                    \
  do {                                                                                                      \
    if (codes) hipLaunchKernelGGL((gemm_lds_kernel<R, T, true>), dim3(grid), dim3(kPThreads), 0, stream, a); \
    else hipLaunchKernelGGL((gemm_lds_kernel<R, T, false>), dim3(grid), dim3(kPThreads), 0, stream, a);     \
  } while (0)
  switch (L.resid_bits) {
    case 0: if (tiled) GLQ_LAUNCH(0, true); else GLQ_LAUNCH(0, false); break;
    case 8: if (tiled) GLQ_LAUNCH(8, true); else GLQ_LAUNCH(8, false); break;
    default: if (tiled) GLQ_LAUNCH(16, true); else GLQ_LAUNCH(16, false); break;
  }
#undef GLQ_LAUNCH
  return hipGetLastError();
}

GLQ_DEBUG_COUNTER(debug_violations_gemm_lds)

}  // namespace glq
