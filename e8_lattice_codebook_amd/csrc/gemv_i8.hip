// Decode matmul for a few activation rows (4 <= B <= 16) on gfx950: z = u W~^T on the
// int8 matrix units (v_mfma_i32_16x16x64_i8), exact integer products of the
// codewords with 15-bit fixed-point activations.
//
// glq 0.5.1 (PyPI project page), "Inference kernels": the matmul reads the indices
// and the cached codebook and never forms W; for more than one activation row the
// product runs on the matrix units; split-K partial sums are reduced in a fixed order.
// "How it works", items 1 and 4; table "Bit widths".
//
// Activations (quant_i8_kernel): row b of u becomes U = rint(u 2^(14 - E_b)) with
// max|u_b| = f 2^E_b, f in [1/2, 1), so |U| <= 2^14, written as two int8 planes
// U = 256 H + L (H = (U + 128) >> 8 in [-64, 64], L in [-128, 127]) in the order the
// MFMA's activation operand reads them (below).  A row with a NaN or infinity gets a
// NaN poison that the epilogue adds to each of its outputs.
//
// Codewords: a slot word holds 2c as eight signed 4-bit lanes.  Shifted to the high
// half of a byte each lane is 16 (2c), an exact int8; the word's even nibbles give one
// dword (w << 4) & 0xF0F0F0F0, its odd nibbles another, w & 0xF0F0F0F0, so a group's
// eight bytes hold the coordinates in the order 0 4 1 5 2 6 3 7 (nibble j, j + 4 =
// coordinates 2j, 2j + 1).  A complemented read (descending page, negative slot code)
// is negated exactly: in offset binary (nibble + 8) the complement plus one per nibble
// carries nowhere (|2c| <= 6), and XOR 0x8 per nibble returns to two's complement.
// The 16 / 256 factors and 2^(E_b - 14) are undone once per output in fp64.
//
// Tile: a wave owns a unit of 16 output rows and one split of the index blocks (256
// columns each).  At step kk of block kb, lane l = 16 q + r takes row 16 rb + r and the
// groups 32 kb + 8 q + 2 kk, + 1: over a block the lane's groups are 8 q .. 8 q + 7,
// one 16-byte load of eight codes per stage.  The activation operand of that step,
// lane l = 16 q + j, holds token j's 16 columns of the same two groups in the same
// order, for each plane (1 KiB per plane and step).  The result lane l = 16 q + j
// holds outputs 16 rb + 4 q + i (i < 4) of token j: one 16-byte store per unit.
// Workgroups of 16 waves are persistent, one per compute unit (the codebook image
// fills the LDS).  A wave's units, with all their blocks, form one stream: index
// vectors are loaded two blocks ahead and activation fragments one block ahead,
// across unit boundaries.
#include "lds_codebook.h"

namespace glq {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kI8Rows = 16;  // the activation operand's token rows

// ---- activation planes ------------------------------------------------------------
// planes: [n_pad / 64 steps][2 planes: H, L][64 lanes] x 16 bytes; step st = 4 kb + kk
constexpr int kQThreads = 1024;

// the 16 activation bytes of fragment (step st, lane quarter q) of row j: U, then its
// planes H and L
__device__ __forceinline__ void quant_frag(const float* row, int st, int q, int sh, u32x4& h, u32x4& l) {
  // byte b of a fragment: group b / 8, coordinate kPerm[b % 8]
  constexpr int kPerm[8] = {0, 4, 1, 5, 2, 6, 3, 7};
  const int g0 = 32 * (st >> 2) + 8 * q + 2 * (st & 3);
  float v[16];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 t = *reinterpret_cast<const float4*>(row + 8 * g0 + 4 * k);
    v[4 * k] = t.x;
    v[4 * k + 1] = t.y;
    v[4 * k + 2] = t.z;
    v[4 * k + 3] = t.w;
  }
  h = u32x4{0u, 0u, 0u, 0u};
  l = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    const int U = int(rintf(__builtin_amdgcn_ldexpf(v[8 * (b >> 3) + kPerm[b & 7]], sh)));
    const int H = (U + 128) >> 8;
    const int L = U - 256 * H;
    h[b >> 2] |= (uint32_t(H) & 0xFFu) << (8 * (b & 3));
    l[b >> 2] |= (uint32_t(L) & 0xFFu) << (8 * (b & 3));
  }
}

// one workgroup per row j of the 16-row operand: the row's largest |u| (and NaN
// poison), then every fragment of the row; rows j >= B are zeros
__global__ __launch_bounds__(kQThreads) void quant_i8_kernel(const float* __restrict__ u, int B, int n_pad,
                                                             u32x4* __restrict__ planes, I8RowInfo* __restrict__ info) {
  const int j = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ float red_mx[kQThreads / 64], red_po[kQThreads / 64];
  const float* row = u + int64_t(j < B ? j : 0) * n_pad;
  float mx = 0.0f, poison = 0.0f;
  if (j < B) {
    // four float4 loads in flight per thread at a time
    for (int c0 = 4 * tid; c0 < n_pad; c0 += 16 * kQThreads) {
      float4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = c0 + 4 * k * kQThreads;
        v[k] = c < n_pad ? *reinterpret_cast<const float4*>(row + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        mx = fmaxf(fmaxf(mx, fabsf(v[k].x)), fmaxf(fabsf(v[k].y), fmaxf(fabsf(v[k].z), fabsf(v[k].w))));
        poison += (v[k].x - v[k].x) + (v[k].y - v[k].y) + (v[k].z - v[k].z) + (v[k].w - v[k].w);  // 0 or NaN
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    poison += __shfl_xor(poison, off, 64);
  }
  if ((tid & 63) == 0) {
    red_mx[tid >> 6] = mx;
    red_po[tid >> 6] = poison;
  }
  __syncthreads();
  mx = 0.0f;
  poison = 0.0f;
#pragma unroll
  for (int w = 0; w < kQThreads / 64; ++w) {  // the same order in every thread
    mx = fmaxf(mx, red_mx[w]);
    poison += red_po[w];
  }
  const bool live = mx > 0.0f && poison == 0.0f;  // finite with a nonzero element
  const int e = live ? __builtin_amdgcn_frexp_expf(mx) : 0;
  const int sh = 14 - e;
  const int frags = (n_pad >> 6) * 4;  // (step, lane quarter)
  // two fragments per thread at a time, both loaded before either is converted
  for (int f0 = tid; f0 < frags; f0 += 2 * kQThreads) {
    u32x4 h[2], l[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int f = f0 + k * kQThreads;
      h[k] = u32x4{0u, 0u, 0u, 0u};
      l[k] = u32x4{0u, 0u, 0u, 0u};
      if (live && f < frags) quant_frag(row, f >> 2, f & 3, sh, h[k], l[k]);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int f = f0 + k * kQThreads;
      if (f < frags) {
        const int st = f >> 2, q = f & 3;
        planes[(2 * st) * 64 + 16 * q + j] = h[k];
        planes[(2 * st + 1) * 64 + 16 * q + j] = l[k];
      }
    }
  }
  if (tid == 0) info[j] = I8RowInfo{e, j < B ? poison : 0.0f};
}

// ---- codeword operand dwords --------------------------------------------------------
// the two dwords (16 x 2c, coordinate order 0 4 1 5 | 2 6 3 7) of slot word n read
// complemented when m = ~0; c = m & 0x11111111 (the +1 of the complement per nibble)
__device__ __forceinline__ u32x2 a_dwords(uint32_t x, uint32_t c) {
  // x = n ^ m: offset binary, plus one per complemented nibble (no carries)
  const uint32_t t = (x ^ 0x88888888u) + c;
  return u32x2{((t << 4) & 0xF0F0F0F0u) ^ 0x80808080u, (t & 0xF0F0F0F0u) ^ 0x80808080u};
}

// the operand (4 dwords: group 2k, then 2k + 1) of the two codes in word w
template <bool CODES>
__device__ __forceinline__ u32x4 stage_operand(const uint32_t* lds, uint32_t w, uint32_t nd, uint32_t two) {
  u32x4 r;
  if constexpr (CODES) {
    uint32_t mm, n0, n1;
    code_pair(lds, w, nd, mm, n0, n1);
    const uint32_t k1 = 0x11111111u;
    uint32_t c0, c1;
    asm("v_and_b32_sdwa %0, sext(%1), %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_0 src1_sel:DWORD"
        : "=v"(c0) : "v"(mm), "v"(k1));
    asm("v_and_b32_sdwa %0, sext(%1), %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1 src1_sel:DWORD"
        : "=v"(c1) : "v"(mm), "v"(k1));
    const u32x2 d0 = a_dwords(xor_half_mask<0>(n0, mm), c0), d1 = a_dwords(xor_half_mask<1>(n1, mm), c1);
    r = u32x4{d0.x, d0.y, d1.x, d1.y};
  } else {
    const uint32_t d0 = page_desc<0>(lds, w, two), d1 = page_desc<1>(lds, w, two);
    const uint32_t m0 = page_mask(d0), m1 = page_mask(d1);
    const uint32_t n0 = slot_word<0>(lds, w, d0, m0, two), n1 = slot_word<1>(lds, w, d1, m1, two);
    const u32x2 e0 = a_dwords(n0 ^ m0, m0 & 0x11111111u), e1 = a_dwords(n1 ^ m1, m1 & 0x11111111u);
    r = u32x4{e0.x, e0.y, e1.x, e1.y};
  }
  return r;
}

struct I8Args {
  const u32x4* planes;        // activation planes (quant_i8_kernel)
  const I8RowInfo* info;      // [16] per token row: exponent, poison
  const uint16_t* idx0;       // [m_pad][G]
  const void* idx1;           // [m_pad][G] u8 or u16
  const uint32_t* pack0_hdr;
  const uint32_t* img0;       // page image (codebook indices) or slot image (slot codes)
  const uint32_t* res_slots;  // 8-bit residual: the 256 slot words of its pack
  float* z;                   // [splits][B][m_pad]
  int B, m_pad, G;
  int kbs, lkbs;              // index blocks per split (a power of two) and its log2
  int row_groups, units;      // units: row groups (16 RB rows) x splits
  double scale;               // s / 2 / 16 (codewords held doubled, operand bytes 16 x)
  double sr;
  int accumulate;             // add to z (second pass of a 5-8 bpw layer)
};

// RB: 16-row blocks per wave (each activation fragment serves RB codeword operands);
// 16 waves per workgroup for RB = 1, 8 (with twice the registers) for RB = 4
template <int RB>
constexpr int i8_threads() {
  return RB <= 2 ? 1024 : 512;
}

// The body of one workgroup: workgroup wg of the nwg that serve this layer.
template <int RESID, bool CODES, int RB>
__device__ __forceinline__ void gemv_i8_body(const I8Args& a, int wg, int nwg) {
  constexpr int kT = i8_threads<RB>();
  constexpr int kW = kT / 64;
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsDwords];
  __shared__ __attribute__((aligned(16))) u32x2 res8[RESID == 8 ? 256 : 1];  // 8-bit stage operand dwords
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const uint32_t two = 2;
  const uint32_t nd = CODES ? pair_ndelta(slot_delta(a.pack0_hdr)) : 0u;

  const int q = lane >> 4;
  const int r16 = lane & 15;
  const int wave_g = __builtin_amdgcn_readfirstlane(wg * kW + (tid >> 6));
  const int nwaves = nwg * kW;
  const int n_mine = wave_g < a.units ? (a.units - 1 - wave_g) / nwaves + 1 : 0;
  const int npos = n_mine << a.lkbs;  // (unit, block) positions of the wave's stream
  const uint8_t* idx1_8 = static_cast<const uint8_t*>(a.idx1);
  const uint16_t* idx1_16 = static_cast<const uint16_t*>(a.idx1);
  const int G = a.G;
  const int kmask = a.kbs - 1;

  // token row of the lane's results: exponent and poison
  const I8RowInfo ri = a.info[r16];

  struct Pos {
    int split, rg, kb;
  };
  auto pos_of = [&](int p) {
    p = p < npos ? p : npos - 1;  // past the stream's end: its last block again (never used)
    const int unit = wave_g + (p >> a.lkbs) * nwaves;
    Pos r;
    r.split = unit / a.row_groups;
    r.rg = unit - r.split * a.row_groups;
    r.kb = (r.split << a.lkbs) + (p & kmask);
    return r;
  };
  struct Idx {
    u32x4 i0[RB], i1w[RB];
    u32x2 i1b[RB];
  };
  auto load_idx = [&](int p, Idx& d) {
    const Pos s = pos_of(p);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int64_t off = int64_t((s.rg * RB + r) * 16 + r16) * G + 32 * s.kb + 8 * q;
      d.i0[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.idx0 + off));
      if (RESID == 16) d.i1w[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(idx1_16 + off));
      if (RESID == 8) d.i1b[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(idx1_8 + off));
    }
  };
  // the activation fragments (both planes) of step kk of block p
  auto act_src = [&](int p) { return a.planes + int64_t(8 * pos_of(p).kb) * 64 + lane; };


  // ---- the image into LDS: every 16-byte part of the thread loaded before any is
  // stored (all in flight at once; parts past the end re-read the last one, which its
  // owner stores with the same value), the last partial uint4 by words; the 8-bit
  // stage's entries as operand dwords
  {
    constexpr int kParts = (kImageMaxDwords / 4 + kT - 1) / kT;
    uint32_t ndw = a.pack0_hdr[CODES ? kHdrSlotDwords : 3];
    ndw = ndw > uint32_t(kImageMaxDwords) ? uint32_t(kImageMaxDwords) : ndw;
    const uint32_t nd4 = ndw >> 2;
    const uint32_t last4 = nd4 > 0 ? nd4 - 1 : 0;
    const u32x4* src4 = reinterpret_cast<const u32x4*>(a.img0);
    u32x4* dst4 = reinterpret_cast<u32x4*>(lds + kImgOff);
    u32x4 t[kParts];
#pragma unroll
    for (int k = 0; k < kParts; ++k) t[k] = src4[min(uint32_t(k * kT + tid), last4)];
    uint32_t tail = 0;
    const uint32_t ti = (nd4 << 2) + tid;
    if (ti < ndw) tail = a.img0[ti];
    if (nd4 > 0) {
#pragma unroll
      for (int k = 0; k < kParts; ++k) dst4[min(uint32_t(k * kT + tid), last4)] = t[k];
    }
    if (ti < ndw) lds[kImgOff + ti] = tail;
  }
  if (RESID == 8 && tid < 256) {
    const uint32_t w = a.res_slots[tid];
    res8[tid] = u32x2{(w << 4) & 0xF0F0F0F0u, w & 0xF0F0F0F0u};
  }
  __syncthreads();

  i32x4 acc[RB][2][2];  // [row block][stage][plane]
  auto zero_acc = [&]() {
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) acc[r][s][pl] = i32x4{0, 0, 0, 0};
  };
  // z[split][j][16 (rg RB + r) + 4 q + i] for the lane's token j = r16 < B
  auto store_unit = [&](int p) {
    const Pos s = pos_of(p);
    if (r16 < a.B) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          double t = double(int64_t(acc[r][0][0][i]) * 256 + acc[r][0][1][i]);
          if (RESID != 0) t += a.sr * double(int64_t(acc[r][1][0][i]) * 256 + acc[r][1][1][i]);
          v[i] = float(ldexp(t * a.scale, ri.e - 14)) + ri.poison;
        }
        float4* zo = reinterpret_cast<float4*>(a.z + (int64_t(s.split) * a.B + r16) * a.m_pad +
                                               (s.rg * RB + r) * 16 + 4 * q);
        float4 o = make_float4(v[0], v[1], v[2], v[3]);
        if (a.accumulate) {
          const float4 z0 = *zo;
          o = make_float4(z0.x + o.x, z0.y + o.y, z0.z + o.z, z0.w + o.w);
        }
        *zo = o;
      }
    }
  };

  auto mfma = [](const u32x4& w, const u32x4& x, i32x4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, w), __builtin_bit_cast(i32x4, x), c, 0, 0,
                                                 0);
  };
  // one block: four steps of the stage operands against the fragments f, each step's
  // registers reloaded with block p + 1's once its products are issued
  auto block = [&](int p, const Idx& ix, u32x4 (&f)[4][2]) {
    const u32x4* next = act_src(p + 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const u32x4 a0 = stage_operand<CODES>(lds, ix.i0[r][kk], nd, two);
        acc[r][0][0] = mfma(a0, f[kk][0], acc[r][0][0]);
        acc[r][0][1] = mfma(a0, f[kk][1], acc[r][0][1]);
        if (RESID != 0) {
          u32x4 a1;
          if (RESID == 16) {
            a1 = stage_operand<CODES>(lds, ix.i1w[r][kk], nd, two);
          } else {
            // the bytes of groups 8 q + 2 kk, + 1: bytes 2 kk, 2 kk + 1 of the lane's eight
            const uint32_t w = ix.i1b[r][kk >> 1];
            const uint32_t b0 = (kk & 1) ? (w >> 16) & 0xFFu : w & 0xFFu;
            const uint32_t b1 = (kk & 1) ? w >> 24 : (w >> 8) & 0xFFu;
            const u32x2 e0 = res8[b0], e1 = res8[b1];
            a1 = u32x4{e0.x, e0.y, e1.x, e1.y};
          }
          acc[r][1][0] = mfma(a1, f[kk][0], acc[r][1][0]);
          acc[r][1][1] = mfma(a1, f[kk][1], acc[r][1][1]);
        }
      }
      f[kk][0] = next[(2 * kk) * 64];
      f[kk][1] = next[(2 * kk + 1) * 64];
    }
    if ((p & kmask) == kmask) {  // the unit's last block
      store_unit(p);
      zero_acc();
    }
  };

  if (npos == 0) return;  // after the barrier: no wave waits for this one again
  // the stream's first index vectors and fragments (after the image copy: its stores
  // would otherwise wait for these first, cold HBM reads)
  Idx x0, x1, x2;
  u32x4 f[4][2];
  load_idx(0, x0);
  load_idx(1, x1);
  {
    const u32x4* src = act_src(0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      f[kk][0] = src[(2 * kk) * 64];
      f[kk][1] = src[(2 * kk + 1) * 64];
    }
  }
  zero_acc();
  // index vectors in a ring of three sets, each loaded two blocks ahead; whole turns of
  // the ring in a loop with no early exit (an exit merged into the loop latch makes the
  // compiler wait for every load at the loop head), then the rest
  int p = 0;
  for (; p + 2 < npos; p += 3) {
    load_idx(p + 2, x2);
    block(p, x0, f);
    load_idx(p + 3, x0);
    block(p + 1, x1, f);
    load_idx(p + 4, x1);
    block(p + 2, x2, f);
  }
  if (p < npos) block(p, x0, f);
  if (p + 1 < npos) block(p + 1, x1, f);
}

template <int RESID, bool CODES, int RB>
__global__ __launch_bounds__(i8_threads<RB>(), 1) void gemv_i8_kernel(I8Args a) {
  gemv_i8_body<RESID, CODES, RB>(a, int(blockIdx.x), int(gridDim.x));
}

// Several layers' GEMVs in one launch: layer k owns the workgroups [end[k-1], end[k])
// of the grid and runs the per-layer body over them.  The layers share RESID, CODES
// and RB; their arguments are their own.
struct I8GroupArgs {
  I8Args L[GLQ_GROUP_MAX];
  int end[GLQ_GROUP_MAX];
  int count;
};

template <int RESID, bool CODES, int RB>
__global__ __launch_bounds__(i8_threads<RB>(), 1) void gemv_i8_group_kernel(I8GroupArgs g) {
  const int bid = int(blockIdx.x);
  int k = 0;
#pragma unroll
  for (int j = 0; j < GLQ_GROUP_MAX - 1; ++j) k += (j < g.count - 1 && bid >= g.end[j]) ? 1 : 0;
  k = __builtin_amdgcn_readfirstlane(k);
  const int start = k > 0 ? g.end[k - 1] : 0;
  gemv_i8_body<RESID, CODES, RB>(g.L[k], bid - start, g.end[k] - start);
}

struct I8Plan {
  int rb, threads, splits, kbs, lkbs, row_groups, units;
};

// cus: the CUs the layer's launch may fill (all of them for a layer on its own)
I8Plan i8_plan(int64_t n_pad, int64_t m_pad, int cus) {
  const int KB = int(n_pad / 256);
  // four row blocks per wave (8 waves per CU) where its units fill every wave slot,
  // else one (16 waves per CU); splits (powers of two dividing KB, at most 16: the
  // output transform sums them per element, and at least 2 blocks per unit) until the
  // units fill the slots
  I8Plan p{};
  for (const int rb : {4, 1}) {
    if (m_pad % (16 * rb) != 0) continue;
    p.rb = rb;
    p.threads = rb == 4 ? i8_threads<4>() : i8_threads<1>();
    p.row_groups = int(m_pad / (16 * rb));
    const int64_t slots = int64_t(cus) * (p.threads / 64);
    int s = 1;
    while (int64_t(p.row_groups) * s < slots && KB % (2 * s) == 0 && KB / (2 * s) >= 2 && s < 16) s *= 2;
    p.splits = s;
    if (rb == 4 && int64_t(p.row_groups) * s < slots) continue;
    break;
  }
  p.kbs = KB / p.splits;
  p.lkbs = 0;
  while ((1 << p.lkbs) < p.kbs) ++p.lkbs;
  p.units = p.row_groups * p.splits;
  return p;
}

template <int RESID, bool CODES>
hipError_t launch_t(const I8Args& a, int rb, hipStream_t stream) {
  const int cus = device_cus();
  const int waves = (rb == 4 ? i8_threads<4>() : i8_threads<1>()) / 64;
  const int need = (a.units + waves - 1) / waves;
  const dim3 grid(unsigned(need < cus ? need : cus)), block(unsigned(waves * 64));
  switch (rb) {
    case 1: hipLaunchKernelGGL((gemv_i8_kernel<RESID, CODES, 1>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((gemv_i8_kernel<RESID, CODES, 4>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace

bool gemv_i8_supported(const glq_layer& L) {
  // whole 256-column index blocks with a power-of-two count, whole 16-row units; the
  // residual from the primary image or an 8-bit table
  const int64_t kb = L.n_pad / 256;
  return L.n_pad % 256 == 0 && kb >= 1 && (kb & (kb - 1)) == 0 && L.m_pad % 16 == 0 &&
         (L.resid_bits != 16 || L.cb2_pack == L.cb_pack);
}

int gemv_i8_splits(int64_t n_pad, int64_t m_pad) { return i8_plan(n_pad, m_pad, device_cus()).splits; }

size_t i8_planes_bytes(int64_t n_pad) { return size_t(n_pad / 64) * 2 * 64 * 16; }

hipError_t launch_quant_i8(const float* u, int64_t B, int64_t n_pad, void* planes, I8RowInfo* info,
                           hipStream_t stream) {
  hipLaunchKernelGGL(quant_i8_kernel, dim3(kI8Rows), dim3(kQThreads), 0, stream, u, int(B), int(n_pad),
                     static_cast<u32x4*>(planes), info);
  return hipGetLastError();
}

namespace {

bool codes_of(const glq_layer& L) { return L.index_format == GLQ_INDEX_SLOT; }

I8Args i8_args(const glq_layer& L, const I8Plan& p, const void* planes, const I8RowInfo* info, int64_t B,
               float* z_parts, bool accumulate) {
  I8Args a;
  a.planes = static_cast<const u32x4*>(planes);
  a.info = info;
  a.idx0 = L.idx0;
  a.idx1 = L.idx1;
  const char* p0 = static_cast<const char*>(L.cb_pack);
  a.pack0_hdr = reinterpret_cast<const uint32_t*>(p0);
  a.img0 = reinterpret_cast<const uint32_t*>(
      p0 + (codes_of(L) ? pack_slot_image_offset(GLQ_CODEBOOK_ENTRIES) : pack_image_offset(GLQ_CODEBOOK_ENTRIES)));
  a.res_slots = L.resid_bits == 8 ? reinterpret_cast<const uint32_t*>(static_cast<const char*>(L.cb2_pack) +
                                                                     pack_image_offset(GLQ_RESID8_ENTRIES)) + kPageCount
                                   : nullptr;
  a.z = z_parts;
  a.B = int(B);
  a.m_pad = int(L.m_pad);
  a.G = int(L.n_pad / 8);
  a.kbs = p.kbs;
  a.lkbs = p.lkbs;
  a.row_groups = p.row_groups;
  a.units = p.units;
  a.scale = 0.5 * double(L.wscale) / 16.0;
  a.sr = double(L.resid_scale);
  a.accumulate = int(accumulate);
  return a;
}

// workgroups of a launch over p's units, at most cus of them
int i8_grid(const I8Plan& p, int cus) {
  const int waves = p.threads / 64;
  const int need = (p.units + waves - 1) / waves;
  return need < cus ? need : cus;
}

// the CUs each layer of a group may fill: its own plan when the layers' grids fit the
// device together, else a share of the CUs in proportion to the layer's index groups
void i8_group_cus(const glq_layer* Ls, int count, int* cus) {
  const int all = device_cus();
  int64_t wgs = 0, work = 0;
  for (int k = 0; k < count; ++k) {
    wgs += i8_grid(i8_plan(Ls[k].n_pad, Ls[k].m_pad, all), all);
    work += Ls[k].m_pad * (Ls[k].n_pad / 8);
  }
  for (int k = 0; k < count; ++k) {
    const int64_t share = int64_t(all) * (Ls[k].m_pad * (Ls[k].n_pad / 8)) / work;
    cus[k] = wgs <= all ? all : int(share > 1 ? share : 1);
  }
}

template <int RESID, bool CODES>
hipError_t launch_group_t(const I8GroupArgs& g, int rb, int wgs, hipStream_t stream) {
  const int threads = rb == 4 ? i8_threads<4>() : i8_threads<1>();
  switch (rb) {
    case 1: hipLaunchKernelGGL((gemv_i8_group_kernel<RESID, CODES, 1>), dim3(unsigned(wgs)), dim3(threads), 0, stream, g); break;
    default: hipLaunchKernelGGL((gemv_i8_group_kernel<RESID, CODES, 4>), dim3(unsigned(wgs)), dim3(threads), 0, stream, g); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_i8(const glq_layer& L, const void* planes, const I8RowInfo* info, int64_t B, float* z_parts,
                          hipStream_t stream, bool accumulate) {
  const I8Plan p = i8_plan(L.n_pad, L.m_pad, device_cus());
  const I8Args a = i8_args(L, p, planes, info, B, z_parts, accumulate);
  switch (L.resid_bits) {
    case 0: return codes_of(L) ? launch_t<0, true>(a, p.rb, stream) : launch_t<0, false>(a, p.rb, stream);
    case 8: return codes_of(L) ? launch_t<8, true>(a, p.rb, stream) : launch_t<8, false>(a, p.rb, stream);
    default: return codes_of(L) ? launch_t<16, true>(a, p.rb, stream) : launch_t<16, false>(a, p.rb, stream);
  }
}

bool gemv_i8_group_plan(const glq_layer* Ls, int count, int* splits) {
  if (count < 1 || count > GLQ_GROUP_MAX) return false;
  int cus[GLQ_GROUP_MAX];
  i8_group_cus(Ls, count, cus);
  int rb = 0;
  for (int k = 0; k < count; ++k) {
    if (!gemv_i8_supported(Ls[k]) || Ls[k].resid_bits != Ls[0].resid_bits || codes_of(Ls[k]) != codes_of(Ls[0]))
      return false;
    const I8Plan p = i8_plan(Ls[k].n_pad, Ls[k].m_pad, cus[k]);
    if (k == 0) rb = p.rb;
    if (p.rb != rb) return false;
    if (splits) splits[k] = p.splits;
  }
  return true;
}

hipError_t launch_gemv_i8_group(const glq_layer* Ls, int count, const void* const* planes,
                                const I8RowInfo* const* info, int64_t B, float* const* z_parts, hipStream_t stream) {
  int cus[GLQ_GROUP_MAX];
  i8_group_cus(Ls, count, cus);
  I8GroupArgs g;
  int wgs = 0, rb = 1;
  for (int k = 0; k < count; ++k) {
    const I8Plan p = i8_plan(Ls[k].n_pad, Ls[k].m_pad, cus[k]);
    g.L[k] = i8_args(Ls[k], p, planes[k], info[k], B, z_parts[k], false);
    wgs += i8_grid(p, cus[k]);
    g.end[k] = wgs;
    rb = p.rb;  // the same for every layer (gemv_i8_group_plan)
  }
  for (int k = count; k < GLQ_GROUP_MAX; ++k) g.end[k] = 0x7FFFFFFF;
  g.count = count;
  const bool codes = codes_of(Ls[0]);
  switch (Ls[0].resid_bits) {
    case 0: return codes ? launch_group_t<0, true>(g, rb, wgs, stream) : launch_group_t<0, false>(g, rb, wgs, stream);
    case 8: return codes ? launch_group_t<8, true>(g, rb, wgs, stream) : launch_group_t<8, false>(g, rb, wgs, stream);
    default: return codes ? launch_group_t<16, true>(g, rb, wgs, stream) : launch_group_t<16, false>(g, rb, wgs, stream);
  }
}

GLQ_DEBUG_COUNTER(debug_violations_gemv_i8)

}  // namespace glq
