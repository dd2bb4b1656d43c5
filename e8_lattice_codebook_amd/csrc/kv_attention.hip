// Decode attention over an E8-compressed paged K/V cache on gfx950.
//
// Glq v0.5.0 release notes, "Highlights": the compressed K/V is dequantized inside
// the attention kernel's tile loop, the inverse Hadamard rotation is an 8-point
// FHT butterfly, and long contexts are split over workgroups (flash-decoding);
// glq 0.5.1, "KV cache compression" -> "E8 lattice cache": the same E8 lattice
// quantizer as the weights, the 4 bpw recipe e8_relaxed:2.
//
// A cached vector (head_dim D) is D/8 groups; group g holds e_g = C[i0] (+ s_r C[i1])
// and reads back as x_g = s H8 e_g / sqrt(8), one fp32 scale s per (token, head).
// The rotation is orthonormal and symmetric, so it never runs per cached token:
//   q . x = s (H8 q_g / sqrt(8)) . e_g   (the query is rotated once), and
//   sum_t p_t x_t = H8 (sum_t p_t s_t e_t) / sqrt(8)   (rotated once, after the sum).
// What remains per token is a codebook lookup (slot image in LDS, as in the
// linear), the codeword's int4 lanes as exact fp16 pairs, and fp32 dot products
// (K) or FMAs (V).
//
// Kernel 1 (kv_split_kernel): persistent workgroups of 512 threads, one per CU, the
// codebook image loaded into LDS once.  A unit is (sequence b, KV head h, chunk of
// T tokens) taken in sub-chunks of up to 256 tokens.  Per unit the G query heads
// of h are rotated and held as fp16 pairs.  Per sub-chunk every wave scores its
// tokens (lanes = token x stage x group, a DPP reduction per token), one wave per
// head updates the running max and exp-sum (an online softmax: earlier V sums are
// rescaled when the max grows), and the same lanes add p s_v 2c into their V sums;
// the next sub-chunk's loads are issued one phase ahead.  At the end of the unit
// the lanes of a group and then the waves (in wave order) are added and the
// unit's (max, sum, o) go to the workspace.  Kernel 2 (kv_combine_kernel) merges a
// sequence's chunks in chunk order, divides, applies the 8-point butterfly and
// 1/sqrt(8), and casts.
#include <math.h>

#include "fwht_lds.h"
#include "lds_codebook.h"

namespace glq {
namespace {

// 8 waves (2 per SIMD, up to 256 registers each): the query digits, the per-head V
// sums and a batch of loads in flight fit without serializing the loads
constexpr int kKvThreads = 512;
constexpr int kKvWaves = kKvThreads / 64;
constexpr int kKvBuf = 1280;  // floats of LDS beside the image: query staging, planes, scores

struct KvArgs {
  const void* q;
  int q_dt;
  const uint16_t* k0;
  const uint16_t* k1;
  const uint16_t* v0;
  const uint16_t* v1;
  const float* ks;
  const float* vs;
  const int32_t* block_table;
  int64_t bt_stride;
  const int32_t* seq_lens;
  const uint32_t* pack_hdr;
  const uint32_t* img;
  float* part_o;   // [units][G][D]
  float* part_ml;  // [units][G][2]: chunk max, sum of exp(score - max)
  int Hkv, lp, T, splits, units;  // T: tokens per unit
  int TS;                          // tokens per sub-chunk (the scores buffer holds TS x G)
  int num_pages;    // page indices are clamped to [0, num_pages)
  int max_len;      // seq_lens are clamped to [0, max_len] (max_seq_len, and the block table's reach)
  float sm_scale, resid_scale;
  int rk;  // two stages with resid_scale = 2^-rk (0 <= rk <= 4): merged exactly in integers
};

__device__ __forceinline__ float q_value(const void* q, int dt, int64_t i) {
  switch (dt) {
    case GLQ_F32: return static_cast<const float*>(q)[i];
    case GLQ_F16: return float(static_cast<const half_t*>(q)[i]);
    default: return __uint_as_float(uint32_t(static_cast<const uint16_t*>(q)[i]) << 16);
  }
}

__device__ __forceinline__ uint32_t img_word(const uint32_t* img, uint32_t byte_addr) {
  GLQ_DCHECK(byte_addr < uint32_t(kImageMaxDwords) * 4u);
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(img) + byte_addr);
}

// The stored word of 16-bit value c and m (all ones: the entry is the word's
// negation, lane by lane).  Slot codes: slot (c ^ m) + (m & delta) with m the sign
// of c as int16.  Codebook indices: the page descriptor (word c >> 8, bit 0 = m),
// then byte ((4 (c & 255)) ^ m) + desc.
template <bool CODES>
__device__ __forceinline__ uint32_t kv_word(const uint32_t* img, uint32_t c, uint32_t delta, uint32_t& m) {
  if constexpr (CODES) {
    const int32_t s = int32_t(int16_t(uint16_t(c)));
    m = uint32_t(s >> 31);
    return img_word(img, ((uint32_t(s) ^ m) + (m & delta)) << 2);
  } else {
    const uint32_t desc = img[c >> 8];
    m = uint32_t(__builtin_amdgcn_sbfe(desc, 0, 1));
    return img_word(img, ((4u * (c & 255u)) ^ m) + desc);
  }
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Decoding.  The workgroup's LDS copy of the image holds every codeword word XOR
// 0x8888_8888, so for stored value c with word w and m (all ones: the entry is the
// word's negation) t = w ^ m has nibble j equal to 2c_j + 8 - mb (mb = m & 1): offset
// binary either way.  Nibbles k and k + 4 hold coordinates 2k and 2k + 1.  A byte N
// <= 255 placed as the low byte of an fp16 with high byte 0x64 reads 1024 + N
// exactly, so the pairs come from byte permutes of the even and odd nibbles and one
// fp16 add of the bias.
constexpr uint32_t kC64 = 0x64646464u;
constexpr uint32_t kSel02 = 0x04020400u;  // (byte 0, 0x64, byte 2, 0x64)
constexpr uint32_t kSel13 = 0x04030401u;  // (byte 1, 0x64, byte 3, 0x64)

// fp16 pairs (N_a + 1024, N_b + 1024) of even-nibble bytes lo and odd-nibble bytes hi,
// plus bias nb: pairs (coordinates 0, 1), (2, 3), (4, 5), (6, 7)
__device__ __forceinline__ void byte_pairs(uint32_t lo, uint32_t hi, uint32_t nb, half2v (&p)[4]) {
  const half2v b = __builtin_bit_cast(half2v, nb);
  p[0] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(kC64, lo, kSel02)) + b;
  p[1] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(kC64, hi, kSel02)) + b;
  p[2] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(kC64, lo, kSel13)) + b;
  p[3] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(kC64, hi, kSel13)) + b;
}

// one stage: 2c as fp16 pairs (bias -(1032 - mb): 0xE408, or 0xE407 negated)
__device__ __forceinline__ void stage_pairs(uint32_t w, uint32_t m, half2v (&p)[4]) {
  const uint32_t t = w ^ m;
  byte_pairs(t & 0x0F0F0F0Fu, (t >> 4) & 0x0F0F0F0Fu, 0xE408E408u + (m & 0xFFFEFFFFu), p);
}

// Decode constants of a call: the residual shift rk and its biases
struct KvDecode {
  int rk;
  uint32_t nbase;  // -(1024 + 8 2^rk + 8) in both halves
  uint32_t nk;     // -(2^rk) in both halves (added when stage 0 is negated)
  half2v rs2;      // resid_scale in both halves (two stages, any scale)
};

// The LDS words of stored values c0, c1 (one codeword, both stages) and their masks
struct CwWords {
  uint32_t w0, m0, w1, m1;
};
template <int MODE, bool CODES>
__device__ __forceinline__ CwWords kv_lookup(const uint32_t* img, uint32_t c0, uint32_t c1, uint32_t delta) {
  CwWords r;
  r.w0 = kv_word<CODES>(img, c0, delta, r.m0);
  r.w1 = 0u;
  r.m1 = 0u;
  if constexpr (MODE != 0) r.w1 = kv_word<CODES>(img, c1, delta, r.m1);
  return r;
}

// The codeword as 8 fp16 (pairs of coordinates), times 2^rk for MODE 1.  MODE 0: one
// stage, 2c0.  MODE 1: resid_scale = 2^-rk, bytes N = 2^rk (2c0 + 8 - mb0) +
// (2c1 + 8 - mb1) <= 255 merged in integers, then one bias: 2^rk 2c0 + 2c1 exactly.
// MODE 2: any resid_scale, 2c0 + s_r 2c1 in fp16.
template <int MODE>
__device__ __forceinline__ void kv_decode(const CwWords& cw, const KvDecode& dc, half2v (&p)[4]) {
  if constexpr (MODE == 0) {
    stage_pairs(cw.w0, cw.m0, p);
  } else if constexpr (MODE == 1) {
    const uint32_t t0 = cw.w0 ^ cw.m0, t1 = cw.w1 ^ cw.m1;
    const uint32_t lo = ((t0 & 0x0F0F0F0Fu) << dc.rk) + (t1 & 0x0F0F0F0Fu);
    const uint32_t hi = (((t0 >> 4) & 0x0F0F0F0Fu) << dc.rk) + ((t1 >> 4) & 0x0F0F0F0Fu);
    byte_pairs(lo, hi, dc.nbase + (cw.m0 & dc.nk) + (cw.m1 & 0xFFFEFFFFu), p);
  } else {
    half2v p1[4];
    stage_pairs(cw.w0, cw.m0, p);
    stage_pairs(cw.w1, cw.m1, p1);
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = p1[j] * dc.rs2 + p[j];
  }
}

// Over the four rows of 16 lanes (lanes l, l ^ 16, l ^ 32, l ^ 48): the max / sum in
// every lane, the same operands in the same order in each (the swaps exchange odd and
// even rows, then the halves of the wave)
__device__ __forceinline__ float xq_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float xq_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

typedef _Float16 half4v __attribute__((ext_vector_type(4)));

// Each wave streams its own tiles of 16 tokens of the unit (tiles wave, wave + 8, ...)
// with its own online softmax; no barrier separates the phases of a tile.  Lane l is
// (c, q) = (l mod 16, l / 16).
//  - scores: one MFMA 16 x 16 x 32 per k-step of 32 dimensions, A = the tile's tokens
//    (rows) x dimensions, B = dimensions x the query heads (columns, zero past G).  At
//    k-step ks lane (c, q) holds group q KS + ks of token c, so its KS k-steps read KS
//    consecutive groups; the query fragments match.  D gives lane (c, q) head c for
//    tokens 4q .. 4q + 3.
//  - softmax: per head, the max of the lane's four scores and then over the four rows
//    of lanes; the running max and exp-sum updated, p = exp(s - max) (0 past the unit).
//  - V: O^T += V^T W^T as GPS / 2 MFMAs 16 x 16 x 16: A = 16 rows of V's columns x the
//    tile's tokens, B = tokens x heads, W the weights p s_v / 2.  Lane (c, q) decodes
//    group c mod GPS of tokens 4q .. 4q + 3 (all 8 coordinates; with D = 64 row c
//    takes coordinates 4 (c / 8) .. + 3) and already holds W for head c and those
//    tokens: no lane exchange.  D gives lane (c, q) head c for the 4 V columns 4q + i
//    of each MFMA, so the rescaling of the sums by exp(max_old - max_new) is the
//    lane's own.  W is fp16 (p <= 1, rounded once); the V scales are taken relative to
//    a running power of two 2^e (the largest scale's exponent so far), which is folded
//    into the rescaling, so W stays in (0, 1/2].
// At the end of the unit the waves are merged in wave order (max, sum and V sums
// rescaled to the common max) in LDS.
// BIG: pages of 16 tokens or more, so a tile (16 aligned tokens) lies on one page and
// its rows are one uniform row plus per-lane constants.
template <int D, int G, int MODE, bool CODES, bool BIG>
__global__ __launch_bounds__(kKvThreads, 1) void kv_split_kernel(KvArgs a) {
  constexpr int GPS = D / 8;  // groups per vector
  constexpr int KS = D / 32;  // score k-steps per vector
  constexpr int NK = GPS / 2; // V MFMAs per tile: 16 columns each, D in all
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  static_assert(G * D <= kKvBuf && G * (D + 2) <= kKvBuf, "query staging and the wave merge fit");

  __shared__ __attribute__((aligned(16))) uint32_t img[kImageMaxDwords];
  __shared__ __attribute__((aligned(16))) float buf[kKvBuf];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the tile loop branches on it
  // The codebook image, copied to LDS in two steps: the loads (issued with the first
  // unit's first reads of the cache, so their latencies overlap), then the stores.
  // Every load is in flight before the first store (clamped addresses: a thread past
  // the end rewrites the last uint4 with the value found there).  Codeword words (all
  // of the slot image; past the page table of the index image) are stored in offset
  // binary: XOR 0x8888_8888.
  uint32_t nd = a.pack_hdr[CODES ? kHdrSlotDwords : 3];
  nd = nd > uint32_t(kImageMaxDwords) ? uint32_t(kImageMaxDwords) : nd;
  const uint32_t nd4 = nd >> 2;
  const uint32_t last4 = nd4 > 0 ? nd4 - 1 : 0;
  constexpr int kParts = (kImageMaxDwords / 4 + kKvThreads - 1) / kKvThreads;
  constexpr uint32_t kFirstWord4 = CODES ? 0u : uint32_t(kPageCount / 4);
  const uint32_t img_ti = (nd4 << 2) + tid;
  auto image_loads = [&](img_x4 (&imt)[kParts], uint32_t& img_tail) {
    const img_x4* src = reinterpret_cast<const img_x4*>(a.img);
#pragma unroll
    for (int k = 0; k < kParts; ++k) imt[k] = src[min(uint32_t(tid + k * kKvThreads), last4)];
    img_tail = img_ti < nd ? a.img[img_ti] : 0u;
  };
  auto image_stores = [&](const img_x4 (&imt)[kParts], uint32_t img_tail) {
    img_x4* dst = reinterpret_cast<img_x4*>(img);
#pragma unroll
    for (int k = 0; k < kParts; ++k) {
      const uint32_t u = min(uint32_t(tid + k * kKvThreads), last4);
      const uint32_t x = u >= kFirstWord4 ? 0x88888888u : 0u;
      dst[u] = img_x4{imt[k].x ^ x, imt[k].y ^ x, imt[k].z ^ x, imt[k].w ^ x};
    }
    if (img_ti < nd) img[img_ti] = img_tail ^ (img_ti >= kFirstWord4 * 4 ? 0x88888888u : 0u);
  };
  bool img_ready = false;
  const uint32_t delta = CODES ? slot_delta(a.pack_hdr) : 0u;
  const int c = lane & 15, q = lane >> 4;
  const int vg = c % GPS;  // V: the lane's group
  const int vh = c / GPS;  // V with D = 64: the half of the group's coordinates
  const int P = 1 << a.lp;
  KvDecode dc;
  dc.rk = MODE == 1 ? a.rk : 0;
  dc.nbase = 0xE400E400u | ((8u << dc.rk) + 8u) * 0x00010001u;
  dc.nk = 0u - (1u << dc.rk) * 0x00010001u;
  dc.rs2 = half2v{_Float16(a.resid_scale), _Float16(a.resid_scale)};
  // the codewords are 2 (2c0 + s_r 2c1), times 2^rk for MODE 1
  const float cw_scale = MODE == 1 ? ldexpf(0.5f, -dc.rk) : 0.5f;
  // per-lane offsets from a tile's first row (BIG): K token c, V / scale tokens 4q + i
  const int vpair = vg & ~1;  // V: the element offset of the lane's 32-bit word in a row
  const int koff = c * a.Hkv * GPS + q * KS;
  const int voff = (4 * q + 2 * (c & 1)) * a.Hkv * GPS + vpair;
  const int soff = (4 * q + (c & 3)) * a.Hkv;
  const int vstep = a.Hkv * GPS;
  const float* sbase = (c & 4) ? a.vs : a.ks;  // the lane's scale array

  for (int unit = blockIdx.x; unit < a.units; unit += gridDim.x) {
    const int split = unit % a.splits;
    const int bh = unit / a.splits;
    const int h = bh % a.Hkv;
    const int b = bh / a.Hkv;
    const int L = min(max(a.seq_lens[b], 0), a.max_len);
    const int t0 = split * a.T;
    if (t0 >= L) continue;  // the same for the whole workgroup
    const int nt_unit = min(a.T, L - t0);
    const int32_t* bt = a.block_table + int64_t(b) * a.bt_stride;

    half8 qb[KS];  // the query fragments, filled before the first tile

    // ---- the wave's tiles.  A tile's rows take two dependent loads (the block table,
    // then the indices), each issued well before its use.  Tiles past the wave's last
    // load a valid tile again and are not used.
    const int ntiles = (nt_unit + 15) >> 4;
    // Per tile a lane reads: K, the KS groups q KS .. + KS - 1 of token c, per stage; V,
    // the 32-bit word of groups (vg & ~1, vg | 1) of tokens 4q + 2 (c & 1) + j (j = 0,
    // 1), per stage, whose halves lanes c and c ^ 1 exchange (a pair of lanes reads
    // the four tokens' words once, in 32-bit loads); one scale, k_scale (c mod 8 < 4)
    // or v_scale of token 4q + (c mod 4), broadcast over the lane's row afterwards.
    struct TilePages {
      int32_t pk, pv[2], ps;  // BIG: pk alone, the tile's page
      int tk, tv[2], ts;      // tokens of the unit (small pages: token 0 past its end)
    };
    struct TileIdx {
      uint32_t k0[KS], k1[KS];  // K indices, per stage
      uint32_t v0[2], v1[2];    // V words, per stage
      float sc;                 // the lane's scale
    };
    auto unit_token = [&](int jj, int t) { return t0 + (jj * 16 + t < nt_unit ? jj * 16 + t : 0); };
    auto load_pages = [&](int j, TilePages& tp) {
      const int jj = j < ntiles ? j : ntiles - 1;
      if constexpr (BIG) {
        tp.tk = t0 + jj * 16;
        // a vector load (the index in a VGPR): a scalar load in flight would make
        // every wait for the LDS reads a wait for all of them
        int pi = tp.tk >> a.lp;
        asm("" : "+v"(pi));
        tp.pk = bt[pi];
      } else {
        tp.tk = unit_token(jj, c);
        tp.pk = bt[tp.tk >> a.lp];
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2) {
          tp.tv[j2] = unit_token(jj, 4 * q + 2 * (c & 1) + j2);
          tp.pv[j2] = bt[tp.tv[j2] >> a.lp];
        }
        tp.ts = unit_token(jj, 4 * q + (c & 3));
        tp.ps = bt[tp.ts >> a.lp];
      }
    };
    // row of token t on page entry pg: (page, slot, head); rows * D / 8 < 2^31 (checked by
    // the caller)
    auto row_at = [&](int32_t pg, int t) {
      pg = min(max(pg, 0), a.num_pages - 1);
      const int r = (pg * P + (t & (P - 1))) * a.Hkv + h;
      GLQ_DCHECK(r >= 0 && int64_t(r) < int64_t(a.num_pages) * P * a.Hkv);
      return r;
    };
    auto word_at = [&](const uint16_t* p) {  // 32 bits at an even element offset
      uint32_t w;
      __builtin_memcpy(&w, p, 4);
      return w;
    };
    auto load_idx = [&](const TilePages& tp, TileIdx& ti) {
      if constexpr (BIG) {
        // the tile's first row, uniform; the lanes' rows are fixed offsets from it
        const int64_t r0 = row_at(__builtin_amdgcn_readfirstlane(tp.pk), tp.tk);
        GLQ_DCHECK(r0 + int64_t(15) * a.Hkv < int64_t(a.num_pages) * P * a.Hkv);
        const uint16_t* pk0 = a.k0 + r0 * GPS + koff;
        const uint16_t* pk1 = a.k1 + r0 * GPS + koff;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          ti.k0[ks] = pk0[ks];
          ti.k1[ks] = MODE != 0 ? uint32_t(pk1[ks]) : 0u;
        }
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2) {
          ti.v0[j2] = word_at(a.v0 + r0 * GPS + voff + j2 * vstep);
          ti.v1[j2] = MODE != 0 ? word_at(a.v1 + r0 * GPS + voff + j2 * vstep) : 0u;
        }
        ti.sc = sbase[r0 + soff];
      } else {
        const int rk = row_at(tp.pk, tp.tk);
        const uint16_t* pk0 = a.k0 + int64_t(rk) * GPS + q * KS;
        const uint16_t* pk1 = a.k1 + int64_t(rk) * GPS + q * KS;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          ti.k0[ks] = pk0[ks];
          ti.k1[ks] = MODE != 0 ? uint32_t(pk1[ks]) : 0u;
        }
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2) {
          const int64_t rv = row_at(tp.pv[j2], tp.tv[j2]);
          ti.v0[j2] = word_at(a.v0 + rv * GPS + vpair);
          ti.v1[j2] = MODE != 0 ? word_at(a.v1 + rv * GPS + vpair) : 0u;
        }
        ti.sc = sbase[row_at(tp.ps, tp.ts)];
      }
    };

    floatx4 oacc[NK];  // lane (c, q): head c, V columns 4q + i of MFMA k
#pragma unroll
    for (int k = 0; k < NK; ++k) oacc[k] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;  // head c; the same in the lanes of a column
    int e_run = 0;                          // the V sums are in units of 2^(e_run - 126)

    // one tile: scores, the online softmax, V (tl holds tile j's indices)
    auto process = [&](const TileIdx& tl, int j) {
      // V indices of tokens 4q + i, group vg: lane c's own words hold tokens 2 (c & 1)
      // + (0, 1), its neighbour's the other two; the lane's half is (c & 1)
      struct {
        uint32_t k0[KS], k1[KS], v0[4], v1[4];
        float ksc[4], vsc[4];
      } ti;
      const bool odd = c & 1;
      const int hs = odd ? 16 : 0;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        ti.k0[ks] = tl.k0[ks];
        ti.k1[ks] = tl.k1[ks];
      }
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
        const uint32_t g0 = uint32_t(__builtin_amdgcn_update_dpp(0, int(tl.v0[j2]), 0xB1, 0xF, 0xF, false));
        ti.v0[j2] = ((odd ? g0 : tl.v0[j2]) >> hs) & 0xFFFFu;
        ti.v0[2 + j2] = ((odd ? tl.v0[j2] : g0) >> hs) & 0xFFFFu;
        if constexpr (MODE != 0) {
          const uint32_t g1 = uint32_t(__builtin_amdgcn_update_dpp(0, int(tl.v1[j2]), 0xB1, 0xF, 0xF, false));
          ti.v1[j2] = ((odd ? g1 : tl.v1[j2]) >> hs) & 0xFFFFu;
          ti.v1[2 + j2] = ((odd ? tl.v1[j2] : g1) >> hs) & 0xFFFFu;
        } else {
          ti.v1[j2] = ti.v1[2 + j2] = 0u;
        }
      }
      // the scales of tokens 4q + i: lanes 16q + i (k) and 16q + 4 + i (v) of the row
      const int sci = __float_as_int(tl.sc);
      ti.ksc[0] = __int_as_float(__builtin_amdgcn_update_dpp(0, sci, 0x150, 0xF, 0xF, false));
      ti.ksc[1] = __int_as_float(__builtin_amdgcn_update_dpp(0, sci, 0x151, 0xF, 0xF, false));
      ti.ksc[2] = __int_as_float(__builtin_amdgcn_update_dpp(0, sci, 0x152, 0xF, 0xF, false));
      ti.ksc[3] = __int_as_float(__builtin_amdgcn_update_dpp(0, sci, 0x153, 0xF, 0xF, false));
      ti.vsc[0] = __int_as_float(__builtin_amdgcn_update_dpp(0, sci, 0x154, 0xF, 0xF, false));
      ti.vsc[1] = __int_as_float(__builtin_amdgcn_update_dpp(0, sci, 0x155, 0xF, 0xF, false));
      ti.vsc[2] = __int_as_float(__builtin_amdgcn_update_dpp(0, sci, 0x156, 0xF, 0xF, false));
      ti.vsc[3] = __int_as_float(__builtin_amdgcn_update_dpp(0, sci, 0x157, 0xF, 0xF, false));

      floatx4 sacc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        half2v pk[4];
        kv_decode<MODE>(kv_lookup<MODE, CODES>(img, ti.k0[ks], ti.k1[ks], delta), dc, pk);
        const half8 ak = half8{pk[0].x, pk[0].y, pk[1].x, pk[1].y, pk[2].x, pk[2].y, pk[3].x, pk[3].y};
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, qb[ks], sacc, 0, 0, 0);
      }
      const int tb = j * 16 + 4 * q;  // the unit's index of the lane's first token
      bool ok[4];
      float sv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ok[i] = tb + i < nt_unit;
        sv[i] = ok[i] ? sacc[i] * (cw_scale * ti.ksc[i]) : -INFINITY;
      }
      // a tile holds at least one token of the unit, so the max is finite
      const float m_new = fmaxf(m_run, xq_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]))));
      const float alpha = __expf(m_run - m_new);  // 0 on the wave's first tile
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __expf(sv[i] - m_new);
      l_run = l_run * alpha + xq_sum((p[0] + p[1]) + (p[2] + p[3]));
      m_run = m_new;
      // the V scales' running exponent: the biased exponent of the largest |s_v| so far
      float vm = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) vm = ok[i] ? fmaxf(vm, fabsf(ti.vsc[i])) : vm;
      const int e_new = max(e_run, int(__float_as_uint(xq_max(vm)) >> 23));
      const float r = ldexpf(alpha, e_run - e_new);
      e_run = e_new;
      half4v wb;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        wb[i] = _Float16(ok[i] ? ldexpf(p[i] * (cw_scale * ti.vsc[i]), 126 - e_new) : 0.0f);
      // the sums rescaled unless every lane's factor is 1 (no new max, no new exponent)
      if (__builtin_amdgcn_ballot_w64(r != 1.0f) != 0) {
#pragma unroll
        for (int k = 0; k < NK; ++k) oacc[k] *= r;
      }
      // V: group vg of the lane's 4 tokens, coordinate k (+ 4 vh) per MFMA
      half2v cw[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kv_decode<MODE>(kv_lookup<MODE, CODES>(img, ti.v0[i], ti.v1[i], delta), dc, cw[i]);
      if constexpr (D == 64) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const half2v lo0 = cw[i][0], lo1 = cw[i][1];
          cw[i][0] = vh ? cw[i][2] : lo0;
          cw[i][1] = vh ? cw[i][3] : lo1;
        }
      }
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        const int pr = k >> 1;
        const half4v va = (k & 1) ? half4v{cw[0][pr].y, cw[1][pr].y, cw[2][pr].y, cw[3][pr].y}
                                  : half4v{cw[0][pr].x, cw[1][pr].x, cw[2][pr].x, cw[3][pr].x};
        oacc[k] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, wb, oacc[k], 0, 0, 0);
      }
    };
    // Two stages run ahead of the tile processed: its pages (two of the wave's tiles
    // ahead) and its indices (one ahead), each in two buffers used in turn.  The loop
    // is unrolled by two, so no buffer is copied (a copy would wait for the loads in
    // flight into it).  The scheduling barriers keep the loads in the same issue order
    // before the loop as at its back edge, so the counted waits leave the newer loads
    // in flight.  The first unit's image loads go out among its first reads.
    constexpr int W = kKvWaves;
    TilePages pg0, pg1;
    TileIdx ix0, ix1;
    load_pages(wave, pg0);
    load_pages(wave + W, pg1);
    __builtin_amdgcn_sched_barrier(0);
    if (!img_ready) {  // the same for the whole workgroup
      img_x4 imt[kParts];
      uint32_t img_tail;
      image_loads(imt, img_tail);
      __builtin_amdgcn_sched_barrier(0);
      load_idx(pg0, ix0);
      __builtin_amdgcn_sched_barrier(0);
      image_stores(imt, img_tail);
      __syncthreads();
      img_ready = true;
    } else {
      load_idx(pg0, ix0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- the query fragments, straight from memory: lane (c, q) holds head c's groups
    // q KS + ks (zero past G), each rotated by the 8-point Hadamard and scaled:
    // q' = H8 q_g / sqrt(8) * sm_scale
    {
      const int64_t qrow = ((int64_t(b) * a.Hkv + h) * G + min(c, G - 1)) * D;
      float qv[KS][8];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) qv[ks][j] = c < G ? q_value(a.q, a.q_dt, qrow + (q * KS + ks) * 8 + j) : 0.0f;
      const float f = a.sm_scale * 0.35355339059327373f;  // 1 / sqrt(8)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        fwht_reg<8>(qv[ks]);
        half8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = _Float16(qv[ks][j] * f);
        qb[ks] = v;
      }
    }
    // step k of the wave (tile j): pages of step k + 2 into the slot k mod 2, indices
    // of step k + 1 from its pages, then tile j itself
    auto step = [&](int j, TilePages& p_load, const TilePages& p_use, TileIdx& i_load, const TileIdx& i_use) {
      load_pages(j + 2 * W, p_load);
      __builtin_amdgcn_sched_barrier(0);
      load_idx(p_use, i_load);
      __builtin_amdgcn_sched_barrier(0);
      process(i_use, j);
    };
    for (int j = wave; j < ntiles; j += 2 * W) {
      step(j, pg0, pg1, ix1, ix0);
      if (j + W >= ntiles) break;
      step(j + W, pg1, pg0, ix0, ix1);
    }

    // ---- the waves' results merged in wave order.  On the workgroup's last unit the
    // image is no longer needed: every wave stores its sums (in units of 1), max and
    // exp-sum there and all threads merge them at once; otherwise the waves take turns
    // on O [G][D], M [G], L [G] in buf.  A wave without tokens has max -inf and adds
    // nothing; wave 0 always has the first tile.
    auto o_dim = [&](int k, int i) {  // dimension of the lane's sum (k, i)
      const int n = 4 * q + i;         // V column of MFMA k
      return D == 128 ? 8 * n + k : 8 * (n % 8) + k + 4 * (n / 8);
    };
    if (unit + int(gridDim.x) >= a.units) {
      __syncthreads();  // every wave is done with the image
      float* so = reinterpret_cast<float*>(img);  // [wave][G][D]
      float* sml = so + kKvWaves * G * D;        // [wave][G][2]
      if (c < G) {
#pragma unroll
        for (int k = 0; k < NK; ++k)
#pragma unroll
          for (int i = 0; i < 4; ++i) so[(wave * G + c) * D + o_dim(k, i)] = ldexpf(oacc[k][i], e_run - 126);
        if (q == 0) {
          sml[(wave * G + c) * 2 + 0] = m_run;
          sml[(wave * G + c) * 2 + 1] = l_run;
        }
      }
      __syncthreads();
      for (int idx = tid; idx < G * D; idx += kKvThreads) {
        const int g = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kKvWaves; ++w) M = fmaxf(M, sml[(w * G + g) * 2]);
        float o = 0.0f, l = 0.0f;
#pragma unroll
        for (int w = 0; w < kKvWaves; ++w) {
          const float mw = sml[(w * G + g) * 2];
          const float aw = mw == -INFINITY ? 0.0f : __expf(mw - M);
          o = fmaf(aw, so[(w * G + g) * D + d], o);
          l = fmaf(aw, sml[(w * G + g) * 2 + 1], l);
        }
        a.part_o[int64_t(unit) * G * D + idx] = o;
        if (d == 0) {
          a.part_ml[(int64_t(unit) * G + g) * 2 + 0] = M;
          a.part_ml[(int64_t(unit) * G + g) * 2 + 1] = l;
        }
      }
      img_ready = false;
      continue;
    }
    float* bO = buf;
    float* bM = buf + G * D;
    float* bL = bM + G;
    for (int ww = 0; ww < kKvWaves; ++ww) {
      if (wave == ww && c < G) {
        const float M0 = ww == 0 ? -INFINITY : bM[c];
        const float Mn = fmaxf(M0, m_run);
        const float a0 = ww == 0 ? 0.0f : __expf(M0 - Mn);
        const float a1 = m_run == -INFINITY ? 0.0f : __expf(m_run - Mn);
#pragma unroll
        for (int k = 0; k < NK; ++k)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float* dp = &bO[c * D + o_dim(k, i)];
            const float o = ldexpf(oacc[k][i], e_run - 126);
            *dp = (ww == 0 ? 0.0f : *dp * a0) + o * a1;
          }
        if (q == 0) {
          bL[c] = (ww == 0 ? 0.0f : bL[c] * a0) + l_run * a1;
          bM[c] = Mn;
        }
      }
      __syncthreads();
    }
    if (tid < G) {
      a.part_ml[(int64_t(unit) * G + tid) * 2 + 0] = bM[tid];
      a.part_ml[(int64_t(unit) * G + tid) * 2 + 1] = bL[tid];
    }
    for (int i = tid; i < G * D; i += kKvThreads) a.part_o[int64_t(unit) * G * D + i] = bO[i];
    __syncthreads();  // buf is reused by the next unit
  }
}

// ---- the chunks of a sequence merged in chunk order ------------------------------------
// One workgroup per (b, query head), thread d = output dimension: out[d] =
// H8 (sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s) / sqrt(8) over the group of d.
template <int D, int G, class OT>
__global__ __launch_bounds__(D) void kv_combine_kernel(const float* __restrict__ part_o,
                                                       const float* __restrict__ part_ml,
                                                       const int32_t* __restrict__ seq_lens, int max_len, int Hkv,
                                                       int T, int splits, OT* __restrict__ out) {
  const int d = threadIdx.x;
  const int hq = blockIdx.x % (Hkv * G);
  const int b = blockIdx.x / (Hkv * G);
  const int h = hq / G, g = hq % G;
  const int n = (min(max(seq_lens[b], 0), max_len) + T - 1) / T;
  const int64_t u0 = (int64_t(b) * Hkv + h) * splits;
  // one pass over batches of 16 chunks, whose loads are in flight together: the
  // running max is raised to the batch's, the sums are rescaled and the batch added
  // in chunk order (up to 16 chunks: the global max, then one ordered sum)
  constexpr int CB = 16;
  float M = -INFINITY, acc = 0.0f, lsum = 0.0f;
  for (int s0 = 0; s0 < n; s0 += CB) {
    float mv[CB], lv[CB], ov[CB];
#pragma unroll
    for (int k = 0; k < CB; ++k) {
      const int64_t u = u0 + min(s0 + k, n - 1);
      mv[k] = part_ml[(u * G + g) * 2];
      lv[k] = part_ml[(u * G + g) * 2 + 1];
      ov[k] = part_o[u * G * D + g * D + d];
    }
    float Mb = M;
#pragma unroll
    for (int k = 0; k < CB; ++k) Mb = s0 + k < n ? fmaxf(Mb, mv[k]) : Mb;
    // every chunk below n holds a token, so Mb is finite; exp(-inf) = 0 on the first batch
    const float r = __expf(M - Mb);
    acc *= r;
    lsum *= r;
#pragma unroll
    for (int k = 0; k < CB; ++k) {
      if (s0 + k >= n) break;
      const float e = __expf(mv[k] - Mb);
      acc = fmaf(e, ov[k], acc);
      lsum = fmaf(e, lv[k], lsum);
    }
    M = Mb;
  }
  float v = n > 0 ? acc / lsum : 0.0f;
  // the 8-point butterfly over the 8 consecutive threads of the group
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const float q = __shfl_xor(v, 1 << k, 64);
    v = ((d >> k) & 1) ? q - v : v + q;
  }
  out[(int64_t(b) * Hkv * G + hq) * D + d] = from_f32<OT>(v * 0.35355339059327373f);
}

template <int D, int G, int MODE, bool CODES>
hipError_t launch_split(const KvArgs& a, int grid, hipStream_t stream) {
  if (a.lp >= 4)
    hipLaunchKernelGGL((kv_split_kernel<D, G, MODE, CODES, true>), dim3(unsigned(grid)), dim3(kKvThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((kv_split_kernel<D, G, MODE, CODES, false>), dim3(unsigned(grid)), dim3(kKvThreads), 0,
                       stream, a);
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_split_dg(const KvArgs& a, int grid, int stages, bool codes, hipStream_t stream) {
  if (stages == 2 && a.rk >= 0)
    return codes ? launch_split<D, G, 1, true>(a, grid, stream) : launch_split<D, G, 1, false>(a, grid, stream);
  if (stages == 2)
    return codes ? launch_split<D, G, 2, true>(a, grid, stream) : launch_split<D, G, 2, false>(a, grid, stream);
  return codes ? launch_split<D, G, 0, true>(a, grid, stream) : launch_split<D, G, 0, false>(a, grid, stream);
}

template <int D, int G>
hipError_t launch_combine(const KvArgs& a, int B, void* out, glq_dtype out_dt, hipStream_t stream) {
  const dim3 grid(unsigned(B * a.Hkv * G)), block(D);
  switch (out_dt) {
    case GLQ_F32:
      hipLaunchKernelGGL((kv_combine_kernel<D, G, float>), grid, block, 0, stream, a.part_o, a.part_ml, a.seq_lens,
                         a.max_len, a.Hkv, a.T, a.splits, static_cast<float*>(out));
      break;
    case GLQ_F16:
      hipLaunchKernelGGL((kv_combine_kernel<D, G, half_t>), grid, block, 0, stream, a.part_o, a.part_ml, a.seq_lens,
                         a.max_len, a.Hkv, a.T, a.splits, static_cast<half_t*>(out));
      break;
    default:
      hipLaunchKernelGGL((kv_combine_kernel<D, G, bf16_t>), grid, block, 0, stream, a.part_o, a.part_ml,
                         a.seq_lens, a.max_len, a.Hkv, a.T, a.splits, static_cast<bf16_t*>(out));
      break;
  }
  return hipGetLastError();
}

template <int D, int G>
hipError_t run_dg(const KvArgs& a, int grid, int B, int stages, bool codes, void* out, glq_dtype out_dt,
                  hipStream_t stream) {
  hipError_t e = launch_split_dg<D, G>(a, grid, stages, codes, stream);
  if (e != hipSuccess) return e;
  return launch_combine<D, G>(a, B, out, out_dt, stream);
}

}  // namespace

// Sub-chunks of TS tokens (the scores beside the image: TS G <= 1024; smaller when the
// sub-chunks would not fill the CUs), units of as many sub-chunks as leave about one
// unit per CU.
KvPlan kv_plan(int64_t B, int64_t Hkv, int64_t G, int64_t max_seq_len) {
  KvPlan p;
  const int64_t cus = device_cus();
  int TS = G <= 4 ? 256 : 128;
  while (TS > 64 && B * Hkv * ((max_seq_len + TS - 1) / TS) < cus) TS >>= 1;
  const int64_t subs = B * Hkv * ((max_seq_len + TS - 1) / TS);
  int64_t ns = subs / cus;
  if (ns < 1) ns = 1;
  if (ns > 64) ns = 64;
  p.TS = TS;
  p.T = int(TS * ns);
  p.splits = int((max_seq_len + p.T - 1) / p.T);
  p.units = B * Hkv * p.splits;
  return p;
}

hipError_t launch_kv_attention(const glq_kv_cache& kv, const void* q, glq_dtype q_dt, int64_t B, int64_t Hq,
                               const int32_t* block_table, int64_t max_pages, const int32_t* seq_lens,
                               int64_t max_seq_len, float sm_scale, void* out, glq_dtype out_dt, float* part_o,
                               float* part_ml, hipStream_t stream) {
  const int64_t G = Hq / kv.num_kv_heads;
  const KvPlan p = kv_plan(B, kv.num_kv_heads, G, max_seq_len);
  KvArgs a;
  a.q = q;
  a.q_dt = q_dt;
  a.k0 = kv.k_idx[0];
  a.k1 = kv.k_idx[1];
  a.v0 = kv.v_idx[0];
  a.v1 = kv.v_idx[1];
  a.ks = kv.k_scale;
  a.vs = kv.v_scale;
  a.block_table = block_table;
  a.bt_stride = max_pages;
  a.seq_lens = seq_lens;
  const bool codes = kv.index_format == GLQ_INDEX_SLOT;
  const char* p0 = static_cast<const char*>(kv.cb_pack);
  a.pack_hdr = reinterpret_cast<const uint32_t*>(p0);
  a.img = reinterpret_cast<const uint32_t*>(
      p0 + (codes ? pack_slot_image_offset(GLQ_CODEBOOK_ENTRIES) : pack_image_offset(GLQ_CODEBOOK_ENTRIES)));
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.Hkv = int(kv.num_kv_heads);
  a.num_pages = int(kv.num_pages);
  a.max_len = int(max_seq_len < max_pages * kv.page_size ? max_seq_len : max_pages * kv.page_size);
  a.lp = log2_exact(kv.page_size);
  a.T = p.T;
  a.TS = p.TS;
  a.splits = p.splits;
  a.units = int(p.units);
  a.sm_scale = sm_scale;
  a.resid_scale = kv.resid_scale;
  // resid_scale = 2^-rk with 0 <= rk <= 4: the stages are merged exactly in integers
  a.rk = -1;
  for (int k = 0; k <= 4; ++k)
    if (kv.resid_scale == std::ldexp(1.0f, -k)) a.rk = k;
  const int grid = int(p.units < device_cus() ? p.units : device_cus());
  const int st = kv.stages;
  if (kv.head_dim == 64) {
    switch (G) {
      case 1: return run_dg<64, 1>(a, grid, int(B), st, codes, out, out_dt, stream);
      case 2: return run_dg<64, 2>(a, grid, int(B), st, codes, out, out_dt, stream);
      case 4: return run_dg<64, 4>(a, grid, int(B), st, codes, out, out_dt, stream);
      default: return run_dg<64, 8>(a, grid, int(B), st, codes, out, out_dt, stream);
    }
  }
  switch (G) {
    case 1: return run_dg<128, 1>(a, grid, int(B), st, codes, out, out_dt, stream);
    case 2: return run_dg<128, 2>(a, grid, int(B), st, codes, out, out_dt, stream);
    case 4: return run_dg<128, 4>(a, grid, int(B), st, codes, out, out_dt, stream);
    default: return run_dg<128, 8>(a, grid, int(B), st, codes, out, out_dt, stream);
  }
}

GLQ_DEBUG_COUNTER(debug_violations_kv_attention)

}  // namespace glq
