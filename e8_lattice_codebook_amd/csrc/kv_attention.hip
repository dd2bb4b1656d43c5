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
};

__device__ __forceinline__ float q_value(const void* q, int dt, int64_t i) {
  switch (dt) {
    case GLQ_F32: return static_cast<const float*>(q)[i];
    case GLQ_F16: return float(static_cast<const half_t*>(q)[i]);
    default: return __uint_as_float(uint32_t(static_cast<const uint16_t*>(q)[i]) << 16);
  }
}

__device__ __forceinline__ uint32_t img_word(const uint32_t* img, uint32_t byte_addr) {
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

// The entry's 2c as four fp16 pairs (2c_2k, 2c_2k+1) from its stored word w and m
// (all ones: the entry is the word's negation): with t = w ^ m ^ 0x8888_8888 each
// nibble is lane + 8 (or 7 - lane), 1024 + nibble is an exact fp16 when placed in
// the mantissa, and the bias -(1024 + 8) (or -(1024 + 7)) leaves the value; nibbles
// k and k + 4 hold coordinates 2k and 2k + 1.
__device__ __forceinline__ void word_pairs(uint32_t w, uint32_t m, half2v (&p)[4]) {
  const uint32_t t = w ^ m ^ 0x88888888u;
  const half2v bias = __builtin_bit_cast(half2v, 0xE408E408u ^ (m & 0x000F000Fu));
#pragma unroll
  for (int k = 0; k < 4; ++k)
    p[k] = __builtin_bit_cast(half2v, ((t >> (4 * k)) & 0x000F000Fu) | 0x64006400u) + bias;
}

__device__ __forceinline__ float dpp_max(float v, int ctrl_sel) {
  int r;
  const int x = __float_as_int(v);
  switch (ctrl_sel) {
    case 0: r = __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false); break;
    case 1: r = __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false); break;
    case 3: r = __builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false); break;
    case 4: r = __builtin_amdgcn_update_dpp(x, x, 0x142, 0xA, 0xF, false); break;
    default: r = __builtin_amdgcn_update_dpp(x, x, 0x143, 0xC, 0xF, false); break;
  }
  return fmaxf(v, __int_as_float(r));
}

// the max / sum over the 64 lanes, valid in lane 63
__device__ __forceinline__ float wave_max63(float v) {
#pragma unroll
  for (int k = 0; k < 6; ++k) v = dpp_max(v, k);
  return v;
}

template <int D, int G, int ST, bool CODES>
__global__ __launch_bounds__(kKvThreads, 1) void kv_split_kernel(KvArgs a) {
  constexpr int GPS = D / 8;          // groups per vector
  constexpr int TPV = 64 / GPS;       // V phase: tokens per wave instruction (lane = token x group)
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  static_assert(G * D <= kKvBuf && G * GPS * 5 <= kKvBuf, "query staging fits");

  __shared__ __attribute__((aligned(16))) uint32_t img[kImageMaxDwords];
  __shared__ __attribute__((aligned(16))) float buf[kKvBuf];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  {
    // every load of the image in flight before the first store (clamped addresses:
    // a thread past the end rewrites the last uint4 with the value found there)
    uint32_t nd = a.pack_hdr[CODES ? kHdrSlotDwords : 3];
    nd = nd > uint32_t(kImageMaxDwords) ? uint32_t(kImageMaxDwords) : nd;
    const uint32_t nd4 = nd >> 2;
    const uint32_t last4 = nd4 > 0 ? nd4 - 1 : 0;
    const img_x4* src = reinterpret_cast<const img_x4*>(a.img);
    img_x4* dst = reinterpret_cast<img_x4*>(img);
    constexpr int kParts = (kImageMaxDwords / 4 + kKvThreads - 1) / kKvThreads;
    img_x4 t[kParts];
#pragma unroll
    for (int k = 0; k < kParts; ++k) t[k] = src[min(uint32_t(tid + k * kKvThreads), last4)];
    uint32_t tail = 0;
    const uint32_t ti = (nd4 << 2) + tid;
    if (ti < nd) tail = a.img[ti];
#pragma unroll
    for (int k = 0; k < kParts; ++k) dst[min(uint32_t(tid + k * kKvThreads), last4)] = t[k];
    if (ti < nd) img[ti] = tail;
  }
  const uint32_t delta = CODES ? slot_delta(a.pack_hdr) : 0u;
  const int vt = lane / GPS;                // V phase: token of the lane in a batch
  const int vg = lane % GPS;                // V phase: group of the lane
  const int P = 1 << a.lp;
  const float rs = a.resid_scale;
  __syncthreads();

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
    // row of token t: (page, slot, head); rows * D / 8 < 2^31 (checked by the caller)
    auto row_of = [&](int t) {
      const int pg = min(max(bt[t >> a.lp], 0), a.num_pages - 1);
      return (pg * P + (t & (P - 1))) * a.Hkv + h;
    };

    // ---- the G query heads of h: q' = H8 q_g / sqrt(8) * sm_scale, as fp16 pairs
    const int64_t qbase = (int64_t(b) * a.Hkv + h) * G * D;
    for (int i = tid; i < G * D; i += kKvThreads) buf[i] = q_value(a.q, a.q_dt, qbase + i);
    __syncthreads();
    const bool qlane = tid < G * GPS;
    float qv[8];
    if (qlane) {
#pragma unroll
      for (int j = 0; j < 8; ++j) qv[j] = buf[tid * 8 + j];
      fwht_reg<8>(qv);
      const float f = a.sm_scale * 0.35355339059327373f;  // 1 / sqrt(8)
#pragma unroll
      for (int j = 0; j < 8; ++j) qv[j] *= f;
    }
    __syncthreads();
    if (qlane) {
#pragma unroll
      for (int j = 0; j < 8; ++j) buf[tid * 8 + j] = qv[j];
    }
    __syncthreads();
    // the scores are an MFMA 16 x 16 x 32 per k-step of 32 dimensions: A = the query
    // heads (rows, zero past G) x dimensions, B = dimensions x 16 tokens, one codeword
    // (8 dimensions of one token) per lane; lane l holds A row l mod 16, dimensions
    // 8 (l / 16) .. + 7 of each k-step
    constexpr int KS = D / 32;
    half8 qa[KS];
    {
      const int hr = lane & 15;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        half8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          v[j] = hr < G ? _Float16(buf[hr * D + ks * 32 + 8 * (lane >> 4) + j]) : _Float16(0.0f);
        qa[ks] = v;
      }
    }
    __syncthreads();  // buf becomes the chunk's scores [T][G]

    // ---- the unit's tokens in sub-chunks of TS: scores, an online softmax (running
    // max and exp-sum per head, the V sums rescaled when the max grows), V sums
    // V: lane (token of the batch, group) sums its group of V, both stages combined
    // exactly in fp16, over the wave's tokens; at the end of the unit the lanes of a
    // group and then the waves are added.
    float o[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) o[g][j] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;  // wave g < G: head g's running statistics
    // Loads run ahead of their use: the next sub-chunk's K indices are issued once
    // this one's scores are done (in flight during its softmax and V), its V indices
    // once this one's V is done (in flight during the next scores).  A wave's KBV
    // batches (wave, wave + 8, ...) cover a sub-chunk of up to 256 tokens; slots past
    // it load a valid row and are not used.
    constexpr int KBV = 256 / TPV / kKvWaves;
    auto load_v = [&](int ts0, int nt, uint32_t (&c)[KBV][ST], float (&sv)[KBV]) {
      int rows[KBV];
#pragma unroll
      for (int k = 0; k < KBV; ++k) {
        const int tt = (wave + k * kKvWaves) * TPV + vt;
        rows[k] = row_of(ts0 + (tt < nt ? tt : 0));
      }
#pragma unroll
      for (int k = 0; k < KBV; ++k) {
        c[k][0] = a.v0[rows[k] * GPS + vg];
        if (ST == 2) c[k][ST - 1] = a.v1[rows[k] * GPS + vg];
        sv[k] = a.vs[rows[k]];
      }
    };
    // K: a wave takes token blocks wave, wave + 8, ... of 16 tokens; lane l loads
    // token l mod 16's group 4 ks + l / 16 of every k-step ks, both stages
    constexpr int KTB = 256 / 16 / kKvWaves;
    const int ktok = lane & 15, kq = lane >> 4;
    auto load_k = [&](int ts0, int nt, uint32_t (&c)[KTB][KS][ST], float (&sv)[KTB]) {
      int rows[KTB];
#pragma unroll
      for (int k = 0; k < KTB; ++k) {
        const int tt = (wave + k * kKvWaves) * 16 + ktok;
        rows[k] = row_of(ts0 + (tt < nt ? tt : 0));
      }
#pragma unroll
      for (int k = 0; k < KTB; ++k) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          c[k][ks][0] = a.k0[rows[k] * GPS + ks * 4 + kq];
          if (ST == 2) c[k][ks][ST - 1] = a.k1[rows[k] * GPS + ks * 4 + kq];
        }
        sv[k] = a.ks[rows[k]];
      }
    };
    uint32_t kc[KTB][KS][ST], vc[KBV][ST];
    float kks[KTB], vvs[KBV];
    load_k(t0, min(a.TS, nt_unit), kc, kks);
    load_v(t0, min(a.TS, nt_unit), vc, vvs);
    const half2v rs2 = half2v{_Float16(rs), _Float16(rs)};
    for (int sc = 0; sc < nt_unit; sc += a.TS) {
      const int nt = min(a.TS, nt_unit - sc);

      // K: scores 0.5 s_k q' . (2 c0 + s_r 2 c1) of the sub-chunk's tokens, by MFMA
      // (2c0 + s_r 2c1 is exact in fp16 for s_r = 1/4: multiples of 1/4 below 8)
#pragma unroll
      for (int k = 0; k < KTB; ++k) {
        const int tb = wave + k * kKvWaves;
        if (tb * 16 >= nt) break;  // the same for the whole wave
        floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          uint32_t m;
          half2v p0[4];
          word_pairs(kv_word<CODES>(img, kc[k][ks][0], delta, m), m, p0);
          if (ST == 2) {
            half2v p1[4];
            word_pairs(kv_word<CODES>(img, kc[k][ks][ST - 1], delta, m), m, p1);
#pragma unroll
            for (int j = 0; j < 4; ++j) p0[j] = p1[j] * rs2 + p0[j];
          }
          const half8 bk = half8{p0[0].x, p0[0].y, p0[1].x, p0[1].y, p0[2].x, p0[2].y, p0[3].x, p0[3].y};
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[ks], bk, acc, 0, 0, 0);
        }
        const int tt = tb * 16 + ktok;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int hh = 4 * kq + i;
          if (hh < G && tt < a.TS) buf[tt * G + hh] = tt < nt ? acc[i] * 0.5f * kks[k] : -INFINITY;
        }
      }
      const int sc2 = sc + a.TS < nt_unit ? sc + a.TS : sc;  // past the unit: this one again, unused
      load_k(t0 + sc2, min(a.TS, nt_unit - sc2), kc, kks);
      __syncthreads();

      // softmax statistics, one wave per head: p = exp(s - m_new), the factor
      // exp(m_run - m_new) for what was summed before (0 on the first sub-chunk)
      if (wave < G) {
        float mx = -INFINITY;
        for (int tt = lane; tt < nt; tt += 64) mx = fmaxf(mx, buf[tt * G + wave]);
        mx = __shfl(wave_max63(mx), 63, 64);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __expf(m_run - m_new);
        float sum = 0.0f;
        for (int tt = lane; tt < nt; tt += 64) {
          const float pv = __expf(buf[tt * G + wave] - m_new);
          buf[tt * G + wave] = pv;
          sum += pv;
        }
        sum = __shfl(lane_reduce(sum, 6), 63, 64);
        l_run = l_run * alpha + sum;
        m_run = m_new;
        if (lane == 0) buf[kKvBuf - 8 + wave] = alpha;
      }
      __syncthreads();

      // V: o += p_t * 0.5 s_v * (2c0 + s_r 2c1) over the wave's tokens
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float al = buf[kKvBuf - 8 + g];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[g][j] *= al;
      }
      const int vbatches = (nt + TPV - 1) / TPV;
#pragma unroll
      for (int k = 0; k < KBV; ++k) {
        const int bi = wave + k * kKvWaves;
        if (bi >= vbatches) break;
        const int tt = bi * TPV + vt;
        const bool valid = tt < nt;
        const int ts = valid ? tt : 0;
        uint32_t m;
        half2v p0[4];
        word_pairs(kv_word<CODES>(img, vc[k][0], delta, m), m, p0);
        if (ST == 2) {
          half2v p1[4];
          word_pairs(kv_word<CODES>(img, vc[k][ST - 1], delta, m), m, p1);
#pragma unroll
          for (int j = 0; j < 4; ++j) p0[j] = p1[j] * rs2 + p0[j];
        }
        const float f = 0.5f * vvs[k];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float sv = valid ? buf[ts * G + g] * f : 0.0f;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            o[g][2 * kk] = fmaf(sv, float(p0[kk].x), o[g][2 * kk]);
            o[g][2 * kk + 1] = fmaf(sv, float(p0[kk].y), o[g][2 * kk + 1]);
          }
        }
      }
      load_v(t0 + sc2, min(a.TS, nt_unit - sc2), vc, vvs);
      __syncthreads();  // the next sub-chunk overwrites the scores
    }

    // ---- the unit's results: statistics; V sums over the lanes of a group (the
    // lane bits above the group), then over the waves in wave order in LDS
    if (wave < G && lane == 63) {
      a.part_ml[(int64_t(unit) * G + wave) * 2 + 0] = m_run;
      a.part_ml[(int64_t(unit) * G + wave) * 2 + 1] = l_run;
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int bit = GPS; bit < 64; bit <<= 1) o[g][j] += __shfl_xor(o[g][j], bit, 64);
    for (int ww = 0; ww < kKvWaves; ++ww) {
      if (wave == ww && lane < GPS) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            float* d = &buf[g * D + lane * 8 + j];
            *d = ww == 0 ? o[g][j] : *d + o[g][j];
          }
      }
      __syncthreads();
    }
    for (int i = tid; i < G * D; i += kKvThreads) a.part_o[int64_t(unit) * G * D + i] = buf[i];
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

template <int D, int G, int ST, bool CODES>
hipError_t launch_split(const KvArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((kv_split_kernel<D, G, ST, CODES>), dim3(unsigned(grid)), dim3(kKvThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_split_dg(const KvArgs& a, int grid, int stages, bool codes, hipStream_t stream) {
  if (stages == 2)
    return codes ? launch_split<D, G, 2, true>(a, grid, stream) : launch_split<D, G, 2, false>(a, grid, stream);
  return codes ? launch_split<D, G, 1, true>(a, grid, stream) : launch_split<D, G, 1, false>(a, grid, stream);
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

}  // namespace glq
