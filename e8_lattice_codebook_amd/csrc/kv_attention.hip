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
// linear) and integer dot products (K) or FMAs (V) on the int4 codeword lanes.
//
// Kernel 1 (kv_split_kernel): persistent workgroups, one per CU, the codebook image
// loaded into LDS once.  A unit is (sequence b, KV head h, chunk of T tokens).  Per
// unit: the G query heads of h are rotated and quantized to 16-bit fixed point
// (four int4 digit planes per group); every wave scores tokens (lanes = token x
// stage x group, exact i32 dot products, a DPP reduction per token); one wave per
// head takes the chunk's max and exp-sums; then wave w accumulates group w mod D/8
// of V over its tokens (lane = token) in fp32.  The unit's (max, sum, o) go to the
// workspace.  Kernel 2 (kv_combine_kernel) merges a sequence's chunks in chunk
// order, divides, applies the 8-point butterfly and 1/sqrt(8), and casts.
#include <math.h>

#include "fwht_lds.h"
#include "lds_codebook.h"

namespace glq {
namespace {

constexpr int kKvThreads = 1024;
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
  int Hkv, lp, T, splits, units;
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
  constexpr int LPT = ST * GPS;       // lanes per token in the K phase
  constexpr int LPT_LOG2 = LPT == 8 ? 3 : LPT == 16 ? 4 : 5;
  constexpr int TPI = 64 / LPT;       // tokens per wave instruction
  constexpr int PARTS = kKvWaves / GPS;  // V-phase waves per group
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
  const int lt = lane >> LPT_LOG2;          // token of the lane in a K-phase batch
  const int lst = (lane / GPS) % ST;        // stage of the lane
  const int lg = lane % GPS;                // group of the lane
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
    const int nt = min(a.T, L - t0);
    const int32_t* bt = a.block_table + int64_t(b) * a.bt_stride;
    auto row_of = [&](int t) {
      const int pg = min(max(bt[t >> a.lp], 0), a.num_pages - 1);
      return (int64_t(pg) * P + (t & (P - 1))) * a.Hkv + h;
    };

    // ---- the G query heads of h: H8 q_g / sqrt(8) * sm_scale, then digit planes
    const int64_t qbase = (int64_t(b) * a.Hkv + h) * G * D;
    for (int i = tid; i < G * D; i += kKvThreads) buf[i] = q_value(a.q, a.q_dt, qbase + i);
    __syncthreads();
    float qv[8];
    const bool qlane = tid < G * GPS;
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
    if (wave < G) {  // the head's max |q'|
      float mx = 0.0f;
      for (int d = lane; d < D; d += 64) mx = fmaxf(mx, fabsf(buf[wave * D + d]));
      mx = wave_max63(mx);
      if (lane == 63) buf[kKvBuf - 8 + wave] = mx;
    }
    __syncthreads();
    uint32_t pl[4];
    int32_t gsum = 0;
    float qsc = 0.0f;
    if (qlane) {
      const float mx = buf[kKvBuf - 8 + tid / GPS];
      quantize_group(qv, mx > 0.0f ? float(kUqMax) / mx : 0.0f, pl, gsum);
      qsc = mx / float(kUqMax);
    }
    __syncthreads();
    if (qlane) {
#pragma unroll
      for (int p = 0; p < 4; ++p) buf[tid * 5 + p] = __uint_as_float(pl[p]);
      buf[tid * 5 + 4] = __int_as_float(gsum);
    }
    if (qlane && tid % GPS == 0) buf[kKvBuf - 16 + tid / GPS] = qsc;
    __syncthreads();
    uint32_t dig[G][4];
    float qs[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int p = 0; p < 4; ++p) dig[g][p] = __float_as_uint(buf[(g * GPS + lg) * 5 + p]);
      qs[g] = buf[kKvBuf - 16 + g];
    }
    __syncthreads();  // buf becomes the chunk's scores [T][G]

    // ---- K: score of every token of the chunk, 0.5 s_k q' . (2 c0 + s_r 2 c1)
    // a wave takes batches wave, wave + 16, ...; KB of them have their loads in
    // flight at once (the page numbers first, then the indices and scales)
    const uint16_t* kidx = lst == 0 ? a.k0 : a.k1;
    const int batches = (nt + TPI - 1) / TPI;
    constexpr int KB = 8;
    for (int bi0 = wave; bi0 < batches; bi0 += kKvWaves * KB) {
      int64_t rows[KB];
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int tt = (bi0 + k * kKvWaves) * TPI + lt;
        rows[k] = row_of(t0 + (tt < nt ? tt : 0));
      }
      uint32_t cs[KB];
      float kss[KB];
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        cs[k] = kidx[rows[k] * GPS + lg];
        kss[k] = a.ks[rows[k]];
      }
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int tt = (bi0 + k * kKvWaves) * TPI + lt;
        if (bi0 + k * kKvWaves >= batches) break;  // the same for the whole wave
        const bool valid = tt < nt;
        uint32_t m;
        const uint32_t w = kv_word<CODES>(img, cs[k], delta, m);
        const float f = (m ? -0.5f : 0.5f) * (lst ? rs : 1.0f);
        float sc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          int acc[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) acc[p] = __builtin_amdgcn_sdot8(int(w), int(dig[g][p]), 0, false);
          const int tot = ((acc[3] * 16 + acc[2]) * 16 + acc[1]) * 16 + acc[0];
          sc[g] = lane_reduce(float(tot) * f, LPT_LOG2);
        }
        if ((lane & (LPT - 1)) == LPT - 1 && tt < a.T) {
#pragma unroll
          for (int g = 0; g < G; ++g) buf[tt * G + g] = valid ? sc[g] * kss[k] * qs[g] : -INFINITY;
        }
      }
    }
    __syncthreads();

    // ---- softmax statistics of the chunk, one wave per head
    if (wave < G) {
      float mx = -INFINITY;
      for (int tt = lane; tt < nt; tt += 64) mx = fmaxf(mx, buf[tt * G + wave]);
      mx = __shfl(wave_max63(mx), 63, 64);
      float sum = 0.0f;
      for (int tt = lane; tt < nt; tt += 64) {
        const float p = __expf(buf[tt * G + wave] - mx);
        buf[tt * G + wave] = p;
        sum += p;
      }
      sum = lane_reduce(sum, 6);
      if (lane == 63) {
        a.part_ml[(int64_t(unit) * G + wave) * 2 + 0] = mx;
        a.part_ml[(int64_t(unit) * G + wave) * 2 + 1] = sum;
      }
    }
    __syncthreads();

    // ---- V: wave w sums group w mod GPS of its tokens, lane = token
    const int gv = wave % GPS;
    const int part = wave / GPS;
    float o[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) o[g][j] = 0.0f;
    constexpr int VB = 4;  // tokens per lane with their loads in flight at once
    for (int tb = part * 64 + lane; tb < nt; tb += 64 * PARTS * VB) {
      int64_t rows[VB];
#pragma unroll
      for (int k = 0; k < VB; ++k) {
        const int tt = tb + k * 64 * PARTS;
        rows[k] = row_of(t0 + (tt < nt ? tt : 0));
      }
      uint32_t cs[VB][ST];
      float vss[VB];
#pragma unroll
      for (int k = 0; k < VB; ++k) {
        cs[k][0] = a.v0[rows[k] * GPS + gv];
        if (ST == 2) cs[k][ST - 1] = a.v1[rows[k] * GPS + gv];
        vss[k] = a.vs[rows[k]];
      }
#pragma unroll
      for (int k = 0; k < VB; ++k) {
        const int tt = tb + k * 64 * PARTS;
        if (tt >= nt) continue;
        const float vsc = 0.5f * vss[k];
        float pw[G];
#pragma unroll
        for (int g = 0; g < G; ++g) pw[g] = buf[tt * G + g] * vsc;
#pragma unroll
        for (int st = 0; st < ST; ++st) {
          uint32_t m;
          const uint32_t w = kv_word<CODES>(img, cs[k][st], delta, m);
          const float f = (m ? -1.0f : 1.0f) * (st ? rs : 1.0f);
          float x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)  // the builtin's result type is unsigned: read it as the signed lane
            x[j] = float(int32_t(__builtin_amdgcn_sbfe(w, 4 * lane_nibble(j), 4)));
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float s = pw[g] * f;
#pragma unroll
            for (int j = 0; j < 8; ++j) o[g][j] = fmaf(s, x[j], o[g][j]);
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) o[g][j] = lane_reduce(o[g][j], 6);
    __syncthreads();  // every wave is done with the scores
    if (PARTS > 1 && part > 0 && lane == 63) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) buf[((part - 1) * GPS + gv) * G * 8 + g * 8 + j] = o[g][j];
    }
    __syncthreads();
    if (part == 0 && lane == 63) {
      float* po = a.part_o + int64_t(unit) * G * D + gv * 8;
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float v = o[g][j];
          for (int pp = 1; pp < PARTS; ++pp) v += buf[((pp - 1) * GPS + gv) * G * 8 + g * 8 + j];
          po[g * D + j] = v;
        }
      }
    }
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
  float M = -INFINITY;
  for (int s = 0; s < n; ++s) M = fmaxf(M, part_ml[((u0 + s) * G + g) * 2]);
  float acc = 0.0f, lsum = 0.0f;
  for (int s = 0; s < n; ++s) {
    const float e = __expf(part_ml[((u0 + s) * G + g) * 2] - M);
    acc = fmaf(e, part_o[(u0 + s) * G * D + g * D + d], acc);
    lsum = fmaf(e, part_ml[((u0 + s) * G + g) * 2 + 1], lsum);
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

int kv_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

}  // namespace

// tokens per chunk: the largest of 256, 128, 64 whose units still fill the CUs
// (and whose scores fit beside the image: T G <= 1024)
KvPlan kv_plan(int64_t B, int64_t Hkv, int64_t G, int64_t max_seq_len) {
  KvPlan p;
  int T = G <= 4 ? 256 : 128;
  while (T > 64 && B * Hkv * ((max_seq_len + T - 1) / T) < kv_cus()) T >>= 1;
  p.T = T;
  p.splits = int((max_seq_len + T - 1) / T);
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
  a.splits = p.splits;
  a.units = int(p.units);
  a.sm_scale = sm_scale;
  a.resid_scale = kv.resid_scale;
  const int grid = int(p.units < kv_cus() ? p.units : kv_cus());
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
