// The whole E8RHTLinear forward for one activation row (B = 1) in one launch on
// gfx950: input RHT, decode matmul against the E8 indices with the codebook
// resident in LDS, fixed-order reduction of the split-K partials, output RHT.
//
// glq 0.5.1 (PyPI project page), "How it works", items 1-4 (sign flips + fast
// Walsh-Hadamard transform on both sides of a weight quantized to 16-bit E8
// codebook indices per 8 weights, optional residual stage); "Inference
// kernels" (the matmul reads the indices and codewords, never W; split-K
// partials reduced in a fixed order, not with atomics).  Glq v0.3.2 release
// notes, "What changed": the input_rht / dequant_matmul / output_rht sequence
// that this kernel performs in one launch.
//
// Workgroup (s, w) of the grid (S splits x W workgroups per split) owns the
// columns [s K, (s + 1) K) of the transformed activation u (K = 8 * 8 * lanes
// per row, 4096 at most) and a contiguous range of output rows:
//  1. its chunk of u, from the Kronecker split H_N = H_{N/K} (x) H_K with the
//     index i = a K + b:  u[s K + b] = (H_K t)[b] / sqrt(N),
//     t[b] = sum_a (-1)^popcount(s & a) sign[a K + b] x[a K + b]
//     (a ascending; x is zero beyond n); t is summed straight from global
//     memory, H_K runs in LDS;
//  2. each lane quantizes its 64 columns of the chunk to 16-bit fixed-point
//     digit planes in registers (one scale per 64 columns);
//  3. the codebook image is copied into the same LDS and the rows are walked
//     as in the staged decode matmul, the partials going to z_parts[s][o];
//  4. every workgroup then adds 1 to an arrival counter; the one that brings it
//     to S W sums z_parts over s = 0 .. S-1 in order, transforms the sum in LDS
//     (H_{m_pad} / sqrt(m_pad), sign flip, truncation to m, cast) and sets the
//     counter back to zero, so the counter is zero again when the launch ends.
// No workgroup waits for another, so the kernel never depends on co-residency.
#include <math.h>

#include "fwht_lds.h"
#include "lds_codebook.h"

namespace glq {
namespace {

constexpr int kThreads = 1024;
// LDS of the chunk of u (4096 fp32 at most), at the top of the LDS array: above
// image parts 0-7 (kImgOff + 4 * 8192 = 33024 <= kLdsDwords - kChunkDwords)
constexpr int kChunkDwords = 4096;
// digit planes of the chunk, between image parts 0-7 and the chunk: uint4
// [8 groups][64 lanes], negated group sums int4 [2][64 lanes], scales [64 lanes]
constexpr int kDigOff = kImgOff + 4 * 8 * 1024;
constexpr int kGsOff = kDigOff + 8 * 64 * 4;
constexpr int kScOff = kGsOff + 2 * 64 * 4;
static_assert(kScOff + 64 <= kLdsDwords - kChunkDwords, "digit region overlaps the chunk");

struct FusedArgs {
  const void* x;
  const int8_t* sign_in;
  const int8_t* sign_out;
  const uint16_t* idx0;
  const void* idx1;
  const uint32_t* pack0_hdr;
  const uint32_t* img0;       // primary pack's LDS image
  const uint32_t* res_slots;  // 8-bit residual slots (8-bit residual stage only)
  float* z_parts;             // [S][m_pad]
  uint32_t* counter;          // arrival counter: zero before and after a launch
  void* y;                    // [m] in y_dt
  int64_t n, m;
  int x_dt, y_dt;
  int ln, lk, lm;  // log2 of n_pad, of the chunk length K, of m_pad
  int vec_in;      // x and sign_in may be read 4 elements at a time
  int vec_out;     // sign_out may be read 32 entries at a time (16-byte aligned, m_pad >= 32)
  int vec_y;       // y may be written 8 outputs at a time (16-byte aligned, m % 8 == 0)
  int G, m_pad, lpr_log2, row_steps, wgs_per_split, rs_per_wg;
  float sc_scale;   // 1 / (sqrt(n_pad) kUqMax): u = t_H / sqrt(n_pad), scale = max|t_H| * sc_scale
  float out_scale;  // s / 2 (codebook entries are held doubled)
  float sr;         // residual scale
  float y_scale;    // 1 / sqrt(m_pad)
};

__device__ __forceinline__ float x_at(const void* x, int dt, int64_t j) {
  switch (dt) {
    case GLQ_F32: return static_cast<const float*>(x)[j];
    case GLQ_F16: return float(static_cast<const half_t*>(x)[j]);
    default: return __uint_as_float(uint32_t(static_cast<const uint16_t*>(x)[j]) << 16);
  }
}

__device__ __forceinline__ float sign_f(uint32_t w, int k) { return float(int8_t(uint8_t(w >> (8 * k)))); }

struct StoreLds {  // element i of the row -> its swizzled LDS position
  float* buf;
  __device__ void operator()(int64_t, int64_t i, float v) const { buf[swz(int(i))] = v; }
};

// Step 1 loads: four consecutive x values (raw) and their signs from column j of
// source chunk; a vector load when aligned and inside n, otherwise the signed
// values themselves (marked `ready`).
struct XRaw {
  img_x4 v;
  uint32_t sgn;
  bool ready;
};

__device__ __forceinline__ void x_issue(const FusedArgs& a, int64_t j, XRaw& r) {
  if (a.vec_in && j + 3 < a.n) {
    r.ready = false;
    if (a.x_dt == GLQ_F32) {
      r.v = *reinterpret_cast<const img_x4*>(static_cast<const float*>(a.x) + j);
    } else {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.x) + j);
      r.v.x = w.x;
      r.v.y = w.y;
    }
    r.sgn = *reinterpret_cast<const uint32_t*>(a.sign_in + j);
  } else {
    r.ready = true;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = (j + e < a.n) ? x_at(a.x, a.x_dt, j + e) * float(a.sign_in[j + e]) : 0.0f;
      r.v[e] = __float_as_uint(v);
    }
  }
}

__device__ __forceinline__ void x_accumulate(const XRaw& r, int dt, bool neg, float (&t)[4]) {
  float v[4];
  if (r.ready || dt == GLQ_F32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(r.v[e]);
  } else if (dt == GLQ_F16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t h = uint16_t(r.v[e >> 1] >> (16 * (e & 1)));
      v[e] = float(__builtin_bit_cast(half_t, h));
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __uint_as_float((e & 1) ? (r.v[e >> 1] & 0xFFFF0000u) : (r.v[e >> 1] << 16));
  }
  if (!r.ready) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] *= sign_f(r.sgn, e);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) t[e] = neg ? t[e] - v[e] : t[e] + v[e];
}

// Step 4: y from sum_s z_parts[s] (s ascending).  Thread t holds the float4s at
// 4 t + 4096 i (i < IT = max(1, m_pad / 4096)): bits 0-1 and the bits of i (12
// and up) are transformed in registers, bits 2-11 in two LDS passes of up to 5
// bits; then every thread writes 8 consecutive outputs at a time, scaled,
// sign-flipped (sign_out packed to one bit per output in LDS beforehand) and
// cast, with 16-byte stores where y allows.
template <class YT>
__device__ __forceinline__ void store8(YT* y, const float (&v)[8]);
template <>
__device__ __forceinline__ void store8<float>(float* y, const float (&v)[8]) {
  reinterpret_cast<float4*>(y)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(y)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
template <class YT>
__device__ __forceinline__ void store8(YT* y, const float (&v)[8]) {
  img_x4 w;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = __builtin_bit_cast(uint16_t, from_f32<YT>(v[2 * k]));
    const uint32_t hi = __builtin_bit_cast(uint16_t, from_f32<YT>(v[2 * k + 1]));
    w[k] = lo | (hi << 16);
  }
  *reinterpret_cast<img_x4*>(y) = w;
}

template <class YT, int IT>
__device__ __forceinline__ void output_transform(const FusedArgs& a, int S, float* buf) {
  const int M = a.m_pad;
  const int tid = threadIdx.x;
  const int c = tid * 4;
  uint32_t* neg = reinterpret_cast<uint32_t*>(buf) + M;  // one bit per output, set = negative
  float t[4 * IT];
  if (c < M) {
    const float* z = a.z_parts;
    float4 acc[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) acc[i] = *reinterpret_cast<const float4*>(z + c + 4096 * i);
    constexpr int UN = IT >= 8 ? 1 : 8 / IT;
    int s = 1;
    for (; s + UN <= S; s += UN) {
      float4 v[UN][IT];
#pragma unroll
      for (int u = 0; u < UN; ++u) {
#pragma unroll
        for (int i = 0; i < IT; ++i) v[u][i] = *reinterpret_cast<const float4*>(z + int64_t(s + u) * M + c + 4096 * i);
      }
#pragma unroll
      for (int u = 0; u < UN; ++u) {
#pragma unroll
        for (int i = 0; i < IT; ++i) {
          acc[i].x += v[u][i].x;
          acc[i].y += v[u][i].y;
          acc[i].z += v[u][i].z;
          acc[i].w += v[u][i].w;
        }
      }
    }
    for (; s < S; ++s) {
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(z + int64_t(s) * M + c + 4096 * i);
        acc[i].x += v.x;
        acc[i].y += v.y;
        acc[i].z += v.z;
        acc[i].w += v.w;
      }
    }
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      t[4 * i + 0] = acc[i].x;
      t[4 * i + 1] = acc[i].y;
      t[4 * i + 2] = acc[i].z;
      t[4 * i + 3] = acc[i].w;
    }
  }
  // sign_out -> bits, while the partials are in flight
  if (a.vec_out) {
    for (int w = tid; w < (M >> 5); w += kThreads) {
      const img_x4 lo = reinterpret_cast<const img_x4*>(a.sign_out)[2 * w];
      const img_x4 hi = reinterpret_cast<const img_x4*>(a.sign_out)[2 * w + 1];
      uint32_t bits = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bits |= ((lo[k] >> (8 * e + 7)) & 1u) << (4 * k + e);
          bits |= ((hi[k] >> (8 * e + 7)) & 1u) << (16 + 4 * k + e);
        }
      }
      neg[w] = bits;
    }
  } else {  // unaligned signs or m_pad < 32: byte loads
    for (int w = tid; w < ((M + 31) >> 5); w += kThreads) {
      uint32_t bits = 0;
      for (int i = 0; i < 32 && 32 * w + i < M; ++i) bits |= uint32_t(a.sign_out[32 * w + i] < 0) << i;
      neg[w] = bits;
    }
  }
  if (c < M) {
    fwht_reg<4 * IT>(t);
#pragma unroll
    for (int i = 0; i < IT; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) buf[swz(c + 4096 * i + e)] = t[4 * i + e];
    }
  }
  const int b_end = a.lm < 12 ? a.lm : 12;
  fwht_lds_passes<StoreLds, 5>(StoreLds{buf}, 0, a.lm, 2, buf, b_end);
  __syncthreads();
  YT* y = static_cast<YT*>(a.y);
  const float scale = a.y_scale;
  if (a.vec_y) {
    for (int o = tid * 8; o < a.m; o += kThreads * 8) {
      const uint32_t nb = neg[o >> 5] >> (o & 31);
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = __uint_as_float(__float_as_uint(buf[swz(o + e)] * scale) ^ (((nb >> e) & 1u) << 31));
      store8<YT>(y + o, v);
    }
  } else {
    for (int o = tid; o < a.m; o += kThreads) {
      const uint32_t bit = (neg[o >> 5] >> (o & 31)) & 1u;
      y[o] = from_f32<YT>(__uint_as_float(__float_as_uint(buf[swz(o)] * scale) ^ (bit << 31)));
    }
  }
}

template <class YT>
__device__ __forceinline__ void output_transform_any(const FusedArgs& a, int S, float* buf) {
  switch (a.lm <= 12 ? 1 : 1 << (a.lm - 12)) {
    case 1: output_transform<YT, 1>(a, S, buf); break;
    case 2: output_transform<YT, 2>(a, S, buf); break;
    case 4: output_transform<YT, 4>(a, S, buf); break;
    default: output_transform<YT, 8>(a, S, buf); break;
  }
}

template <int RESID, bool FULL>
__global__ __launch_bounds__(kThreads) void fused_decode_kernel(FusedArgs a) {
  constexpr int GL = 8;
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsDwords];
  __shared__ int s_last;
  float* fbuf = reinterpret_cast<float*>(lds);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int split = int(blockIdx.x) / a.wgs_per_split;
  const int wg = int(blockIdx.x) - split * a.wgs_per_split;
  const int lpr = FULL ? 6 : a.lpr_log2;
  const int LPR = 1 << lpr;
  const int RPS = 64 >> lpr;
  const int lane_in_row = lane & (LPR - 1);
  const int row_in_step = lane >> lpr;
  const int G = a.G;
  const int g0 = split * (LPR * GL) + lane_in_row * GL;
  const uint8_t* idx1_8 = static_cast<const uint8_t*>(a.idx1);
  const uint16_t* idx1_16 = static_cast<const uint16_t*>(a.idx1);

  // the wave's row-steps
  const int wave = tid >> 6;
  const int r_wg0 = wg * a.rs_per_wg;
  const int r_wg1 = min(r_wg0 + a.rs_per_wg, a.row_steps);
  const int per_wave = (a.rs_per_wg + (kThreads / 64) - 1) / (kThreads / 64);
  const int r_begin = min(r_wg0 + wave * per_wave, r_wg1);
  const int r_end = min(r_begin + per_wave, r_wg1);
  auto row_off = [&](int r) {
    const int o = r * RPS + row_in_step;
    return (o < a.m_pad ? o : 0) * G + g0;
  };

  // ---- steps 1-2.  The x loads go first, then the codebook image fetch; the
  // chunk of u sits in the top kChunkDwords of LDS and the digit planes in the
  // region above image parts 0-7, so those parts are stored as soon as they
  // arrive and only parts 8-9 wait until every lane has its digits.
  float* chunk = reinterpret_cast<float*>(lds + (kLdsDwords - kChunkDwords));
  const int K = 1 << a.lk;
  const int nsrc = 1 << (a.ln - a.lk);
  const int c4 = tid * 4;  // the thread's four columns of the chunk (K <= 4096)
  float t[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  XRaw xr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i < nsrc && c4 < K) x_issue(a, (int64_t(i) << a.lk) + c4, xr[i]);
  ImageRegs img;
  image_issue<RESID>(img, a.pack0_hdr, a.img0, a.res_slots, tid);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i < nsrc && c4 < K) x_accumulate(xr[i], a.x_dt, __popc(unsigned(split & i)) & 1, t);
  for (int src0 = 8; src0 < nsrc; src0 += 8) {  // n_pad > 8 * 4096
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (src0 + i < nsrc && c4 < K) x_issue(a, (int64_t(src0 + i) << a.lk) + c4, xr[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (src0 + i < nsrc && c4 < K) x_accumulate(xr[i], a.x_dt, __popc(unsigned(split & (src0 + i))) & 1, t);
  }
  if (c4 < K) {
    fwht_reg<4>(t);
#pragma unroll
    for (int e = 0; e < 4; ++e) chunk[swz(c4 + e)] = t[e];
  }
  fwht_lds_passes(StoreLds{chunk}, 0, a.lk, 2, chunk);
  __syncthreads();
  image_store<0, 8, false, RESID>(img, lds, tid);

  // the chunk's 8 * LPR groups, one per thread; threads 8l .. 8l+7 hold lane l's
  // 64 columns (one scale block)
  if (tid < 8 * LPR) {
    const int l = tid >> 3, q = tid & 7;
    float v[8];
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = chunk[swz(tid * 8 + j)];
      mx = fmaxf(mx, fabsf(v[j]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
    const float inv = mx > 0.0f ? float(kUqMax) / mx : 0.0f;
    uint32_t planes[4];
    int32_t gsum;
    quantize_group(v, inv, planes, gsum);
    img_x4 pv;
    pv.x = planes[0];
    pv.y = planes[1];
    pv.z = planes[2];
    pv.w = planes[3];
    *reinterpret_cast<img_x4*>(lds + kDigOff + 4 * (q * LPR + l)) = pv;
    lds[kGsOff + 4 * ((q >> 2) * LPR + l) + (q & 3)] = uint32_t(-gsum);  // negated: added on complemented reads
    if (q == 0) lds[kScOff + l] = __float_as_uint(mx * a.sc_scale);
  }
  __syncthreads();
  uint32_t dig[1][GL][4];
  int32_t gs[1][GL];
  float sc[1];
#pragma unroll
  for (int q = 0; q < GL; ++q) {
    const img_x4 d = *reinterpret_cast<const img_x4*>(lds + kDigOff + 4 * (q * LPR + lane_in_row));
    dig[0][q][0] = d.x;
    dig[0][q][1] = d.y;
    dig[0][q][2] = d.z;
    dig[0][q][3] = d.w;
  }
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const img_x4 g = *reinterpret_cast<const img_x4*>(lds + kGsOff + 4 * (qq * LPR + lane_in_row));
    gs[0][4 * qq + 0] = int32_t(g.x);
    gs[0][4 * qq + 1] = int32_t(g.y);
    gs[0][4 * qq + 2] = int32_t(g.z);
    gs[0][4 * qq + 3] = int32_t(g.w);
  }
  sc[0] = __uint_as_float(lds[kScOff + lane_in_row]);
  __syncthreads();  // every lane has its digits before image parts 8-9 overwrite them

  // ---- step 3: the rest of the image, then the rows; the first row-step's
  // index vectors are in flight meanwhile
  image_store<8, 10, true, RESID>(img, lds, tid);
  IdxRow<GL> n0, n1w;
  Idx8Row<GL> n1b;
  if (r_begin < r_end) {
    const int off = row_off(r_begin);
    load_idx16<GL>(a.idx0 + off, n0);
    if (RESID == 16) load_idx16<GL>(idx1_16 + off, n1w);
    if (RESID == 8) load_idx8<GL>(idx1_8 + off, n1b);
  }
  __syncthreads();

  for (int r = r_begin; r < r_end; ++r) {
    const int o = r * RPS + row_in_step;
    const bool valid = o < a.m_pad;
    const IdxRow<GL> i0 = n0;
    const IdxRow<GL> i1w = n1w;
    const Idx8Row<GL> i1b = n1b;
    if (r + 1 < r_end) {
      const int off = row_off(r + 1);
      load_idx16<GL>(a.idx0 + off, n0);
      if (RESID == 16) load_idx16<GL>(idx1_16 + off, n1w);
      if (RESID == 8) load_idx8<GL>(idx1_8 + off, n1b);
    }
    float vv[1];
    row_dots<1, GL, RESID>(lds, i0, i1w, i1b, dig, gs, a.sr, vv);
    float v = vv[0] * sc[0];
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
    if (valid && lane_in_row == LPR - 1) a.z_parts[int64_t(split) * a.m_pad + o] = v * a.out_scale;
  }

  // ---- step 4: arrival; the last workgroup reduces and transforms.  Every wave
  // waits for its partial-sum stores, then one release (thread 0's add: the L2
  // write-back) publishes the workgroup's stores; only the last workgroup
  // acquires (L2 invalidate), once, before its waves read the partials.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(a.counter, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev + 1 == gridDim.x;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_last = last ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  const int S = int(gridDim.x) / a.wgs_per_split;
  switch (a.y_dt) {
    case GLQ_F32: output_transform_any<float>(a, S, fbuf); break;
    case GLQ_F16: output_transform_any<half_t>(a, S, fbuf); break;
    default: output_transform_any<bf16_t>(a, S, fbuf); break;
  }
  if (tid == 0) __hip_atomic_store(a.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int device_cus() {
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

struct FusedPlan {
  int lpr_log2, splits, rps, row_steps, wgs_per_split, rs_per_wg;
};

FusedPlan fused_plan(const glq_layer& L) {
  FusedPlan p;
  const int64_t G = L.n_pad / 8;
  const int64_t lanes = G / 8;
  int l = 0;
  while ((int64_t(1) << l) < lanes && l < 6) ++l;
  p.lpr_log2 = l;
  p.splits = int(G / (int64_t(8) << l));
  p.rps = 64 >> l;
  p.row_steps = int((L.m_pad + p.rps - 1) / p.rps);
  int w = device_cus() / p.splits;
  if (w < 1) w = 1;
  const int min_per_wg = kThreads / 64;  // at least one row-step per wave
  const int wmax = (p.row_steps + min_per_wg - 1) / min_per_wg;
  if (w > wmax) w = wmax;
  p.rs_per_wg = (p.row_steps + w - 1) / w;
  p.wgs_per_split = (p.row_steps + p.rs_per_wg - 1) / p.rs_per_wg;
  return p;
}

}  // namespace

bool fused_decode_supported(const glq_layer& L, int64_t B) {
  // one activation row; 64 <= n_pad (8 groups per lane); the chunk of u fits
  // (K <= 4096 always holds); m_pad floats fit the LDS of the output transform
  return B == 1 && L.n_pad >= 64 && L.m_pad <= 32768 && (L.resid_bits != 16 || L.cb2_pack == L.cb_pack);
}

size_t fused_decode_z_bytes(const glq_layer& L) {
  const FusedPlan p = fused_plan(L);
  return size_t(p.splits) * size_t(L.m_pad) * 4;
}

hipError_t launch_fused_decode(const glq_layer& L, const void* x, glq_dtype x_dt, void* y, glq_dtype y_dt,
                               uint32_t* counter, float* z_parts, hipStream_t stream) {
  const FusedPlan p = fused_plan(L);
  FusedArgs a;
  a.x = x;
  a.sign_in = L.sign_in;
  a.sign_out = L.sign_out;
  a.idx0 = L.idx0;
  a.idx1 = L.idx1;
  const char* p0 = static_cast<const char*>(L.cb_pack);
  a.pack0_hdr = reinterpret_cast<const uint32_t*>(p0);
  a.img0 = reinterpret_cast<const uint32_t*>(p0 + pack_image_offset(GLQ_CODEBOOK_ENTRIES));
  a.res_slots = nullptr;
  if (L.resid_bits == 8)
    a.res_slots = reinterpret_cast<const uint32_t*>(static_cast<const char*>(L.cb2_pack) +
                                                    pack_image_offset(GLQ_RESID8_ENTRIES)) + kPageCount;
  a.z_parts = z_parts;
  a.counter = counter;
  a.y = y;
  a.n = L.n;
  a.m = L.m;
  a.x_dt = x_dt;
  a.y_dt = y_dt;
  a.ln = log2_exact(L.n_pad);
  a.lm = log2_exact(L.m_pad);
  a.lk = a.ln - log2_exact(p.splits);
  const size_t xal = x_dt == GLQ_F32 ? 16 : 8;
  a.vec_in = (reinterpret_cast<uintptr_t>(x) % xal == 0) && (reinterpret_cast<uintptr_t>(L.sign_in) % 4 == 0);
  a.vec_out = (reinterpret_cast<uintptr_t>(L.sign_out) % 16 == 0) && L.m_pad >= 32;
  a.vec_y = (reinterpret_cast<uintptr_t>(y) % 16 == 0) && L.m % 8 == 0;
  a.G = int(L.n_pad / 8);
  a.m_pad = int(L.m_pad);
  a.lpr_log2 = p.lpr_log2;
  a.row_steps = p.row_steps;
  a.wgs_per_split = p.wgs_per_split;
  a.rs_per_wg = p.rs_per_wg;
  a.sc_scale = float(1.0 / (sqrt(double(L.n_pad)) * double(kUqMax)));
  a.out_scale = 0.5f * L.wscale;
  a.sr = L.resid_scale;
  a.y_scale = float(1.0 / sqrt(double(L.m_pad)));
  const dim3 grid(unsigned(p.splits * p.wgs_per_split)), block(kThreads);
  const bool full = p.lpr_log2 == 6;
  switch (L.resid_bits) {
    case 0:
      if (full) hipLaunchKernelGGL((fused_decode_kernel<0, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((fused_decode_kernel<0, false>), grid, block, 0, stream, a);
      break;
    case 8:
      if (full) hipLaunchKernelGGL((fused_decode_kernel<8, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((fused_decode_kernel<8, false>), grid, block, 0, stream, a);
      break;
    default:
      if (full) hipLaunchKernelGGL((fused_decode_kernel<16, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((fused_decode_kernel<16, false>), grid, block, 0, stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace glq
