// The E8RHTLinear forward for one activation row (B = 1) in two launches on
// gfx950: input RHT, decode matmul against the E8 indices with the codebook
// resident in LDS and the row-local part of the output RHT in the first; the
// fixed-order reduction of the split-K partials and the rest of the output RHT
// in the second.
//
// glq 0.5.1 (PyPI project page), "How it works", items 1-4 (sign flips + fast
// Walsh-Hadamard transform on both sides of a weight quantized to 16-bit E8
// codebook indices per 8 weights, optional residual stage); "Inference
// kernels" (the matmul reads the indices and codewords, never W; split-K
// partials reduced in a fixed order, not with atomics).  Glq v0.3.2 release
// notes, "What changed": the input_rht / dequant_matmul / output_rht sequence
// that these two kernels perform.
//
// fused_decode_kernel: workgroup (s, w) of the grid (S splits x W workgroups per
// split) owns the columns [s K, (s + 1) K) of the transformed activation u
// (K = 8 * 8 * lanes per row, 4096 at most) and the R output rows [w R, (w+1) R):
//  1. its chunk of u, from the Kronecker split H_N = H_{N/K} (x) H_K with the
//     index i = a K + b:  u[s K + b] = (H_K t)[b] / sqrt(N),
//     t[b] = sum_a (-1)^popcount(s & a) sign[a K + b] x[a K + b]
//     (a ascending; x is zero beyond n); t is summed straight from global
//     memory, H_K runs in LDS;
//  2. the chunk is quantized to 16-bit fixed-point digit planes (one scale per
//     64 columns), which every lane keeps in registers;
//  3. the codebook image is copied into the same LDS and the rows are walked
//     as in the staged decode matmul, the row partials kept in LDS;
//  4. H_R of the R row partials (the output index is i = a R + b and
//     H_{m_pad} = H_W (x) H_R, linear in the partials) goes to z_parts[s].
// output_blocks_kernel: for every column b, T = sum_s z_parts[s] in order, then
// the W-point transform over the blocks a, 1/sqrt(m_pad), sign flip, truncation
// to m and cast.
#include <math.h>

#include <type_traits>

#include "fwht_lds.h"
#include "lds_codebook.h"

namespace glq {
namespace {

constexpr int kThreads = 1024;
// LDS of the chunk of u (4096 fp32 at most), at the top of the LDS array: above
// image parts 0-7 (kImgOff + 4 * 8192 = 33024 <= kLdsDwords - kChunkDwords)
constexpr int kChunkDwords = 4096;
constexpr int kLenLog2s = 21;  // transform block lengths 2^0 .. 2^20
// rows of the workgroup kept in LDS for its share of the output transform
constexpr int kRowBuf = 1024;
// digit planes of the chunk, between image parts 0-7 and the chunk: uint4
// [8 groups][64 lanes], negated group sums int4 [2][64 lanes], scales [64 lanes]
constexpr int kDigOff = kImgOff + 4 * 8 * 1024;
constexpr int kGsOff = kDigOff + 8 * 64 * 4;
constexpr int kScOff = kGsOff + 2 * 64 * 4;
// per scale block: the binary exponent of its max (int32 [64 lanes]); then the
// workgroup's largest such exponent (one int32, LDS max)
constexpr int kFeOff = kScOff + 64;
constexpr int kExpOff = kFeOff + 64;
static_assert(kExpOff + 1 <= kLdsDwords - kChunkDwords, "digit region overlaps the chunk");
// the workgroup exponent before any block has reported one (all-zero chunks)
constexpr int kNoExp = -1024;

struct FusedArgs {
  const void* x;
  const int8_t* sign_in;
  const uint16_t* idx0;
  const void* idx1;
  const uint32_t* pack0_hdr;
  const uint32_t* img0;       // primary pack's LDS image
  const uint32_t* res_slots;  // 8-bit residual slots (8-bit residual stage only)
  float* z_parts;             // [S][m_pad]: H_R of each workgroup's row block
  int64_t n;
  int x_dt;
  int n_pad;   // transform length (block-diagonal over its binary expansion)
  int lk;      // log2 of the chunk length K (K divides every block of n_pad)
  int vec_in;  // x and sign_in may be read 4 elements at a time
  int G, m_pad, lpr_log2, row_steps, wgs_per_split, rs_per_wg;
  int lr;           // log2 R, the rows of a workgroup's block
  float sc_tab[kLenLog2s];  // [log2 L] 1 / (sqrt(L) kUqMax): u = t_H / sqrt(L), scale = max|t_H| * sc_tab
  float out_scale;  // s / 2 (codebook entries are held doubled)
  float sr;         // residual scale
  // further stages of a 5-8 bpw layer in one pass: 16-bit stages (primary image) and an
  // 8-bit stage (the residual slots), each with its scale relative to s
  const uint16_t* idx_x16[2];
  const uint8_t* idx_x8;
  float sc_x16[2];
  float sc_x8;
};

// The index words of one row-step for every stage of the layer.
template <int GL, int X16>
struct RowIdx {
  IdxRow<GL> i0, i1w;
  Idx8Row<GL> i1b;
  IdxRow<GL> x16[X16 > 0 ? X16 : 1];
  Idx8Row<GL> x8;
};

__device__ __forceinline__ float x_at(const void* x, int dt, int64_t j) {
  switch (dt) {
    case GLQ_F32: return static_cast<const float*>(x)[j];
    case GLQ_F16: return float(static_cast<const half_t*>(x)[j]);
    default: return __uint_as_float(uint32_t(static_cast<const uint16_t*>(x)[j]) << 16);
  }
}

__device__ __forceinline__ float sign_f(uint32_t w, int k) { return float(int8_t(uint8_t(w >> (8 * k)))); }

struct StoreZ {  // element i < lim of a workgroup's rows -> its place in z_parts
  float* p;
  int lim;
  __device__ void operator()(int64_t, int64_t i, float v) const {
    if (i < lim) p[i] = v;
  }
};

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
// H_R on the R = 64 E rows base .. base + R - 1 of the workgroup's rows in rowbuf
// by one wave: lane l holds rows base + l E .. + E - 1 (bits below log2 E in
// registers, the six lane bits by shuffles), then stores them to p with 16-byte
// stores.
template <int E>
__device__ __forceinline__ void wave_block_transform(const float* rowbuf, int base, float* p, int lane) {
  float v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = rowbuf[swz(base + lane * E + e)];
  fwht_reg<E>(v);
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    const bool upper = (lane >> k) & 1;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float q = __shfl_xor(v[e], 1 << k, 64);
      v[e] = upper ? q - v[e] : v[e] + q;
    }
  }
#pragma unroll
  for (int e = 0; e < E; e += 4) {
    *reinterpret_cast<float4*>(p + lane * E + e) = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
  }
}

// Butterfly of the chunk transform on lane bit k of the wave (column bit k + 2:
// thread t holds columns 4 t .. 4 t + 3): v + partner on the lower lane of each
// pair, partner - v on the upper one (s = -1 there); the partner comes from DPP
// (quad permutes, row rotates; lane bit 2 takes the rotate by 12 on rows' banks
// 0 and 2 and by 4 on banks 1 and 3), a swizzle (bit 4) or a permute (bit 5).
__device__ __forceinline__ float lane_butterfly(float v, int k, float s, int lane) {
  const int x = __float_as_int(v);
  int pv;
  switch (k) {
    case 0: pv = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false); break;   // quad_perm [1,0,3,2]
    case 1: pv = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false); break;   // quad_perm [2,3,0,1]
    case 2:
      pv = __builtin_amdgcn_update_dpp(0, x, 0x12C, 0xF, 0x5, false);               // row_ror:12 -> lanes i + 4
      pv = __builtin_amdgcn_update_dpp(pv, x, 0x124, 0xF, 0xA, false);              // row_ror:4  -> lanes i - 4
      break;
    case 3: pv = __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false); break;  // row_ror:8
    case 4: pv = __builtin_amdgcn_ds_swizzle(x, 0x401F); break;                      // lane ^ 16 within 32
    default: pv = __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, x); break;          // lane ^ 32
  }
  return fmaf(s, v, __int_as_float(pv));
}

__device__ __forceinline__ int dpp_partner1(int x) { return __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false); }

// RESID: the first residual stage (0, 8 or 16 bits); X16, X8: further 16-bit stages
// (0-2) and a trailing 8-bit stage (0-1) of a 5-8 bpw layer (after RESID 16)
// The body of one workgroup; bid is the workgroup's number within its layer's grid.
template <int RESID, int X16, int X8, bool FULL, bool CODES>
__device__ __forceinline__ void fused_decode_body(const FusedArgs& a, int bid) {
  constexpr int GL = 8;
  constexpr int R8 = (RESID == 8 || X8) ? 8 : 0;  // the 8-bit table in LDS
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsDwords];
  __shared__ __attribute__((aligned(16))) float rowbuf[kRowBuf];  // the workgroup's row block (swizzled)
  float* fbuf = reinterpret_cast<float*>(lds);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const uint32_t delta = CODES ? slot_delta(a.pack0_hdr) : 0u;
  const int split = bid / a.wgs_per_split;
  const int wg = bid - split * a.wgs_per_split;
  const int lpr = FULL ? 6 : a.lpr_log2;
  const int LPR = 1 << lpr;
  const int RPS = 64 >> lpr;
  const int lane_in_row = lane & (LPR - 1);
  const int row_in_step = lane >> lpr;
  const int G = a.G;
  const int g0 = split * (LPR * GL) + lane_in_row * GL;
  const uint8_t* idx1_8 = static_cast<const uint8_t*>(a.idx1);
  const uint16_t* idx1_16 = static_cast<const uint16_t*>(a.idx1);

  // the wave's row-steps.  With at most two index stages per row, the waves take the
  // workgroup's row-steps dynamically, in chunks of three from a counter in LDS, so
  // that no wave of a SIMD idles while another still has rows: the counter is LDS
  // word 0 without an 8-bit stage (whose residual slots live there), else the last
  // word of the image budget, which a slot image never reaches (slot images are at
  // most kSlotImageMaxDwords); a page image with an 8-bit stage may fill the budget,
  // and there, as for 5-8 bpw rows, each wave takes a fixed share.
  // Only a workgroup with at least six row-steps per wave does so: below that, chunks of
  // three would leave waves without rows.
  constexpr bool kDynOk = X16 == 0 && X8 == 0 && (RESID != 8 || CODES);
  constexpr int kCtr = RESID != 8 ? kResOff : kImgOff + kImageMaxDwords - 1;
  static_assert(kSlotImageMaxDwords < kImageMaxDwords, "the counter word lies above every slot image");
  const bool dyn = kDynOk && a.rs_per_wg >= 6 * (kThreads / 64);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r_wg0 = wg * a.rs_per_wg;
  const int r_wg1 = min(r_wg0 + a.rs_per_wg, a.row_steps);
  const int per_wave = dyn ? 3 : (a.rs_per_wg + (kThreads / 64) - 1) / (kThreads / 64);
  const int r_begin = min(r_wg0 + wave * per_wave, r_wg1);  // dyn: the wave's first chunk
  const int r_end = min(r_begin + per_wave, r_wg1);
  auto row_off = [&](int r) {
    const int o = r * RPS + row_in_step;
    return (o < a.m_pad ? o : 0) * G + g0;
  };
  // with 64 lanes per row the row is wave-uniform: a scalar row base plus the
  // lane's 32-bit offset (g0 elements) addresses the index loads
  const uint32_t g0b = uint32_t(g0);
  auto load16 = [&](const uint16_t* base, int64_t rb, IdxRow<GL>& d) {
    load_idx16<GL>(reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(base + rb) + 2 * g0b), d);
  };
  auto load_full = [&](int r, RowIdx<GL, X16>& n) {
    const int64_t rb = int64_t(r < a.m_pad ? r : 0) * G;
    load16(a.idx0, rb, n.i0);
    if (RESID == 16) load16(idx1_16, rb, n.i1w);
    if (RESID == 8) load_idx8<GL>(idx1_8 + rb + g0b, n.i1b);
#pragma unroll
    for (int k = 0; k < X16; ++k) load16(a.idx_x16[k], rb, n.x16[k]);
    if (X8) load_idx8<GL>(a.idx_x8 + rb + g0b, n.x8);
  };
  auto load_off = [&](int off, RowIdx<GL, X16>& n) {
    load_idx16<GL>(a.idx0 + off, n.i0);
    if (RESID == 16) load_idx16<GL>(idx1_16 + off, n.i1w);
    if (RESID == 8) load_idx8<GL>(idx1_8 + off, n.i1b);
#pragma unroll
    for (int k = 0; k < X16; ++k) load_idx16<GL>(a.idx_x16[k] + off, n.x16[k]);
    if (X8) load_idx8<GL>(a.idx_x8 + off, n.x8);
  };

  // ---- steps 1-2.  The x loads go first, then the codebook image fetch; the
  // chunk of u sits in the top kChunkDwords of LDS and the digit planes in the
  // region above image parts 0-7, so those parts are stored as soon as they
  // arrive and only parts 8-9 wait until every lane has its digits.
  // the first row-step's index vectors go first of all: their latency overlaps
  // the whole prologue
  RowIdx<GL, X16> n;
  if (r_begin < r_end) {
    if (FULL)
      load_full(r_begin, n);
    else
      load_off(row_off(r_begin), n);
  }
  float* chunk = reinterpret_cast<float*>(lds + (kLdsDwords - kChunkDwords));
  // the split's chunk lies in the transform block of length 2^lb that starts at
  // column blk0: the block of a column c < n_pad is the highest set bit of
  // n_pad ^ c (the blocks are n_pad's binary expansion, largest first); the
  // chunk is number s_loc of the block's nsrc chunks
  const int K = 1 << a.lk;
  const int col0 = split << a.lk;
  const int lb = 31 - __clz(a.n_pad ^ col0);
  const int blk0 = col0 & ~((1 << lb) - 1);
  const int s_loc = (col0 - blk0) >> a.lk;
  const int nsrc = 1 << (lb - a.lk);
  const int c4 = tid * 4;  // the thread's four columns of the chunk (K <= 4096)
  float t[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  XRaw xr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i < nsrc && c4 < K) x_issue(a, blk0 + (int64_t(i) << a.lk) + c4, xr[i]);
  ImageRegs img;
  image_issue<R8>(img, a.pack0_hdr, a.img0, a.res_slots, tid, CODES ? kHdrSlotDwords : 3);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i < nsrc && c4 < K) x_accumulate(xr[i], a.x_dt, __popc(unsigned(s_loc & i)) & 1, t);
  for (int src0 = 8; src0 < nsrc; src0 += 8) {  // n_pad > 8 * 4096
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (src0 + i < nsrc && c4 < K) x_issue(a, blk0 + (int64_t(src0 + i) << a.lk) + c4, xr[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (src0 + i < nsrc && c4 < K) x_accumulate(xr[i], a.x_dt, __popc(unsigned(s_loc & (src0 + i))) & 1, t);
  }
  // bits 0-1 in registers, bits 2-7 across the lanes of the wave (threads past
  // the chunk hold zeros and never pair with one inside it), bits 8-11 in one
  // LDS pass; the same butterflies in the same order as a transform of the row
  fwht_reg<4>(t);
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    if (k + 2 < a.lk) {
      const float sk = ((lane >> k) & 1) ? -1.0f : 1.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = lane_butterfly(t[e], k, sk, lane);
    }
  }
  if (c4 < K) {
#pragma unroll
    for (int e = 0; e < 4; ++e) chunk[swz(c4 + e)] = t[e];
  }
  if (tid == 0) lds[kExpOff] = uint32_t(kNoExp);  // published by the barrier below
  fwht_lds_passes(StoreLds{chunk}, 0, a.lk, 8, chunk);
  __syncthreads();
  image_store<0, 8, false, R8>(img, lds, tid);

  // quantization: thread t < 16 LPR takes half h = t & 1 (columns 4 h .. 4 h + 3)
  // of group g = t >> 1, the group q = g & 7 of lane l = g >> 3; the 16 threads of
  // a lane's 64 columns (one scale block) are one DPP row.  U = rint(u kUqMax / max)
  // has the balanced base-16 digits d_p = nibble p of (U + 0x8888) minus 8, whose
  // 4-bit two's complement is nibble p of W = (U + 0x8888) ^ 0x8888.
  //
  // The block is normalized by a power of two first: with max = f 2^fe, f in
  // [1/2, 1), U = rint(v 2^-fe * kUqMax / f), the same U as rint(v kUqMax / max)
  // wherever that is finite, but never inf for a tiny max.  The block's scale
  // f / (sqrt(L) kUqMax) is kept relative to the workgroup's largest exponent E
  // (2^(fe - E) of it), and the row partials are multiplied by 2^E once, so no
  // scale leaves the normal range however small the chunk is.  A non-finite value
  // makes its block's scale NaN (poison = sum of v - v is 0 or NaN), and every
  // row partial with it.
  if (tid < 16 * LPR) {
    const int g = tid >> 1, h = tid & 1;
    const int l = g >> 3, q = g & 7;
    float v[4];
    float mx = 0.0f, poison = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = chunk[swz(4 * tid + e)];
      mx = fmaxf(mx, fabsf(v[e]));
      poison += v[e] - v[e];
    }
    mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(mx), 0x128, 0xF, 0xF, false)));
    mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(mx), 0x124, 0xF, 0xF, false)));
    mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(mx), 0x122, 0xF, 0xF, false)));
    mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(mx), 0x121, 0xF, 0xF, false)));
    poison += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(poison), 0x128, 0xF, 0xF, false));
    poison += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(poison), 0x124, 0xF, 0xF, false));
    poison += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(poison), 0x122, 0xF, 0xF, false));
    poison += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(poison), 0x121, 0xF, 0xF, false));
    const bool live = mx > 0.0f && poison == 0.0f;  // a finite block with a nonzero value
    const int fe = live ? __builtin_amdgcn_frexp_expf(mx) : 0;
    const float inv = live ? float(kUqMax) / __builtin_amdgcn_frexp_mantf(mx) : 0.0f;
    uint32_t w[4];
    int32_t gsum = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int U = int(rintf(__builtin_amdgcn_ldexpf(v[e], -fe) * inv));
      U = U > kUqMax ? kUqMax : (U < -kUqMax ? -kUqMax : U);
      gsum += U;
      w[e] = uint32_t(U + 0x8888) ^ 0x8888u;
    }
    gsum += dpp_partner1(gsum);
    // columns 4 h + e sit in nibble (h 2) + lane_nibble(e) of the plane word
    const uint32_t r0 = w[0] | (w[1] << 16), r1 = w[2] | (w[3] << 16);
    uint32_t pl[4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const uint32_t part = ((r0 >> (4 * pp)) & 0x000F000Fu) | (((r1 >> (4 * pp)) & 0x000F000Fu) << 4);
      const uint32_t mine = part << (8 * h);
      pl[pp] = mine | uint32_t(dpp_partner1(int(mine)));
    }
    if (h == 0) {
      img_x4 pv;
      pv.x = pl[0];
      pv.y = pl[1];
      pv.z = pl[2];
      pv.w = pl[3];
      *reinterpret_cast<img_x4*>(lds + kDigOff + 4 * (q * LPR + l)) = pv;
      lds[kGsOff + 4 * ((q >> 2) * LPR + l) + (q & 3)] = uint32_t(-gsum);  // negated: added on complemented reads
      if (q == 0) {
        lds[kScOff + l] = __float_as_uint((live ? __builtin_amdgcn_frexp_mantf(mx) : 0.0f) * a.sc_tab[lb] + poison);
        lds[kFeOff + l] = uint32_t(fe);
        if (live) atomicMax(reinterpret_cast<int*>(lds + kExpOff), fe);
      }
    }
  }
  __syncthreads();
  uint32_t dig[1][GL][4];
  GroupSumsFor<1, GL, CODES> gs;
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
    gs.set(0, 4 * qq + 0, int32_t(g.x));
    gs.set(0, 4 * qq + 1, int32_t(g.y));
    gs.set(0, 4 * qq + 2, int32_t(g.z));
    gs.set(0, 4 * qq + 3, int32_t(g.w));
  }
  // the chunk exponent E (wave-uniform) and the lane's scale relative to 2^E
  const int chunk_exp = __builtin_amdgcn_readfirstlane(int(lds[kExpOff]));
  sc[0] = __builtin_amdgcn_ldexpf(__uint_as_float(lds[kScOff + lane_in_row]),
                                  int(lds[kFeOff + lane_in_row]) - chunk_exp);
  __syncthreads();  // every lane has its digits before image parts 8-9 overwrite them

  // ---- step 3: the rest of the image (and the chunk counter, its word free now that
  // the chunk of u is consumed), then the rows
  image_store<8, 10, true, R8>(img, lds, tid);
  if (dyn && tid == 0) lds[kCtr] = 0u;
  __syncthreads();

  // one row-step: the lane's groups of row r against the digit planes, the
  // fixed-order lane reduction, the row partial into rowbuf
  auto row_step = [&](const RowIdx<GL, X16>& ix, int r) {
    const int o = r * RPS + row_in_step;
    float vv[1];
    row_dots<1, GL, RESID, CODES>(lds, ix.i0, ix.i1w, ix.i1b, dig, gs, a.sr, vv, delta);
#pragma unroll
    for (int k = 0; k < X16; ++k)
      vv[0] = fmaf(a.sc_x16[k], float(stage16_total<GL, CODES>(lds, ix.x16[k], dig, gs, delta)), vv[0]);
    if (X8) vv[0] = fmaf(a.sc_x8, float(stage8_total<GL>(lds, ix.x8, dig)), vv[0]);
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
    if (o < a.m_pad && lane_in_row == LPR - 1)
      rowbuf[swz(o - wg * (a.rs_per_wg * RPS))] = __builtin_amdgcn_ldexpf(v * a.out_scale, chunk_exp);
  };
  auto load_row = [&](int r, RowIdx<GL, X16>& ix) {
    if (FULL)
      load_full(r < r_end ? r : r_end - 1, ix);  // past the end: reload the last row
    else
      load_off(row_off(r < r_end ? r : r_end - 1), ix);
  };
  // The rows' index vectors are loaded ahead into a ring of register sets (rows past
  // r_end load the last row again): with at most two index stages per row, three
  // sets, each loaded two row-steps ahead; with more stages (5-8 bpw, whose rows
  // already carry 3-4 vectors) two sets, one step ahead, so the sets stay in
  // registers.  Whole turns of the ring run in a loop with no early exit (an exit
  // merged into the loop latch makes the compiler wait for every load at the loop
  // head), then the remaining rows.
  constexpr bool kDeep = X16 == 0 && X8 == 0;
  RowIdx<GL, X16> m, p;
  int r = r_begin;
  if (kDynOk && dyn) {
    // chunk ch holds row-steps r_wg0 + 3 ch .. + 2 (rows past r_wg1 load the last row
    // again and are not computed); chunks 0 .. kW-1 go to the waves in order, the rest
    // by the counter, each taken one chunk ahead so that the ring's loads run on
    // across chunks.  The loop's only exit is at its head.
    constexpr int kW = kThreads / 64;
    const int nch = (r_wg1 - r_wg0 + 2) / 3;
    auto take = [&]() {
      uint32_t t = 0;
      if (lane == 0) t = atomicAdd(lds + kCtr, 1u);
      return kW + int(__builtin_amdgcn_readfirstlane(t));
    };
    auto load_at = [&](int ch, int k, RowIdx<GL, X16>& ix) {
      int rr = r_wg0 + 3 * ch + k;
      rr = rr < r_wg1 ? rr : r_wg1 - 1;
      if (FULL)
        load_full(rr, ix);
      else
        load_off(row_off(rr), ix);
    };
    auto step_at = [&](const RowIdx<GL, X16>& ix, int ch, int k) {
      const int rr = r_wg0 + 3 * ch + k;
      if (rr < r_wg1) row_step(ix, rr);
    };
    int ch = wave;
    if (ch < nch) {
      int nx = take();
      load_at(ch, 1, m);
      while (ch < nch) {
        load_at(ch, 2, p);
        step_at(n, ch, 0);
        // without a next chunk the ring's loads reread the row just requested into p
        // (its lines are already on their way into L2), not rows of HBM a chunk old
        load_at(nx < nch ? nx : ch, nx < nch ? 0 : 2, n);
        step_at(m, ch, 1);
        load_at(nx < nch ? nx : ch, nx < nch ? 1 : 2, m);
        step_at(p, ch, 2);
        ch = nx;
        if (ch < nch) nx = take();
      }
    }
  } else if (kDeep) {
    if (r_begin < r_end) load_row(r_begin + 1, m);
    for (; r + 2 < r_end; r += 3) {
      load_row(r + 2, p);
      row_step(n, r);
      load_row(r + 3, n);
      row_step(m, r + 1);
      load_row(r + 4, m);
      row_step(p, r + 2);
    }
    if (r < r_end) row_step(n, r);
    if (r + 1 < r_end) row_step(m, r + 1);
  } else {
    (void)p;
    for (; r + 1 < r_end; r += 2) {
      load_row(r + 1, m);
      row_step(n, r);
      load_row(r + 2, n);
      row_step(m, r + 1);
    }
    if (r < r_end) row_step(n, r);
  }

  // ---- step 4: H_R of each of the workgroup's row blocks into z_parts[split]
  {
    const int rows_wg = a.rs_per_wg * RPS;
    const int row0 = wg * rows_wg;
    const int rows = min(rows_wg, a.m_pad - row0);  // whole row blocks: R divides m_pad
    float* zb = a.z_parts + int64_t(split) * a.m_pad + row0;
    if (a.lr >= 8) {
      __syncthreads();
      const int nrb = rows >> a.lr;
      for (int j = wave; j < nrb; j += kThreads / 64) {
        const int base = j << a.lr;
        switch (a.lr) {
          case 8: wave_block_transform<4>(rowbuf, base, zb + base, lane); break;
          case 9: wave_block_transform<8>(rowbuf, base, zb + base, lane); break;
          default: wave_block_transform<16>(rowbuf, base, zb + base, lane); break;
        }
      }
    } else {
      // the butterflies on bits 0 .. lr-1 of every row block at once, over the
      // power-of-two span of rowbuf that covers the rows (rows past them unused)
      int span = a.lr;
      while ((1 << span) < rows) ++span;
      fwht_lds_passes<StoreZ, 4>(StoreZ{zb, rows}, 0, span, 0, rowbuf, a.lr);
    }
  }
}

template <int RESID, int X16, int X8, bool FULL, bool CODES>
__global__ __launch_bounds__(kThreads) void fused_decode_kernel(FusedArgs a) {
  fused_decode_body<RESID, X16, X8, FULL, CODES>(a, int(blockIdx.x));
}

// Several layers of one launch: layer k owns the workgroups [end[k-1], end[k]) of the
// grid.  Every layer has the same stage layout (RESID, X16, X8) and lanes per row
// (FULL); the arguments of each are its own.
constexpr int kGroupMax = 4;
struct FusedGroupArgs {
  FusedArgs L[kGroupMax];
  int end[kGroupMax];
  int count;
};

__device__ __forceinline__ int group_member(const int* end, int count, int bid) {
  int k = 0;
#pragma unroll
  for (int j = 0; j < kGroupMax - 1; ++j) k += (j < count - 1 && bid >= end[j]) ? 1 : 0;
  return k;
}

template <int RESID, int X16, int X8, bool FULL, bool CODES>
__global__ __launch_bounds__(kThreads) void fused_group_kernel(FusedGroupArgs g) {
  const int bid = int(blockIdx.x);
  const int k = __builtin_amdgcn_readfirstlane(group_member(g.end, g.count, bid));
  fused_decode_body<RESID, X16, X8, FULL, CODES>(g.L[k], bid - (k > 0 ? g.end[k - 1] : 0));
}

// ---- the cross-block part of the output transform ------------------------------------
// Output i = a R + b (row block a < W = m_pad / R, column b < R).  z_parts[s] holds
// H_R of every row block, so for a power-of-two m_pad
// y[a R + b] = sign[i] / sqrt(m_pad) * sum_a' H_W[a][a'] T[a' R + b] with
// T = sum over s = 0 .. S-1, in order, of z_parts[s].  A block-diagonal m_pad
// (R divides its smallest block) does the same inside each of its blocks: the
// butterfly on bit k of a joins a and a ^ 2^k only when both lie in one block,
// i.e. when that block holds more than 2^k row blocks, and the scale is
// 1 / sqrt(block length).  One wave per CB consecutive columns; lane l holds row
// blocks a = l E + e (e < E, 64 E >= W; blocks past W are idle): the bits of e in
// registers, the lane bits by shuffles.
struct BlocksArgs {
  const float* z;
  const int8_t* sign;
  void* y;
  int64_t m;
  int S, m_pad, lr, lw, W;  // lw = ceil(log2 W)
  int vec_sign;  // sign_out 4-byte aligned: one 32-bit load per CB = 4 signs
  int vec_y;     // y aligned for CB-element stores
  float sc_tab[kLenLog2s];  // [log2 L] 1 / sqrt(L)
};

template <int CB>
__device__ __forceinline__ void add_parts(float (&v)[CB], const float* zs) {
  if constexpr (CB == 4) {
    const float4 q = *reinterpret_cast<const float4*>(zs);
    v[0] += q.x;
    v[1 % CB] += q.y;
    v[2 % CB] += q.z;
    v[3 % CB] += q.w;
  } else {
#pragma unroll
    for (int c = 0; c < CB; ++c) v[c] += zs[c];
  }
}

__device__ __forceinline__ uint32_t bits16(half_t v) { return __builtin_bit_cast(uint16_t, v); }
__device__ __forceinline__ uint32_t bits16(bf16_t v) { return v.bits; }

// CB consecutive outputs with one store (p aligned to CB elements)
template <class YT, int CB>
__device__ __forceinline__ void store_vec(YT* p, const YT (&o)[CB]) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  if constexpr (std::is_same<YT, float>::value) {
    if constexpr (CB == 4) *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
    else if constexpr (CB == 2) *reinterpret_cast<float2*>(p) = make_float2(o[0], o[1]);
    else p[0] = o[0];
  } else {
    if constexpr (CB == 4) {
      u32x2 w;
      w.x = bits16(o[0]) | (bits16(o[1]) << 16);
      w.y = bits16(o[2]) | (bits16(o[3]) << 16);
      *reinterpret_cast<u32x2*>(p) = w;
    } else if constexpr (CB == 2) {
      *reinterpret_cast<uint32_t*>(p) = bits16(o[0]) | (bits16(o[1]) << 16);
    } else {
      p[0] = o[0];
    }
  }
}

template <class YT, int E, int CB>
__device__ __forceinline__ void output_blocks_body(const BlocksArgs& a, int bid) {
  const int lane = threadIdx.x;
  const int b0 = bid * CB;
  const bool live = (lane * E) < a.W;
  float v[E][CB];
  uint32_t sg[E];  // sign bytes of the lane's CB outputs per block (sign_out has m_pad entries)
  int gl[E];       // log2 of the length of the transform block holding row block l E + e
#pragma unroll
  for (int e = 0; e < E; ++e) {
#pragma unroll
    for (int c = 0; c < CB; ++c) v[e][c] = 0.0f;
    sg[e] = 0;
    const int ab = lane * E + e;
    gl[e] = ab < a.W ? 31 - __clz(a.m_pad ^ (ab << a.lr)) : 0;
  }
  if (live) {
    // every load is issued before the first use: signs, then the partials of
    // four splits at a time, summed in split order; row blocks past W (only in
    // the last live lane) read a valid address and are not summed
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int64_t i0 = (int64_t(min(lane * E + e, a.W - 1)) << a.lr) + b0;
      if (CB == 4 && a.vec_sign) {
        sg[e] = *reinterpret_cast<const uint32_t*>(a.sign + i0);
      } else {
#pragma unroll
        for (int c = 0; c < CB; ++c) sg[e] |= uint32_t(uint8_t(a.sign[i0 + c])) << (8 * c);
      }
    }
    for (int s = 0; s < a.S; s += 4) {
      float t[4][E][CB];
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < E; ++e) {
#pragma unroll
          for (int c = 0; c < CB; ++c) t[k][e][c] = 0.0f;
          const int sk = s + k < a.S ? s + k : a.S - 1;  // past the last split: a valid address, not summed
          add_parts<CB>(t[k][e], a.z + int64_t(sk) * a.m_pad + (int64_t(min(lane * E + e, a.W - 1)) << a.lr) + b0);
        }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bool in = s + k < a.S;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const bool use = in && lane * E + e < a.W;
#pragma unroll
          for (int c = 0; c < CB; ++c) v[e][c] += use ? t[k][e][c] : 0.0f;
        }
      }
    }
  }
  // register bits: the butterfly (e, e + h) acts when its transform block holds
  // more than h row blocks (both then lie in it; always for a power-of-two m_pad)
#pragma unroll
  for (int h = 1; h < E; h <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if ((e & h) == 0) {
        const bool act = gl[e] - a.lr > log2_exact_dev(h);
#pragma unroll
        for (int c = 0; c < CB; ++c) {
          const float x0 = v[e][c], x1 = v[e + h][c];
          v[e][c] = act ? x0 + x1 : x0;
          v[e + h][c] = act ? x0 - x1 : x1;
        }
      }
    }
  }
  int le = 0;
  while ((1 << le) < E) ++le;
  for (int k = 0; k < a.lw - le; ++k) {
    const bool upper = (lane >> k) & 1;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool act = gl[e] - a.lr > k + le;  // the same on both lanes of the pair
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const float q = __shfl_xor(v[e][c], 1 << k, 64);
        const float r = upper ? q - v[e][c] : v[e][c] + q;
        v[e][c] = act ? r : v[e][c];
      }
    }
  }
  if (!live) return;
  YT* y = static_cast<YT*>(a.y);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (lane * E + e >= a.W) continue;
    const int64_t i0 = (int64_t(lane * E + e) << a.lr) + b0;
    const float scale = a.sc_tab[gl[e]];
    YT o[CB];
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      const uint32_t neg = (sg[e] >> (8 * c + 7)) << 31;  // sign bit of the c-th byte
      o[c] = from_f32<YT>(__uint_as_float(__float_as_uint(v[e][c] * scale) ^ neg));
    }
    if (a.vec_y && i0 + CB <= a.m) {
      store_vec<YT, CB>(y + i0, o);
    } else {
#pragma unroll
      for (int c = 0; c < CB; ++c)
        if (i0 + c < a.m) y[i0 + c] = o[c];
    }
  }
}

template <class YT, int E, int CB>
__global__ __launch_bounds__(64) void output_blocks_kernel(BlocksArgs a) {
  output_blocks_body<YT, E, CB>(a, int(blockIdx.x));
}

// the cross-block launches of several layers in one: layer k owns the waves
// [end[k-1], end[k]); E covers the largest W of the group, CB divides every R
struct BlocksGroupArgs {
  BlocksArgs L[kGroupMax];
  int end[kGroupMax];
  int count;
};

template <class YT, int E, int CB>
__global__ __launch_bounds__(64) void blocks_group_kernel(BlocksGroupArgs g) {
  const int bid = int(blockIdx.x);
  const int k = __builtin_amdgcn_readfirstlane(group_member(g.end, g.count, bid));
  output_blocks_body<YT, E, CB>(g.L[k], bid - (k > 0 ? g.end[k - 1] : 0));
}

template <class YT, int CB>
hipError_t launch_blocks_e(BlocksArgs a, hipStream_t stream) {
  const dim3 grid(unsigned((1 << a.lr) / CB)), block(64);
  a.vec_sign = CB == 4 && reinterpret_cast<uintptr_t>(a.sign) % 4 == 0;
  a.vec_y = reinterpret_cast<uintptr_t>(a.y) % (sizeof(YT) * CB) == 0;
  switch (a.lw <= 6 ? 1 : 1 << (a.lw - 6)) {
    case 1: hipLaunchKernelGGL((output_blocks_kernel<YT, 1, CB>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((output_blocks_kernel<YT, 2, CB>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((output_blocks_kernel<YT, 4, CB>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((output_blocks_kernel<YT, 8, CB>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((output_blocks_kernel<YT, 16, CB>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

// CB columns per wave: 4 when R >= 256, fewer below so that the launch keeps R / CB
// >= 64 waves (each element is computed the same way whatever CB is)
template <class YT>
hipError_t launch_blocks(const BlocksArgs& a, hipStream_t stream) {
  if (a.lr >= 8) return launch_blocks_e<YT, 4>(a, stream);
  if (a.lr == 7) return launch_blocks_e<YT, 2>(a, stream);
  return launch_blocks_e<YT, 1>(a, stream);
}

template <int R_, int X_, int Y_>
struct Stages {
  static constexpr int R = R_, X = X_, Y = Y_;
};

struct FusedPlan {
  int lpr_log2, splits, rps, row_steps, wgs_per_split, rs_per_wg, lr;
  int W;  // row blocks of R = 2^lr rows (the cross-block transform's length)
  bool ok;
};

// cus: the CUs the layer's launch may fill (all of them for a layer on its own)
FusedPlan fused_plan(const glq_layer& L, int cus) {
  FusedPlan p;
  const int64_t G = L.n_pad / 8;
  const int64_t lanes = G / 8;
  int l = 0;
  while ((int64_t(1) << l) < lanes && l < 6) ++l;
  // a split's chunk (64 columns per lane) must lie in one transform block: the
  // smallest block of a block-diagonal n_pad bounds it
  while (l > 0 && L.n_pad % (int64_t(64) << l) != 0) --l;
  p.lpr_log2 = l;
  p.splits = int(G / (int64_t(8) << l));
  p.rps = 64 >> l;
  p.row_steps = int((L.m_pad + p.rps - 1) / p.rps);
  int w = cus / p.splits;
  if (w < 1) w = 1;
  const int min_per_wg = kThreads / 64;  // at least one row-step per wave
  const int wmax = (p.row_steps + min_per_wg - 1) / min_per_wg;
  if (w > wmax) w = wmax;
  // power-of-two m_pad and splits: one row block of R = m_pad / w rows per workgroup
  if (is_pow2(L.m_pad)) {
    p.rs_per_wg = (p.row_steps + w - 1) / w;
    p.wgs_per_split = (p.row_steps + p.rs_per_wg - 1) / p.rs_per_wg;
    int64_t R = int64_t(p.rs_per_wg) * p.rps;
    if (p.wgs_per_split == 1 && R > L.m_pad) R = L.m_pad;
    p.ok = is_pow2(R) && R <= kRowBuf && R * p.wgs_per_split == L.m_pad && p.wgs_per_split <= 1024;
    p.lr = p.ok ? log2_exact(R) : 0;
    p.W = p.wgs_per_split;
    if (p.ok) return p;
  }
  // otherwise (a block-diagonal m_pad, or a split count that does not divide the
  // CUs): a workgroup takes c row blocks of R rows, R a power of two dividing every
  // transform block of m_pad, with c R rows covering m_pad in at most CUs / splits
  // workgroups per split (one round).  Cost in rows of the first launch: its
  // rows per workgroup, plus 16 per row block above 2 that each lane of the
  // cross-block launch sums and transforms (W / 64 of them), plus a quarter for
  // R < 64 (fewer than 64 waves there); ties go to the larger R.
  const int64_t wps = cus / p.splits > 0 ? cus / p.splits : 1;
  const int64_t T = (L.m_pad + wps - 1) / wps;
  const int64_t cap = smallest_block(L.m_pad) < kRowBuf ? smallest_block(L.m_pad) : kRowBuf;
  int64_t best_rows = 0, best_R = 0;
  for (int64_t R = p.rps > 8 ? p.rps : 8; R <= cap; R *= 2) {
    if (L.m_pad % R != 0 || L.m_pad / R > 1024) continue;
    const int64_t rows = (T + R - 1) / R * R;
    if (rows > kRowBuf) continue;
    auto cost_of = [&](int64_t rw, int64_t r) {
      const int64_t e = (L.m_pad / r + 63) / 64;
      return rw + 16 * (e > 2 ? e - 2 : 0) + (r < 64 ? rw / 4 : 0);
    };
    if (best_R == 0 || cost_of(rows, R) <= cost_of(best_rows, best_R)) {
      best_rows = rows;
      best_R = R;
    }
  }
  p.ok = best_R > 0;
  if (!p.ok) return p;
  p.rs_per_wg = int(best_rows / p.rps);
  p.wgs_per_split = int((L.m_pad + best_rows - 1) / best_rows);
  p.lr = log2_exact(best_R);
  p.W = int(L.m_pad / best_R);
  return p;
}

// the stage layout of a layer as (RESID, further 16-bit stages, further 8-bit stages)
void stage_layout(const glq_layer& L, int& x16, int& x8) {
  x16 = (L.n_extra >= 1 && L.extra_bits[0] == 16 ? 1 : 0) + (L.n_extra == 2 && L.extra_bits[1] == 16 ? 1 : 0);
  x8 = L.n_extra >= 1 && L.extra_bits[L.n_extra - 1] == 8 ? 1 : 0;
}

// the first launch's arguments of one layer under plan p
FusedArgs fused_args(const glq_layer& L, const FusedPlan& p, const void* x, glq_dtype x_dt, float* z_parts) {
  FusedArgs a;
  a.x = x;
  a.sign_in = L.sign_in;
  a.idx0 = L.idx0;
  a.idx1 = L.idx1;
  const char* p0 = static_cast<const char*>(L.cb_pack);
  a.pack0_hdr = reinterpret_cast<const uint32_t*>(p0);
  const bool codes = L.index_format == GLQ_INDEX_SLOT;
  a.img0 = reinterpret_cast<const uint32_t*>(
      p0 + (codes ? pack_slot_image_offset(GLQ_CODEBOOK_ENTRIES) : pack_image_offset(GLQ_CODEBOOK_ENTRIES)));
  // further stages (5-8 bpw in one pass): 16-bit ones index the primary pack, an
  // 8-bit one (always the last) the 256-entry residual pack
  int x16, x8;
  stage_layout(L, x16, x8);
  for (int k = 0; k < 2; ++k) {
    a.idx_x16[k] = k < x16 ? static_cast<const uint16_t*>(L.extra_idx[k]) : nullptr;
    a.sc_x16[k] = k < x16 ? L.extra_scale[k] : 0.0f;
  }
  a.idx_x8 = x8 ? static_cast<const uint8_t*>(L.extra_idx[L.n_extra - 1]) : nullptr;
  a.sc_x8 = x8 ? L.extra_scale[L.n_extra - 1] : 0.0f;
  a.res_slots = nullptr;
  const void* res8 = L.resid_bits == 8 ? L.cb2_pack : x8 ? L.cb8_pack : nullptr;
  if (res8)
    a.res_slots = reinterpret_cast<const uint32_t*>(static_cast<const char*>(res8) +
                                                    pack_image_offset(GLQ_RESID8_ENTRIES)) + kPageCount;
  a.z_parts = z_parts;
  a.n = L.n;
  a.x_dt = x_dt;
  a.n_pad = int(L.n_pad);
  a.lk = 6 + p.lpr_log2;
  const size_t xal = x_dt == GLQ_F32 ? 16 : 8;
  a.vec_in = (reinterpret_cast<uintptr_t>(x) % xal == 0) && (reinterpret_cast<uintptr_t>(L.sign_in) % 4 == 0);
  a.G = int(L.n_pad / 8);
  a.m_pad = int(L.m_pad);
  a.lpr_log2 = p.lpr_log2;
  a.row_steps = p.row_steps;
  a.wgs_per_split = p.wgs_per_split;
  a.rs_per_wg = p.rs_per_wg;
  a.lr = p.lr;
  for (int k = 0; k < kLenLog2s; ++k)
    a.sc_tab[k] = float(1.0 / (sqrt(double(int64_t(1) << k)) * double(kUqMax)));
  a.out_scale = 0.5f * L.wscale;
  a.sr = L.resid_scale;
  return a;
}

// the second launch's arguments of one layer under plan p (vec_sign and vec_y are set
// by the launcher, which knows its columns per wave)
BlocksArgs blocks_args(const glq_layer& L, const FusedPlan& p, const float* z_parts, void* y) {
  BlocksArgs b;
  b.z = z_parts;
  b.sign = L.sign_out;
  b.y = y;
  b.m = L.m;
  b.S = p.splits;
  b.m_pad = int(L.m_pad);
  b.lr = p.lr;
  b.W = p.W;
  b.lw = log2_exact(b.W);
  b.vec_sign = 0;
  b.vec_y = 0;
  for (int k = 0; k < kLenLog2s; ++k) b.sc_tab[k] = float(1.0 / sqrt(double(int64_t(1) << k)));
  return b;
}

// The cross-block launch's shape for a layer: E = W / 64 row blocks per lane (at least
// 1; W = 2^lw row blocks), and CB columns per wave for row blocks of 2^lr rows (as
// launch_blocks picks them).  A group takes the largest E and the smallest CB.
int blocks_e(int lw) { return lw <= 6 ? 1 : 1 << (lw - 6); }
int blocks_cb(int lr) { return lr >= 8 ? 4 : lr == 7 ? 2 : 1; }

template <class YT, int E, int CB>
hipError_t launch_blocks_group_ecb(BlocksGroupArgs g, int waves, hipStream_t stream) {
  for (int k = 0; k < g.count; ++k) {
    g.L[k].vec_sign = CB == 4 && reinterpret_cast<uintptr_t>(g.L[k].sign) % 4 == 0;
    g.L[k].vec_y = reinterpret_cast<uintptr_t>(g.L[k].y) % (sizeof(YT) * CB) == 0;
  }
  hipLaunchKernelGGL((blocks_group_kernel<YT, E, CB>), dim3(unsigned(waves)), dim3(64), 0, stream, g);
  return hipGetLastError();
}

template <class YT, int CB>
hipError_t launch_blocks_group_cb(BlocksGroupArgs& g, int E, hipStream_t stream) {
  int waves = 0;
  for (int k = 0; k < g.count; ++k) {
    waves += (1 << g.L[k].lr) / CB;
    g.end[k] = waves;
  }
  switch (E) {
    case 1: return launch_blocks_group_ecb<YT, 1, CB>(g, waves, stream);
    case 2: return launch_blocks_group_ecb<YT, 2, CB>(g, waves, stream);
    case 4: return launch_blocks_group_ecb<YT, 4, CB>(g, waves, stream);
    case 8: return launch_blocks_group_ecb<YT, 8, CB>(g, waves, stream);
    default: return launch_blocks_group_ecb<YT, 16, CB>(g, waves, stream);
  }
}

template <class YT>
hipError_t launch_blocks_group(BlocksGroupArgs& g, int E, int CB, hipStream_t stream) {
  if (CB == 4) return launch_blocks_group_cb<YT, 4>(g, E, stream);
  if (CB == 2) return launch_blocks_group_cb<YT, 2>(g, E, stream);
  return launch_blocks_group_cb<YT, 1>(g, E, stream);
}

// the CUs each layer of a group may fill: every layer its own plan when their grids
// fit the device together, else shares of the CUs in proportion to the layers'
// index groups (at least one workgroup per split)
void group_cus(const glq_layer* Ls, int count, int* cus) {
  const int all = device_cus();
  int64_t wgs = 0, work = 0;
  for (int k = 0; k < count; ++k) {
    const FusedPlan p = fused_plan(Ls[k], all);
    wgs += int64_t(p.splits) * p.wgs_per_split;
    work += Ls[k].m_pad * (Ls[k].n_pad / 8);
  }
  for (int k = 0; k < count; ++k) {
    if (wgs <= all) {
      cus[k] = all;
    } else {
      const int64_t share = int64_t(all) * (Ls[k].m_pad * (Ls[k].n_pad / 8)) / work;
      const int splits = fused_plan(Ls[k], all).splits;
      cus[k] = int(share > splits ? share : splits);
    }
  }
}

}  // namespace

bool fused_decode_supported(const glq_layer& L, int64_t B) {
  // one activation row; 64 <= n_pad (8 groups per lane; the chunk of u, K <= 4096,
  // always fits); the residual stage in the LDS image; row blocks as fused_plan needs
  return B == 1 && L.n_pad >= 64 && (L.resid_bits != 16 || L.cb2_pack == L.cb_pack) &&
         fused_plan(L, device_cus()).ok;
}

size_t fused_decode_z_bytes(const glq_layer& L) {
  const FusedPlan p = fused_plan(L, device_cus());
  return size_t(p.splits) * size_t(L.m_pad) * 4;
}

hipError_t launch_fused_decode(const glq_layer& L, const void* x, glq_dtype x_dt, void* y, glq_dtype y_dt,
                               float* z_parts, hipStream_t stream) {
  const FusedPlan p = fused_plan(L, device_cus());
  const FusedArgs a = fused_args(L, p, x, x_dt, z_parts);
  int x16, x8;
  stage_layout(L, x16, x8);
  const bool codes = L.index_format == GLQ_INDEX_SLOT;
  const dim3 grid(unsigned(p.splits * p.wgs_per_split)), block(kThreads);
  const bool full = p.lpr_log2 == 6;
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, 0, stream, a); };
  // the stage layout: (RESID, X16, X8)
  auto launch_fc = [&](auto tag) {
    constexpr int R = decltype(tag)::R, X = decltype(tag)::X, Y = decltype(tag)::Y;
    if (full)
      codes ? go(fused_decode_kernel<R, X, Y, true, true>) : go(fused_decode_kernel<R, X, Y, true, false>);
    else
      codes ? go(fused_decode_kernel<R, X, Y, false, true>) : go(fused_decode_kernel<R, X, Y, false, false>);
  };
  switch (L.resid_bits * 16 + x16 * 2 + x8) {
    case 0: launch_fc(Stages<0, 0, 0>{}); break;
    case 128: launch_fc(Stages<8, 0, 0>{}); break;
    case 256: launch_fc(Stages<16, 0, 0>{}); break;
    case 257: launch_fc(Stages<16, 0, 1>{}); break;  // 16 + 16 + 8
    case 258: launch_fc(Stages<16, 1, 0>{}); break;  // 16 + 16 + 16
    case 259: launch_fc(Stages<16, 1, 1>{}); break;  // 16 + 16 + 16 + 8
    default: launch_fc(Stages<16, 2, 0>{}); break;   // 16 + 16 + 16 + 16
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const BlocksArgs b = blocks_args(L, p, z_parts, y);
  switch (y_dt) {
    case GLQ_F32: return launch_blocks<float>(b, stream);
    case GLQ_F16: return launch_blocks<half_t>(b, stream);
    default: return launch_blocks<bf16_t>(b, stream);
  }
}

bool fused_group_supported(const glq_layer* Ls, int count) {
  if (count < 1 || count > kGroupMax) return false;
  for (int k = 0; k < count; ++k) {
    const glq_layer& L = Ls[k];
    if (!fused_decode_supported(L, 1)) return false;
    if (L.n_pad != Ls[0].n_pad || L.resid_bits != Ls[0].resid_bits || L.index_format != Ls[0].index_format)
      return false;
    int x16, x8, x16_0, x8_0;
    stage_layout(L, x16, x8);
    stage_layout(Ls[0], x16_0, x8_0);
    if (x16 != x16_0 || x8 != x8_0) return false;
  }
  int cus[kGroupMax];
  group_cus(Ls, count, cus);
  for (int k = 0; k < count; ++k)
    if (!fused_plan(Ls[k], cus[k]).ok) return false;
  return true;
}

size_t fused_group_z_bytes(const glq_layer* Ls, int count, int k) {
  int cus[kGroupMax];
  group_cus(Ls, count, cus);
  return size_t(fused_plan(Ls[k], cus[k]).splits) * size_t(Ls[k].m_pad) * 4;
}

hipError_t launch_fused_group(const glq_layer* Ls, int count, const void* const* x, glq_dtype x_dt, void* const* y,
                              glq_dtype y_dt, float* const* z_parts, hipStream_t stream) {
  int cus[kGroupMax];
  group_cus(Ls, count, cus);
  FusedGroupArgs g;
  BlocksGroupArgs bg;
  int wgs = 0, E = 1, CB = 4;
  bool full = false;
  for (int k = 0; k < count; ++k) {
    const FusedPlan p = fused_plan(Ls[k], cus[k]);
    g.L[k] = fused_args(Ls[k], p, x[k], x_dt, z_parts[k]);
    wgs += p.splits * p.wgs_per_split;
    g.end[k] = wgs;
    bg.L[k] = blocks_args(Ls[k], p, z_parts[k], y[k]);
    E = blocks_e(bg.L[k].lw) > E ? blocks_e(bg.L[k].lw) : E;
    CB = blocks_cb(p.lr) < CB ? blocks_cb(p.lr) : CB;
    full = p.lpr_log2 == 6;  // the same for every layer: one n_pad
  }
  for (int k = count; k < kGroupMax; ++k) g.end[k] = bg.end[k] = 0x7FFFFFFF;
  g.count = bg.count = count;
  const bool codes = Ls[0].index_format == GLQ_INDEX_SLOT;
  const dim3 grid(static_cast<unsigned>(wgs)), block(kThreads);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, 0, stream, g); };
  auto launch_r = [&](auto tag) {
    constexpr int R = decltype(tag)::R, X = decltype(tag)::X, Y = decltype(tag)::Y;
    if (full)
      codes ? go(fused_group_kernel<R, X, Y, true, true>) : go(fused_group_kernel<R, X, Y, true, false>);
    else
      codes ? go(fused_group_kernel<R, X, Y, false, true>) : go(fused_group_kernel<R, X, Y, false, false>);
  };
  int x16, x8;
  stage_layout(Ls[0], x16, x8);
  switch (Ls[0].resid_bits * 16 + x16 * 2 + x8) {
    case 0: launch_r(Stages<0, 0, 0>{}); break;
    case 128: launch_r(Stages<8, 0, 0>{}); break;
    case 256: launch_r(Stages<16, 0, 0>{}); break;
    case 257: launch_r(Stages<16, 0, 1>{}); break;  // 16 + 16 + 8
    case 258: launch_r(Stages<16, 1, 0>{}); break;  // 16 + 16 + 16
    case 259: launch_r(Stages<16, 1, 1>{}); break;  // 16 + 16 + 16 + 8
    default: launch_r(Stages<16, 2, 0>{}); break;   // 16 + 16 + 16 + 16
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (y_dt) {
    case GLQ_F32: return launch_blocks_group<float>(bg, E, CB, stream);
    case GLQ_F16: return launch_blocks_group<half_t>(bg, E, CB, stream);
    default: return launch_blocks_group<bf16_t>(bg, E, CB, stream);
  }
}

GLQ_DEBUG_COUNTER(debug_violations_fused_decode)

}  // namespace glq
