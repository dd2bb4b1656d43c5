// Randomized Hadamard transforms on gfx950: the input RHT (sign flip, FWHT,
// 1/sqrt(n_pad)) and the output RHT (fixed-order sum of split partials, FWHT,
// 1/sqrt(m_pad), sign flip, truncation to m, cast).
//
// glq 0.5.1 (PyPI project page), "How it works", item 2: random sign flips
// followed by a fast Walsh-Hadamard transform.  Glq v0.3.2 release notes, "What
// changed": separate input_rht / output_rht operations, one-workgroup transforms
// up to 16384 and a separate path above that.
//
// A length that is not a power of two is transformed block-diagonally: its
// blocks are the powers of two of its binary expansion, largest first, each
// transformed on its own and scaled by 1/sqrt(block length) (glq 0.5.1, table
// "Bit widths" and the note below it: 2688 = 2048 + 512 + 128, no padding).  A
// power of two is one block.
//
// Transform order is Sylvester's: butterflies (a, b) -> (a + b, a - b) on every
// index bit.  One workgroup transforms one row of up to 2^14 fp32 values in LDS:
// the first 4 bits in registers straight from global memory, then radix-16
// passes over LDS (XOR-swizzled so strided passes spread over the banks), the
// last pass writing to global memory.  Longer rows use H_{N1 N2} = H_{N1} (x) H_{N2}
// with index i = a * N2 + c: a row pass of length N2 for every a, then a column
// pass of length N1 <= 64 per c held in registers.
#include <math.h>

#include <atomic>

#include "fwht_lds.h"

namespace glq {
namespace {

// ---- element loaders / storers ------------------------------------------------
template <class XT>
struct LoadSignedX {  // x [B][n] -> sign[c] * x[b][c] at c = off + i, zero beyond n
  const XT* x;
  int64_t n, off;
  const int8_t* sign;
  __device__ float operator()(int64_t b, int64_t i) const {
    const int64_t c = off + i;
    // both loads unconditional (sign has n_pad entries, x's column is clamped into its
    // row, n >= 1), so that a thread's loads are in flight together; zero beyond n
    const float v = to_f32<XT>(x[b * n + (c < n ? c : n - 1)]) * float(sign[c]);
    return c < n ? v : 0.0f;
  }
};

// LoadSignedX with row b scaled by 2^-rexp[b] (exact: a power of two), the fp16
// prefill operands' row scales; a non-finite row (kRowExpNaN) is not scaled
template <class XT>
struct LoadSignedXRow {
  LoadSignedX<XT> in;
  const int32_t* rexp;
  __device__ float operator()(int64_t b, int64_t i) const {
    const int32_t e = rexp[b];
    return __builtin_amdgcn_ldexpf(in(b, i), e == kRowExpNaN ? 0 : -e);
  }
};

struct LoadF32 {  // p [B][N]
  const float* p;
  int64_t N;
  __device__ float operator()(int64_t b, int64_t i) const { return p[b * N + i]; }
};

template <class UT>
struct StoreScaled {  // u[b][off + i] = RN(v * scale), rows of N
  UT* u;
  int64_t N, off;
  float scale;
  __device__ void operator()(int64_t b, int64_t i, float v) const { u[b * N + off + i] = from_f32<UT>(v * scale); }
};

// u16 in the prefill matmul's fragment order: token b, column c = off + i of group
// g = c / 8 (k-step ks = g mod KS, lane quarter q = g / KS, KS = n_pad / 32) at
// (((b / 16) KS + ks) 4 + q) 128 + (b mod 16) 8 + c mod 8
// u in the prefill matmuls' fragment order, fp16: 16-token blocks; the groups
// interleave by 4 over the four lane quarters, g = 16 (ks / 4) + 4 q + ks % 4,
// KS = N / 32 k-steps.
struct StoreTiledHalf {
  half_t* u;
  uint32_t KS;
  int64_t off;
  float scale;
  __device__ void operator()(int64_t b, int64_t i, float v) const {
    const int64_t c = off + i;
    const uint32_t g = uint32_t(c >> 3);
    const uint32_t q = (g >> 2) & 3u, ks = ((g >> 4) << 2) | (g & 3u);
    const int64_t o = ((((b >> 4) * KS + ks) * 4 + q) * 16 + (b & 15)) * 8 + (c & 7);
    u[o] = from_f32<half_t>(v * scale);
  }
  // the 8 columns i .. i + 7 of one group (i a multiple of 8): one 16-byte store
  __device__ void store8(int64_t b, int64_t i, const float (&v)[8]) const {
    const uint32_t g = uint32_t((off + i) >> 3);
    const uint32_t q = (g >> 2) & 3u, ks = ((g >> 4) << 2) | (g & 3u);
    const int64_t o = ((((b >> 4) * KS + ks) * 4 + q) * 16 + (b & 15)) * 8;
    uint32_t h[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) h[k] = __builtin_bit_cast(uint16_t, from_f32<half_t>(v[k] * scale));
    uint4 w;
    w.x = h[0] | (h[1] << 16);
    w.y = h[2] | (h[3] << 16);
    w.z = h[4] | (h[5] << 16);
    w.w = h[6] | (h[7] << 16);
    *reinterpret_cast<uint4*>(u + o) = w;
  }
};

struct StoreLdsRow {  // element i of the row -> its swizzled LDS position
  float* buf;
  __device__ void operator()(int64_t, int64_t i, float v) const { buf[swz(int(i))] = v; }
};

struct StoreF32 {
  float* p;
  int64_t N;
  __device__ void operator()(int64_t b, int64_t i, float v) const { p[b * N + i] = v; }
};

// Row r of a segmented pass is (b, a) = (r >> nseg_log2, r & (N1 - 1)); element c of
// it is element a * N2 + c of row b.
template <class Inner>
struct SegLoad {
  Inner in;
  int seg_log2, nseg_log2;
  __device__ float operator()(int64_t r, int64_t c) const {
    const int64_t a = r & ((int64_t(1) << nseg_log2) - 1);
    return in(r >> nseg_log2, (a << seg_log2) + c);
  }
  // a span never crosses a segment (R divides the segment length)
  template <int R>
  __device__ void load_span(int64_t r, int64_t c0, float (&v)[R]) const {
    const int64_t a = r & ((int64_t(1) << nseg_log2) - 1);
    load_elems<R>(in, r >> nseg_log2, (a << seg_log2) + c0, v);
  }
};
template <class Inner>
struct SegStore {
  Inner in;
  int seg_log2, nseg_log2;
  __device__ void operator()(int64_t r, int64_t c, float v) const {
    const int64_t a = r & ((int64_t(1) << nseg_log2) - 1);
    in(r >> nseg_log2, (a << seg_log2) + c, v);
  }
};

template <class Load, class Store>
__global__ __launch_bounds__(1024) void fwht_rows_kernel(Load ld, Store st, int L) {
  extern __shared__ float buf[];
  fwht_row_lds(ld, st, int64_t(blockIdx.x), L, buf);
}

// ---- column pass of the two-pass transform ------------------------------------
template <int N1, class Load, class Store>
__global__ __launch_bounds__(256) void fwht_cols_kernel(Load ld, Store st, int64_t B, int seg_log2) {
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= (B << seg_log2)) return;
  const int64_t b = t >> seg_log2;
  const int64_t c = t & ((int64_t(1) << seg_log2) - 1);
  float v[N1];
#pragma unroll
  for (int a = 0; a < N1; ++a) v[a] = ld(b, (int64_t(a) << seg_log2) + c);
  fwht_reg<N1>(v);
#pragma unroll
  for (int a = 0; a < N1; ++a) st(b, (int64_t(a) << seg_log2) + c, v[a]);
}

template <class Load, class Store>
hipError_t run_rows(const Load& ld, const Store& st, int64_t rows, int L, hipStream_t stream) {
  int threads = (1 << L) / 16;
  if (threads < 64) threads = 64;
  if (threads > 1024) threads = 1024;
  const size_t shmem = L > 4 ? (size_t(4) << L) : 0;
  hipLaunchKernelGGL((fwht_rows_kernel<Load, Store>), dim3(unsigned(rows)), dim3(threads), shmem, stream, ld, st,
                     L);
  return hipGetLastError();
}

template <class Load, class Store>
hipError_t run_cols(const Load& ld, const Store& st, int64_t B, int seg_log2, int l_col, hipStream_t stream) {
  const int64_t total = B << seg_log2;
  const dim3 grid(unsigned((total + 255) / 256)), block(256);
  switch (l_col) {
    case 1: hipLaunchKernelGGL((fwht_cols_kernel<2, Load, Store>), grid, block, 0, stream, ld, st, B, seg_log2); break;
    case 2: hipLaunchKernelGGL((fwht_cols_kernel<4, Load, Store>), grid, block, 0, stream, ld, st, B, seg_log2); break;
    case 3: hipLaunchKernelGGL((fwht_cols_kernel<8, Load, Store>), grid, block, 0, stream, ld, st, B, seg_log2); break;
    case 4: hipLaunchKernelGGL((fwht_cols_kernel<16, Load, Store>), grid, block, 0, stream, ld, st, B, seg_log2); break;
    case 5: hipLaunchKernelGGL((fwht_cols_kernel<32, Load, Store>), grid, block, 0, stream, ld, st, B, seg_log2); break;
    case 6: hipLaunchKernelGGL((fwht_cols_kernel<64, Load, Store>), grid, block, 0, stream, ld, st, B, seg_log2); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// One block of 2^L columns at column `off`: one-workgroup rows up to 2^14, else the
// row pass into `mid` (rows of 2^L floats) and the column pass from it.
template <class Load, class Store>
hipError_t run_block(const Load& ld, const Store& st, int64_t B, int L, float* mid, hipStream_t stream) {
  const int64_t N = int64_t(1) << L;
  int lr, lc;
  fwht_split(B, L, &lr, &lc);
  if (lc == 0) return run_rows(ld, st, B, L, stream);
  hipError_t e = run_rows(SegLoad<Load>{ld, lr, lc}, SegStore<StoreF32>{StoreF32{mid, N}, lr, lc}, B << lc, lr,
                          stream);
  if (e != hipSuccess) return e;
  return run_cols(LoadF32{mid, N}, st, B, lr, lc, stream);
}

// the blocks of length N, largest first: calls f(offset, log2 length)
template <class F>
hipError_t for_blocks(int64_t N, F f) {
  int64_t off = 0;
  for (int L = 62; L >= 0; --L) {
    if (!((N >> L) & 1)) continue;
    hipError_t e = f(off, L);
    if (e != hipSuccess) return e;
    off += int64_t(1) << L;
  }
  return hipSuccess;
}

template <class XT, class UT>
hipError_t rht_in_typed(const void* x, int64_t B, int64_t n, int64_t N, const int8_t* sign, void* u, float* ws,
                        hipStream_t stream, const int32_t* rexp) {
  return for_blocks(N, [&](int64_t off, int L) {
    const float scale = float(1.0 / sqrt(double(int64_t(1) << L)));
    const LoadSignedX<XT> ld{static_cast<const XT*>(x), n, off, sign};
    // an fp32 u is its own two-pass buffer when it is one block
    float* mid = (sizeof(UT) == 4 && off == 0 && N == (int64_t(1) << L)) ? reinterpret_cast<float*>(u) : ws;
    const StoreScaled<UT> st{static_cast<UT*>(u), N, off, scale};
    if (rexp) return run_block(LoadSignedXRow<XT>{ld, rexp}, st, B, L, mid, stream);
    return run_block(ld, st, B, L, mid, stream);
  });
}

template <class XT>
hipError_t rht_in_x(const void* x, int64_t B, int64_t n, int64_t N, const int8_t* sign, void* u, glq_dtype u_dt,
                    float* ws, hipStream_t stream, const int32_t* rexp) {
  switch (u_dt) {
    case GLQ_F32: return rht_in_typed<XT, float>(x, B, n, N, sign, u, ws, stream, rexp);
    case GLQ_F16: return rht_in_typed<XT, half_t>(x, B, n, N, sign, u, ws, stream, rexp);
    case GLQ_BF16: return rht_in_typed<XT, bf16_t>(x, B, n, N, sign, u, ws, stream, rexp);
  }
  return hipErrorInvalidValue;
}

// ---- the rows' power-of-two exponents of the fp16 prefill operands ---------------------
// One workgroup per row: m = max |x[b]| (fmax ignores NaN; poison, the sum of v - v,
// is 0 or NaN and catches NaN and inf), then rexp[b] = frexp exponent of m + add,
// add = ceil(log2 sqrt(n)) - 14, so that |u| <= ||x[b]|| <= sqrt(n) m < 2^(rexp + 14).
// With VEC the row is read as 16-byte vectors, VEC elements each, four loads in flight
// per thread before any is used.
template <class XT, int VEC>
__global__ __launch_bounds__(1024) void row_exp_kernel(const XT* __restrict__ x, int64_t n, int add,
                                                       int32_t* __restrict__ rexp) {
  __shared__ float red[2][16];
  const int64_t b = blockIdx.x;
  const XT* xr = x + b * n;
  const int nt = int(blockDim.x);
  float mx = 0.0f, poison = 0.0f;
  auto take = [&](float v) {
    mx = fmaxf(mx, fabsf(v));
    poison += v - v;
  };
  if constexpr (VEC > 1) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4* xv = reinterpret_cast<const u32x4*>(xr);
    const int64_t nv = n / VEC;
    for (int64_t i0 = threadIdx.x; i0 < nv; i0 += 4 * int64_t(nt)) {
      u32x4 t[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t i = i0 + int64_t(k) * nt;
        t[k] = xv[i < nv ? i : nv - 1];  // past the end: the last vector again (a repeat)
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const XT* e = reinterpret_cast<const XT*>(&t[k]);
#pragma unroll
        for (int j = 0; j < VEC; ++j) take(to_f32<XT>(e[j]));
      }
    }
  } else {
    for (int64_t i = threadIdx.x; i < n; i += nt) take(to_f32<XT>(xr[i]));
  }
  for (int off = 1; off < 64; off <<= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    poison += __shfl_xor(poison, off, 64);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wave] = mx;
    red[1][wave] = poison;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    mx = 0.0f;
    poison = 0.0f;
    for (int w = 0; w < (nt >> 6); ++w) {
      mx = fmaxf(mx, red[0][w]);
      poison += red[1][w];
    }
    rexp[b] = poison != 0.0f ? kRowExpNaN : mx > 0.0f ? __builtin_amdgcn_frexp_expf(mx) + add : 0;
  }
}

// One row per workgroup (block of 2^L columns, 3 <= L <= kSingleLog2) into the
// fragment order: the one-workgroup transform with its last pass writing back to
// LDS, then each thread stores whole 8-column groups as single 16-byte stores.
// The 16 rows of a 16-token block share every 256-byte span of the output, so the
// rows go to the XCDs (workgroups are dispatched to them round-robin) in runs of
// whole blocks, per_xcd blocks each: a span is assembled in one L2 and written back
// whole.  Workgroups past the last row exit at once.
template <class XT>
__global__ __launch_bounds__(1024) void rht_in_tiled_kernel(LoadSignedXRow<XT> ld, StoreTiledHalf st, int L,
                                                            int64_t B, int per_xcd) {
  extern __shared__ float buf[];
  const int64_t b = int64_t(blockIdx.x & 7u) * per_xcd * 16 + (blockIdx.x >> 3);
  if (b >= B) return;
  // the last pass reads and writes the same LDS positions in the same thread
  fwht_row_lds(ld, StoreLdsRow{buf}, b, L, buf);
  __syncthreads();
  const int groups = (1 << L) >> 3;
  for (int g = threadIdx.x; g < groups; g += blockDim.x) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = buf[swz(8 * g + j)];
    st.store8(b, int64_t(8) * g, v);
  }
}

// input transform into the prefill matmul's fragment order (fp16), rows scaled by
// 2^-rexp[b]
template <class XT>
hipError_t rht_in_tiled_x(const void* x, int64_t B, int64_t n, int64_t N, const int8_t* sign, const int32_t* rexp,
                          half_t* u16, float* ws, hipStream_t stream) {
  return for_blocks(N, [&](int64_t off, int L) {
    const float scale = float(1.0 / sqrt(double(int64_t(1) << L)));
    const LoadSignedXRow<XT> ld{LoadSignedX<XT>{static_cast<const XT*>(x), n, off, sign}, rexp};
    const StoreTiledHalf st{u16, uint32_t(N / 32), off, scale};
    int lr, lc;
    fwht_split(B, L, &lr, &lc);
    if (L < 3 || lc > 0) return run_block(ld, st, B, L, ws, stream);
    int threads = (1 << L) / 16;
    if (threads < 64) threads = 64;
    if (threads > 1024) threads = 1024;
    const int64_t per_xcd = ((B + 15) / 16 + 7) / 8;  // 16-row blocks per XCD
    hipLaunchKernelGGL((rht_in_tiled_kernel<XT>), dim3(unsigned(8 * per_xcd * 16)), dim3(threads), size_t(4) << L,
                       stream, ld, st, L, B, int(per_xcd));
    return hipGetLastError();
  });
}

// ---- output transform, one row at a time per workgroup, 4096 <= N <= 32768 -------------
// Thread t holds the float4s at 4 t + 4096 i (i < IT = N / 4096) of the row's split
// sum (s = 0 .. S-1 in order, all loads of a split in flight), so bits 0-1 and the
// bits of i (12 and up) are transformed in registers and bits 2-11 in two LDS passes
// of 5 bits; then each thread writes 8 consecutive outputs at a time (16-byte stores
// where y allows), sign-flipped, scaled and cast.  Workgroups are persistent (one per
// CU, at most B): once a row is in LDS, the loads of the workgroup's next row are
// issued, so they overlap the LDS passes and stores (up to 2^14-point rows).
template <class YT>
__device__ __forceinline__ void store8(YT* y, const float (&v)[8]);
template <>
__device__ __forceinline__ void store8<float>(float* y, const float (&v)[8]) {
  reinterpret_cast<float4*>(y)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(y)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
template <class YT>
__device__ __forceinline__ void store8(YT* y, const float (&v)[8]) {
  uint4 w;
  uint32_t h[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) h[k] = __builtin_bit_cast(uint16_t, from_f32<YT>(v[k]));
  w.x = h[0] | (h[1] << 16);
  w.y = h[2] | (h[3] << 16);
  w.z = h[4] | (h[5] << 16);
  w.w = h[6] | (h[7] << 16);
  *reinterpret_cast<uint4*>(y) = w;
}

// The block is columns off .. off + N - 1 of rows of ldz partials (z + off and
// sign + off are passed in) and of m outputs, mv = min(N, m - off) of them kept.
// acc = sum over s = 0 .. S-1, in order, of the float4s at 4 t + 4096 i of row `row`
// of split s (all loads of a group of splits in flight together)
template <int IT>
__device__ __forceinline__ void split_sum_row(const float* __restrict__ z, int64_t ldz, int S, int B, int row, int c,
                                              float4 (&acc)[IT]) {
  const float* zr = z + int64_t(row) * ldz;
#pragma unroll
  for (int i = 0; i < IT; ++i) acc[i] = *reinterpret_cast<const float4*>(zr + c + 4096 * i);
  constexpr int UN = IT >= 8 ? 1 : 8 / IT;
  int s = 1;
  for (; s + UN <= S; s += UN) {
    float4 v[UN][IT];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
#pragma unroll
      for (int i = 0; i < IT; ++i)
        v[u][i] = *reinterpret_cast<const float4*>(zr + (int64_t(s + u) * B) * ldz + c + 4096 * i);
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
      const float4 v = *reinterpret_cast<const float4*>(zr + (int64_t(s) * B) * ldz + c + 4096 * i);
      acc[i].x += v.x;
      acc[i].y += v.y;
      acc[i].z += v.z;
      acc[i].w += v.w;
    }
  }
}

template <class YT, int IT>
__global__ __launch_bounds__(1024) void rows_out_kernel(const float* __restrict__ z, int64_t ldz, int S, int B,
                                                       int64_t m, int mv, const int8_t* __restrict__ sign,
                                                       YT* __restrict__ y, float scale, int vec_y) {
  extern __shared__ float buf[];
  const int tid = threadIdx.x;
  const int c = tid * 4;
  float4 acc[IT];
  int row = blockIdx.x;  // rows blockIdx.x, + gridDim.x, ... (the grid holds at most B workgroups)
  split_sum_row<IT>(z, ldz, S, B, row, c, acc);
  for (;;) {
    float t[4 * IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      t[4 * i + 0] = acc[i].x;
      t[4 * i + 1] = acc[i].y;
      t[4 * i + 2] = acc[i].z;
      t[4 * i + 3] = acc[i].w;
    }
    fwht_reg<4 * IT>(t);  // bits 0-1 and 12 + log2 i
#pragma unroll
    for (int i = 0; i < IT; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) buf[swz(c + 4096 * i + e)] = t[4 * i + e];
    }
    // the next row's loads are in flight during this row's LDS passes and stores
    // (not for 2^15-point rows, whose registers are all taken by the passes)
    const int next = row + int(gridDim.x);
    if constexpr (IT <= 4) {
      if (next < B) split_sum_row<IT>(z, ldz, S, B, next, c, acc);
    }
    fwht_lds_passes<StoreLdsRow, 5>(StoreLdsRow{buf}, 0, 12 + log2_exact_dev(IT), 2, buf, 12);
    __syncthreads();
    YT* yr = y + int64_t(row) * m;
    if (vec_y) {
      for (int o = tid * 8; o < mv; o += 1024 * 8) {
        const uint2 sg = *reinterpret_cast<const uint2*>(sign + o);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t neg = ((e < 4 ? sg.x : sg.y) >> (8 * (e & 3) + 7)) & 1u;
          v[e] = __uint_as_float(__float_as_uint(buf[swz(o + e)] * scale) ^ (neg << 31));
        }
        store8<YT>(yr + o, v);
      }
    } else {
      for (int o = tid; o < mv; o += 1024) {
        const uint32_t neg = sign[o] < 0 ? 0x80000000u : 0u;
        yr[o] = from_f32<YT>(__uint_as_float(__float_as_uint(buf[swz(o)] * scale) ^ neg));
      }
    }
    if (next >= B) break;
    row = next;
    __syncthreads();  // every thread's reads of buf are done before the next row's writes
    if constexpr (IT > 4) split_sum_row<IT>(z, ldz, S, B, row, c, acc);
  }
}

template <class YT>
hipError_t rht_out_block(const float* z, int64_t S, int64_t B, int64_t m, int64_t ldz, int64_t off, int L,
                         const int8_t* sign, void* y, float* ws, hipStream_t stream) {
  const float scale = float(1.0 / sqrt(double(int64_t(1) << L)));
  if (L >= 12 && L <= 15 && B >= kMinRowWgs) {
    const int64_t mv = m - off < (int64_t(1) << L) ? m - off : (int64_t(1) << L);
    // 16-byte output stores need y + off 16-byte aligned, mv % 8 == 0 and 8-byte aligned signs
    YT* yp = static_cast<YT*>(y) + off;
    const int8_t* sg = sign + off;
    const int vec_y = (reinterpret_cast<uintptr_t>(static_cast<YT*>(y) + off) % 16 == 0) && m % 8 == 0 &&
                      mv % 8 == 0 && (reinterpret_cast<uintptr_t>(sg) % 8 == 0);
    const float* zb = z + off;
    const size_t shmem = size_t(4) << L;
    // resident workgroups: one per CU (16 waves holding over 64 registers each)
    const int64_t wgs = int64_t(device_cus());
    const dim3 grid{unsigned(B < wgs ? B : wgs)}, block{1024};
    const int S_ = int(S), B_ = int(B), mv_ = int(mv);
    switch (L) {
      case 12: hipLaunchKernelGGL((rows_out_kernel<YT, 1>), grid, block, shmem, stream, zb, ldz, S_, B_, m, mv_, sg, yp, scale, vec_y); break;
      case 13: hipLaunchKernelGGL((rows_out_kernel<YT, 2>), grid, block, shmem, stream, zb, ldz, S_, B_, m, mv_, sg, yp, scale, vec_y); break;
      case 14: hipLaunchKernelGGL((rows_out_kernel<YT, 4>), grid, block, shmem, stream, zb, ldz, S_, B_, m, mv_, sg, yp, scale, vec_y); break;
      default: {
        // 128 KiB of dynamic LDS: raise the kernel's limit once per device (threads
        // racing on the first call both set it: harmless, and the flag is atomic)
        static std::atomic<uint64_t> lds_set{0};
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) dev = 0;
        const uint64_t bit = uint64_t(1) << (dev & 63);
        if (!(lds_set.load(std::memory_order_relaxed) & bit)) {
          hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&rows_out_kernel<YT, 8>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, int(shmem));
          if (e != hipSuccess) return e;
          lds_set.fetch_or(bit, std::memory_order_relaxed);
        }
        hipLaunchKernelGGL((rows_out_kernel<YT, 8>), grid, block, shmem, stream, zb, ldz, S_, B_, m, mv_, sg, yp,
                           scale, vec_y);
        break;
      }
    }
    return hipGetLastError();
  }
  const LoadSplitSum ld{z, S, B, ldz, off};
  const StoreOut<YT> st{static_cast<YT*>(y), m, off, sign, scale};
  return run_block(ld, st, B, L, ws, stream);
}

template <class YT>
hipError_t rht_out_typed(const float* z, int64_t S, int64_t B, int64_t m, int64_t N, const int8_t* sign, void* y,
                         float* ws, hipStream_t stream) {
  return for_blocks(N, [&](int64_t off, int L) {
    // blocks wholly past m (possible only with padding) are not computed
    if (off >= m) return hipSuccess;
    return rht_out_block<YT>(z, S, B, m, N, off, L, sign, y, ws, stream);
  });
}

}  // namespace

hipError_t launch_rht_in(const void* x, glq_dtype x_dt, int64_t B, int64_t n, int64_t N, const int8_t* sign,
                         void* u, glq_dtype u_dt, float* ws, hipStream_t stream, const int32_t* rexp) {
  switch (x_dt) {
    case GLQ_F32: return rht_in_x<float>(x, B, n, N, sign, u, u_dt, ws, stream, rexp);
    case GLQ_F16: return rht_in_x<half_t>(x, B, n, N, sign, u, u_dt, ws, stream, rexp);
    case GLQ_BF16: return rht_in_x<bf16_t>(x, B, n, N, sign, u, u_dt, ws, stream, rexp);
  }
  return hipErrorInvalidValue;
}

template <class XT>
hipError_t row_exp_t(const void* x, int64_t B, int64_t n, int add, int32_t* rexp, hipStream_t stream) {
  constexpr int VEC = 16 / int(sizeof(XT));
  const bool vec = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (n % VEC == 0);
  const int64_t items = vec ? n / VEC : n;
  int threads = int(((items + 3) / 4 + 63) / 64 * 64);  // about four loads per thread
  threads = threads < 64 ? 64 : threads > 1024 ? 1024 : threads;
  const XT* xp = static_cast<const XT*>(x);
  if (vec)
    hipLaunchKernelGGL((row_exp_kernel<XT, VEC>), dim3(unsigned(B)), dim3(threads), 0, stream, xp, n, add, rexp);
  else
    hipLaunchKernelGGL((row_exp_kernel<XT, 1>), dim3(unsigned(B)), dim3(threads), 0, stream, xp, n, add, rexp);
  return hipGetLastError();
}

hipError_t launch_row_exp(const void* x, glq_dtype x_dt, int64_t B, int64_t n, int32_t* rexp, hipStream_t stream) {
  int c = 0;  // ceil(log2 sqrt(n))
  while ((int64_t(1) << (2 * c)) < n) ++c;
  const int add = c - 14;
  switch (x_dt) {
    case GLQ_F32: return row_exp_t<float>(x, B, n, add, rexp, stream);
    case GLQ_F16: return row_exp_t<half_t>(x, B, n, add, rexp, stream);
    case GLQ_BF16: return row_exp_t<bf16_t>(x, B, n, add, rexp, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_rht_in_tiled(const void* x, glq_dtype x_dt, int64_t B, int64_t n, int64_t N, const int8_t* sign,
                               const int32_t* rexp, half_t* u16, float* ws, hipStream_t stream) {
  switch (x_dt) {
    case GLQ_F32: return rht_in_tiled_x<float>(x, B, n, N, sign, rexp, u16, ws, stream);
    case GLQ_F16: return rht_in_tiled_x<half_t>(x, B, n, N, sign, rexp, u16, ws, stream);
    case GLQ_BF16: return rht_in_tiled_x<bf16_t>(x, B, n, N, sign, rexp, u16, ws, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_rht_out(const float* z, int64_t S, int64_t B, int64_t m, int64_t N, const int8_t* sign, void* y,
                          glq_dtype y_dt, float* ws, hipStream_t stream) {
  switch (y_dt) {
    case GLQ_F32: return rht_out_typed<float>(z, S, B, m, N, sign, y, ws, stream);
    case GLQ_F16: return rht_out_typed<half_t>(z, S, B, m, N, sign, y, ws, stream);
    case GLQ_BF16: return rht_out_typed<bf16_t>(z, S, B, m, N, sign, y, ws, stream);
  }
  return hipErrorInvalidValue;
}

GLQ_DEBUG_COUNTER(debug_violations_rht)

}  // namespace glq
