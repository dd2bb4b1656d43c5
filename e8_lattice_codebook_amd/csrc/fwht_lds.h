// Fast Walsh-Hadamard transform building blocks shared by the transform kernels
// and the fused decode kernel: in-register butterflies, the XOR swizzle of LDS
// rows, the split-sum loader and the output storer, and the register-blocked
// passes of a one-workgroup transform of a row held in LDS.
//
// Order is Sylvester's: butterflies (a, b) -> (a + b, a - b) on every index bit.
#pragma once

#include <type_traits>

#include "internal.h"

namespace glq {
namespace {

template <int R>
__device__ __forceinline__ void fwht_reg(float* v) {
#pragma unroll
  for (int h = 1; h < R; h <<= 1) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

__device__ __forceinline__ int swz(int i) { return i ^ ((i >> 5) & 31); }

// LDS position of element i of a row: XOR of the low 5 bits with bits 5..9, so
// strided passes spread over the banks (a permutation inside each 32-block).

// The loaders and storers address element i of a transform block that starts at
// column `off` of its row (off = 0 and one block for a power-of-two length).
struct LoadSplitSum {  // sum over s = 0..S-1, in order, of z[s][b][off + i]; rows of N
  const float* z;
  int64_t S, B, N, off;
  __device__ float operator()(int64_t b, int64_t i) const {
    const float* p = z + b * N + off + i;
    const int64_t step = B * N;
    float acc = p[0];
    int64_t s = 1;
    // eight partials in flight at a time, added in split order
    for (; s + 8 <= S; s += 8) {
      float t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = p[(s + j) * step];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += t[j];
    }
    for (; s < S; ++s) acc += p[s * step];
    return acc;
  }
  template <int R>
  __device__ void load_span(int64_t b, int64_t i0, float (&v)[R]) const {
    const float* p = z + b * N + off + i0;
    const int64_t step = B * N;
#pragma unroll
    for (int j = 0; j < R; ++j) v[j] = p[j];
    for (int64_t s = 1; s < S; ++s) {
      float t[R];
#pragma unroll
      for (int j = 0; j < R; ++j) t[j] = p[s * step + j];
#pragma unroll
      for (int j = 0; j < R; ++j) v[j] += t[j];
    }
  }
};

template <class YT>
struct StoreOut {  // y[b][c] = RN(sign[c] * v * scale) for c = off + i < m
  YT* y;
  int64_t m, off;
  const int8_t* sign;
  float scale;
  __device__ void operator()(int64_t b, int64_t i, float v) const {
    const int64_t c = off + i;
    if (c < m) y[b * m + c] = from_f32<YT>(v * scale * float(sign[c]));
  }
};

// ---- R consecutive elements i0 .. i0 + R - 1 of a row ----------------------------------
// By default one load call per element.  A loader with load_span(row, i0, v) (R a
// template parameter) takes them together: the split-sum loader issues the R loads of
// one split at a time, so a thread's loads of a split are in flight together (the sums
// keep their split order, so the result is the same bit for bit).
template <class Load, class = void>
struct HasSpan : std::false_type {};
template <class Load>
struct HasSpan<Load, decltype(void(&Load::template load_span<1>))> : std::true_type {};

template <int R, class Load>
__device__ __forceinline__ void load_elems(const Load& ld, int64_t row, int64_t i0, float (&v)[R]) {
  if constexpr (HasSpan<Load>::value) {
    ld.template load_span<R>(row, i0, v);
  } else {
#pragma unroll
    for (int j = 0; j < R; ++j) v[j] = ld(row, i0 + j);
  }
}

// ---- one row per workgroup -------------------------------------------------------
template <int R, class Load, class Store>
__device__ __forceinline__ void first_pass(const Load& ld, const Store& st, int64_t row, int L, float* buf,
                                           bool last) {
  const int chunks = (1 << L) / R;
  for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
    float v[R];
    load_elems<R>(ld, row, int64_t(c) * R, v);
    fwht_reg<R>(v);
    if (last) {
#pragma unroll
      for (int j = 0; j < R; ++j) st(row, c * R + j, v[j]);
    } else {
#pragma unroll
      for (int j = 0; j < R; ++j) buf[swz(c * R + j)] = v[j];
    }
  }
}

template <int LR, class Store>
__device__ __forceinline__ void mid_pass(const Store& st, int64_t row, int L, int b0, float* buf, bool last) {
  constexpr int R = 1 << LR;
  const int groups = (1 << L) >> LR;
  const int lowmask = (1 << b0) - 1;
  for (int g = threadIdx.x; g < groups; g += blockDim.x) {
    const int base = (g & lowmask) | ((g >> b0) << (b0 + LR));
    float v[R];
#pragma unroll
    for (int j = 0; j < R; ++j) v[j] = buf[swz(base + (j << b0))];
    fwht_reg<R>(v);
    if (last) {
#pragma unroll
      for (int j = 0; j < R; ++j) st(row, base + (j << b0), v[j]);
    } else {
#pragma unroll
      for (int j = 0; j < R; ++j) buf[swz(base + (j << b0))] = v[j];
    }
  }
}

// The passes over bits b0 .. b_end-1 (b_end = L by default) of a row of 2^L
// elements in buf (swizzled) whose other bits are done; the last pass stores
// through `st`.
// Every pass starts with a workgroup barrier.
// Passes take up to MAXB bits each (4: 16 values per thread, 5: 32).
template <class Store, int MAXB = 4>
__device__ __forceinline__ void fwht_lds_passes(const Store& st, int64_t row, int L, int b0, float* buf,
                                                int b_end = -1) {
  static_assert(MAXB == 4 || MAXB == 5, "4 or 5 bits per pass");
  if (b_end < 0) b_end = L;
  for (; b0 < b_end; b0 += MAXB) {
    __syncthreads();
    const int rb = (b_end - b0) < MAXB ? (b_end - b0) : MAXB;
    const bool last = (b0 + rb == b_end);
    switch (rb) {
      case 1: mid_pass<1>(st, row, L, b0, buf, last); break;
      case 2: mid_pass<2>(st, row, L, b0, buf, last); break;
      case 3: mid_pass<3>(st, row, L, b0, buf, last); break;
      case 4: mid_pass<4>(st, row, L, b0, buf, last); break;
      default:
        if constexpr (MAXB == 5) mid_pass<5>(st, row, L, b0, buf, last);
        break;
    }
  }
}

// A one-workgroup transform of row `row` (length 2^L) from `ld` to `st`, through
// buf (2^L floats of LDS); the first pass reads 4 bits' worth of elements per
// thread straight from `ld`, the last pass stores straight to `st`.
template <class Load, class Store>
__device__ __forceinline__ void fwht_row_lds(const Load& ld, const Store& st, int64_t row, int L, float* buf) {
  const int r0 = L < 4 ? L : 4;
  const bool last0 = (r0 == L);
  switch (r0) {
    case 0: if (threadIdx.x == 0) st(row, 0, ld(row, 0)); break;
    case 1: first_pass<2>(ld, st, row, L, buf, last0); break;
    case 2: first_pass<4>(ld, st, row, L, buf, last0); break;
    case 3: first_pass<8>(ld, st, row, L, buf, last0); break;
    default: first_pass<16>(ld, st, row, L, buf, last0); break;
  }
  fwht_lds_passes(st, row, L, r0, buf);
}

}  // namespace
}  // namespace glq
