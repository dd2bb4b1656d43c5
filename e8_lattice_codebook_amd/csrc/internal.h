// Internal declarations shared by the HIP sources of the E8RHTLinear library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "glq.h"

namespace glq {

// ---- debug builds (GLQ_DEBUG) -------------------------------------------------------
// Device-side bounds checks: a failed check adds one to its source file's counter and
// the kernel runs on (no trap); glq_debug_violations() reads and clears the counters.
// Release builds compile the checks away.
#if defined(GLQ_DEBUG) && defined(__HIP__)
static __device__ unsigned int g_debug_violations;
#define GLQ_DCHECK(cond)                                            \
  do {                                                              \
    if (!(cond)) atomicAdd(&::glq::g_debug_violations, 1u);         \
  } while (0)
#define GLQ_DEBUG_COUNTER(fn)                                                       \
  uint32_t fn() {                                                                   \
    uint32_t v = 0;                                                                 \
    const uint32_t zero = 0;                                                        \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_debug_violations), 4) != hipSuccess)   \
      return 0xFFFFFFFFu;                                                           \
    (void)hipMemcpyToSymbol(HIP_SYMBOL(g_debug_violations), &zero, 4);              \
    return v;                                                                       \
  }
#else
#define GLQ_DCHECK(cond) \
  do {                   \
  } while (0)
#define GLQ_DEBUG_COUNTER(fn) \
  uint32_t fn() { return 0; }
#endif
// the counter of each HIP source file (debug builds; 0 otherwise)
uint32_t debug_violations_rht();
uint32_t debug_violations_dequant();
uint32_t debug_violations_gemv();
uint32_t debug_violations_gemv_lds();
uint32_t debug_violations_fused_decode();
uint32_t debug_violations_gemm();
uint32_t debug_violations_gemm_lds();
uint32_t debug_violations_gemm_shared();
uint32_t debug_violations_kv_attention();
uint32_t debug_violations_noalloc();
uint32_t debug_violations_gemv_i8();

// Longest transform done by one workgroup in LDS (16384 fp32 = 64 KiB).  Longer
// transforms use the Kronecker split H_{a*b} = H_a (x) H_b in two passes.
constexpr int kSingleLog2 = 14;
// Split point of the two-pass transform: the row pass has length 2^kSplitLog2
// (or n_pad / 64 when that is longer), the column pass the rest (<= 64).
constexpr int kSplitLog2 = 12;

inline int log2_exact(int64_t v) {
  int l = 0;
  while ((int64_t(1) << l) < v) ++l;
  return l;
}
inline bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
// A transform length: a power of two (one block), or a multiple of 64 that is
// transformed block-diagonally over its binary expansion (largest block first).
inline int64_t largest_block(int64_t v) {
  int64_t b = 1;
  while (b <= v / 2) b *= 2;
  return b;
}
inline int64_t smallest_block(int64_t v) { return v & -v; }
__host__ __device__ constexpr int log2_exact_dev(int v) { return v <= 1 ? 0 : 1 + log2_exact_dev(v >> 1); }
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Rows of a transform launch below which one workgroup per row leaves most of the
// GPU idle; such launches split every row into segments instead.
constexpr int64_t kMinRowWgs = 128;
// Split of a length-2^L transform over B rows: (row pass log2, column pass log2), the
// column pass (2^l_col <= 64 points per column, in registers) empty when one workgroup
// per row does the whole row.  Above 2^kSingleLog2 points the row pass is 2^kSplitLog2
// (or 2^(L-6)) long; from 2^13 points with fewer than kMinRowWgs rows it is shortened
// (to 2^kSplitLog2 points at least) until B 2^l_col reaches kMinRowWgs.
inline void fwht_split(int64_t B, int L, int* l_row, int* l_col) {
  int r = L;
  if (L > kSingleLog2) r = L - 6 > kSplitLog2 ? L - 6 : kSplitLog2;
  while (L >= 13 && (B << (L - r)) < kMinRowWgs && L - r < 6 && r - 1 >= kSplitLog2) --r;
  *l_row = r;
  *l_col = L - r;
}

// ---- numeric storage types -------------------------------------------------
typedef _Float16 half_t;
struct bf16_t {
  uint16_t bits;
};

template <class T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<half_t>(half_t v) { return (float)v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) {
  return __uint_as_float(uint32_t(v.bits) << 16);
}

template <class T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ half_t from_f32<half_t>(float v) {
  // v rounded to fp32 first: the empty constraint keeps the compiler from fusing the
  // product that made v into a mixed-precision FMA rounded once to fp16
  asm("" : "+v"(v));
  return (half_t)v;
}
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) {
  // nearest, ties to even (finite values)
  uint32_t b = __float_as_uint(v);
  b += 0x7FFFu + ((b >> 16) & 1u);
  bf16_t r;
  r.bits = uint16_t(b >> 16);
  return r;
}

// ---- codebook pack layout ----------------------------------------------------
// header (256 B) | int8 table [entries][8] = 2c | LDS image (page table + slots)
constexpr uint32_t kPackMagic = 0x32514C47u;  // "GLQ2"
constexpr uint32_t kPackVersion = 5;
constexpr int kPageSize = 256;                 // indices per page
constexpr int kPageCount = 256;                // pages of a 16-bit index
constexpr int kImageMaxDwords = 39680;         // LDS image budget: 155 KiB
constexpr int kResidDwords = 256;              // 8-bit residual slots (direct)
// A slot word holds the 8 coordinates 2c as signed 4-bit lanes; coordinate e sits
// in nibble lane_nibble(e), so that nibbles j and j + 4 (16 bits apart) hold the
// adjacent coordinates 2j and 2j + 1.
__host__ __device__ constexpr int lane_nibble(int e) { return (e >> 1) + 4 * (e & 1); }
inline size_t pack_i8_offset() { return 256; }
inline size_t pack_image_offset(int64_t entries) { return align256(256 + size_t(entries) * 8); }
// Slot-code format (header words 5 and 6: slot image dwords, 0 when the codebook
// has no slot format, and delta): a 16-bit code c, read as int16 with m = c >> 15
// (0 or all ones), names slot (c ^ m) + (m & delta) of the slot image, a plain
// 4-byte word like a page slot, read complemented when m is all ones.  code_of
// [entries] maps an index to its code and index_of [65536] a code to its index.
constexpr int kHdrSlotDwords = 5;
constexpr int kHdrSlotDelta = 6;
constexpr int kSlotShared = 32768;  // codes below, and complemented codes, both reach [delta, 32768)
// Slot images larger than this get no slot format: the shared-tile prefill kernel
// keeps the slot image, an fp16 residual table and two codeword tiles in LDS.
constexpr int kSlotImageMaxDwords = 37632;
inline size_t pack_slot_image_offset(int64_t entries) { return pack_image_offset(entries) + size_t(kImageMaxDwords) * 4; }
inline size_t pack_code_of_offset(int64_t entries) { return pack_slot_image_offset(entries) + size_t(kImageMaxDwords) * 4; }
inline size_t pack_index_of_offset(int64_t entries) { return pack_code_of_offset(entries) + align256(size_t(entries) * 2); }
size_t pack_total_bytes(int64_t entries);
glq_status build_pack(const uint16_t* cb_host, int64_t entries, void* pack_host, size_t pack_bytes);

// ---- launchers (return the launch status) -----------------------------------

// Transforms of length N (block-diagonal when N is not a power of two).
// Input transform; ws: fp32 [B][N] scratch, used only when a block is longer than
// 2^kSingleLog2 and u is not fp32 of one block.
// rexp (may be NULL): row b of x is scaled by 2^-rexp[b] as it is loaded
hipError_t launch_rht_in(const void* x, glq_dtype x_dt, int64_t B, int64_t n, int64_t N, const int8_t* sign,
                         void* u, glq_dtype u_dt, float* ws, hipStream_t stream, const int32_t* rexp = nullptr);
// Output transform of sum_s z[s] (rows of N); ws: fp32 [B][N] scratch used only
// when a block is longer than 2^kSingleLog2.
hipError_t launch_rht_out(const float* z, int64_t S, int64_t B, int64_t m, int64_t N, const int8_t* sign,
                          void* y, glq_dtype y_dt, float* ws, hipStream_t stream);

hipError_t launch_dequant(const glq_layer& layer, void* w, glq_dtype w_dt, hipStream_t stream);
hipError_t launch_slot_codes(const void* cb_pack, const uint16_t* idx, int64_t count, uint16_t* codes,
                             hipStream_t stream);

// Decode matmul, codewords gathered from the packs' int8 tables in global memory
// (used when a 16-bit residual stage has its own codebook): z_parts [S][B][m_pad].
int gemv_splits(int64_t n_pad, int64_t B);
hipError_t launch_gemv(const glq_layer& layer, const float* u, int64_t B, float* z_parts,
                       hipStream_t stream);

// Decode matmul with the codebook image resident in LDS.  u is first quantized to
// 16-bit fixed point (4 int4 digit planes per 8-column group, one scale per 64
// columns) into uq_bytes(B, n_pad) of scratch; z_parts [S][B][m_pad] with
// S = gemv_lds_splits(n_pad, B).
size_t uq_bytes(int64_t B, int64_t n_pad);
int gemv_lds_splits(int64_t n_pad, int64_t B);
hipError_t launch_quant_u(const float* u, int64_t B, int64_t n_pad, void* uq, hipStream_t stream);
// accumulate: add to z_parts instead of storing (the second pass of a 5-8 bpw layer)
hipError_t launch_gemv_lds(const glq_layer& layer, const void* uq, int64_t B, float* z_parts, hipStream_t stream,
                           bool accumulate = false);

// Decode matmul for a few activation rows (4 <= B <= 16) on the int8 matrix units.  u
// (fp32 [B][n_pad]) is quantized per row to 15-bit fixed point, two int8 planes in the
// operand order (i8_planes_bytes(n_pad)) plus an I8RowInfo per row of the 16-row
// operand; z_parts [S][B][m_pad] with S = gemv_i8_splits(n_pad, m_pad).
struct I8RowInfo {
  int32_t e;     // U = rint(u 2^(14 - e))
  float poison;  // 0, or NaN for a row with a NaN or infinity
};
bool gemv_i8_supported(const glq_layer& layer);
int gemv_i8_splits(int64_t n_pad, int64_t m_pad);
size_t i8_planes_bytes(int64_t n_pad);
hipError_t launch_quant_i8(const float* u, int64_t B, int64_t n_pad, void* planes, I8RowInfo* info,
                           hipStream_t stream);
hipError_t launch_gemv_i8(const glq_layer& layer, const void* planes, const I8RowInfo* info, int64_t B,
                          float* z_parts, hipStream_t stream, bool accumulate = false);
// Up to GLQ_GROUP_MAX layers' int8 GEMVs in one launch, the CUs shared among them:
// gemv_i8_group_plan says whether the layers can share one (every layer supported, one
// residual stage, index format and row blocks per wave) and gives each layer's split
// count (its z_parts hold splits[k] x B x m_pad); one pass per layer, no accumulation.
bool gemv_i8_group_plan(const glq_layer* layers, int count, int* splits);
hipError_t launch_gemv_i8_group(const glq_layer* layers, int count, const void* const* planes,
                                const I8RowInfo* const* info, int64_t B, float* const* z_parts, hipStream_t stream);

// The whole linear for B = 1 in two launches (input RHT, decode matmul with the
// LDS codebook and the row-local part of the output RHT; then the fixed-order
// split reduction and the rest of the output RHT).  z_parts:
// fused_decode_z_bytes(layer) of scratch.
bool fused_decode_supported(const glq_layer& layer, int64_t B);
size_t fused_decode_z_bytes(const glq_layer& layer);
// Every stage of the layer (5-8 bpw included) is summed in the one pass.
hipError_t launch_fused_decode(const glq_layer& layer, const void* x, glq_dtype x_dt, void* y, glq_dtype y_dt,
                               float* z_parts, hipStream_t stream);
// Up to four such layers at B = 1 in one pair of launches: same n_pad, stage layout
// and index format; each layer its own x, y and z_parts
// (fused_group_z_bytes(layers, count, k) for layer k), the CUs shared among them.
bool fused_group_supported(const glq_layer* layers, int count);
size_t fused_group_z_bytes(const glq_layer* layers, int count, int k);
hipError_t launch_fused_group(const glq_layer* layers, int count, const void* const* x, glq_dtype x_dt,
                              void* const* y, glq_dtype y_dt, float* const* z_parts, hipStream_t stream);

// Compute units of the current device (256 if the query fails), cached per device.
int device_cus();

// Prefill matmul: z [M][m_pad] fp32 from u16 fp16, either in fragment order
// [ceil(M/16)][n_pad/32][4][16][8] (tiled_u_bytes), as launch_rht_in_tiled writes it,
// or [M][n_pad].  launch_gemm_shared: slot-code layers (gemm_shared_supported), u16
// in fragment order.  launch_gemm_lds: the per-wave LDS-codebook kernel on either
// order (tiled).  launch_gemm: u16 [M][n_pad]; launch_gemm_lds when
// gemm_lds_supported(layer), else the kernel that gathers codewords from the pack's
// int8 tables.
bool gemm_shared_supported(const glq_layer& layer);
size_t tiled_u_bytes(int64_t M, int64_t n_pad);
// fp16 prefill operands carry a power-of-two scale per row: u[b] = 2^rexp[b] * (the
// fp16 values stored), rexp[b] chosen from max |x[b]| so that no stored value
// exceeds 2^14 (see launch_row_exp); the matmuls apply 2^rexp[b] to row b of z in
// fp32.  kRowExpNaN marks a row holding a value that is not finite: its z row is NaN.
constexpr int32_t kRowExpNaN = 0x7FFFFFFF;
// Fragment-order u16 followed (at a 256-byte boundary) by int32 rexp [ceil(M/16) 16].
inline size_t prefill_rexp_offset(int64_t M, int64_t n_pad) { return align256(tiled_u_bytes(M, n_pad)); }
inline size_t prefill_u_total_bytes(int64_t M, int64_t n_pad) {
  return prefill_rexp_offset(M, n_pad) + align256(size_t((M + 15) / 16) * 16 * 4);
}
// rexp[b] = e with max |x[b]| < 2^(e + 14) / sqrt(n) (so |u| <= ||x[b]|| < 2^(e + 14)
// after the orthonormal transform); 0 for a zero row, kRowExpNaN for a non-finite one
hipError_t launch_row_exp(const void* x, glq_dtype x_dt, int64_t B, int64_t n, int32_t* rexp, hipStream_t stream);
// z of a row with exponent e: v 2^e (NaN for a non-finite row)
__device__ __forceinline__ float row_scaled(float v, int32_t e) {
  return e == kRowExpNaN ? __builtin_nanf("") : __builtin_amdgcn_ldexpf(v, e);
}
hipError_t launch_gemm_shared(const glq_layer& layer, const half_t* u16, const int32_t* rexp, int64_t M, float* z,
                              hipStream_t stream, bool accumulate = false);
bool gemm_lds_supported(const glq_layer& layer);
hipError_t launch_gemm_lds(const glq_layer& layer, const half_t* u16, const int32_t* rexp, int64_t M, bool tiled,
                           float* z, hipStream_t stream, bool accumulate = false);
// rexp: the rows' exponents (launch_row_exp), applied to x as it is loaded
hipError_t launch_rht_in_tiled(const void* x, glq_dtype x_dt, int64_t B, int64_t n, int64_t N, const int8_t* sign,
                               const int32_t* rexp, half_t* u16, float* ws, hipStream_t stream);
// rexp may be NULL (no row scales)
hipError_t launch_gemm(const glq_layer& layer, const half_t* u16, const int32_t* rexp, int64_t M, float* z,
                       hipStream_t stream, bool accumulate = false);

// Decode attention over an E8-compressed paged K/V cache: chunks of T tokens per
// (sequence, KV head) in a persistent kernel, then the chunks merged in order.
// Workspace: units * G * D floats of partial outputs, then units * G * 2 floats of
// (max, exp-sum), units = B * num_kv_heads * splits.
struct KvPlan {
  int T, TS, splits;  // tokens per unit, per sub-chunk; units per (sequence, KV head)
  int64_t units;
};
KvPlan kv_plan(int64_t B, int64_t Hkv, int64_t G, int64_t max_seq_len);
hipError_t launch_kv_attention(const glq_kv_cache& kv, const void* q, glq_dtype q_dt, int64_t B, int64_t Hq,
                               const int32_t* block_table, int64_t max_pages, const int32_t* seq_lens,
                               int64_t max_seq_len, float sm_scale, void* out, glq_dtype out_dt, float* part_o,
                               float* part_ml, hipStream_t stream);

}  // namespace glq
