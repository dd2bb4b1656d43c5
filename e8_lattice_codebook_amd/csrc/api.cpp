// C ABI entry points: argument validation, workspace layout and dispatch to
// the gfx950 kernels.  Nothing here allocates, frees or synchronizes.
#include <atomic>
#include <cstdint>
#include <cstring>

#include "internal.h"

using namespace glq;

// A per-device cache; threads that race on a device's first call each query the
// attribute and store the same value (relaxed atomics: no data race).
int glq::device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cus[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

namespace {

bool valid_dtype(glq_dtype d) { return d == GLQ_F32 || d == GLQ_F16 || d == GLQ_BF16; }

// a transform length: a power of two in [8, GLQ_MAX_PAD], or a multiple of 64 below
// GLQ_MAX_PAD (block-diagonal transform over its binary expansion)
bool valid_pad(int64_t p) {
  return p >= 8 && p <= GLQ_MAX_PAD && (is_pow2(p) || p % 64 == 0);
}

// scratch of the two-pass transform of B rows of length N: some block runs in two
// passes (longer than one workgroup's, or split for want of rows), unless the output
// is fp32 of one block (its own scratch)
bool rht_needs_ws(int64_t B, int64_t N, bool f32_out) {
  bool two = false;
  for (int L = 0; L < 63; ++L) {
    if (!((N >> L) & 1)) continue;
    int lr, lc;
    fwht_split(B, L, &lr, &lc);
    two = two || lc > 0;
  }
  return two && !(f32_out && is_pow2(N));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

glq_status from_hip(hipError_t e) { return e == hipSuccess ? GLQ_OK : GLQ_ERR_HIP; }

// Validation of a layer descriptor.  need_signs: the RHT steps use the signs.
glq_status check_layer(const glq_layer* L, bool need_signs) {
  if (!L) return GLQ_ERR_NULL;
  if (!L->idx0 || !L->cb_pack) return GLQ_ERR_NULL;
  if (need_signs && (!L->sign_in || !L->sign_out)) return GLQ_ERR_NULL;
  if (!valid_pad(L->n_pad) || !valid_pad(L->m_pad)) return GLQ_ERR_SHAPE;
  if (L->m_pad * (L->n_pad / 8) >= (int64_t(1) << 31)) return GLQ_ERR_SHAPE;  // 32-bit group offsets
  if (need_signs && (L->n < 1 || L->n > L->n_pad || L->m < 1 || L->m > L->m_pad)) return GLQ_ERR_SHAPE;
  if (L->resid_bits != 0 && L->resid_bits != 8 && L->resid_bits != 16) return GLQ_ERR_RECIPE;
  if (L->resid_bits != 0 && (!L->idx1 || !L->cb2_pack)) return GLQ_ERR_NULL;
  if (!aligned(L->idx0, 16) || !aligned(L->cb_pack, 256)) return GLQ_ERR_ALIGN;
  if (L->resid_bits != 0 && (!aligned(L->idx1, 16) || !aligned(L->cb2_pack, 256))) return GLQ_ERR_ALIGN;
  if (L->index_format != GLQ_INDEX_CODEBOOK && L->index_format != GLQ_INDEX_SLOT) return GLQ_ERR_RECIPE;
  // further residual stages: the 5-8 bpw rows of "Bit widths"
  if (L->n_extra < 0 || L->n_extra > 2) return GLQ_ERR_RECIPE;
  if (L->n_extra > 0) {
    if (L->resid_bits != 16 || L->cb2_pack != L->cb_pack) return GLQ_ERR_RECIPE;
    if (L->n_extra == 2 && L->extra_bits[0] != 16) return GLQ_ERR_RECIPE;
    for (int k = 0; k < L->n_extra; ++k) {
      if (L->extra_bits[k] != 8 && L->extra_bits[k] != 16) return GLQ_ERR_RECIPE;
      if (!(L->extra_scale[k] == L->extra_scale[k]) || L->extra_scale[k] == 0.0f) return GLQ_ERR_RECIPE;
      if (!L->extra_idx[k]) return GLQ_ERR_NULL;
      if (!aligned(L->extra_idx[k], 16)) return GLQ_ERR_ALIGN;
      if (L->extra_bits[k] == 8 && !L->cb8_pack) return GLQ_ERR_NULL;
      if (L->extra_bits[k] == 8 && !aligned(L->cb8_pack, 256)) return GLQ_ERR_ALIGN;
    }
  }
  // slot codes of a 16-bit residual stage name entries of the primary pack
  if (L->index_format == GLQ_INDEX_SLOT && L->resid_bits == 16 && L->cb2_pack != L->cb_pack) return GLQ_ERR_RECIPE;
  return GLQ_OK;
}

// A 5-8 bpw layer as two passes shaped like 2-4 bpw layers whose partial outputs
// add (every kernel then needs only an accumulating store): pass a is the primary
// with one residual stage, pass b the remaining stages with their scale folded
// into wscale.
//   16+16+8:    a = (0, 2 [8 bit]),  b = (1)
//   16+16+16:   a = (0, 1),          b = (2)
//   16+16+16+x: a = (0, 1),          b = (2, 3 [x bit])
struct Passes {
  glq_layer a, b;
  bool two;
};

Passes split_passes(const glq_layer& L) {
  Passes P{L, L, false};
  P.a.n_extra = P.b.n_extra = 0;
  if (L.n_extra == 0) return P;
  P.two = true;
  if (L.n_extra == 1 && L.extra_bits[0] == 8) {
    P.a.idx1 = L.extra_idx[0];
    P.a.resid_bits = 8;
    P.a.resid_scale = L.extra_scale[0];
    P.a.cb2_pack = L.cb8_pack;
    P.b.idx0 = static_cast<const uint16_t*>(L.idx1);
    P.b.idx1 = nullptr;
    P.b.resid_bits = 0;
    P.b.cb2_pack = nullptr;
    P.b.wscale = L.wscale * L.resid_scale;
  } else if (L.n_extra == 1) {
    P.b.idx0 = static_cast<const uint16_t*>(L.extra_idx[0]);
    P.b.idx1 = nullptr;
    P.b.resid_bits = 0;
    P.b.cb2_pack = nullptr;
    P.b.wscale = L.wscale * L.extra_scale[0];
  } else {
    P.b.idx0 = static_cast<const uint16_t*>(L.extra_idx[0]);
    P.b.idx1 = L.extra_idx[1];
    P.b.resid_bits = L.extra_bits[1];
    P.b.resid_scale = L.extra_scale[1] / L.extra_scale[0];
    P.b.cb2_pack = L.extra_bits[1] == 8 ? L.cb8_pack : L.cb_pack;
    P.b.wscale = L.wscale * L.extra_scale[0];
  }
  return P;
}

// fp16 prefill operands of the linear: fragment order (with the row exponents as
// its trailer) for the LDS-codebook matmuls, else row order followed by them
bool prefill_tiled(const glq_layer& L) { return gemm_shared_supported(L) || gemm_lds_supported(L); }
size_t prefill_u_region(const glq_layer& L, int64_t B) {
  return prefill_tiled(L) ? prefill_u_total_bytes(B, L.n_pad)
                          : align256(size_t(B) * size_t(L.n_pad) * 2) + align256(size_t(B) * 4);
}
size_t prefill_rexp_off(const glq_layer& L, int64_t B) {
  return prefill_tiled(L) ? prefill_rexp_offset(B, L.n_pad) : align256(size_t(B) * size_t(L.n_pad) * 2);
}

// Linear workspace: the buffers of the B = 1 two-launch path or of the staged path.
struct LinearWs {
  size_t u_off, uq_off, rin_off, z_off, rout_off, total;
  int splits;
  bool prefill, lds, fused, skinny;
};



constexpr int64_t kDecodeMaxB = 16;
// The decode matmul runs on the int8 matrix units for 2 <= B <= kDecodeMaxB on layers
// of at least 2^21 groups, and from 4 rows on layers of at least 2^17 groups (its cost
// per codeword does not grow with B; smaller layers and batches are bound by launches
// and the transforms, where the staged integer GEMV path measured faster), for every
// pass of the layer.
bool skinny_ok(const glq_layer& L, int64_t B) {
  if (B < 2 || B > kDecodeMaxB) return false;
  const int64_t groups = L.m_pad * (L.n_pad / 8);
  if (groups < (int64_t(1) << 17) || (B < 4 && groups < (int64_t(1) << 21))) return false;
  const Passes P = split_passes(L);
  return gemv_i8_supported(P.a) && (!P.two || gemv_i8_supported(P.b));
}

// the decode kernel with the LDS codebook needs the 16-bit residual stage (if
// any) to use the primary codebook; otherwise codewords come from global memory
bool decode_uses_lds(const glq_layer& L) { return L.resid_bits != 16 || L.cb2_pack == L.cb_pack; }

int matmul_splits(const glq_layer& L, int64_t B) {
  if (B > kDecodeMaxB) return 1;
  return decode_uses_lds(L) ? gemv_lds_splits(L.n_pad, B) : gemv_splits(L.n_pad, B);
}

// scratch of glq_e8_matmul: the quantized activations of the LDS decode kernel
size_t matmul_ws_bytes(const glq_layer& L, int64_t B) {
  return (B <= kDecodeMaxB && decode_uses_lds(L)) ? uq_bytes(B, L.n_pad) : 0;
}

// the int8 path's workspace: fp32 u, its int8 planes (+ row info), split partials
// (splits of them), output scratch
void skinny_layout(const glq_layer& L, int64_t B, int splits, LinearWs& w) {
  size_t off = 0;
  w.u_off = off;
  off += align256(size_t(B) * size_t(L.n_pad) * 4);
  w.uq_off = off;
  off += align256(i8_planes_bytes(L.n_pad)) + align256(16 * sizeof(I8RowInfo));
  w.rin_off = off;
  if (rht_needs_ws(B, L.n_pad, true)) off += align256(size_t(B) * size_t(L.n_pad) * 4);
  w.splits = splits;
  w.z_off = off;
  off += align256(size_t(w.splits) * size_t(B) * size_t(L.m_pad) * 4);
  w.rout_off = off;
  if (rht_needs_ws(B, L.m_pad, false)) off += align256(size_t(B) * size_t(L.m_pad) * 4);
  w.total = off;
}

LinearWs linear_ws(const glq_layer& L, int64_t B) {
  LinearWs w{};
  w.prefill = B > kDecodeMaxB;
  w.lds = !w.prefill && decode_uses_lds(L);
  w.fused = fused_decode_supported(L, B);
  w.skinny = !w.fused && skinny_ok(L, B);
  size_t off = 0;
  if (w.fused) {
    w.z_off = off;
    w.total = off + align256(fused_decode_z_bytes(L));
    return w;
  }
  if (w.skinny) {
    skinny_layout(L, B, gemv_i8_splits(L.n_pad, L.m_pad), w);
    return w;
  }
  w.u_off = off;
  off += !w.prefill ? align256(size_t(B) * size_t(L.n_pad) * 4) : prefill_u_region(L, B);
  w.uq_off = off;
  if (w.lds) off += align256(uq_bytes(B, L.n_pad));
  w.rin_off = off;
  if (rht_needs_ws(B, L.n_pad, !w.prefill)) off += align256(size_t(B) * size_t(L.n_pad) * 4);
  w.splits = matmul_splits(L, B);
  w.z_off = off;
  off += align256(size_t(w.splits) * size_t(B) * size_t(L.m_pad) * 4);
  w.rout_off = off;
  if (rht_needs_ws(B, L.m_pad, false)) off += align256(size_t(B) * size_t(L.m_pad) * 4);
  w.total = off;
  return w;
}

// decode matmul from fp32 u: quantize into uq (LDS kernel) or gather from global
hipError_t decode_matmul(const glq_layer& L, const float* u, int64_t B, void* uq, float* z, hipStream_t stream) {
  if (decode_uses_lds(L)) {  // always for 5-8 bpw (their 16-bit stages use the primary pack)
    const Passes P = split_passes(L);
    hipError_t e = launch_quant_u(u, B, L.n_pad, uq, stream);
    if (e != hipSuccess) return e;
    e = launch_gemv_lds(P.a, uq, B, z, stream);
    if (e != hipSuccess || !P.two) return e;
    return launch_gemv_lds(P.b, uq, B, z, stream, true);
  }
  return launch_gemv(L, u, B, z, stream);
}

// prefill matmul of every pass.  u16 in fragment order: the shared-tile kernel
// (slot codes), else the per-wave kernel; u16 in row order: launch_gemm.  rexp:
// the rows' power-of-two exponents (NULL: none).
hipError_t prefill_pass(const glq_layer& L, const half_t* u16, const int32_t* rexp, int64_t M, bool tiled, float* z,
                        hipStream_t stream, bool acc) {
  if (!tiled) return launch_gemm(L, u16, rexp, M, z, stream, acc);
  if (gemm_shared_supported(L)) return launch_gemm_shared(L, u16, rexp, M, z, stream, acc);
  return launch_gemm_lds(L, u16, rexp, M, true, z, stream, acc);
}

hipError_t prefill_matmul(const glq_layer& L, const half_t* u16, const int32_t* rexp, int64_t M, bool tiled, float* z,
                          hipStream_t stream) {
  const Passes P = split_passes(L);
  hipError_t e = prefill_pass(P.a, u16, rexp, M, tiled, z, stream, false);
  if (e != hipSuccess || !P.two) return e;
  return prefill_pass(P.b, u16, rexp, M, tiled, z, stream, true);
}


template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

}  // namespace

extern "C" {

int glq_abi_version(void) { return GLQ_ABI_VERSION; }

int64_t glq_debug_violations(void) {
#ifdef GLQ_DEBUG
  (void)hipDeviceSynchronize();
  using namespace glq;
  const uint32_t parts[] = {debug_violations_rht(),       debug_violations_dequant(),   debug_violations_gemv(),
                            debug_violations_gemv_lds(),  debug_violations_fused_decode(),
                            debug_violations_gemm(),      debug_violations_gemm_lds(),  debug_violations_gemm_shared(),
                            debug_violations_kv_attention(), debug_violations_noalloc(), debug_violations_gemv_i8()};
  int64_t total = 0;
  for (uint32_t v : parts) total += v == 0xFFFFFFFFu ? int64_t(1) << 32 : int64_t(v);
  return total;
#else
  return -1;
#endif
}

const char* glq_status_string(glq_status s) {
  switch (s) {
    case GLQ_OK: return "ok";
    case GLQ_ERR_NULL: return "a required pointer is NULL";
    case GLQ_ERR_SHAPE: return "a size is out of range or sizes disagree";
    case GLQ_ERR_DTYPE: return "dtype not supported by this entry point";
    case GLQ_ERR_RECIPE: return "not a recipe of the bit-width table, or a bad index_format";
    case GLQ_ERR_ALIGN: return "a pointer is not aligned as documented";
    case GLQ_ERR_WORKSPACE: return "workspace missing or too small";
    case GLQ_ERR_HIP: return "a HIP launch failed";
    case GLQ_ERR_CODEBOOK: return "codebook entries outside the representable range";
  }
  return "unknown status";
}

size_t glq_codebook_pack_bytes(int64_t entries) {
  if (entries < 1 || entries > GLQ_CODEBOOK_ENTRIES) return 0;
  return pack_total_bytes(entries);
}

glq_status glq_codebook_pack(const uint16_t* cb_host, int64_t entries, void* pack_host, size_t pack_bytes_given) {
  return build_pack(cb_host, entries, pack_host, pack_bytes_given);
}

glq_status glq_slot_codes(const void* cb_pack, const uint16_t* idx, int64_t count, uint16_t* codes,
                          hipStream_t stream) {
  if (!cb_pack || (count > 0 && (!idx || !codes))) return GLQ_ERR_NULL;
  if (count < 0) return GLQ_ERR_SHAPE;
  if (!aligned(cb_pack, 256) || !aligned(idx, 2) || !aligned(codes, 2)) return GLQ_ERR_ALIGN;
  return from_hip(launch_slot_codes(cb_pack, idx, count, codes, stream));
}

size_t glq_input_rht_workspace_bytes(int64_t B, int64_t n_pad, glq_dtype u_dt) {
  if (B < 1 || !valid_pad(n_pad)) return 0;
  if (rht_needs_ws(B, n_pad, u_dt == GLQ_F32)) return align256(size_t(B) * size_t(n_pad) * 4);
  return 0;
}

glq_status glq_input_rht(const void* x, glq_dtype x_dt, int64_t B, int64_t n, int64_t n_pad, const int8_t* sign_in,
                         void* u, glq_dtype u_dt, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!x || !sign_in || !u) return GLQ_ERR_NULL;
  if (B < 1 || !valid_pad(n_pad) || n < 1 || n > n_pad || B > int64_t(1) << 31) return GLQ_ERR_SHAPE;
  if (!valid_dtype(x_dt) || !valid_dtype(u_dt)) return GLQ_ERR_DTYPE;
  const size_t need = glq_input_rht_workspace_bytes(B, n_pad, u_dt);
  if (need > 0 && (!workspace || workspace_bytes < need)) return GLQ_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 256)) return GLQ_ERR_ALIGN;
  return from_hip(launch_rht_in(x, x_dt, B, n, n_pad, sign_in, u, u_dt,
                                static_cast<float*>(workspace), stream));
}

size_t glq_output_rht_workspace_bytes(int64_t B, int64_t m_pad) {
  if (B < 1 || !valid_pad(m_pad)) return 0;
  if (rht_needs_ws(B, m_pad, false)) return align256(size_t(B) * size_t(m_pad) * 4);
  return 0;
}

glq_status glq_output_rht(const float* z_parts, int64_t splits, int64_t B, int64_t m, int64_t m_pad,
                          const int8_t* sign_out, void* y, glq_dtype y_dt, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  if (!z_parts || !sign_out || !y) return GLQ_ERR_NULL;
  if (B < 1 || splits < 1 || !valid_pad(m_pad) || m < 1 || m > m_pad || B > int64_t(1) << 31)
    return GLQ_ERR_SHAPE;
  if (!valid_dtype(y_dt)) return GLQ_ERR_DTYPE;
  const size_t need = glq_output_rht_workspace_bytes(B, m_pad);
  if (need > 0 && (!workspace || workspace_bytes < need)) return GLQ_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 256)) return GLQ_ERR_ALIGN;
  return from_hip(launch_rht_out(z_parts, splits, B, m, m_pad, sign_out, y, y_dt,
                                 static_cast<float*>(workspace), stream));
}

glq_status glq_e8_dequant(const glq_layer* layer, void* w, glq_dtype w_dt, hipStream_t stream) {
  glq_status st = check_layer(layer, false);
  if (st != GLQ_OK) return st;
  if (!w) return GLQ_ERR_NULL;
  if (!valid_dtype(w_dt)) return GLQ_ERR_DTYPE;
  if (!aligned(w, 16)) return GLQ_ERR_ALIGN;
  return from_hip(launch_dequant(*layer, w, w_dt, stream));
}

int64_t glq_e8_matmul_splits(const glq_layer* layer, int64_t B) {
  if (!layer || B < 1 || !valid_pad(layer->n_pad)) return 0;
  return matmul_splits(*layer, B);
}

size_t glq_e8_matmul_workspace_bytes(const glq_layer* layer, int64_t B) {
  if (!layer || B < 1 || !valid_pad(layer->n_pad) || !valid_pad(layer->m_pad)) return 0;
  return matmul_ws_bytes(*layer, B);
}

glq_status glq_e8_matmul(const glq_layer* layer, const void* u, glq_dtype u_dt, int64_t B, float* z_parts,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  glq_status st = check_layer(layer, false);
  if (st != GLQ_OK) return st;
  if (!u || !z_parts) return GLQ_ERR_NULL;
  if (B < 1 || B > int64_t(1) << 31) return GLQ_ERR_SHAPE;
  if (u_dt != (B > kDecodeMaxB ? GLQ_F16 : GLQ_F32)) return GLQ_ERR_DTYPE;
  if (!aligned(u, 16)) return GLQ_ERR_ALIGN;
  const size_t need = matmul_ws_bytes(*layer, B);
  if (need > 0 && (!workspace || workspace_bytes < need)) return GLQ_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 256)) return GLQ_ERR_ALIGN;
  if (B > kDecodeMaxB)
    return from_hip(prefill_matmul(*layer, static_cast<const half_t*>(u), nullptr, B, false, z_parts, stream));
  return from_hip(decode_matmul(*layer, static_cast<const float*>(u), B, workspace, z_parts, stream));
}

size_t glq_prefill_u_bytes(int64_t B, int64_t n_pad) {
  if (B < 1 || !valid_pad(n_pad) || n_pad % 128 != 0) return 0;
  return prefill_u_total_bytes(B, n_pad);
}

size_t glq_prefill_row_exp_offset(int64_t B, int64_t n_pad) {
  if (B < 1 || !valid_pad(n_pad) || n_pad % 128 != 0) return 0;
  return prefill_rexp_offset(B, n_pad);
}

int glq_e8_matmul_prefill_supported(const glq_layer* layer) {
  if (!layer || check_layer(layer, false) != GLQ_OK) return 0;
  return gemm_shared_supported(*layer) || gemm_lds_supported(*layer) ? 1 : 0;
}

glq_status glq_input_rht_prefill(const void* x, glq_dtype x_dt, int64_t B, int64_t n, int64_t n_pad,
                                 const int8_t* sign_in, void* u16, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  if (!x || !sign_in || !u16) return GLQ_ERR_NULL;
  if (B < 1 || !valid_pad(n_pad) || n_pad < 256 || n_pad % 128 != 0 || n < 1 || n > n_pad || B > int64_t(1) << 31)
    return GLQ_ERR_SHAPE;
  if (!valid_dtype(x_dt)) return GLQ_ERR_DTYPE;
  if (!aligned(u16, 16)) return GLQ_ERR_ALIGN;
  const size_t need = glq_input_rht_workspace_bytes(B, n_pad, GLQ_F16);
  if (need > 0 && (!workspace || workspace_bytes < need)) return GLQ_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 256)) return GLQ_ERR_ALIGN;
  int32_t* rexp = at<int32_t>(u16, prefill_rexp_offset(B, n_pad));
  hipError_t e = launch_row_exp(x, x_dt, B, n, rexp, stream);
  if (e != hipSuccess) return GLQ_ERR_HIP;
  return from_hip(launch_rht_in_tiled(x, x_dt, B, n, n_pad, sign_in, rexp, static_cast<half_t*>(u16),
                                      static_cast<float*>(workspace), stream));
}

glq_status glq_e8_matmul_prefill(const glq_layer* layer, const void* u16, int64_t B, float* z, hipStream_t stream) {
  glq_status st = check_layer(layer, false);
  if (st != GLQ_OK) return st;
  if (!u16 || !z) return GLQ_ERR_NULL;
  if (B < 1 || B > int64_t(1) << 31 || !(gemm_shared_supported(*layer) || gemm_lds_supported(*layer)))
    return GLQ_ERR_SHAPE;
  if (!aligned(u16, 16)) return GLQ_ERR_ALIGN;
  const int32_t* rexp =
      reinterpret_cast<const int32_t*>(static_cast<const char*>(u16) + prefill_rexp_offset(B, layer->n_pad));
  return from_hip(prefill_matmul(*layer, static_cast<const half_t*>(u16), rexp, B, true, z, stream));
}

size_t glq_e8rht_linear_workspace_bytes(const glq_layer* layer, int64_t B) {
  if (!layer || B < 1 || !valid_pad(layer->n_pad) || !valid_pad(layer->m_pad)) return 0;
  return linear_ws(*layer, B).total;
}

glq_status glq_e8rht_linear(const glq_layer* layer, const void* x, glq_dtype x_dt, int64_t B, void* y,
                            glq_dtype y_dt, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  glq_status st = check_layer(layer, true);
  if (st != GLQ_OK) return st;
  if (!x || !y) return GLQ_ERR_NULL;
  if (B < 1 || B > int64_t(1) << 31) return GLQ_ERR_SHAPE;
  if (!valid_dtype(x_dt) || !valid_dtype(y_dt)) return GLQ_ERR_DTYPE;
  const LinearWs w = linear_ws(*layer, B);
  if (!workspace || workspace_bytes < w.total) return GLQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return GLQ_ERR_ALIGN;
  const glq_layer& L = *layer;
  if (w.fused)  // every stage in one pass (5-8 bpw included)
    return from_hip(launch_fused_decode(L, x, x_dt, y, y_dt, at<float>(workspace, w.z_off), stream));
  hipError_t e;
  float* z = at<float>(workspace, w.z_off);
  if (w.skinny) {
    // u in fp32, then 15-bit fixed point per row as two int8 planes; every pass of the
    // layer on the int8 matrix units
    float* u = at<float>(workspace, w.u_off);
    char* planes = at<char>(workspace, w.uq_off);
    I8RowInfo* info = reinterpret_cast<I8RowInfo*>(planes + align256(i8_planes_bytes(L.n_pad)));
    e = launch_rht_in(x, x_dt, B, L.n, L.n_pad, L.sign_in, u, GLQ_F32, at<float>(workspace, w.rin_off), stream);
    if (e != hipSuccess) return GLQ_ERR_HIP;
    e = launch_quant_i8(u, B, L.n_pad, planes, info, stream);
    if (e != hipSuccess) return GLQ_ERR_HIP;
    const Passes P = split_passes(L);
    e = launch_gemv_i8(P.a, planes, info, B, z, stream, false);
    if (e == hipSuccess && P.two) e = launch_gemv_i8(P.b, planes, info, B, z, stream, true);
    if (e != hipSuccess) return GLQ_ERR_HIP;
  } else if (!w.prefill) {
    float* u = at<float>(workspace, w.u_off);
    e = launch_rht_in(x, x_dt, B, L.n, L.n_pad, L.sign_in, u, GLQ_F32, at<float>(workspace, w.rin_off), stream);
    if (e != hipSuccess) return GLQ_ERR_HIP;
    e = decode_matmul(L, u, B, at<char>(workspace, w.uq_off), z, stream);
    if (e != hipSuccess) return GLQ_ERR_HIP;
  } else {
    // fp16 operands with a power-of-two scale per row (the row exponents), undone
    // in the matmul's fp32 epilogue
    half_t* u = at<half_t>(workspace, w.u_off);
    int32_t* rexp = at<int32_t>(workspace, w.u_off + prefill_rexp_off(L, B));
    e = launch_row_exp(x, x_dt, B, L.n, rexp, stream);
    if (e != hipSuccess) return GLQ_ERR_HIP;
    if (prefill_tiled(L)) {  // u in the matmuls' fragment order
      e = launch_rht_in_tiled(x, x_dt, B, L.n, L.n_pad, L.sign_in, rexp, u, at<float>(workspace, w.rin_off), stream);
      if (e != hipSuccess) return GLQ_ERR_HIP;
      e = prefill_matmul(L, u, rexp, B, true, z, stream);
    } else {
      e = launch_rht_in(x, x_dt, B, L.n, L.n_pad, L.sign_in, u, GLQ_F16, at<float>(workspace, w.rin_off), stream,
                        rexp);
      if (e != hipSuccess) return GLQ_ERR_HIP;
      e = prefill_matmul(L, u, rexp, B, false, z, stream);
    }
    if (e != hipSuccess) return GLQ_ERR_HIP;
  }
  e = launch_rht_out(z, w.splits, B, L.m, L.m_pad, L.sign_out, y, y_dt, at<float>(workspace, w.rout_off), stream);
  return from_hip(e);
}

// How a group runs: GROUP_FUSED (B = 1, the fused launches), GROUP_I8 (2 <= B <= 16,
// every layer on the int8 path in one GEMV launch), else GROUP_EACH (one call per layer).
enum GroupMode { GROUP_EACH, GROUP_FUSED, GROUP_I8 };

static GroupMode group_mode(const glq_layer* layers, int32_t count, int64_t B) {
  if (B == 1 && fused_group_supported(layers, count)) return GROUP_FUSED;
  if (B < 2 || B > kDecodeMaxB || count < 2) return GROUP_EACH;
  for (int32_t k = 0; k < count; ++k) {
    const glq_layer& L = layers[k];
    // one pass per layer (no further stages), one n_pad, each on the int8 path alone
    if (!skinny_ok(L, B) || L.n_extra != 0 || L.n_pad != layers[0].n_pad) return GROUP_EACH;
  }
  return gemv_i8_group_plan(layers, count, nullptr) ? GROUP_I8 : GROUP_EACH;
}

// the group's workspace: one z_parts region per layer (the fused launches), one int8
// path workspace per layer (the GEMV launch shared), or the largest single-layer
// workspace (one layer after another); base[k] is layer k's offset
static size_t group_ws(const glq_layer* layers, int32_t count, int64_t B, GroupMode mode, size_t* base,
                       LinearWs* lw) {
  size_t total = 0;
  int splits[GLQ_GROUP_MAX];
  if (mode == GROUP_I8) gemv_i8_group_plan(layers, count, splits);
  for (int32_t k = 0; k < count; ++k) {
    if (mode == GROUP_FUSED) {
      if (base) base[k] = total;
      total += align256(fused_group_z_bytes(layers, count, k));
    } else if (mode == GROUP_I8) {
      LinearWs w{};
      skinny_layout(layers[k], B, splits[k], w);
      if (base) base[k] = total;
      if (lw) lw[k] = w;
      total += align256(w.total);
    } else {
      const size_t t = linear_ws(layers[k], B).total;
      total = t > total ? t : total;
    }
  }
  return total;
}

size_t glq_e8rht_linear_group_workspace_bytes(const glq_layer* layers, int32_t count, int64_t B) {
  if (!layers || count < 1 || count > GLQ_GROUP_MAX || B < 1) return 0;
  for (int32_t k = 0; k < count; ++k)
    if (check_layer(&layers[k], true) != GLQ_OK) return 0;
  return group_ws(layers, count, B, group_mode(layers, count, B), nullptr, nullptr);
}

glq_status glq_e8rht_linear_group(const glq_layer* layers, int32_t count, const void* const* x, glq_dtype x_dt,
                                  int64_t B, void* const* y, glq_dtype y_dt, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  if (!layers || !x || !y) return GLQ_ERR_NULL;
  if (count < 1 || count > GLQ_GROUP_MAX) return GLQ_ERR_SHAPE;
  for (int32_t k = 0; k < count; ++k) {
    const glq_status st = check_layer(&layers[k], true);
    if (st != GLQ_OK) return st;
    if (!x[k] || !y[k]) return GLQ_ERR_NULL;
  }
  if (B < 1 || B > int64_t(1) << 31) return GLQ_ERR_SHAPE;
  if (!valid_dtype(x_dt) || !valid_dtype(y_dt)) return GLQ_ERR_DTYPE;
  const GroupMode mode = group_mode(layers, count, B);
  size_t base[GLQ_GROUP_MAX];
  LinearWs lw[GLQ_GROUP_MAX];
  const size_t need = group_ws(layers, count, B, mode, base, lw);
  if (!workspace || workspace_bytes < need) return GLQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return GLQ_ERR_ALIGN;
  if (mode == GROUP_FUSED) {
    float* z[GLQ_GROUP_MAX];
    for (int32_t k = 0; k < count; ++k) z[k] = at<float>(workspace, base[k]);
    return from_hip(launch_fused_group(layers, count, x, x_dt, y, y_dt, z, stream));
  }
  if (mode == GROUP_I8) {
    // per layer: u, then its int8 planes; one GEMV launch for all; per layer the output RHT
    const void* planes[GLQ_GROUP_MAX];
    const I8RowInfo* info[GLQ_GROUP_MAX];
    float* z[GLQ_GROUP_MAX];
    for (int32_t k = 0; k < count; ++k) {
      const glq_layer& L = layers[k];
      char* ws = at<char>(workspace, base[k]);
      float* u = at<float>(ws, lw[k].u_off);
      char* pl = at<char>(ws, lw[k].uq_off);
      I8RowInfo* inf = reinterpret_cast<I8RowInfo*>(pl + align256(i8_planes_bytes(L.n_pad)));
      hipError_t e = launch_rht_in(x[k], x_dt, B, L.n, L.n_pad, L.sign_in, u, GLQ_F32, at<float>(ws, lw[k].rin_off),
                                   stream);
      if (e == hipSuccess) e = launch_quant_i8(u, B, L.n_pad, pl, inf, stream);
      if (e != hipSuccess) return GLQ_ERR_HIP;
      planes[k] = pl;
      info[k] = inf;
      z[k] = at<float>(ws, lw[k].z_off);
    }
    if (launch_gemv_i8_group(layers, count, planes, info, B, z, stream) != hipSuccess) return GLQ_ERR_HIP;
    for (int32_t k = 0; k < count; ++k) {
      const glq_layer& L = layers[k];
      char* ws = at<char>(workspace, base[k]);
      if (launch_rht_out(z[k], lw[k].splits, B, L.m, L.m_pad, L.sign_out, y[k], y_dt, at<float>(ws, lw[k].rout_off),
                         stream) != hipSuccess)
        return GLQ_ERR_HIP;
    }
    return GLQ_OK;
  }
  for (int32_t k = 0; k < count; ++k) {
    const glq_status st = glq_e8rht_linear(&layers[k], x[k], x_dt, B, y[k], y_dt, workspace, workspace_bytes, stream);
    if (st != GLQ_OK) return st;
  }
  return GLQ_OK;
}

static glq_status check_kv(const glq_kv_cache* kv) {
  if (!kv) return GLQ_ERR_NULL;
  if (!kv->k_idx[0] || !kv->v_idx[0] || !kv->k_scale || !kv->v_scale || !kv->cb_pack) return GLQ_ERR_NULL;
  if (kv->stages != 1 && kv->stages != 2) return GLQ_ERR_RECIPE;
  if (kv->stages == 2 && (!kv->k_idx[1] || !kv->v_idx[1])) return GLQ_ERR_NULL;
  if (kv->stages == 2 && !(kv->resid_scale == kv->resid_scale)) return GLQ_ERR_RECIPE;
  if (kv->index_format != GLQ_INDEX_CODEBOOK && kv->index_format != GLQ_INDEX_SLOT) return GLQ_ERR_RECIPE;
  if (kv->head_dim != 64 && kv->head_dim != 128) return GLQ_ERR_SHAPE;
  if (kv->num_kv_heads < 1 || kv->num_pages < 1 || kv->page_size < 1 || kv->page_size > 1024 ||
      !is_pow2(kv->page_size))
    return GLQ_ERR_SHAPE;
  // 32-bit rows of the kernel: pages * page_size * heads * D / 8 groups
  if (kv->num_pages * kv->page_size * kv->num_kv_heads * (kv->head_dim / 8) >= (int64_t(1) << 31))
    return GLQ_ERR_SHAPE;
  if (!aligned(kv->cb_pack, 256) || !aligned(kv->k_scale, 4) || !aligned(kv->v_scale, 4)) return GLQ_ERR_ALIGN;
  for (int s = 0; s < kv->stages; ++s)
    if (!aligned(kv->k_idx[s], 2) || !aligned(kv->v_idx[s], 2)) return GLQ_ERR_ALIGN;
  return GLQ_OK;
}

static bool kv_heads_ok(const glq_kv_cache* kv, int32_t num_q_heads) {
  if (num_q_heads < 1 || num_q_heads % kv->num_kv_heads != 0) return false;
  const int32_t G = num_q_heads / kv->num_kv_heads;
  return G == 1 || G == 2 || G == 4 || G == 8;
}

size_t glq_e8kv_attention_workspace_bytes(const glq_kv_cache* kv, int64_t B, int32_t num_q_heads,
                                          int64_t max_seq_len) {
  if (!kv || B < 1 || max_seq_len < 1 || kv->num_kv_heads < 1 || !kv_heads_ok(kv, num_q_heads)) return 0;
  if (kv->head_dim != 64 && kv->head_dim != 128) return 0;
  const int64_t G = num_q_heads / kv->num_kv_heads;
  const KvPlan p = kv_plan(B, kv->num_kv_heads, G, max_seq_len);
  return align256(size_t(p.units) * size_t(G) * size_t(kv->head_dim) * 4) + align256(size_t(p.units) * size_t(G) * 8);
}

glq_status glq_e8kv_attention_decode(const glq_kv_cache* kv, const void* q, glq_dtype q_dt, int64_t B,
                                     int32_t num_q_heads, const int32_t* block_table, int64_t max_pages,
                                     const int32_t* seq_lens, int64_t max_seq_len, float sm_scale, void* out,
                                     glq_dtype out_dt, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  glq_status st = check_kv(kv);
  if (st != GLQ_OK) return st;
  if (!q || !block_table || !seq_lens || !out) return GLQ_ERR_NULL;
  if (B < 1 || B > (int64_t(1) << 20) || max_pages < 1 || max_seq_len < 1 || max_seq_len > (int64_t(1) << 30) ||
      !kv_heads_ok(kv, num_q_heads))
    return GLQ_ERR_SHAPE;
  if (!valid_dtype(q_dt) || !valid_dtype(out_dt)) return GLQ_ERR_DTYPE;
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4)) return GLQ_ERR_ALIGN;
  const size_t need = glq_e8kv_attention_workspace_bytes(kv, B, num_q_heads, max_seq_len);
  if (!workspace || workspace_bytes < need) return GLQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return GLQ_ERR_ALIGN;
  const int64_t G = num_q_heads / kv->num_kv_heads;
  const KvPlan p = kv_plan(B, kv->num_kv_heads, G, max_seq_len);
  float* part_o = static_cast<float*>(workspace);
  float* part_ml = at<float>(workspace, align256(size_t(p.units) * size_t(G) * size_t(kv->head_dim) * 4));
  return from_hip(launch_kv_attention(*kv, q, q_dt, B, num_q_heads, block_table, max_pages, seq_lens, max_seq_len,
                                      sm_scale, out, out_dt, part_o, part_ml, stream));
}

}  // extern "C"
