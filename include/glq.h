/*
 * glq.h — C ABI of the MI355X (gfx950) E8RHTLinear library.
 *
 * The operation (glq 0.5.1, PyPI project page):
 *   "How it works", item 1: each 8-weight group of a weight matrix is one 16-bit
 *     index into a 65,536-entry E8 lattice codebook; 3-8 bpw add 8-bit
 *     (256-entry) or 16-bit residual stages.
 *   "How it works", item 2: a randomized Hadamard transform (random sign flips,
 *     then a fast Walsh-Hadamard transform) rotates the weights, so the layer
 *     applies one to its input and one to its output.
 *   "How it works", item 4 and "Inference kernels": the matmul is taken directly
 *     against the indices, Y = X dequant(W)^T, without forming W in memory.
 *   table "Bit widths": 2 bpw = 16b; 3 bpw = 16b + 8b; 4 bpw = 16b + 16b; one
 *     global scale per layer.
 *   Glq v0.3.2 release notes, "What changed": the input and output transforms
 *     are separate operations (input_rht, output_rht).
 *
 * The layer forward computed here, for x [B][n] and y [B][m]:
 *   u  = H_{n_pad} (sign_in * [x, 0 ... 0]) / sqrt(n_pad)               (input RHT)
 *   W~[o][8g + j] = s * (C0[idx0[o][g]][j] + s_r * C1[idx1[o][g]][j])    (dequant, never stored)
 *   z  = u W~^T                                                          ([B][m_pad])
 *   y  = (sign_out * H_{m_pad} z / sqrt(m_pad))[:, 0:m]                  (output RHT)
 * with H the Sylvester-ordered Hadamard matrix, H[i][j] = (-1)^popcount(i & j).
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are HIP device pointers on the current device;
 *     "host" pointers are ordinary host memory.  The caller owns every buffer;
 *     the library allocates and frees nothing.  Its mutable state: a per-device
 *     cache of the compute-unit count and of one kernel attribute, updated
 *     atomically, so calls from several host threads are safe; the device array
 *     that glq_e8rht_linear_noalloc uses as its workspace (one per device, shared
 *     by its calls); and, in debug builds only, the bounds-check counters that
 *     glq_debug_violations reads.
 *   - Device work is enqueued asynchronously on `stream` (0 = null stream); the
 *     library never synchronizes, so calls are safe under stream capture.
 *   - Arrays are dense and row-major.  n_pad and m_pad are powers of two in
 *     [8, 2^20]; n <= n_pad, m <= m_pad; batch sizes are >= 1.
 *   - Every argument is validated before anything is launched; on an error the
 *     call returns that status and leaves every output untouched.  A failed
 *     launch returns GLQ_ERR_HIP.  Faults inside kernels surface on the stream.
 *   - Results are deterministic: the same inputs give bit-identical outputs on
 *     every call (fixed-order reductions, no atomics on the data path).
 *   - Range: the transforms run in fp32, so sqrt(n_pad) * max |x| must stay below
 *     FLT_MAX (about 3.4e38); within it the result scales with x (y(2^k x) =
 *     2^k y(x) while y stays in the fp32 range).  Every reduced-precision step
 *     carries a power-of-two scale: the decode path's 16-bit fixed point per 64
 *     columns, and the prefill path's fp16 operands per row.  A NaN or infinity in
 *     a row of x makes that row of y NaN.
 */
#ifndef GLQ_H
#define GLQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GLQ_ABI_VERSION 5
#define GLQ_CODEBOOK_ENTRIES 65536
#define GLQ_RESID8_ENTRIES 256
#define GLQ_MAX_PAD (1 << 20)

typedef enum glq_status {
  GLQ_OK = 0,
  GLQ_ERR_NULL = 1,      /* a required pointer is NULL */
  GLQ_ERR_SHAPE = 2,     /* a size is out of range or sizes disagree */
  GLQ_ERR_DTYPE = 3,     /* dtype code not supported by this entry point */
  GLQ_ERR_RECIPE = 4,    /* not a recipe of "Bit widths" (resid_bits, further stages) or bad index_format */
  GLQ_ERR_ALIGN = 5,     /* a pointer is not aligned as documented */
  GLQ_ERR_WORKSPACE = 6, /* workspace missing or smaller than the size query says */
  GLQ_ERR_HIP = 7,       /* a HIP launch failed */
  GLQ_ERR_CODEBOOK = 8   /* codebook entries outside what the pack can hold */
} glq_status;

/* What the layer's 16-bit index arrays hold (glq_layer.index_format). */
typedef enum glq_index_format {
  GLQ_INDEX_CODEBOOK = 0, /* indices into the 65,536-entry codebook ("How it works", item 1) */
  GLQ_INDEX_SLOT = 1      /* the same entries relabelled as slot codes by glq_slot_codes */
} glq_index_format;

typedef enum glq_dtype {
  GLQ_F32 = 0,  /* IEEE binary32 */
  GLQ_F16 = 1,  /* IEEE binary16 */
  GLQ_BF16 = 2  /* bfloat16 */
} glq_dtype;

/*
 * One quantized layer.  All pointers are device pointers.
 *   n, n_pad        input features and the input transform's length, n <= n_pad
 *   m, m_pad        output features and the output transform's length, m <= m_pad
 *                   A transform length is a power of two in [8, GLQ_MAX_PAD]
 *                   (x zero-padded to it, y truncated from it), or a multiple of
 *                   64 below GLQ_MAX_PAD whose transform is block-diagonal: its
 *                   blocks are the powers of two of its binary expansion, largest
 *                   first, each transformed on its own and orthonormal ("Bit
 *                   widths", note below the table: non-power-of-two sizes use a
 *                   block-diagonal transform, e.g. 2688 = 2048 + 512 + 128, so
 *                   nothing is padded).  n_pad = n and m_pad = m store no padding.
 *   resid_bits      0: 2 bpw, primary stage only ("Bit widths", row 2)
 *                   8: 3 bpw, + 8-bit index into a 256-entry residual codebook
 *                   16: 4 bpw, + 16-bit index into a 65,536-entry residual codebook
 *   wscale          s, the one scale of the layer ("Bit widths", note below the table)
 *   resid_scale     s_r, the residual stage's scale (the inv_resid_scale argument
 *                   of glq_dequant_matmul, "Inference kernels"); unused when
 *                   resid_bits == 0
 *   sign_in         int8 [n_pad], each +1 or -1 (values other than +-1 are a
 *                   precondition violation and are not checked)
 *   sign_out        int8 [m_pad], each +1 or -1
 *   idx0            uint16 [m_pad][n_pad/8]: group g of output row o covers input
 *                   columns 8g .. 8g+7; 16-byte aligned
 *   idx1            uint8 (resid_bits 8) or uint16 (resid_bits 16), same shape
 *                   as idx0, 16-byte aligned; NULL when resid_bits == 0
 *   cb_pack         primary codebook pack (glq_codebook_pack of 65,536 entries)
 *   cb2_pack        residual codebook pack: 256 entries for resid_bits 8, 65,536
 *                   for resid_bits 16 (it may be the same buffer as cb_pack);
 *                   NULL when resid_bits == 0
 *   index_format    GLQ_INDEX_CODEBOOK, or GLQ_INDEX_SLOT: idx0 (and idx1 when
 *                   resid_bits == 16) hold slot codes of cb_pack, written by
 *                   glq_slot_codes; with resid_bits 16 cb2_pack must then be
 *                   cb_pack.  8-bit residual indices are never relabelled.
 *   n_extra         further residual stages, 5-8 bpw ("Bit widths": 16b + 16b + 8b,
 *                   16b + 16b + 16b, 16b + 16b + 16b + 8b, 16b x 4): 0, 1 or 2; with
 *                   1 or 2, resid_bits is 16 and cb2_pack is cb_pack
 *   extra_bits      per further stage: 8, or 16 (16 for the first of two)
 *   extra_scale     per further stage: its scale relative to s, like resid_scale
 *                   (W~ = s (C0 + s_r C1 + sum_k extra_scale[k] C_k))
 *   extra_idx       per further stage: uint8 / uint16 [m_pad][n_pad/8], 16-byte
 *                   aligned; 16-bit stages index cb_pack (slot codes with
 *                   GLQ_INDEX_SLOT), 8-bit stages cb8_pack
 *   cb8_pack        the 256-entry pack of an 8-bit further stage; NULL otherwise
 */
typedef struct glq_layer {
  int64_t n;
  int64_t n_pad;
  int64_t m;
  int64_t m_pad;
  int32_t resid_bits;
  float wscale;
  float resid_scale;
  const int8_t* sign_in;
  const int8_t* sign_out;
  const uint16_t* idx0;
  const void* idx1;
  const void* cb_pack;
  const void* cb2_pack;
  int32_t index_format;
  int32_t n_extra;
  int32_t extra_bits[2];
  float extra_scale[2];
  const void* extra_idx[2];
  const void* cb8_pack;
} glq_layer;

/*
 * An E8-compressed paged K/V cache for decode attention (Glq v0.5.0 release notes,
 * "Highlights"; glq 0.5.1, "KV cache compression" -> "E8 lattice cache": the same
 * E8 quantizer as the weights, e8_relaxed:1 / e8_relaxed:2 with the 4 bpw
 * e8_relaxed:2 the inline-dequant recipe).  All pointers are device pointers.
 * A cached K or V vector of head_dim D is D/8 groups of 8; group g reads back as
 * s * H8 e_g / sqrt(8) (H8 the Sylvester 8-point Hadamard), e_g = C[i0] for one
 * stage or C[i0] + resid_scale * C[i1] for two, with one scale s per vector.
 *   num_pages       physical pages; page indices read from a block table are
 *                   clamped to [0, num_pages)
 *   page_size       tokens per page, a power of two in [1, 1024]
 *   num_kv_heads    KV heads (H_kv)
 *   head_dim        D, 64 or 128
 *   stages          1 (2 bpw) or 2 (4 bpw)
 *   resid_scale     the second stage's scale (ignored with one stage)
 *   index_format    GLQ_INDEX_CODEBOOK or GLQ_INDEX_SLOT (codes of cb_pack, as for
 *                   a layer)
 *   k_idx[s], v_idx[s]   uint16 [num_pages][page_size][num_kv_heads][D/8] per stage
 *                   (index 1 unused with one stage), 2-byte aligned
 *   k_scale, v_scale     fp32 [num_pages][page_size][num_kv_heads]
 *   cb_pack         a 65,536-entry pack from glq_codebook_pack, 256-byte aligned
 */
typedef struct glq_kv_cache {
  int64_t num_pages;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t stages;
  float resid_scale;
  int32_t index_format;
  const uint16_t* k_idx[2];
  const uint16_t* v_idx[2];
  const float* k_scale;
  const float* v_scale;
  const void* cb_pack;
} glq_kv_cache;

/* GLQ_ABI_VERSION of the built library. */
int glq_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* glq_status_string(glq_status s);

/*
 * glq_debug_violations — debug builds only (libglq_mi355x_debug.so and
 * libglq_mi355x_asan.so, compiled with GLQ_DEBUG): the number of device-side bounds
 * checks that failed since the previous call (reads of the LDS codebook image and
 * residual slots, prefill operand fragments, KV cache rows), summed over the
 * library's kernels, and clears the counts.  A failed check does not stop its kernel.
 * Synchronizes the current device.  Returns -1 in release builds, and UINT32_MAX
 * counts as an error reading a counter.  Not a data path: for tests and debugging.
 */
int64_t glq_debug_violations(void);

/*
 * glq_e8_codebook — build the E8 codebook on the host ("How it works", item 1).
 * Writes the first `entries` points (entries in [1, 65536]) of E8 =
 * D8 u (D8 + 1/2) ordered by squared norm, then lexicographically ascending on
 * the coordinates (coordinate 0 most significant), origin first, as fp16 bit
 * patterns: cb_host is host memory of entries * 8 uint16.  The 256-entry residual
 * codebook is the first 256 entries of the same table.  Synchronous, host only.
 * Errors: GLQ_ERR_NULL, GLQ_ERR_SHAPE.
 */
glq_status glq_e8_codebook(uint16_t* cb_host, int64_t entries);

/*
 * glq_codebook_pack — build the kernels' representation of an fp16 codebook, on
 * the host ("Inference kernels": the kernels gather 8-D codewords from a compact
 * cached codebook).  The pack holds 2c as an int8 table and an LDS image that
 * stores each codeword in 4 bytes (eight signed 4-bit values) and every
 * negation-symmetric shell once, behind a 256-entry page table; the E8 codebook's
 * image takes about 151 KiB, which the decode kernel keeps in LDS.
 *   cb_host     host, fp16 bits [entries][8]; every coordinate a multiple of 1/2
 *               in [-4, 3.5] (true for all E8 points of norm^2 <= 12)
 *   entries     1 .. 65536 (the layer uses 65,536-entry packs for the primary and
 *               16-bit residual stages, a 256-entry pack for the 8-bit residual)
 *   pack_host   host, pack_bytes >= glq_codebook_pack_bytes(entries); the caller
 *               copies it to device memory (256-byte aligned) for the layer
 * Synchronous, host only.  Errors: GLQ_ERR_NULL, GLQ_ERR_SHAPE, GLQ_ERR_WORKSPACE,
 * GLQ_ERR_CODEBOOK (a coordinate outside the set above, or an image larger than
 * the LDS budget).
 */
size_t glq_codebook_pack_bytes(int64_t entries);
glq_status glq_codebook_pack(const uint16_t* cb_host, int64_t entries, void* pack_host, size_t pack_bytes);

/*
 * glq_slot_codes — relabel a layer's 16-bit codebook indices as slot codes, once,
 * when the layer is loaded.  A slot code names the same codebook entry (the map
 * is a bijection of the 65,536 values, kept in the pack) in the form the LDS
 * kernels read without a page table: as int16 c with m = c >> 15, the entry is
 * slot (c ^ m) + (m & delta) of the pack's slot image, negated when m is all
 * ones; each codeword whose negation is also an entry shares its slot with it.
 * The pages' decode is unchanged: one 16-bit value per 8-weight group, decoded
 * in registers/LDS ("How it works", item 1; "Inference kernels").
 *   cb_pack     device, a 65,536-entry pack from glq_codebook_pack, 256-byte aligned
 *   idx         device uint16 [count] codebook indices
 *   codes       device uint16 [count]; may be idx itself (in place)
 * Asynchronous on stream.  Errors: GLQ_ERR_NULL, GLQ_ERR_SHAPE (count < 0),
 * GLQ_ERR_ALIGN, GLQ_ERR_HIP.  A pack whose codebook has no slot format (header
 * word 5 is 0; the E8 codebook always has one) yields codes that decode wrongly:
 * build layers for it in GLQ_INDEX_CODEBOOK.
 */
glq_status glq_slot_codes(const void* cb_pack, const uint16_t* idx, int64_t count, uint16_t* codes,
                          hipStream_t stream);

/*
 * glq_input_rht — u = H_{n_pad} (sign_in * [x, 0...]) / sqrt(n_pad) for each of B
 * rows ("How it works", item 2; Glq v0.3.2 "What changed": input_rht).  When
 * n_pad is not a power of two (a multiple of 64), H_{n_pad} / sqrt(n_pad) stands
 * for the block-diagonal transform of the layer description: block b of length L
 * gets H_L / sqrt(L).
 *   x          device [B][n] in x_dt (F32, F16 or BF16)
 *   sign_in    device int8 [n_pad]
 *   u          device [B][n_pad] in u_dt (F32, F16 or BF16); rounded to nearest-even
 *   workspace  device, workspace_bytes >= glq_input_rht_workspace_bytes(B, n_pad, u_dt)
 *              (0 bytes for most shapes; NULL allowed then), 256-byte aligned
 * Accumulation is fp32.  A block above 16384 runs as two passes (H = H_a (x) H_b).
 * Errors: GLQ_ERR_NULL, GLQ_ERR_SHAPE, GLQ_ERR_DTYPE, GLQ_ERR_WORKSPACE, GLQ_ERR_HIP.
 */
size_t glq_input_rht_workspace_bytes(int64_t B, int64_t n_pad, glq_dtype u_dt);
glq_status glq_input_rht(const void* x, glq_dtype x_dt, int64_t B, int64_t n, int64_t n_pad,
                         const int8_t* sign_in, void* u, glq_dtype u_dt, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * glq_output_rht — y = (sign_out * H_{m_pad} z / sqrt(m_pad))[:, 0:m] with
 * z = sum over s = 0 .. splits-1, in that order, of z_parts[s] (Glq v0.3.2,
 * "What changed": output_rht; "Inference kernels": fixed-order reduction of
 * split partial sums instead of atomics); block-diagonal when m_pad is not a
 * power of two, as for glq_input_rht.
 *   z_parts    device fp32 [splits][B][m_pad]
 *   y          device [B][m] in y_dt (F32, F16 or BF16)
 *   workspace  device, >= glq_output_rht_workspace_bytes(B, m_pad), 256-byte aligned
 * Errors: GLQ_ERR_NULL, GLQ_ERR_SHAPE, GLQ_ERR_DTYPE, GLQ_ERR_WORKSPACE, GLQ_ERR_HIP.
 */
size_t glq_output_rht_workspace_bytes(int64_t B, int64_t m_pad);
glq_status glq_output_rht(const float* z_parts, int64_t splits, int64_t B, int64_t m, int64_t m_pad,
                          const int8_t* sign_out, void* y, glq_dtype y_dt, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * glq_e8_dequant — write the dequantized weight W~ [m_pad][n_pad] ("How it works",
 * items 1 and 4; "Bit widths").  For tests and debugging: the linear never
 * forms W~.  In fp32, e = c0 + s_r * c1 is computed exactly and
 * w = RN(s * e) is the one rounding; F16 / BF16 output is the nearest-even
 * rounding of that fp32 value.
 *   layer      idx0, idx1, cb_pack, cb2_pack, resid_bits, wscale, resid_scale,
 *              n_pad and m_pad are used (signs, n and m are ignored)
 *   w          device [m_pad][n_pad] in w_dt, 16-byte aligned
 * Errors: GLQ_ERR_NULL, GLQ_ERR_SHAPE, GLQ_ERR_DTYPE, GLQ_ERR_RECIPE, GLQ_ERR_ALIGN, GLQ_ERR_HIP.
 */
glq_status glq_e8_dequant(const glq_layer* layer, void* w, glq_dtype w_dt, hipStream_t stream);

/*
 * glq_e8_matmul — z = u W~^T without the transforms, the counterpart of
 * glq_dequant_matmul ("Inference kernels": Y = X dequant(W)^T, N/8 codebook
 * blocks per output row, gathered and accumulated without forming W; split-K
 * partial sums in a scratch buffer, reduced in a fixed order instead of with
 * atomics).  This is the middle step of glq_e8rht_linear, exposed on its own.
 *   u          device [B][n_pad]: fp32 when B <= 16 (decode kernel: u quantized
 *              to 16-bit fixed point per 64 columns, exact integer dot products
 *              against the codewords), fp16 when B > 16 (prefill kernel, fp16
 *              MFMA, fp32 accumulate)
 *   z_parts    device fp32 [S][B][m_pad], S = glq_e8_matmul_splits(layer, B):
 *              z = sum over s = 0 .. S-1 of z_parts[s]; glq_output_rht takes
 *              z_parts and S as they are
 *   workspace  device, >= glq_e8_matmul_workspace_bytes(layer, B) (may be 0 and
 *              NULL), 256-byte aligned
 * Only idx0, idx1, packs, resid_bits, wscale, resid_scale, n_pad, m_pad are used.
 * Errors: GLQ_ERR_NULL, GLQ_ERR_SHAPE, GLQ_ERR_DTYPE (u_dt not the one above),
 * GLQ_ERR_RECIPE, GLQ_ERR_ALIGN, GLQ_ERR_WORKSPACE, GLQ_ERR_HIP.
 */
int64_t glq_e8_matmul_splits(const glq_layer* layer, int64_t B);
size_t glq_e8_matmul_workspace_bytes(const glq_layer* layer, int64_t B);
glq_status glq_e8_matmul(const glq_layer* layer, const void* u, glq_dtype u_dt, int64_t B, float* z_parts,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The prefill (B > 16) steps of glq_e8rht_linear on their own, with u in the
 * matmul's fragment order ("Inference kernels": the tensor-core path for B >= 2;
 * "How it works", item 2 for the transform).  Fragment order, for n_pad = 32 KS
 * with KS a multiple of 4 (n_pad a multiple of 128): element (b, i) of u, with
 * group g = i / 8, k-step ks = 4 floor(g / 16) + g mod 4 and quarter
 * q = floor(g / 4) mod 4, sits at half index
 * (((b / 16) KS + ks) 4 + q) 128 + (b mod 16) 8 + i mod 8;
 * a buffer holds ceil(B / 16) * 16 rows (rows past B are never read into y).
 *
 * Each row b carries a power-of-two scale: the buffer holds the fp16 values of
 * u[b] * 2^-e[b], followed, at byte offset glq_prefill_row_exp_offset(B, n_pad), by
 * int32 e[ceil(B / 16) * 16].  e[b] is chosen from the input row so that no stored
 * value exceeds 2^14 in magnitude: e = frexp exponent of max |x[b]| + ceil(log2
 * sqrt(n)) - 14 (|u| <= ||x[b]||_2 <= sqrt(n) max |x[b]|), 0 for a zero row and
 * 0x7FFFFFFF for a row holding a NaN or an infinity (its z row is then NaN).  The
 * fp16 values keep their relative precision at any input scale, and the matmul
 * multiplies row b of z by 2^e[b] in fp32.
 *
 * glq_prefill_u_bytes — bytes of fragment-order u for B rows, the row exponents
 *   included (0 for an invalid n_pad or one that is not a multiple of 128).
 * glq_prefill_row_exp_offset — byte offset of the row exponents in that buffer.
 * glq_e8_matmul_prefill_supported — 1 if glq_e8_matmul_prefill takes the layer:
 *   n_pad >= 256 and a multiple of 128, residual stage 0, 8 bits or 16 bits in the
 *   primary pack, and m_pad a multiple of 64 (slot codes) or of 256 (codebook
 *   indices).
 * glq_input_rht_prefill — u = H (sign_in * [x, 0]) / sqrt(n_pad), each row scaled
 *   by its 2^-e[b] and rounded to fp16, written in fragment order with the row
 *   exponents after it.
 *   x          device [B][n] in x_dt (F32, F16 or BF16)
 *   u16        device, >= glq_prefill_u_bytes(B, n_pad), 16-byte aligned
 *   workspace  device fp32 [B][n_pad] when n_pad > 16384 (else may be NULL),
 *              glq_input_rht_workspace_bytes(B, n_pad, GLQ_F16) bytes, 256-byte aligned
 * glq_e8_matmul_prefill — z [B][m_pad] fp32 = u W~^T from fragment-order u16 and
 *   its row exponents (codewords dequantized from the LDS-resident codebook into
 *   fp16 MFMA operands, fp32 accumulation, row b times 2^e[b]; one split:
 *   glq_output_rht takes z with S = 1).  Slot codes:
 *   per k-step a 64-row codeword tile is dequantized into LDS once and shared by
 *   four waves; codebook indices (a larger LDS image): each wave dequantizes its
 *   own fragments.
 * Errors: GLQ_ERR_NULL, GLQ_ERR_SHAPE (B < 1, n_pad below 256 or not a multiple
 * of 128, or a layer the prefill matmul does not take), GLQ_ERR_DTYPE,
 * GLQ_ERR_RECIPE, GLQ_ERR_ALIGN, GLQ_ERR_WORKSPACE, GLQ_ERR_HIP.
 */
size_t glq_prefill_u_bytes(int64_t B, int64_t n_pad);
size_t glq_prefill_row_exp_offset(int64_t B, int64_t n_pad);
int glq_e8_matmul_prefill_supported(const glq_layer* layer);
glq_status glq_input_rht_prefill(const void* x, glq_dtype x_dt, int64_t B, int64_t n, int64_t n_pad,
                                 const int8_t* sign_in, void* u16, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);
glq_status glq_e8_matmul_prefill(const glq_layer* layer, const void* u16, int64_t B, float* z,
                                 hipStream_t stream);

/*
 * glq_e8rht_linear — the E8RHTLinear forward, y = RHT_out(RHT_in(x) W~^T)
 * (glq 0.5.1, "How it works" and "Inference kernels"; E8RHTLinear is the page's
 * drop-in replacement for a linear layer, "Architecture").
 *   x          device [B][n] in x_dt (F32, F16 or BF16)
 *   y          device [B][m] in y_dt (F32, F16 or BF16)
 *   workspace  device, >= glq_e8rht_linear_workspace_bytes(layer, B), 256-byte aligned;
 *              scratch whose contents need not be initialized.  Calls that may
 *              overlap (different streams) need separate workspaces.
 * B = 1, n_pad >= 64 and every 16-bit residual stage in the primary pack (8-bit
 * stages always qualify; the further stages of a 5-8 bpw layer are added in the
 * same pass): two launches.  The first forms, in every workgroup, its column chunk
 * of the input transform in LDS via H_N = H_{N/K} (x) H_K, quantizes it, walks its
 * rows against the LDS codebook and applies H_R to its block of R output rows
 * (H_{m_pad} = H_W (x) H_R); the second sums the split partials in a fixed order
 * and applies the W-point transform across the blocks, the sign flip and the cast.
 * B <= 16 otherwise: decode path (transformed activations quantized to 16-bit fixed point
 * per 64 columns, exact integer dot products against codewords gathered from the
 * LDS-resident codebook, split-K partial sums reduced in a fixed order).
 * The fixed-point step of a 64-column block is max |u| / 30583 over the block,
 * formed as a power of two times a normal fp32 value, so tiny blocks neither
 * overflow nor lose precision.
 * B > 16: prefill path (transformed activations rounded to fp16 with a power-of-two
 * scale per row, as for glq_input_rht_prefill; codeword tiles dequantized into LDS
 * feeding fp16 MFMA with fp32 accumulation).
 * Errors: GLQ_ERR_NULL, GLQ_ERR_SHAPE, GLQ_ERR_DTYPE, GLQ_ERR_RECIPE, GLQ_ERR_ALIGN,
 * GLQ_ERR_WORKSPACE, GLQ_ERR_HIP.
 */
size_t glq_e8rht_linear_workspace_bytes(const glq_layer* layer, int64_t B);
glq_status glq_e8rht_linear(const glq_layer* layer, const void* x, glq_dtype x_dt, int64_t B, void* y,
                            glq_dtype y_dt, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * glq_e8rht_linear_group — count independent E8RHTLinear forwards,
 * y[k] = glq_e8rht_linear(&layers[k], x[k]) for k < count, in as few launches as the
 * layers allow.  For linears that read the same activations (q, k and v; gate and
 * up) or any others whose inputs are ready together.  glq 0.5.1 (PyPI project page),
 * "Advanced -> CUDA-graph decode wrapper": a B = 1 decode step of a small model is
 * bound by per-kernel dispatch, not by its bytes; here the layers share the launches
 * instead.
 *   layers     host array of count layer descriptors (1 <= count <= GLQ_GROUP_MAX)
 *   x, y       host arrays of count device pointers, x[k] [B][layers[k].n] in x_dt and
 *              y[k] [B][layers[k].m] in y_dt (x[k] may be the same pointer for several
 *              k; no y[k] may overlap another buffer of the call)
 *   workspace  device, >= glq_e8rht_linear_group_workspace_bytes(layers, count, B),
 *              256-byte aligned, uninitialized scratch; calls that may overlap need
 *              separate workspaces
 * B = 1 and layers of one n_pad, one stage layout (the residual stage and any further
 * stages of 5-8 bpw) and one index format, each one the two-launch B = 1 path would
 * take: one pair of launches for all of them, the device's CUs shared among the
 * layers in proportion to their index bytes when their own plans would not fit
 * together.  2 <= B <= 16 with at least two layers of one n_pad, one residual stage
 * and index format and no further stages, each on the int8 matrix-unit path: the input
 * transforms and activation planes per layer, one GEMV launch for all layers (CUs
 * shared the same way), the output transforms per layer.  Otherwise the layers run one
 * after another as glq_e8rht_linear on the same stream and workspace.  Every y[k] is
 * bit-identical to the single call's result when the layers keep their own plans and
 * equal to it within rounding order otherwise (the reductions follow each layer's plan).
 * Errors: as glq_e8rht_linear for any layer (nothing is launched when one fails
 * validation), GLQ_ERR_SHAPE for count outside [1, GLQ_GROUP_MAX].
 */
#define GLQ_GROUP_MAX 4
size_t glq_e8rht_linear_group_workspace_bytes(const glq_layer* layers, int32_t count, int64_t B);
glq_status glq_e8rht_linear_group(const glq_layer* layers, int32_t count, const void* const* x, glq_dtype x_dt,
                                  int64_t B, void* const* y, glq_dtype y_dt, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * glq_e8rht_linear_noalloc — glq_e8rht_linear without a caller's workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The workspace is a device array
 * of GLQ_NOALLOC_SCRATCH_BYTES inside the library, one per device, held until the
 * process ends; nothing is allocated by the call.  It fits every B <= 16 call of the
 * SmolLM2, SmolLM3 and Devstral-Small layer shapes (Devstral at B = 16 takes about
 * 35 MiB) and prefill calls of modest M; a call whose
 * glq_e8rht_linear_workspace_bytes(layer, B) exceeds it returns GLQ_ERR_WORKSPACE
 * and launches nothing.  Every call on one device shares that device's array, so
 * calls that may overlap on one device (several streams or host threads) race and
 * must be serialized by the caller.  The array needs no initial contents and keeps
 * whatever the last call left.
 * Arguments, results and errors otherwise as glq_e8rht_linear (GLQ_ERR_HIP also when
 * the array's device address cannot be obtained).
 */
#define GLQ_NOALLOC_SCRATCH_BYTES (64 << 20)
glq_status glq_e8rht_linear_noalloc(const glq_layer* layer, const void* x, glq_dtype x_dt, int64_t B, void* y,
                                    glq_dtype y_dt, hipStream_t stream);

/*
 * glq_e8kv_attention_decode — one decode step of attention over an E8-compressed
 * paged K/V cache, the cache dequantized inside the kernel (Glq v0.5.0 release
 * notes, "Highlights": the cache is never expanded into a separate buffer, a
 * length-8 Hadamard transform inverts the rotation, long contexts are split over
 * workgroups as in flash decoding).
 *   out[b][hq] = softmax_t(sm_scale q[b][hq] . K_t) . V_t over the tokens
 *   t < seq_lens[b] of sequence b, with K_t, V_t the vectors of KV head
 *   hq / (num_q_heads / num_kv_heads) at slot t mod page_size of page
 *   block_table[b][t / page_size].
 *   q            device [B][num_q_heads][head_dim] in q_dt (F32, F16 or BF16)
 *   num_q_heads  a multiple of num_kv_heads with num_q_heads / num_kv_heads in
 *                {1, 2, 4, 8}
 *   block_table  device int32 [B][max_pages]
 *   seq_lens     device int32 [B]; clamped to [0, min(max_seq_len, max_pages *
 *                page_size)]; a sequence of 0 tokens gives zeros
 *   max_seq_len  host bound on seq_lens (sizes the split of the contexts)
 *   out          device [B][num_q_heads][head_dim] in out_dt (F32, F16 or BF16)
 *   workspace    device, >= glq_e8kv_attention_workspace_bytes(...), 256-byte
 *                aligned; scratch (the chunks' partial results), no initial contents
 * Each chunk's softmax statistics and partial output are merged in chunk order:
 * run-to-run bit identity.  Accumulation is fp32; q is rotated once (the rotation is
 * orthonormal and symmetric, so no cached vector is rotated) and held in fp16, whose
 * products with the codewords' exact fp16 values accumulate in fp32.
 * Errors: GLQ_ERR_NULL, GLQ_ERR_SHAPE, GLQ_ERR_DTYPE, GLQ_ERR_RECIPE, GLQ_ERR_ALIGN,
 * GLQ_ERR_WORKSPACE, GLQ_ERR_HIP.
 */
size_t glq_e8kv_attention_workspace_bytes(const glq_kv_cache* kv, int64_t B, int32_t num_q_heads,
                                          int64_t max_seq_len);
glq_status glq_e8kv_attention_decode(const glq_kv_cache* kv, const void* q, glq_dtype q_dt, int64_t B,
                                     int32_t num_q_heads, const int32_t* block_table, int64_t max_pages,
                                     const int32_t* seq_lens, int64_t max_seq_len, float sm_scale, void* out,
                                     glq_dtype out_dt, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GLQ_H */
