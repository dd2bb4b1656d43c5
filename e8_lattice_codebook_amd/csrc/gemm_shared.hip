// Prefill matmul (B > 16) for slot-code layers on gfx950: z = u W~^T with each
// k-step's codeword tile dequantized once per workgroup into LDS and shared by its
// four waves (fp16 MFMA v_mfma_f32_16x16x32_f16, fp32 accumulation).
//
// glq 0.5.1 (PyPI project page), "Inference kernels": for B >= 2 the matmul runs on
// the matrix units against codebook-loaded operands, without forming W; "How it
// works", items 1 and 4; table "Bit widths".
//
// Tile: 64 output rows x 512 tokens per workgroup.  At each k-step (32 of K: four
// groups per row) the 256 threads look one codeword up each (row t / 4, lane
// quarter t % 4) in the LDS slot image, turn its eight signed 4-bit lanes 2c into
// fp16 (plus s_r times the residual stage, exact in fp16 for s_r = 1/4) and write
// the 16 bytes to an LDS tile in the MFMA's A-operand order.  Every wave reads the
// four 16-row fragments and multiplies them with its own 128 tokens (eight 16-token
// blocks of u, the B operand, loaded from global memory three k-steps ahead): 32
// MFMAs per k-step and wave, so each lookup serves 32 MFMAs of 16x16x32 (all 512
// tokens).  Two tiles alternate between k-steps and the work is pipelined over four
// k-steps (fragments of ks + 1 read, tile of ks + 2 written, codeword of ks + 3
// converted, LDS reads of ks + 4 issued, all among the MFMAs of ks), so one barrier
// per k-step suffices and no VALU waits on LDS.
//
// LDS: the 8-bit residual stage's 256 slot words (1 KiB), the slot image (at most
// kSlotImageMaxDwords: the pack gives larger images no slot format), two 4 KiB
// tiles.  The residual entries are read as 4-byte slot words and converted like the
// primary ones: a random 16-byte read of an fp16 table costs the LDS four times as
// much.
//
// K order (the matmuls' fragment order): at k-step ks, lane quarter q = lane / 16
// takes group 16 (ks / 4) + 4 q + ks % 4 (KS = n_pad / 32 k-steps, a multiple of 4).
// Over a block of 4 k-steps a dequantizing thread's groups are 4 consecutive ones
// (one 8-byte index load) and the row's four threads read 32 consecutive bytes.  u
// is in the same order: the fragment of 16-token block tb at k-step ks is 1 KiB at
// half (tb KS + ks) 512, lane l = 16 q + (token mod 16) holding 8 halves
// (tiled_u_bytes; the input transform writes it so).
#include "mfma_dequant.h"

namespace glq {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kSThreads = 256;  // 4 waves, one per SIMD
constexpr int kSRB = 4;         // 16-row blocks per tile (all waves)
constexpr int kSTB = 8;         // 16-token blocks per wave
constexpr int kSRows = 16 * kSRB;          // output rows per tile
constexpr int kSTok = 4 * 16 * kSTB;       // tokens per tile
constexpr int kSKB = 4;         // k-steps per index block

struct SharedArgs {
  const half_t* u;            // fragment order, tiled_u_bytes(M, n_pad)
  const uint16_t* idx0;       // [m_pad][G] slot codes
  const void* idx1;           // [m_pad][G] u8 or u16
  const uint32_t* pack0_hdr;
  const uint32_t* img0;       // slot image
  const uint32_t* res_slots;  // 8-bit residual: the 256 slot words of its pack
  const int32_t* rexp;        // the rows' power-of-two exponents (NULL: none)
  float* z;                   // [M][m_pad] fp32
  int64_t M;
  int m_pad, G, KS;
  int out_tiles, tiles;
  float scale;                // s / 2
  float sr;
  int accumulate;             // add to z (second pass of a 5-8 bpw layer)
};

template <int RESID>
__global__ __launch_bounds__(kSThreads, 1) void gemm_shared_kernel(SharedArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[kImgOff + kSlotImageMaxDwords];  // residual slots, image
  __shared__ __attribute__((aligned(16))) u32x4 wtile[2][kSRB * 64];                    // [rb][q][16 rows] x 8 halves
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint32_t two = 2;
  uint32_t delta = a.pack0_hdr[kHdrSlotDelta];
  delta = delta < uint32_t(kSlotImageMaxDwords - kSlotShared) ? delta : uint32_t(kSlotImageMaxDwords - kSlotShared);

  // ---- the slot image (and the residual slots) into LDS, once per workgroup
  {
    uint32_t nd = a.pack0_hdr[kHdrSlotDwords];
    nd = nd > uint32_t(kSlotImageMaxDwords) ? uint32_t(kSlotImageMaxDwords) : nd;
    const uint32_t nd4 = nd >> 2;
    const u32x4* src4 = reinterpret_cast<const u32x4*>(a.img0);
    u32x4* dst4 = reinterpret_cast<u32x4*>(lds + kImgOff);
    const uint32_t last4 = nd4 > 0 ? nd4 - 1 : 0;
    for (uint32_t base = 0; base < nd4; base += 8 * kSThreads) {
      u32x4 t[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) t[k] = src4[min(base + k * kSThreads + tid, last4)];
#pragma unroll
      for (int k = 0; k < 8; ++k) dst4[min(base + k * kSThreads + tid, last4)] = t[k];
    }
    for (uint32_t i = (nd4 << 2) + tid; i < nd; i += kSThreads) lds[kImgOff + i] = a.img0[i];
    if (RESID == 8) lds[kResOff + tid] = a.res_slots[tid];  // 256 threads, 256 slots
  }
  __syncthreads();

  const int G = a.G;
  const int KS = a.KS;
  const int NB = KS / kSKB;  // index blocks
  const half2v sr2 = half2v{_Float16(a.sr), _Float16(a.sr)};
  const int dr = tid >> 2, dq = tid & 3;                   // dequantizing role: tile row, lane quarter
  const int wpos = (dr >> 4) * 64 + dq * 16 + (dr & 15);   // its place in a tile
  const int64_t tbc = (a.M + 15) / 16;                     // 16-token blocks held by u

  for (int tile = blockIdx.x; tile < a.tiles; tile += gridDim.x) {
    // workgroups are dealt to the 8 XCDs in turn: XCD x takes a contiguous eighth of
    // the output tiles for every token tile, token-tile major, so the workgroups
    // running at once on one XCD share a few u tiles and index rows in its L2
    int out_tile, tok_tile;
    if ((a.out_tiles & 7) == 0) {
      const int per = a.out_tiles >> 3;
      const int i = tile >> 3;
      tok_tile = i / per;
      out_tile = (tile & 7) * per + (i - tok_tile * per);
    } else {
      out_tile = tile % a.out_tiles;
      tok_tile = tile / a.out_tiles;
    }
    const int o0 = out_tile * kSRows;
    const int64_t tfirst = int64_t(tok_tile) * (kSTok / 16);  // the tile's first token block
    const int64_t tb0 = tfirst + kSTB * wave;                 // this wave's blocks tb0 .. tb0 + 7

    // index rows: tile row dr, groups 16 b + 4 dq .. + 3 of block b
    const int64_t irow = int64_t(o0 + dr) * G + 4 * dq;
    auto load_idx = [&](int b, u32x2& i0, uint32_t& i1b, u32x2& i1w) {
      const int64_t off = irow + 16 * int64_t(b < NB ? b : NB - 1);  // past the end: the last block
      i0 = *reinterpret_cast<const u32x2*>(a.idx0 + off);
      if (RESID == 8) i1b = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(a.idx1) + off);
      if (RESID == 16) i1w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.idx1) + off);
    };
    // the codeword of k-step kk of a block in two steps: the LDS reads (slot words of
    // the stages) and, a k-step later, the conversion to 8 fp16 values, so that no
    // VALU waits on LDS
    struct Raw {
      uint32_t w0, m0, w1, m1;
    };
    auto lookup = [&](const u32x2& i0, uint32_t i1b, const u32x2& i1w, int kk) -> Raw {
      Raw x;
      const uint32_t c0 = i0[kk >> 1];
      x.w0 = (kk & 1) ? code_word<1>(lds, c0, delta, x.m0) : code_word<0>(lds, c0, delta, x.m0);
      x.w1 = 0;
      x.m1 = 0;  // 8-bit entries are never complemented
      if (RESID == 8) {
        uint32_t ra;
        switch (kk & 3) {
          case 0: ra = byte_x4<0>(i1b, two); break;
          case 1: ra = byte_x4<1>(i1b, two); break;
          case 2: ra = byte_x4<2>(i1b, two); break;
          default: ra = byte_x4<3>(i1b, two); break;
        }
        x.w1 = lds_res(lds, ra);
      }
      if (RESID == 16) {
        const uint32_t c1 = i1w[kk >> 1];
        x.w1 = (kk & 1) ? code_word<1>(lds, c1, delta, x.m1) : code_word<0>(lds, c1, delta, x.m1);
      }
      return x;
    };
    auto convert = [&](const Raw& x) -> half8 {
      half8 b = word_to_half8(x.w0, x.m0);
      if (RESID != 0) {
        const half8 r = word_to_half8(x.w1, x.m1);
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const half2v f = half2v{r[j], r[j + 1]} * sr2 + half2v{b[j], b[j + 1]};
          b[j] = f.x;
          b[j + 1] = f.y;
        }
      }
      return b;
    };
    // u fragments of the wave's token blocks (blocks past the buffer read the tile's
    // first block, which exists; their outputs are not stored)
    const u32x4* ubase = reinterpret_cast<const u32x4*>(a.u) + lane;
    int64_t uoff[kSTB];
#pragma unroll
    for (int j = 0; j < kSTB; ++j) uoff[j] = (tb0 + j < tbc ? tb0 + j : tfirst) * KS * 64;
    auto uload = [&](int ks, u32x4 (&f)[kSTB]) {
      const int64_t k = int64_t(ks < KS ? ks : KS - 1) * 64;  // past the end: in-bounds, never used
#pragma unroll
      for (int j = 0; j < kSTB; ++j) {
        GLQ_DCHECK(uoff[j] + k + lane < tbc * KS * 64);
        f[j] = ubase[uoff[j] + k];
      }
    };

    floatx4 acc[kSRB][kSTB];
#pragma unroll
    for (int rb = 0; rb < kSRB; ++rb)
#pragma unroll
      for (int j = 0; j < kSTB; ++j) acc[rb][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // ---- tile prologue: index blocks 0 and 1, u of k-steps 0-2 (k-step k in set
    // k & 3), the codeword tiles of k-steps 0 and 1 in LDS, the fragments of k-step 0
    // in registers, the codeword of k-step 2 and the LDS reads of k-step 3
    u32x4 uf[4][kSTB];
    half8 wa[kSRB], wb[kSRB];
    u32x2 i0, i0n, i1w, i1wn;
    uint32_t i1b = 0, i1bn = 0;
    load_idx(0, i0, i1b, i1w);
    load_idx(1, i0n, i1bn, i1wn);
    uload(0, uf[0]);
    uload(1, uf[1]);
    uload(2, uf[2]);
    const half8 d0 = convert(lookup(i0, i1b, i1w, 0));
    const half8 d1 = convert(lookup(i0, i1b, i1w, 1));
    half8 dn = convert(lookup(i0, i1b, i1w, 2));
    Raw rn = lookup(i0, i1b, i1w, 3);
    __syncthreads();  // the previous tile's last reads of both tiles are done
    wtile[0][wpos] = __builtin_bit_cast(u32x4, d0);
    wtile[1][wpos] = __builtin_bit_cast(u32x4, d1);
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < kSRB; ++rb) wa[rb] = __builtin_bit_cast(half8, wtile[0][rb * 64 + lane]);
    __syncthreads();  // every wave has its fragments of k-step 0: tile slot 0 is free

    // ---- k-step ks: its fragments are in registers (set ks & 1); LDS holds the
    // tile of ks + 1 (published by the last barrier) in slot (ks + 1) & 1, and slot
    // ks & 1 is free (its fragments were read during the previous step).  The step
    // issues the LDS reads of ks + 4 (the next index block, same position), reads the
    // fragments of ks + 1, writes the tile of ks + 2 into slot ks & 1, converts the
    // codeword of ks + 3, loads u of ks + 3 and runs its 32 MFMAs, each followed by a
    // share of that work; one barrier per step publishes the tile of ks + 2.
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int kk = 0; kk < kSKB; ++kk) {
        const int ks = b * kSKB + kk;
        half8* wc = (kk & 1) ? wb : wa;
        half8* wn = (kk & 1) ? wa : wb;
        const Raw rnew = lookup(i0n, i1bn, i1wn, kk);  // k-step ks + 4: first, done before the barrier
#pragma unroll
        for (int rb = 0; rb < kSRB; ++rb) wn[rb] = __builtin_bit_cast(half8, wtile[(kk + 1) & 1][rb * 64 + lane]);
        wtile[kk & 1][wpos] = __builtin_bit_cast(u32x4, dn);
        dn = convert(rn);
        rn = rnew;
        uload(ks + 3, uf[(kk + 3) & 3]);
#pragma unroll
        for (int j = 0; j < kSTB; ++j)
#pragma unroll
          for (int rb = 0; rb < kSRB; ++rb)
            acc[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wc[rb], __builtin_bit_cast(half8, uf[kk & 3][j]),
                                                               acc[rb][j], 0, 0, 0);
        // interleave: each MFMA followed by one VALU and, in the first quarter of
        // the step, one LDS access; a global load after every fourth MFMA
#pragma unroll
        for (int g = 0; g < kSRB * kSTB; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // VALU
          if (g < 8) __builtin_amdgcn_sched_group_barrier(0x080, 1, 0);  // LDS
          if ((g & 3) == 3) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // global memory
        }
        // the step boundary: nothing of one step moves past the barrier into another
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();  // the tile of ks + 2 is complete; every wave has read that of ks + 1
        __builtin_amdgcn_sched_barrier(0);
      }
      i0 = i0n;
      i1b = i1bn;
      i1w = i1wn;
      load_idx(b + 2, i0n, i1bn, i1wn);
    }

    // ---- z = acc * s / 2 * 2^rexp[t].  D of a 16x16 block: lane l holds token
    // l % 16 and outputs 4 (l / 16) .. + 3 of the row block
#pragma unroll
    for (int j = 0; j < kSTB; ++j) {
      const int64_t t = (tb0 + j) * 16 + (lane & 15);
      if (t < a.M) {
        const int32_t e = a.rexp ? a.rexp[t] : 0;
        float* zr = a.z + t * a.m_pad + o0 + 4 * (lane >> 4);
#pragma unroll
        for (int rb = 0; rb < kSRB; ++rb) {
          floatx4* p = reinterpret_cast<floatx4*>(zr + 16 * rb);
          floatx4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = row_scaled(acc[rb][j][i] * a.scale, e);
          *p = a.accumulate ? *p + v : v;
        }
      }
    }
  }
}

}  // namespace

bool gemm_shared_supported(const glq_layer& L) {
  // slot codes (the slot image leaves LDS for the tiles), n_pad a multiple of 128
  // (whole index blocks of 4 k-steps), whole 64-row tiles, residual from the image
  // or an 8-bit table
  return L.index_format == GLQ_INDEX_SLOT && L.n_pad >= 256 && L.n_pad % 128 == 0 && L.m_pad % kSRows == 0 &&
         (L.resid_bits != 16 || L.cb2_pack == L.cb_pack);
}

size_t tiled_u_bytes(int64_t M, int64_t n_pad) { return size_t((M + 15) / 16) * 16 * size_t(n_pad) * 2; }

hipError_t launch_gemm_shared(const glq_layer& L, const half_t* u16, const int32_t* rexp, int64_t M, float* z,
                              hipStream_t stream, bool accumulate) {
  SharedArgs a;
  a.u = u16;
  a.rexp = rexp;
  a.idx0 = L.idx0;
  a.idx1 = L.idx1;
  const char* p0 = static_cast<const char*>(L.cb_pack);
  a.pack0_hdr = reinterpret_cast<const uint32_t*>(p0);
  a.img0 = reinterpret_cast<const uint32_t*>(p0 + pack_slot_image_offset(GLQ_CODEBOOK_ENTRIES));
  a.res_slots = L.resid_bits == 8 ? reinterpret_cast<const uint32_t*>(static_cast<const char*>(L.cb2_pack) +
                                                                     pack_image_offset(GLQ_RESID8_ENTRIES)) + kPageCount
                                   : nullptr;
  a.z = z;
  a.M = M;
  a.m_pad = int(L.m_pad);
  a.G = int(L.n_pad / 8);
  a.KS = int(L.n_pad / 32);
  a.out_tiles = int(L.m_pad / kSRows);
  a.tiles = int(a.out_tiles * ((M + kSTok - 1) / kSTok));
  a.scale = 0.5f * L.wscale;
  a.sr = L.resid_scale;
  a.accumulate = int(accumulate);
  const int cus = device_cus();
  const dim3 grid(unsigned(a.tiles < cus ? a.tiles : cus)), block(kSThreads);
  switch (L.resid_bits) {
    case 0: hipLaunchKernelGGL(gemm_shared_kernel<0>, grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL(gemm_shared_kernel<8>, grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL(gemm_shared_kernel<16>, grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

GLQ_DEBUG_COUNTER(debug_violations_gemm_shared)

}  // namespace glq
