// Host construction of the E8 codebook table (glq_e8_codebook).
//
// glq 0.5.1 (PyPI project page), "How it works", item 1: the table has 2^16 points
// of E8, the lattice points of smallest norm up to the seventh norm value counting
// the origin, addressed by a 16-bit index per group of 8 weights; "Inference
// kernels": stored in fp16 the table takes 1 MB.  E8 = D8 u (D8 + 1/2): all
// coordinates integers or all half-integers, with an even coordinate sum.
//
// Points are enumerated by depth-first search on doubled coordinates t = 2v
// (|t_j| <= 6, every t_j of one parity, sum(t) = 0 mod 4, sum(t^2) <= 48), sorted
// by (sum(t^2), t_0, ..., t_7) ascending, and the first `entries` are written
// as fp16 bit patterns.
#include <algorithm>
#include <array>
#include <cstdint>
#include <vector>

#include "glq.h"

namespace {

typedef std::array<int8_t, 8> Pt;

void dfs(int depth, int parity, int sum, int norm, Pt& cur, std::vector<Pt>& out) {
  if (depth == 8) {
    if (((sum % 4) + 4) % 4 == 0) out.push_back(cur);
    return;
  }
  for (int t = -6 - (parity ? -1 : 0); t <= 6; ++t) {
    if ((t & 1) != parity) continue;
    const int nn = norm + t * t;
    if (nn > 48) continue;
    cur[depth] = int8_t(t);
    dfs(depth + 1, parity, sum + t, nn, cur, out);
  }
}

// fp16 bit pattern of t / 2 for |t| <= 6 (every such value is exact in fp16).
uint16_t half_bits_of_doubled(int t) {
  if (t == 0) return 0;
  const uint16_t sign = t < 0 ? 0x8000 : 0;
  int a = t < 0 ? -t : t;  // value = a / 2
  // normalise: value = (a / 2^k) * 2^(k-1) with 1 <= a / 2^k < 2
  int k = 0;
  while ((a >> (k + 1)) > 0) ++k;
  const int exponent = k - 1;                     // value = 1.f * 2^exponent
  const int mant = (a << (10 - k)) & 0x3FF;       // fraction bits of a / 2^k
  return uint16_t(sign | uint16_t((exponent + 15) << 10) | uint16_t(mant));
}

}  // namespace

extern "C" glq_status glq_e8_codebook(uint16_t* cb_host, int64_t entries) {
  if (!cb_host) return GLQ_ERR_NULL;
  if (entries < 1 || entries > GLQ_CODEBOOK_ENTRIES) return GLQ_ERR_SHAPE;
  std::vector<Pt> pts;
  pts.reserve(120000);
  Pt cur{};
  dfs(0, 0, 0, 0, cur, pts);  // integer type
  dfs(0, 1, 0, 0, cur, pts);  // half-integer type
  auto key_less = [](const Pt& a, const Pt& b) {
    int na = 0, nb = 0;
    for (int j = 0; j < 8; ++j) {
      na += a[j] * a[j];
      nb += b[j] * b[j];
    }
    if (na != nb) return na < nb;
    return a < b;  // lexicographic on signed coordinates, t_0 first
  };
  std::sort(pts.begin(), pts.end(), key_less);
  if (int64_t(pts.size()) < entries) return GLQ_ERR_SHAPE;
  for (int64_t i = 0; i < entries; ++i)
    for (int j = 0; j < 8; ++j) cb_host[i * 8 + j] = half_bits_of_doubled(pts[size_t(i)][j]);
  return GLQ_OK;
}
