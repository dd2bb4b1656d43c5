// Host construction of a codebook pack (glq_codebook_pack).
//
// glq 0.5.1 (PyPI project page), "How it works", item 1 and "Inference kernels":
// the kernels gather 8-D codewords from a compact cached codebook.  On gfx950 the
// codebook is gathered from LDS, which holds 160 KB per CU, so the pack carries
// an LDS image in which every codeword takes 4 bytes (eight signed 4-bit values
// 2c, c in Z/2, |2c| <= 8) and each negation-symmetric shell is stored once.
//
// Layout (offsets in bytes, all 256-byte aligned):
//   0                header: kPackMagic, version, entries, image dwords, slots, flags
//   256              int8 table [entries][8], value 2c (kernels that dequantize)
//   image_offset     LDS image: page table [256] u32, then slot words
//
// Page table: index i falls in page p = i >> 8 at offset t = i & 255.  A page is
// ascending (slot = base + t) or descending (slot = base + (255 - t)).  With
// B = 4 * (base + 256), the byte address of slot `base` in the image (the slots
// follow the 256-dword page table), its descriptor is desc = B on an ascending
// page and desc = B + 1021 on a descending one, so bit 0 flags the direction and
// with m = -(desc & 1) (0 or all ones) the kernels read the image word at byte
// offset ((4 t) ^ m) + desc, i.e. B + 4 t or B + 1020 - 4 t, one xor-add.  A
// symmetric shell (entries M + r and M - 1 - r are negatives of each other, M its
// centre) stores its upper half once: its upper-half pages ascend, its lower-half
// pages descend and read the negated words (the kernels complement every lane,
// m again).  Non-symmetric runs ascend; pages that hold a run boundary or a shell
// centre are stored whole, ascending.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <unordered_map>
#include <utility>
#include <vector>

#include "internal.h"

namespace {

struct Run {
  int64_t start, size;
  bool mirrored;
  int64_t center;  // M
  int64_t base;    // R (slot of distance 0, or of the run start); -1 until allocated
};

}  // namespace

namespace glq {

size_t pack_total_bytes(int64_t entries) { return pack_index_of_offset(entries) + size_t(65536) * 2; }

glq_status build_pack(const uint16_t* cb, int64_t entries, void* out_pack, size_t out_bytes) {
  if (!cb || !out_pack) return GLQ_ERR_NULL;
  if (entries < 1 || entries > GLQ_CODEBOOK_ENTRIES) return GLQ_ERR_SHAPE;
  if (out_bytes < pack_total_bytes(entries)) return GLQ_ERR_WORKSPACE;
  // doubled coordinates
  std::vector<int> t(size_t(entries) * 8);
  for (int64_t i = 0; i < entries * 8; ++i) {
    const uint16_t h = cb[i];
    const int sign = (h >> 15) & 1, ex = (h >> 10) & 31, man = h & 1023;
    if (ex == 31) return GLQ_ERR_CODEBOOK;  // inf / nan
    // value = (-1)^sign * (ex ? (1024 + man) * 2^(ex - 25) : man * 2^-24); need 2 * value integer
    int64_t mant = ex ? (1024 + man) : man;
    int shift = (ex ? ex : 1) - 25 + 1;  // doubled value = mant * 2^shift
    int64_t v;
    if (shift >= 0) {
      if (shift > 8) return GLQ_ERR_CODEBOOK;
      v = mant << shift;
    } else {
      if (-shift >= 40) {
        if (mant != 0) return GLQ_ERR_CODEBOOK;
        v = 0;
      } else {
        if (mant & ((int64_t(1) << -shift) - 1)) return GLQ_ERR_CODEBOOK;  // not a multiple of 1/2
        v = mant >> -shift;
      }
    }
    if (sign) v = -v;
    if (v < -8 || v > 7) return GLQ_ERR_CODEBOOK;
    t[size_t(i)] = int(v);
  }
  auto word = [&](int64_t i) {
    uint32_t w = 0;
    for (int j = 0; j < 8; ++j) w |= uint32_t(t[size_t(i * 8 + j)] & 15) << (4 * lane_nibble(j));
    return w;
  };
  auto norm2 = [&](int64_t i) {
    int s = 0;
    for (int j = 0; j < 8; ++j) s += t[size_t(i * 8 + j)] * t[size_t(i * 8 + j)];
    return s;
  };

  // maximal runs of equal squared norm; symmetric runs (entry O + k is the
  // negation of entry O + N - 1 - k, N even) are stored by distance from the centre
  std::vector<Run> runs;
  for (int64_t i = 0; i < entries;) {
    int64_t j = i + 1;
    const int nn = norm2(i);
    while (j < entries && norm2(j) == nn) ++j;
    Run r{i, j - i, false, i, -1};
    if (r.size >= 2 && r.size % 2 == 0) {
      bool sym = true;
      for (int64_t k = 0; k < r.size / 2 && sym; ++k)
        for (int c = 0; c < 8 && sym; ++c)
          if (t[size_t((i + k) * 8 + c)] != -t[size_t((i + r.size - 1 - k) * 8 + c)]) sym = false;
      if (sym) {
        r.mirrored = true;
        r.center = i + r.size / 2;
      }
    }
    runs.push_back(r);
    i = j;
  }
  auto run_of = [&](int64_t i) {
    int64_t lo = 0, hi = int64_t(runs.size()) - 1;
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) / 2;
      if (runs[size_t(mid)].start <= i) lo = mid; else hi = mid - 1;
    }
    return lo;
  };

  // pages: a page whose indices (those below `entries`) lie in one run uses that
  // run's descriptor; packs of at most 256 entries and straddling pages are direct
  const int64_t n_pages = (entries + kPageSize - 1) / kPageSize;
  std::vector<int64_t> page_run(size_t(kPageCount), -1);
  for (int64_t p = 0; p < n_pages; ++p) {
    const int64_t a = p * kPageSize, b = std::min<int64_t>(entries, a + kPageSize) - 1;
    const int64_t ra = run_of(a), rb = run_of(b);
    if (ra != rb || entries <= kPageSize) continue;
    const Run& r = runs[size_t(ra)];
    if (r.mirrored && a < r.center && b >= r.center) continue;  // holds the centre
    page_run[size_t(p)] = ra;
  }
  std::vector<uint32_t> slots;
  std::vector<uint32_t> desc(size_t(kPageCount), 0);
  auto make_desc = [](int64_t base, bool descending) {
    return uint32_t(4 * (base + kPageCount)) + (descending ? 1021u : 0u);
  };
  // exception (direct) pages first, in page order: a pack of <= 256 entries is slot = index
  for (int64_t p = 0; p < n_pages; ++p) {
    if (page_run[size_t(p)] >= 0) continue;
    const int64_t a = p * kPageSize;
    const int64_t R = int64_t(slots.size());
    for (int64_t k = 0; k < kPageSize; ++k) slots.push_back(a + k < entries ? word(a + k) : 0u);
    desc[size_t(p)] = make_desc(R, false);
  }
  for (int64_t p = 0; p < n_pages; ++p) {
    const int64_t ri = page_run[size_t(p)];
    if (ri < 0) continue;
    Run& r = runs[size_t(ri)];
    if (r.base < 0) {
      r.base = int64_t(slots.size());
      if (r.mirrored) {
        for (int64_t k = 0; k < r.size / 2; ++k) slots.push_back(word(r.center + k));
      } else {
        for (int64_t k = 0; k < r.size; ++k) slots.push_back(word(r.start + k));
      }
    }
    const int64_t a = p * kPageSize;
    if (!r.mirrored) {
      desc[size_t(p)] = make_desc(r.base + a - r.start, false);           // slot = R + i - start
    } else if (a >= r.center) {
      desc[size_t(p)] = make_desc(r.base + a - r.center, false);          // slot = R + i - M
    } else {
      // slot = R + (M - 1 - i) = (R + M - 1 - a - 255) + (255 - t)
      desc[size_t(p)] = make_desc(r.base + r.center - 1 - a - (kPageSize - 1), true);
    }
  }
  const int64_t image_dwords = kPageCount + int64_t(slots.size());
  if (image_dwords > kImageMaxDwords) return GLQ_ERR_CODEBOOK;

  // self-check: every index resolves to its own codeword
  for (int64_t i = 0; i < entries; ++i) {
    const uint32_t dsc = desc[size_t(i >> 8)];
    const bool m = (dsc & 1u) != 0;
    const uint32_t ba = ((uint32_t(i & 0xFF) * 4) ^ (m ? 0xFFFFFFFFu : 0u)) + dsc;  // byte offset in the image
    if (ba < 4u * kPageCount || ba % 4 != 0) return GLQ_ERR_CODEBOOK;
    const uint32_t slot = ba / 4 - kPageCount;
    if (slot >= slots.size()) return GLQ_ERR_CODEBOOK;
    uint32_t w = slots[slot];
    if (m) {  // negate every 4-bit lane
      uint32_t neg = 0;
      for (int j = 0; j < 8; ++j) {
        const int v = int32_t(((w >> (4 * j)) & 15u) << 28) >> 28;
        neg |= uint32_t(-v & 15) << (4 * j);
      }
      w = neg;
    }
    if (w != word(i)) return GLQ_ERR_CODEBOOK;
  }

  // ---- slot-code format: every codeword whose negation is also an entry shares
  // one slot with it (the pair's second member reads it complemented); the other
  // entries fill [0, delta) plain and [32768, 32768 + delta) negated
  std::unordered_map<uint32_t, int64_t> pos;
  for (int64_t i = 0; i < entries; ++i) pos.emplace(word(i), i);
  auto neg_word = [&](int64_t i, bool& ok) {  // the negated codeword's word, if its lanes fit
    uint32_t w = 0;
    ok = true;
    for (int j = 0; j < 8; ++j) {
      const int v = -t[size_t(i * 8 + j)];
      if (v > 7) ok = false;
      w |= uint32_t(v & 15) << (4 * lane_nibble(j));
    }
    return w;
  };
  std::vector<int64_t> partner(size_t(entries), -1);
  std::vector<std::pair<int64_t, int64_t>> pairs;  // (plain member, complemented member)
  for (int64_t i = 0; i < entries; ++i) {
    if (partner[size_t(i)] >= 0) continue;
    bool ok;
    const uint32_t nw = neg_word(i, ok);
    if (!ok) continue;
    auto it = pos.find(nw);
    if (it == pos.end() || it->second == i || partner[size_t(it->second)] >= 0) continue;
    const int64_t j = it->second;
    partner[size_t(i)] = j;
    partner[size_t(j)] = i;
    pairs.emplace_back(std::max(i, j), std::min(i, j));
  }
  const int64_t F = int64_t(pairs.size());
  const int64_t delta = kSlotShared - F;
  std::vector<int64_t> lone_plain, lone_neg;
  for (int64_t i = 0; i < entries; ++i) {  // entries that cannot be negated stay plain
    if (partner[size_t(i)] >= 0) continue;
    bool ok;
    neg_word(i, ok);
    if (!ok) lone_plain.push_back(i);
  }
  for (int64_t i = 0; i < entries; ++i) {
    if (partner[size_t(i)] >= 0) continue;
    bool ok;
    neg_word(i, ok);
    if (!ok) continue;
    if (int64_t(lone_plain.size()) < delta) lone_plain.push_back(i);
    else lone_neg.push_back(i);
  }
  const int64_t slot_dwords = kSlotShared + int64_t(lone_neg.size());
  const bool slot_ok = int64_t(lone_plain.size()) <= delta && int64_t(lone_neg.size()) <= delta &&
                       slot_dwords <= kSlotImageMaxDwords;
  std::vector<uint32_t> slot_img;
  std::vector<uint16_t> code_of(size_t(entries), 0), index_of(65536, 0);
  if (slot_ok) {
    slot_img.assign(size_t(slot_dwords), 0u);
    for (size_t r = 0; r < lone_plain.size(); ++r) {
      slot_img[r] = word(lone_plain[r]);
      code_of[size_t(lone_plain[r])] = uint16_t(r);
    }
    for (size_t k = 0; k < pairs.size(); ++k) {
      slot_img[size_t(delta) + k] = word(pairs[k].first);
      code_of[size_t(pairs[k].first)] = uint16_t(delta + int64_t(k));
      code_of[size_t(pairs[k].second)] = uint16_t(0xFFFFu - uint32_t(k));  // int16 ~k
    }
    for (size_t r = 0; r < lone_neg.size(); ++r) {
      bool ok;
      slot_img[size_t(kSlotShared) + r] = neg_word(lone_neg[r], ok);
      const uint32_t x = uint32_t(kSlotShared) + uint32_t(r) - uint32_t(delta);
      code_of[size_t(lone_neg[r])] = uint16_t(0xFFFFu - x);
    }
    // self-check: every code decodes, as the kernels read it, to its entry
    std::vector<uint8_t> used(65536, 0);
    for (int64_t i = 0; i < entries; ++i) {
      const int32_t c = int16_t(code_of[size_t(i)]);
      const uint32_t m = uint32_t(c >> 15);
      const uint32_t P = (uint32_t(c) ^ m) + (m & uint32_t(delta));
      if (P >= uint32_t(slot_dwords) || used[code_of[size_t(i)]]) return GLQ_ERR_CODEBOOK;
      used[code_of[size_t(i)]] = 1;
      index_of[code_of[size_t(i)]] = uint16_t(i);
      const uint32_t w = slot_img[P];
      for (int j = 0; j < 8; ++j) {
        const int v = int32_t(((w >> (4 * lane_nibble(j))) & 15u) << 28) >> 28;
        if ((m ? -v : v) != t[size_t(i * 8 + j)]) return GLQ_ERR_CODEBOOK;
      }
    }
  }

  // write the pack
  std::memset(out_pack, 0, pack_total_bytes(entries));
  uint32_t* hdr = static_cast<uint32_t*>(out_pack);
  hdr[0] = kPackMagic;
  hdr[1] = kPackVersion;
  hdr[2] = uint32_t(entries);
  hdr[3] = uint32_t(image_dwords);
  hdr[4] = uint32_t(slots.size());
  int8_t* i8 = static_cast<int8_t*>(out_pack) + pack_i8_offset();
  for (int64_t i = 0; i < entries * 8; ++i) i8[i] = int8_t(t[size_t(i)]);
  uint32_t* img = reinterpret_cast<uint32_t*>(static_cast<char*>(out_pack) + pack_image_offset(entries));
  std::memcpy(img, desc.data(), size_t(kPageCount) * 4);
  std::memcpy(img + kPageCount, slots.data(), slots.size() * 4);
  if (slot_ok) {
    hdr[kHdrSlotDwords] = uint32_t(slot_dwords);
    hdr[kHdrSlotDelta] = uint32_t(delta);
    char* base = static_cast<char*>(out_pack);
    std::memcpy(base + pack_slot_image_offset(entries), slot_img.data(), slot_img.size() * 4);
    std::memcpy(base + pack_code_of_offset(entries), code_of.data(), code_of.size() * 2);
    std::memcpy(base + pack_index_of_offset(entries), index_of.data(), index_of.size() * 2);
  }
  return GLQ_OK;
}

}  // namespace glq
