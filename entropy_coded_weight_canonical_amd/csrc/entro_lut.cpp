// Host side of the decode table (LUT): codebook validation, canonical codes,
// table layout, bf16 dequantized values, status strings.
//
// Method: EntroLLM builds one Huffman code per weight tensor from the value
// frequencies of its quantized codes (gist.science technical summary,
// Methodology item 2) and dequantizes with the tensor's scale and zero point
// (tensor-level unsigned/asymmetric quantization, abstract).  The canonical
// assignment of codewords to lengths and the bf16 rounding are readings (the
// pages are silent): codes of one length are consecutive in symbol order,
// shorter codes first, first code zero, MSB-first; bf16 = RNE(f32 product).
//
// Table layout (uint32 words):
//   [0] magic "ECW1"            [1] K | sym_bits << 8 | max_len << 16 | shortest length << 24
//   [2] number of entries E     [3] 2^K (first-level entries)
//   [4 .. 4+E) entries.  Entry bits: [4:0] code length (0 = no codeword),
//   [7] second-level pointer, [15:8] code value (pointer: index bits of the
//   subtable), [31:16] bf16 value (pointer: absolute entry index of the
//   subtable).  First level is indexed by the next K stream bits; a code of
//   length l <= K fills the 2^(K-l) entries that start with it.  A K-bit
//   prefix of codes longer than K points to a subtable indexed by the next
//   (longest length under the prefix - K) bits.
#include <algorithm>
#include <cstring>
#include <vector>

#include "entro.h"
#include "entro_internal.h"

namespace entro {

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

struct Plan {
  uint32_t K = 0;
  uint32_t entries = 0;
  uint32_t codes[256] = {};
  uint32_t max_used = 0;
};

// Validate a codebook and compute its canonical codes and table size.
static entro_status plan_lut(const entro_codebook *cb, Plan *p) {
  if (!cb || !cb->code_len) return ENTRO_E_INVAL;
  if (cb->sym_bits != 4 && cb->sym_bits != 8) return ENTRO_E_FORMAT;
  if (cb->max_len < 1 || cb->max_len > kMaxCodeLen) return ENTRO_E_FORMAT;
  const uint32_t nsym = 1u << cb->sym_bits;
  uint32_t count[kMaxCodeLen + 1] = {};
  uint32_t used = 0;
  for (uint32_t s = 0; s < nsym; ++s) {
    uint32_t l = cb->code_len[s];
    if (l > cb->max_len) return ENTRO_E_CODEBOOK;
    if (l) {
      count[l]++;
      used++;
      if (l > p->max_used) p->max_used = l;
    }
  }
  if (!used) return ENTRO_E_CODEBOOK;
  // Kraft sum <= 1, in units of 2^-16 (exact).
  uint64_t kraft = 0;
  for (uint32_t l = 1; l <= kMaxCodeLen; ++l) kraft += (uint64_t)count[l] << (kMaxCodeLen - l);
  if (kraft > (1ull << kMaxCodeLen)) return ENTRO_E_CODEBOOK;
  // canonical codes: first code of each length, then symbols in order
  uint32_t next[kMaxCodeLen + 2] = {};
  uint32_t code = 0;
  for (uint32_t l = 1; l <= kMaxCodeLen; ++l) {
    code = (code + count[l - 1]) << 1;
    next[l] = code;
  }
  for (uint32_t s = 0; s < nsym; ++s)
    if (cb->code_len[s]) p->codes[s] = next[cb->code_len[s]]++;
  // First-level width: the smallest k >= kFirstLevelMin whose longer codes
  // have an estimated probability (sum of 2^-len, in units of 2^-16) of at
  // most 2^-10; never wider than the longest code, nor than 12 bits (11 when
  // longer codes need second-level room).
  const uint32_t kmax = p->max_used <= kSingleLevelMax ? p->max_used : kFirstLevelBits;
  uint32_t K = kmax;
  for (uint32_t k = std::min(kFirstLevelMin, kmax); k < kmax; ++k) {
    uint64_t mass = 0;
    for (uint32_t l = k + 1; l <= kMaxCodeLen; ++l) mass += (uint64_t)count[l] << (kMaxCodeLen - l);
    if (mass <= (1ull << (kMaxCodeLen - 10))) {
      K = k;
      break;
    }
  }
  // widen until the two levels fit the table size
  for (;; ++K) {
    uint32_t entries = 1u << K;
    if (p->max_used > K) {
      // one subtable per K-bit prefix shared by codes longer than K
      std::vector<uint32_t> deepest(1u << K, 0);
      for (uint32_t s = 0; s < nsym; ++s) {
        uint32_t l = cb->code_len[s];
        if (l > K) {
          uint32_t pre = p->codes[s] >> (l - K);
          if (l > deepest[pre]) deepest[pre] = l;
        }
      }
      for (uint32_t pre = 0; pre < (1u << K); ++pre)
        if (deepest[pre]) entries += 1u << (deepest[pre] - K);
    }
    if (entries <= kLutMaxEntries) {
      p->K = K;
      p->entries = entries;
      return ENTRO_OK;
    }
    if (K >= kmax) return ENTRO_E_UNSUPPORTED;
  }
}

}  // namespace entro

using namespace entro;

extern "C" size_t entro_lut_bytes(const entro_codebook *cb) {
  Plan p;
  if (plan_lut(cb, &p) != ENTRO_OK) return 0;
  return sizeof(uint32_t) * (kLutHeaderWords + p.entries);
}

extern "C" entro_status entro_lut_build(const entro_codebook *cb, void *host_lut, size_t cap) {
  Plan p;
  entro_status st = plan_lut(cb, &p);
  if (st != ENTRO_OK) return st;
  if (!host_lut || ((uintptr_t)host_lut & 3u)) return ENTRO_E_INVAL;
  const size_t bytes = sizeof(uint32_t) * (kLutHeaderWords + p.entries);
  if (cap < bytes) return ENTRO_E_INVAL;
  uint32_t *out = (uint32_t *)host_lut;
  std::memset(out, 0, bytes);
  out[0] = kLutMagic;
  uint32_t l_min = 0;
  for (uint32_t s = 0; s < (1u << cb->sym_bits); ++s)
    if (cb->code_len[s] && (l_min == 0 || cb->code_len[s] < l_min)) l_min = cb->code_len[s];
  out[1] = p.K | (cb->sym_bits << 8) | (cb->max_len << 16) | (l_min << 24);
  out[2] = p.entries;
  out[3] = 1u << p.K;
  uint32_t *e = out + kLutHeaderWords;
  const uint32_t nsym = 1u << cb->sym_bits;
  const uint32_t K = p.K;
  // value field of every code: bf16 of f32(scale) * f32(q - zp), one rounding each
  auto value = [&](uint32_t s) -> uint32_t {
    float v = (float)((int32_t)s - cb->zero_point);
    float prod = cb->scale * v;
    return (uint32_t)f32_to_bf16_rne(prod);
  };
  // subtable placement
  std::vector<uint32_t> deepest(1u << K, 0), base(1u << K, 0);
  for (uint32_t s = 0; s < nsym; ++s) {
    uint32_t l = cb->code_len[s];
    if (l > K) {
      uint32_t pre = p.codes[s] >> (l - K);
      if (l > deepest[pre]) deepest[pre] = l;
    }
  }
  uint32_t cursor = 1u << K;
  for (uint32_t pre = 0; pre < (1u << K); ++pre) {
    if (!deepest[pre]) continue;
    const uint32_t sb = deepest[pre] - K;
    base[pre] = cursor;
    e[pre] = kEntryPointer | (sb << 8) | (cursor << 16);
    cursor += 1u << sb;
  }
  for (uint32_t s = 0; s < nsym; ++s) {
    const uint32_t l = cb->code_len[s];
    if (!l) continue;
    const uint32_t entry = l | (s << 8) | (value(s) << 16);
    if (l <= K) {
      const uint32_t first = p.codes[s] << (K - l);
      for (uint32_t i = 0; i < (1u << (K - l)); ++i) e[first + i] = entry;
    } else {
      const uint32_t pre = p.codes[s] >> (l - K);
      const uint32_t sb = deepest[pre] - K;
      const uint32_t low = p.codes[s] & ((1u << (l - K)) - 1u);
      const uint32_t first = low << (sb - (l - K));
      for (uint32_t i = 0; i < (1u << (sb - (l - K))); ++i) e[base[pre] + first + i] = entry;
    }
  }
  return ENTRO_OK;
}

extern "C" const char *entro_status_str(entro_status s) {
  switch (s) {
    case ENTRO_OK: return "ok";
    case ENTRO_E_INVAL: return "invalid argument";
    case ENTRO_E_CODEBOOK: return "invalid codebook";
    case ENTRO_E_FORMAT: return "stream layout parameters out of range";
    case ENTRO_E_UNSUPPORTED: return "unsupported configuration";
    case ENTRO_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

// ---------------------------------------------------------------------------
// Two-code table for the fused GEMV of 4-bit tensors, built on the host from
// a decode table: entry i (the next kPairBitsWide stream bits, MSB first)
// holds the bf16 values of the two codewords those bits begin with (first
// word: A | B << 16), and in the second word their summed length in byte 1
// and the alignbit shift 32 - length in bits [4:0]; where the two codewords
// do not both lie within the index bits, or the bits begin no codeword, the
// entry is {0, kPairFallback | 0xFF00}.  The lookups follow the decode table
// exactly as the kernels do (first level by the top K bits, pointer entries
// to the subtable of the next bits).
// ---------------------------------------------------------------------------

namespace entro {

static uint32_t raw_lookup(const uint32_t *ent, uint32_t n_ent, uint32_t K, uint32_t hi) {
  uint32_t e = ent[hi >> (32u - K)];
  if (e & kEntryPointer) {
    const uint32_t sb = (e >> 8) & 31u;
    const uint32_t i2 = sb ? (hi << K) >> (32u - sb) : 0u;
    const uint32_t j = (e >> 16) + i2;
    e = j < n_ent ? ent[j] : 0u;
    if (e & kEntryPointer) e = 0u;   // two levels at most
  }
  return e;
}

}  // namespace entro

extern "C" size_t entro_pair_lut_bytes(void) {
  return sizeof(uint32_t) * (kPairLutHeaderWords + (2u << kPairBitsWide));
}

extern "C" entro_status entro_pair_lut_build(const void *host_lut, size_t lut_bytes, void *host_out, size_t cap) {
  if (!host_lut || !host_out || ((uintptr_t)host_lut & 3u) || ((uintptr_t)host_out & 3u)) return ENTRO_E_INVAL;
  if (cap < entro_pair_lut_bytes() || lut_bytes < sizeof(uint32_t) * kLutHeaderWords) return ENTRO_E_INVAL;
  const uint32_t *h = static_cast<const uint32_t *>(host_lut);
  const uint32_t K = h[1] & 0xFFu, sym_bits = (h[1] >> 8) & 0xFFu, n_ent = h[2];
  if (h[0] != kLutMagic || K < 1 || K > kSingleLevelMax || h[3] != (1u << K) || n_ent < h[3] ||
      n_ent > kLutMaxEntries || (uint64_t)n_ent + kLutHeaderWords > lut_bytes / 4)
    return ENTRO_E_INVAL;
  if (sym_bits != 4) return ENTRO_E_UNSUPPORTED;
  const uint32_t *ent = h + kLutHeaderWords;
  uint32_t *out = static_cast<uint32_t *>(host_out);
  uint32_t *pe = out + kPairLutHeaderWords;
  bool whole = true;
  for (uint32_t i = 0; i < (1u << kPairBitsWide); ++i) {
    const uint32_t hi = i << (32u - kPairBitsWide);
    uint32_t x = 0u, y = kPairFallback | 0xFF00u;
    const uint32_t eA = raw_lookup(ent, n_ent, K, hi);
    const uint32_t lA = eA & 31u;
    if (lA && lA <= kPairBitsWide) {
      const uint32_t eB = raw_lookup(ent, n_ent, K, hi << lA);
      const uint32_t lB = eB & 31u;
      if (lB && lA + lB <= kPairBitsWide) {
        const uint32_t lab = lA + lB;
        x = (eA >> 16) | (eB & 0xFFFF0000u);
        y = (lab << 8) | ((32u - lab) & 31u);
      }
    }
    whole &= (y & kPairFallback) == 0u;
    pe[2u * i] = x;
    pe[2u * i + 1u] = y;
  }
  out[0] = kPairLutMagic;
  out[1] = whole ? kPairLutWhole : 0u;
  out[2] = h[1];
  out[3] = 0u;
  return ENTRO_OK;
}
