// Host side of the interleaved rANS variant (ECR v1, layout in entro_rans.h):
// frequency scaling, the slot table, and the encoder.  The encoder runs each
// chunk backwards (steps from last to first, lanes from last to first), so
// that the renormalization units, reversed, come out in the order a lockstep
// decoder takes them.
#include <algorithm>
#include <cstring>
#include <thread>
#include <vector>

#include "entro_rans.h"

namespace {

constexpr uint32_t kM = 1u << ENTRO_RANS_M_BITS;
constexpr uint32_t kL = 1u << 16;
constexpr uint32_t kMagic = 0x31524345u;   // "ECR1", little-endian
constexpr size_t kHeaderBytes = 16;

uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

bool freqs_ok(const uint32_t *freqs, uint32_t alphabet) {
  uint64_t s = 0;
  for (uint32_t i = 0; i < alphabet; ++i) s += freqs[i];
  return s == kM;
}

// Run body(begin, end) over [0, n) in up to `threads` contiguous ranges.
template <typename F>
void parallel_ranges(uint64_t n, uint32_t threads, F body) {
  uint32_t hw = std::max(1u, std::thread::hardware_concurrency());
  uint32_t t = threads ? threads : hw;
  t = (uint32_t)std::min<uint64_t>(std::max(1u, t), std::max<uint64_t>(1, n));
  if (t <= 1) {
    body(0, n);
    return;
  }
  std::vector<std::thread> pool;
  for (uint32_t i = 0; i < t; ++i) pool.emplace_back(body, n * i / t, n * (i + 1) / t);
  for (auto &th : pool) th.join();
}

}  // namespace

extern "C" entro_status entro_rans_freqs(const uint64_t *counts, uint32_t alphabet, uint32_t *freqs) {
  if (!counts || !freqs || alphabet < 1 || alphabet > 256) return ENTRO_E_INVAL;
  unsigned __int128 n = 0;
  uint32_t present = 0;
  for (uint32_t s = 0; s < alphabet; ++s) {
    n += counts[s];
    present += counts[s] ? 1u : 0u;
  }
  if (n == 0) return ENTRO_E_INVAL;
  if (present > kM) return ENTRO_E_CODEBOOK;
  uint64_t total = 0;
  for (uint32_t s = 0; s < alphabet; ++s) {
    if (!counts[s]) {
      freqs[s] = 0;
      continue;
    }
    const unsigned __int128 f = ((unsigned __int128)kM * counts[s]) / n;
    freqs[s] = (uint32_t)std::max<unsigned __int128>(1, f);
    total += freqs[s];
  }
  // shortfall of s: M c / N - f, compared exactly as M c - f N
  while (total < kM) {
    uint32_t best = alphabet;
    __int128 best_v = 0;
    for (uint32_t s = 0; s < alphabet; ++s) {
      if (!counts[s]) continue;
      const __int128 v = (__int128)kM * counts[s] - (__int128)freqs[s] * (__int128)n;
      if (best == alphabet || v > best_v) best = s, best_v = v;
    }
    ++freqs[best];
    ++total;
  }
  while (total > kM) {
    uint32_t best = alphabet;
    for (uint32_t s = 0; s < alphabet; ++s)
      if (counts[s] && freqs[s] > 1 && (best == alphabet || freqs[s] > freqs[best])) best = s;
    --freqs[best];
    --total;
  }
  return ENTRO_OK;
}

extern "C" size_t entro_rans_table_bytes(void) { return kHeaderBytes + (size_t)kM * 8u; }

extern "C" entro_status entro_rans_table_build(uint32_t sym_bits, const uint32_t *freqs, float scale,
                                               int32_t zero_point, void *host_table, size_t cap) {
  if (!freqs || !host_table || cap < entro_rans_table_bytes()) return ENTRO_E_INVAL;
  if (sym_bits != 4 && sym_bits != 8) return ENTRO_E_FORMAT;
  const uint32_t a = 1u << sym_bits;
  if (!freqs_ok(freqs, a)) return ENTRO_E_CODEBOOK;
  uint32_t *w = static_cast<uint32_t *>(host_table);
  w[0] = kMagic;
  w[1] = sym_bits | (ENTRO_RANS_M_BITS << 8);
  w[2] = kM;
  w[3] = 0;
  uint32_t slot = 0;
  for (uint32_t s = 0; s < a; ++s) {
    const float prod = scale * (float)((int32_t)s - zero_point);
    const uint32_t bf = f32_to_bf16_rne(prod);
    for (uint32_t k = 0; k < freqs[s]; ++k, ++slot) {
      w[4 + 2 * slot] = (bf << 16) | s;
      w[4 + 2 * slot + 1] = freqs[s] | (k << 16);
    }
  }
  return ENTRO_OK;
}

extern "C" entro_status entro_rans_encode(const uint8_t *q, uint64_t n, const uint32_t *freqs, uint32_t sym_bits,
                                          uint32_t chunk, uint32_t lanes, uint64_t *chunk_unit_off, uint16_t *units,
                                          uint64_t cap_units, uint64_t *n_units, uint32_t threads) {
  if ((!q && n) || !freqs || !chunk_unit_off || !n_units) return ENTRO_E_INVAL;
  if (sym_bits != 4 && sym_bits != 8) return ENTRO_E_FORMAT;
  if (lanes < 1 || lanes > 64 || (lanes & (lanes - 1)) || chunk == 0 || chunk % lanes) return ENTRO_E_FORMAT;
  const uint32_t a = 1u << sym_bits;
  if (!freqs_ok(freqs, a)) return ENTRO_E_CODEBOOK;
  for (uint64_t i = 0; i < n; ++i)
    if (q[i] >= a || freqs[q[i]] == 0) return ENTRO_E_CODEBOOK;
  uint32_t cum[257];
  cum[0] = 0;
  for (uint32_t s = 0; s < a; ++s) cum[s + 1] = cum[s] + freqs[s];
  const uint64_t nc = (n + chunk - 1) / chunk;
  std::vector<std::vector<uint16_t>> per(nc);
  parallel_ranges(nc, threads, [&](uint64_t c0, uint64_t c1) {
    std::vector<uint32_t> x(lanes);
    std::vector<uint16_t> rev;
    for (uint64_t c = c0; c < c1; ++c) {
      const uint64_t base = c * chunk;
      const uint32_t cc = (uint32_t)std::min<uint64_t>(chunk, n - base);
      const uint32_t steps = (cc + lanes - 1) / lanes;
      std::fill(x.begin(), x.end(), kL);
      rev.clear();
      for (uint32_t t = steps; t-- > 0;) {
        for (uint32_t j = lanes; j-- > 0;) {
          const uint32_t k = t * lanes + j;
          if (k >= cc) continue;
          const uint32_t s = q[base + k];
          const uint32_t f = freqs[s];
          uint32_t v = x[j];
          if ((uint64_t)v >= ((uint64_t)f << 20)) {
            rev.push_back((uint16_t)(v & 0xFFFFu));
            v >>= 16;
          }
          x[j] = (v / f) * kM + (v % f) + cum[s];
        }
      }
      std::vector<uint16_t> &out = per[c];
      out.reserve(2u * lanes + rev.size());
      for (uint32_t j = 0; j < lanes; ++j) {
        out.push_back((uint16_t)(x[j] & 0xFFFFu));
        out.push_back((uint16_t)(x[j] >> 16));
      }
      out.insert(out.end(), rev.rbegin(), rev.rend());
    }
  });
  uint64_t total = 0;
  for (uint64_t c = 0; c < nc; ++c) {
    chunk_unit_off[c] = total;
    total += per[c].size();
  }
  chunk_unit_off[nc] = total;
  *n_units = total;
  if (units) {
    if (cap_units < total) return ENTRO_E_INVAL;
    uint64_t p = 0;
    for (uint64_t c = 0; c < nc; ++c) {
      std::copy(per[c].begin(), per[c].end(), units + p);
      p += per[c].size();
    }
  }
  return ENTRO_OK;
}
