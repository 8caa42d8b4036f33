// Offline encoder of the library (host only): tensor-level quantization,
// optimal length-limited code lengths, ECW v1 stream writer.  See
// include/entro_encode.h for the contract and the pages it follows.
#include "entro_encode.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

namespace {

constexpr uint32_t kMaxLen = 16;

uint32_t pick_threads(uint32_t threads, uint64_t work_items) {
  uint32_t hw = std::max(1u, std::thread::hardware_concurrency());
  uint32_t t = threads ? threads : hw;
  if (work_items < t) t = (uint32_t)std::max<uint64_t>(1, work_items);
  return t;
}

// Run body(begin, end) over [0, n) split into `threads` contiguous ranges.
template <class F>
void parallel_ranges(uint64_t n, uint32_t threads, F body) {
  if (threads <= 1 || n < 2) {
    body(0, n);
    return;
  }
  std::vector<std::thread> pool;
  for (uint32_t i = 0; i < threads; ++i) {
    const uint64_t b = n * i / threads, e = n * (i + 1) / threads;
    pool.emplace_back([=] { body(b, e); });
  }
  for (auto &th : pool) th.join();
}

double code_entropy(const uint64_t *hist, uint32_t nsym, uint64_t n) {
  double h = 0.0;
  for (uint32_t s = 0; s < nsym; ++s) {
    if (!hist[s]) continue;
    const double p = (double)hist[s] / (double)n;
    h -= p * std::log2(p);
  }
  return h;
}

struct QuantResult {
  float scale;
  int32_t zp;
};

// q = clamp(rint(w / s) + zp, 0, Q) in float64, s already rounded to float32
void quantize_with(const float *w, uint64_t n, double s, int32_t zp, uint32_t Q, uint8_t *q,
                   uint64_t *hist, uint32_t threads) {
  const uint32_t nsym = Q + 1;
  std::vector<std::vector<uint64_t>> part(threads, std::vector<uint64_t>(nsym, 0));
  std::atomic<uint32_t> slot{0};
  parallel_ranges(n, threads, [&](uint64_t b, uint64_t e) {
    std::vector<uint64_t> &h = part[slot.fetch_add(1)];
    for (uint64_t i = b; i < e; ++i) {
      double v = std::nearbyint((double)w[i] / s) + (double)zp;
      v = v < 0.0 ? 0.0 : (v > (double)Q ? (double)Q : v);
      const uint8_t c = (uint8_t)v;
      q[i] = c;
      h[c]++;
    }
  });
  std::fill(hist, hist + nsym, 0);
  for (auto &h : part)
    for (uint32_t s2 = 0; s2 < nsym; ++s2) hist[s2] += h[s2];
}

}  // namespace

extern "C" entro_status entro_quantize(const float *w, uint64_t n, uint32_t bits, entro_qscheme scheme,
                                       float clip, uint8_t *q_out, float *scale_out, int32_t *zero_point_out,
                                       entro_qscheme *chosen) {
  if (!w || !q_out || !scale_out || !zero_point_out || n == 0) return ENTRO_E_INVAL;
  if (bits != 4 && bits != 8) return ENTRO_E_FORMAT;
  if (scheme != ENTRO_Q_ASYMMETRIC && scheme != ENTRO_Q_UNSIGNED && scheme != ENTRO_Q_MIXED) return ENTRO_E_FORMAT;
  const uint32_t Q = (1u << bits) - 1u;
  const int32_t half = 1 << (bits - 1);
  const uint32_t threads = pick_threads(0, n / (1u << 16));

  // range statistics
  std::vector<float> lo(threads, w[0]), hi(threads, w[0]), amax(threads, 0.f);
  std::atomic<uint32_t> slot{0};
  parallel_ranges(n, threads, [&](uint64_t b, uint64_t e) {
    const uint32_t k = slot.fetch_add(1);
    float l = w[b], h = w[b], a = 0.f;
    for (uint64_t i = b; i < e; ++i) {
      l = std::min(l, w[i]);
      h = std::max(h, w[i]);
      a = std::max(a, std::fabs(w[i]));
    }
    lo[k] = l;
    hi[k] = h;
    amax[k] = a;
  });
  const double wmin = *std::min_element(lo.begin(), lo.end());
  const double wmax = *std::max_element(hi.begin(), hi.end());
  const double wabs = *std::max_element(amax.begin(), amax.end());

  QuantResult asym{1.f, 0}, uns{1.f, half};
  if (wmax != wmin) {
    asym.scale = (float)((wmax - wmin) / (double)Q);
    double z = std::nearbyint(-wmin / (double)asym.scale);
    asym.zp = (int32_t)(z < 0.0 ? 0.0 : (z > (double)Q ? (double)Q : z));
  }
  const double m = clip > 0.f ? (double)clip : wabs;
  if (m != 0.0) uns.scale = (float)(m / (double)(half - 1));

  uint64_t hist[256];
  if (scheme == ENTRO_Q_ASYMMETRIC || scheme == ENTRO_Q_UNSIGNED) {
    const QuantResult &r = scheme == ENTRO_Q_ASYMMETRIC ? asym : uns;
    quantize_with(w, n, (double)r.scale, r.zp, Q, q_out, hist, threads);
    *scale_out = r.scale;
    *zero_point_out = r.zp;
    if (chosen) *chosen = scheme;
    return ENTRO_OK;
  }
  // mixed: unsigned first into a scratch copy, asymmetric into q_out
  std::vector<uint8_t> qu(n);
  uint64_t hu[256];
  quantize_with(w, n, (double)uns.scale, uns.zp, Q, qu.data(), hu, threads);
  quantize_with(w, n, (double)asym.scale, asym.zp, Q, q_out, hist, threads);
  const double ha = code_entropy(hist, Q + 1, n), hun = code_entropy(hu, Q + 1, n);
  if (hun < ha) {
    std::memcpy(q_out, qu.data(), n);
    *scale_out = uns.scale;
    *zero_point_out = uns.zp;
    if (chosen) *chosen = ENTRO_Q_UNSIGNED;
  } else {
    *scale_out = asym.scale;
    *zero_point_out = asym.zp;
    if (chosen) *chosen = ENTRO_Q_ASYMMETRIC;
  }
  return ENTRO_OK;
}

extern "C" entro_status entro_code_lengths(const uint8_t *q, uint64_t n, uint32_t bits, uint32_t max_len,
                                           uint8_t *code_len_out) {
  if (!q || !code_len_out || n == 0) return ENTRO_E_INVAL;
  if (bits != 4 && bits != 8) return ENTRO_E_FORMAT;
  if (max_len < 1 || max_len > kMaxLen) return ENTRO_E_FORMAT;
  const uint32_t nsym = 1u << bits;
  uint64_t hist[256] = {};
  for (uint64_t i = 0; i < n; ++i) {
    if (q[i] >= nsym) return ENTRO_E_INVAL;
    hist[q[i]]++;
  }
  std::memset(code_len_out, 0, nsym);
  // leaves ordered by (count, value)
  std::vector<uint32_t> leaf;
  for (uint32_t s = 0; s < nsym; ++s)
    if (hist[s]) leaf.push_back(s);
  std::stable_sort(leaf.begin(), leaf.end(), [&](uint32_t a, uint32_t b) { return hist[a] < hist[b]; });
  const uint32_t nl = (uint32_t)leaf.size();
  if (nl == 1) {
    code_len_out[leaf[0]] = 1;
    return ENTRO_OK;
  }
  if (max_len < 32 && (1ull << max_len) < nl) return ENTRO_E_CODEBOOK;
  // Package-merge.  Level max_len holds the leaves; every shallower level is
  // the leaves merged with packages (adjacent pairs) of the level below, the
  // leaf first when weights tie.  Items only record whether they are
  // packages: a selection of the first m items of a level uses its first
  // (m - packages) leaves and 2 * packages items of the level below.
  struct Item {
    uint64_t w;
    bool pkg;
  };
  std::vector<std::vector<Item>> lists(max_len + 1);
  for (uint32_t s : leaf) lists[max_len].push_back({hist[s], false});
  for (uint32_t lev = max_len - 1; lev >= 1; --lev) {
    const std::vector<Item> &deep = lists[lev + 1];
    std::vector<Item> &cur = lists[lev];
    size_t ip = 0, il = 0;
    const size_t npk = deep.size() / 2;
    while (il < nl || ip < npk) {
      const bool take_leaf =
          ip >= npk || (il < nl && hist[leaf[il]] <= deep[2 * ip].w + deep[2 * ip + 1].w);
      if (take_leaf) {
        cur.push_back({hist[leaf[il]], false});
        ++il;
      } else {
        cur.push_back({deep[2 * ip].w + deep[2 * ip + 1].w, true});
        ++ip;
      }
    }
    if (lev == 1) break;
  }
  std::vector<uint32_t> len(nl, 0);
  size_t m = 2 * (size_t)nl - 2;
  for (uint32_t lev = 1; lev <= max_len && m; ++lev) {
    const std::vector<Item> &cur = lists[lev];
    size_t leaves_used = 0, pk = 0;
    for (size_t i = 0; i < m && i < cur.size(); ++i) (cur[i].pkg ? pk : leaves_used)++;
    for (size_t i = 0; i < leaves_used; ++i) len[i]++;
    m = 2 * pk;
  }
  for (uint32_t i = 0; i < nl; ++i) code_len_out[leaf[i]] = (uint8_t)len[i];
  return ENTRO_OK;
}

namespace {

bool lanes_ok(uint32_t w) { return w >= 1 && w <= 64 && (w & (w - 1)) == 0; }

entro_status check_layout(const uint8_t *q, uint64_t n, const uint8_t *code_len, uint32_t bits, uint32_t chunk,
                          uint32_t lanes) {
  if ((!q && n) || !code_len) return ENTRO_E_INVAL;
  if (bits != 4 && bits != 8) return ENTRO_E_FORMAT;
  if (!lanes_ok(lanes) || chunk == 0 || chunk % lanes) return ENTRO_E_FORMAT;
  for (uint32_t s = 0; s < (1u << bits); ++s)
    if (code_len[s] > kMaxLen) return ENTRO_E_CODEBOOK;
  return ENTRO_OK;
}

}  // namespace

extern "C" entro_status entro_encode_layout(const uint8_t *q, uint64_t n, const uint8_t *code_len, uint32_t bits,
                                            uint32_t chunk, uint32_t lanes, uint64_t *chunk_bit_off,
                                            uint64_t *n_words) {
  entro_status st = check_layout(q, n, code_len, bits, chunk, lanes);
  if (st != ENTRO_OK) return st;
  if (!chunk_bit_off || !n_words) return ENTRO_E_INVAL;
  const uint64_t nc = (n + chunk - 1) / chunk;
  const uint32_t nsym = 1u << bits;
  std::vector<uint64_t> words(nc, 0);
  std::atomic<bool> bad{false};
  parallel_ranges(nc, pick_threads(0, nc / 64), [&](uint64_t c0, uint64_t c1) {
    uint64_t lane_bits[64];
    for (uint64_t c = c0; c < c1; ++c) {
      const uint64_t beg = c * chunk, cc = std::min<uint64_t>(chunk, n - beg);
      std::fill(lane_bits, lane_bits + lanes, 0);
      for (uint64_t k = 0; k < cc; ++k) {
        const uint8_t s = q[beg + k];
        if (s >= nsym || !code_len[s]) bad = true;
        lane_bits[k & (lanes - 1)] += code_len[s < nsym ? s : 0];
      }
      uint64_t wsum = 0;
      for (uint32_t j = 0; j < lanes; ++j) wsum += (lane_bits[j] + 31) / 32;
      words[c] = wsum;
    }
  });
  if (bad) return ENTRO_E_CODEBOOK;
  uint64_t acc = 0;
  chunk_bit_off[0] = 0;
  for (uint64_t c = 0; c < nc; ++c) {
    acc += words[c];
    chunk_bit_off[c + 1] = 32 * acc;
  }
  *n_words = acc;
  return ENTRO_OK;
}

extern "C" entro_status entro_encode(const uint8_t *q, uint64_t n, const uint8_t *code_len, uint32_t bits,
                                     uint32_t chunk, uint32_t lanes, uint32_t refill_steps, uint32_t refill_ahead,
                                     const uint64_t *chunk_bit_off, uint32_t *words, uint32_t threads) {
  entro_status st = check_layout(q, n, code_len, bits, chunk, lanes);
  if (st != ENTRO_OK) return st;
  if (refill_steps == 0) refill_steps = 1;
  if (refill_steps > 2 || refill_ahead > 1) return ENTRO_E_FORMAT;
  if (!chunk_bit_off || (!words && n)) return ENTRO_E_INVAL;
  const uint32_t nsym = 1u << bits;
  // canonical codewords
  uint32_t count[kMaxLen + 1] = {}, next[kMaxLen + 1] = {}, code[256] = {};
  for (uint32_t s = 0; s < nsym; ++s)
    if (code_len[s]) count[code_len[s]]++;
  uint32_t c = 0;
  for (uint32_t l = 1; l <= kMaxLen; ++l) {
    c = (c + count[l - 1]) << 1;
    next[l] = c;
  }
  for (uint32_t s = 0; s < nsym; ++s)
    if (code_len[s]) code[s] = next[code_len[s]]++;
  // refilling ahead: a lane is "early" while codes_left * l_min >= 32
  uint32_t l_min = 0;
  for (uint32_t s = 0; s < nsym; ++s)
    if (code_len[s] && (l_min == 0 || code_len[s] < l_min)) l_min = code_len[s];
  if (l_min == 0) l_min = 1;

  const uint64_t nc = (n + chunk - 1) / chunk;
  std::atomic<bool> bad{false};
  parallel_ranges(nc, pick_threads(threads, nc / 16), [&](uint64_t c0, uint64_t c1) {
    // Per lane: bit accumulator of the word being filled, its assigned slot,
    // the slot of the next word (assigned at the step that first needs it),
    // and the count of loaded, unconsumed bits the decoder will hold.
    uint64_t acc[64];
    uint32_t nacc[64], avail[64];
    uint64_t slot_cur[64], slot_next[64];
    bool has_cur[64], has_next[64];
    for (uint64_t ch = c0; ch < c1; ++ch) {
      const uint64_t beg = ch * chunk, cc = std::min<uint64_t>(chunk, n - beg);
      uint64_t out = chunk_bit_off[ch] / 32;
      const uint64_t end = chunk_bit_off[ch + 1] / 32;
      for (uint32_t j = 0; j < lanes; ++j) {
        acc[j] = 0;
        nacc[j] = 0;
        avail[j] = 0;
        has_cur[j] = has_next[j] = false;
      }
      const uint64_t steps = (cc + lanes - 1) / lanes;
      for (uint64_t k = 0; k < cc; ++k) {
        const uint32_t j = (uint32_t)(k & (lanes - 1));
        const uint64_t t = k / lanes;
        const uint8_t s = q[beg + k];
        const uint32_t l = s < nsym ? code_len[s] : 0;
        if (!l || out > end) {
          bad = true;
          return;
        }
        // bits the lane needs at this decision point (its codewords of the
        // next refill_steps steps), only at the first step of the group
        uint32_t need = 0;
        if (t % refill_steps == 0) {
          need = l;
          for (uint32_t d = 1; d < refill_steps && t + d < steps; ++d) {
            const uint64_t k2 = k + (uint64_t)d * lanes;
            if (k2 < cc) need += q[beg + k2] < nsym ? code_len[q[beg + k2]] : 0;
          }
        }
        bool take = false;
        if (t % refill_steps == 0) {
          const uint64_t codes_left = (cc - j + lanes - 1) / lanes - t;
          take = (refill_ahead && codes_left * l_min >= 32) ? avail[j] < 32u : need > avail[j];
        }
        if (take) {                  // the decoder takes the next word here
          if (has_next[j]) {         // (never: a lane holds under 64 loaded bits)
            bad = true;
            return;
          }
          if (!has_cur[j]) {
            slot_cur[j] = out++;
            has_cur[j] = true;
          } else {
            slot_next[j] = out++;
            has_next[j] = true;
          }
          avail[j] += 32;
        }
        avail[j] -= l;   // (the group's later codewords find avail already covering them)
        acc[j] = (acc[j] << l) | code[s];
        nacc[j] += l;
        if (nacc[j] >= 32) {
          nacc[j] -= 32;
          words[slot_cur[j]] = (uint32_t)(acc[j] >> nacc[j]);
          acc[j] &= (nacc[j] ? ((1ull << nacc[j]) - 1ull) : 0ull);
          slot_cur[j] = slot_next[j];
          has_cur[j] = has_next[j];
          has_next[j] = false;
        }
      }
      for (uint32_t j = 0; j < lanes; ++j)
        if (nacc[j]) words[slot_cur[j]] = (uint32_t)(acc[j] << (32 - nacc[j]));
      if (out != end) {
        bad = true;
        return;
      }
    }
  });
  return bad ? ENTRO_E_CODEBOOK : ENTRO_OK;
}
