/*
 * Plain C encoder and bit-serial decoder for the chunked, lane-interleaved
 * canonical-Huffman stream ("ECW v1").  TEST INFRASTRUCTURE ONLY: part of the
 * CPU oracle, used by the tests and by the benchmark's CPU baseline.  It
 * shares no code with the GPU library.
 *
 * What the pages fix: encoded weights are split into independent chunks that
 * keep the tensor's structure and are decoded concurrently (EntroLLM,
 * gist.science technical summary, Methodology item 3); codes are Huffman-coded
 * losslessly in interleaved lanes and decoded bit-exactly (LazyWeights
 * abstract, arXiv 2611.17108).  The layout is the reading spelled out in
 * oracle/ecw.py; this file implements the same steps without tables:
 *
 *   - canonical codes from lengths (codes of one length consecutive in symbol
 *     order, shorter codes first, first code zero; MSB-first);
 *   - lane j of a chunk holds symbols k = j (mod W); its codewords are cut
 *     into 32-bit words, first bit in bit 31, last word zero-padded;
 *   - refill decisions every D = refill_steps steps (1 or 2): at a step t with
 *     t mod D == 0 a lane takes its next word when its codewords of steps
 *     t .. t+D-1 are together longer than its count n of loaded, unconsumed
 *     bits; with `ahead`, a lane that still has R codes to go with
 *     R * l_min >= 32 (l_min: shortest code length) takes its next word
 *     exactly when n < 32 instead; words are stored in the order they are
 *     taken, lanes of one decision point in increasing lane index;
 *   - chunk_bit_off[c] = 32 * (words before chunk c), plus a final entry.
 *
 * The decoder reads one bit at a time and compares against the canonical
 * first code of each length; at a decision point a lane tries to read its
 * next D codewords from the bits it holds and, if it runs dry, takes the
 * chunk's next word and reads them again.  It never builds a lookup table.
 *
 * Plain C99, no intrinsics, no threads (callers run chunk ranges in parallel).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OC_OK 0
#define OC_E_PARAM 1
#define OC_E_CODEBOOK 2
#define OC_E_STREAM 3
#define OC_E_NOMEM 4
#define OC_MAXLEN 32

static int check_params(uint32_t chunk, uint32_t lanes, uint32_t refill_steps) {
  if (lanes < 1 || lanes > 64 || (lanes & (lanes - 1))) return OC_E_PARAM;
  if (chunk < 1 || chunk % lanes) return OC_E_PARAM;
  if (refill_steps != 1 && refill_steps != 2) return OC_E_PARAM;
  return OC_OK;
}

/* Canonical codes; returns max length or -1 on bad lengths. */
static int canonical(const uint8_t *len, uint32_t nsym, uint32_t *code) {
  uint32_t bl_count[OC_MAXLEN + 1], next[OC_MAXLEN + 1];
  int max_len = 0;
  uint32_t s, l, c;
  memset(bl_count, 0, sizeof bl_count);
  for (s = 0; s < nsym; s++) {
    if (len[s] > OC_MAXLEN) return -1;
    if (len[s]) bl_count[len[s]]++;
    if (len[s] > max_len) max_len = len[s];
  }
  c = 0;
  next[0] = 0;
  for (l = 1; l <= OC_MAXLEN; l++) {
    c = (c + (l >= 2 ? bl_count[l - 1] : 0)) << 1;
    next[l] = c;
  }
  for (s = 0; s < nsym; s++) {
    code[s] = 0;
    if (len[s]) code[s] = next[len[s]]++;
  }
  return max_len;
}

/* Shortest nonzero code length (1 if none). */
static uint32_t min_len(const uint8_t *len, uint32_t nsym) {
  uint32_t s, m = 0;
  for (s = 0; s < nsym; s++)
    if (len[s] && (m == 0 || len[s] < m)) m = len[s];
  return m ? m : 1;
}

/* Steps lane j of a chunk of cc codes has. */
static uint64_t lane_steps(uint64_t cc, uint32_t j, uint32_t lanes) {
  return cc > j ? (cc - j + lanes - 1) / lanes : 0;
}

/* Words of one chunk = sum over lanes of ceil(bits / 32). */
static uint64_t chunk_words(const uint8_t *q, uint64_t cc, const uint8_t *len, uint32_t lanes) {
  uint64_t total = 0, k;
  uint32_t j;
  for (j = 0; j < lanes; j++) {
    uint64_t bits = 0;
    for (k = j; k < cc; k += lanes) bits += len[q[k]];
    total += (bits + 31) / 32;
  }
  return total;
}

/* Number of words the whole stream takes; fills chunk_bit_off[0..n_chunks]. */
int oc_layout(const uint8_t *q, uint64_t n, const uint8_t *len, uint32_t nsym,
              uint32_t chunk, uint32_t lanes, uint64_t *chunk_bit_off, uint64_t *n_words) {
  uint64_t nc, c, acc = 0, i;
  if (check_params(chunk, lanes, 1)) return OC_E_PARAM;
  for (i = 0; i < n; i++)
    if (q[i] >= nsym || len[q[i]] == 0) return OC_E_CODEBOOK;
  nc = (n + chunk - 1) / chunk;
  chunk_bit_off[0] = 0;
  for (c = 0; c < nc; c++) {
    uint64_t beg = c * chunk, cc = n - beg < chunk ? n - beg : chunk;
    acc += chunk_words(q + beg, cc, len, lanes);
    chunk_bit_off[c + 1] = 32 * acc;
  }
  *n_words = acc;
  return OC_OK;
}

/* Encode chunks [c0, c1) into words; chunk_bit_off must come from oc_layout. */
int oc_encode(const uint8_t *q, uint64_t n, const uint8_t *len, uint32_t nsym,
              uint32_t chunk, uint32_t lanes, uint32_t refill_steps, uint32_t ahead,
              const uint64_t *chunk_bit_off, uint32_t *words, uint64_t c0, uint64_t c1) {
  uint32_t code[256];
  uint64_t c, k;
  uint32_t j;
  uint64_t lane_cap;
  uint32_t *lane_buf;
  uint64_t lane_n[64], taken[64];
  int32_t avail[64];
  uint32_t lmin;
  if (check_params(chunk, lanes, refill_steps) || nsym > 256) return OC_E_PARAM;
  if (canonical(len, nsym, code) < 0) return OC_E_CODEBOOK;
  lmin = min_len(len, nsym);
  /* per-lane word buffer: at most ceil(chunk/lanes) codewords of <= 32 bits */
  lane_cap = ((uint64_t)chunk / lanes) + 2;
  lane_buf = (uint32_t *)calloc((size_t)(lane_cap * lanes), sizeof(uint32_t));
  if (!lane_buf) return OC_E_NOMEM;
  for (c = c0; c < c1; c++) {
    uint64_t beg = c * chunk, cc = n - beg < chunk ? n - beg : chunk;
    uint64_t out = chunk_bit_off[c] / 32, steps;
    uint32_t t;
    /* 1. each lane's bit sequence, MSB-first, into its own word buffer */
    memset(lane_buf, 0, (size_t)(lane_cap * lanes) * sizeof(uint32_t));
    for (j = 0; j < lanes; j++) {
      uint64_t bitpos = 0;
      uint32_t *lw = lane_buf + (uint64_t)j * lane_cap;
      for (k = j; k < cc; k += lanes) {
        uint32_t s = q[beg + k], l = len[s], b;
        if (l == 0) { free(lane_buf); return OC_E_CODEBOOK; }
        for (b = 0; b < l; b++) {
          uint32_t bit = (code[s] >> (l - 1 - b)) & 1u;
          if (bit) lw[bitpos / 32] |= 1u << (31 - (bitpos % 32));
          bitpos++;
        }
      }
      lane_n[j] = (bitpos + 31) / 32;
      taken[j] = 0;
      avail[j] = 0;
    }
    /* 2. store the words in the order the lanes take them */
    steps = (cc + lanes - 1) / lanes;
    for (t = 0; t < steps; t += refill_steps) {
      for (j = 0; j < lanes; j++) {
        uint64_t kk = (uint64_t)t * lanes + j;
        int32_t l = 0;
        uint32_t d;
        if (kk >= cc) continue;
        int take;
        for (d = 0; d < refill_steps; d++)
          if (kk + (uint64_t)d * lanes < cc) l += len[q[beg + kk + (uint64_t)d * lanes]];
        if (ahead && (lane_steps(cc, j, lanes) - t) * lmin >= 32) take = avail[j] < 32;
        else take = l > avail[j];
        if (take) {
          if (taken[j] >= lane_n[j]) { free(lane_buf); return OC_E_STREAM; }
          words[out++] = lane_buf[(uint64_t)j * lane_cap + taken[j]++];
          avail[j] += 32;
        }
        avail[j] -= l;
      }
    }
    for (j = 0; j < lanes; j++)
      if (taken[j] != lane_n[j]) { free(lane_buf); return OC_E_STREAM; }
    if (out != chunk_bit_off[c + 1] / 32) { free(lane_buf); return OC_E_STREAM; }
  }
  free(lane_buf);
  return OC_OK;
}

/* Read the next `count` codewords from the `nbits` bits at the top of `buf`
 * (first bit = bit 63) one bit at a time.  Returns the bits used, 0 if the
 * bits end first, -1 if no codeword matches. */
static int read_codewords(uint64_t buf, int nbits, uint32_t count_, int max_len, const uint32_t *count,
                          const uint32_t *first, const uint32_t *offset, const uint8_t *sorted_syms,
                          uint8_t *syms) {
  int p = 0;
  uint32_t i, l, code;
  for (i = 0; i < count_; i++) {
    int found = 0;
    code = 0;
    for (l = 1; l <= (uint32_t)max_len; l++) {
      if (p >= nbits) return 0;
      code = (code << 1) | (uint32_t)((buf >> (63 - p)) & 1u);
      p++;
      if (code >= first[l] && code - first[l] < count[l]) {
        syms[i] = sorted_syms[offset[l] + code - first[l]];
        found = 1;
        break;
      }
    }
    if (!found) return -1;
  }
  return p;
}

/* Decode chunks [c0, c1) bit by bit into out[c*chunk ...]. */
int oc_decode(const uint32_t *words, uint64_t n_words, const uint64_t *chunk_bit_off,
              uint64_t n, const uint8_t *len, uint32_t nsym, uint32_t chunk, uint32_t lanes,
              uint32_t refill_steps, uint32_t ahead, uint8_t *out, uint64_t c0, uint64_t c1) {
  uint32_t count[OC_MAXLEN + 1], first[OC_MAXLEN + 1], offset[OC_MAXLEN + 1];
  uint8_t sorted_syms[256];
  uint64_t buf[64];      /* unconsumed bits of each lane, first bit at bit 63 */
  int32_t nb[64];        /* how many */
  int max_len = 0;
  uint32_t s, l, code, acc, j, lmin;
  uint64_t c;
  if (check_params(chunk, lanes, refill_steps) || nsym > 256) return OC_E_PARAM;
  lmin = min_len(len, nsym);
  memset(count, 0, sizeof count);
  for (s = 0; s < nsym; s++) {
    if (len[s] > OC_MAXLEN) return OC_E_CODEBOOK;
    if (len[s]) count[len[s]]++;
    if (len[s] > max_len) max_len = len[s];
  }
  code = 0;
  acc = 0;
  for (l = 1; l <= (uint32_t)max_len; l++) {
    code = (code + (l >= 2 ? count[l - 1] : 0)) << 1;
    first[l] = code;
    offset[l] = acc;
    acc += count[l];
  }
  acc = 0;
  for (l = 1; l <= (uint32_t)max_len; l++)
    for (s = 0; s < nsym; s++)
      if (len[s] == l) sorted_syms[acc++] = (uint8_t)s;
  /* one word must cover the codewords of a decision point */
  if ((int)refill_steps * max_len > 32) return OC_E_CODEBOOK;
  for (c = c0; c < c1; c++) {
    uint64_t beg = c * chunk, cc = n - beg < chunk ? n - beg : chunk;
    uint64_t pos = chunk_bit_off[c] / 32, end = chunk_bit_off[c + 1] / 32, t, steps;
    if (chunk_bit_off[c] % 32 || end < pos || end > n_words) return OC_E_STREAM;
    for (j = 0; j < lanes; j++) { buf[j] = 0; nb[j] = 0; }
    steps = (cc + lanes - 1) / lanes;
    for (t = 0; t < steps; t += refill_steps) {
      for (j = 0; j < lanes; j++) {
        uint64_t k = t * lanes + j;
        uint8_t syms[2];
        uint32_t cnt = 0, d;
        int used;
        if (k >= cc) continue;
        for (d = 0; d < refill_steps; d++)
          if (k + (uint64_t)d * lanes < cc) cnt++;
        if (ahead && (lane_steps(cc, j, lanes) - t) * lmin >= 32) {
          /* take a word whenever fewer than 32 bits are loaded, then read */
          if (nb[j] < 32) {
            if (pos >= end) return OC_E_STREAM;
            buf[j] |= (uint64_t)words[pos++] << (32 - nb[j]);
            nb[j] += 32;
          }
          used = read_codewords(buf[j], nb[j], cnt, max_len, count, first, offset, sorted_syms, syms);
          if (used <= 0) return OC_E_STREAM;
        } else {
          used = read_codewords(buf[j], nb[j], cnt, max_len, count, first, offset, sorted_syms, syms);
        }
        if (used == 0) {
          if (pos >= end || nb[j] > 32) return OC_E_STREAM;
          buf[j] |= (uint64_t)words[pos++] << (32 - nb[j]);
          nb[j] += 32;
          used = read_codewords(buf[j], nb[j], cnt, max_len, count, first, offset, sorted_syms, syms);
        }
        if (used <= 0) return OC_E_STREAM;
        for (d = 0; d < cnt; d++) out[beg + k + (uint64_t)d * lanes] = syms[d];
        buf[j] = used == 64 ? 0 : buf[j] << used;
        nb[j] -= used;
      }
    }
    if (pos != end) return OC_E_STREAM;
    for (j = 0; j < lanes; j++)
      if (buf[j]) return OC_E_STREAM;
  }
  return OC_OK;
}
