// HIP kernels (gfx950) and the device entry points of the C ABI:
// entro_decode, entro_decode_dequant, entro_decode_gemv.
//
// Method: EntroLLM splits Huffman-coded weights into independent chunks that
// are decoded in parallel (gist.science technical summary, Methodology
// item 3); LazyWeights codes them in interleaved lanes and decodes them on
// demand so that only coded bytes cross the memory bus (abstract).  Here one
// wavefront (64 lanes) decodes 64 / W chunks of W lanes each, in lockstep:
//
//   per step t, every active lane
//     1. looks up the next K bits of its 64-bit bit buffer in the LDS table
//        (second level for long codes);
//     2. needs a word iff that codeword is longer than its loaded bits (an
//        entry without codeword counts as "longer" while fewer than 16 bits
//        are loaded);
//     3. the lanes needing a word take consecutive words of their chunk,
//        word index = chunk word pointer + number of lower lanes of the same
//        chunk needing one (a prefix count over the wave's ballot mask);
//     4. after a refill the lookup is repeated; the codeword is consumed and
//        the result emitted (code byte, bf16 value, or an FMA into the GEMV
//        accumulators).
//
// Writes of one step are contiguous: lane j of a chunk emits symbol t*W + j.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "entro.h"
#include "entro_internal.h"

namespace entro {

__device__ __forceinline__ uint32_t lut_lookup(const uint32_t *lut, uint32_t hi, uint32_t K) {
  uint32_t e = lut[hi >> (32u - K)];
  if (e & kEntryPointer) {
    const uint32_t sb = (e >> 8) & 31u;
    const uint32_t i2 = (hi << K) >> (32u - sb);
    e = lut[((e >> 16) + i2) & (kLutMaxEntries - 1u)];
  }
  return e;
}

template <int MODE, int LOG2W, int BATCH>
__global__ __launch_bounds__(kBlockThreads) void ecw_decode_kernel(const LaunchArgs a) {
  __shared__ uint32_t lut[kLutMaxEntries];
  constexpr uint32_t W = 1u << LOG2W;
  constexpr uint32_t G = 64u / W;   // chunks per wavefront

  // tensor of this block (uniform scan over at most 32 entries)
  const uint32_t b = blockIdx.x;
  uint32_t ti = 0;
  while (ti + 1 < a.n_tensors && a.block_begin[ti + 1] <= b) ++ti;
  const TensorArg &d = a.t[ti];
  const uint32_t blk = b - a.block_begin[ti];

  // table header
  if (d.lut_words < kLutHeaderWords) {
    if (threadIdx.x == 0) atomicOr(d.status, kFLut);
    return;
  }
  const uint32_t h0 = d.lut[0], h1 = d.lut[1], n_entries = d.lut[2], l1 = d.lut[3];
  const uint32_t K = h1 & 0xFFu;
  const bool lut_ok = h0 == kLutMagic && (h1 & 0xFFFFFF00u) == d.expect_hdr && K >= 1 &&
                      K <= kSingleLevelMax && l1 == (1u << K) && n_entries >= l1 &&
                      n_entries <= kLutMaxEntries && n_entries <= d.lut_words - kLutHeaderWords;
  if (!lut_ok) {
    if (threadIdx.x == 0) atomicOr(d.status, kFLut);
    return;
  }
  for (uint32_t i = threadIdx.x; i < n_entries; i += kBlockThreads) lut[i] = d.lut[kLutHeaderWords + i];
  __syncthreads();

  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = threadIdx.x >> 6;
  const uint32_t grp = lane >> LOG2W;
  const uint32_t j = lane & (W - 1u);
  const uint64_t grp_mask = (W == 64u) ? ~0ull : (((1ull << W) - 1ull) << (grp * W));
  const uint64_t grp_below = grp_mask & ((1ull << lane) - 1ull);

  const uint64_t task = (uint64_t)blk * kWavesPerBlock + wave;
  const uint64_t c = task * G + grp;
  uint32_t flags = 0;
  bool chunk_ok = c < d.n_chunks;
  uint64_t wb = 0, nw = 0;
  uint32_t cc = 0;
  if (chunk_ok) {
    const uint64_t o0 = d.offs[c], o1 = d.offs[c + 1];
    if ((o0 & 31u) || (o1 & 31u) || o1 < o0 || (o1 >> 5) > d.n_words) {
      flags |= kFOffsets;
      chunk_ok = false;
    } else {
      wb = o0 >> 5;
      nw = (o1 - o0) >> 5;
      const uint64_t first = c * d.chunk;
      cc = (uint32_t)min((uint64_t)d.chunk, d.n_symbols - first);
    }
  }
  const uint32_t my_steps = (chunk_ok && j < cc) ? ((cc - j + W - 1u) >> LOG2W) : 0u;
  const uint32_t steps = d.chunk >> LOG2W;
  const uint64_t sym0 = c * d.chunk;   // first symbol of this lane's chunk

  uint64_t buf = 0;      // loaded, unconsumed bits, first bit at bit 63
  uint32_t n = 0;        // number of such bits
  uint64_t P = 0;        // words of the chunk taken so far (same in all lanes of a chunk)

  float acc[BATCH];
#pragma unroll
  for (int i = 0; i < BATCH; ++i) acc[i] = 0.f;
  uint32_t col = j;
  uint64_t row = 0;
  if (MODE == kModeGemv) row = sym0 / d.cols;

  for (uint32_t t = 0; t < steps; ++t) {
    const bool act = t < my_steps;
    uint32_t e = lut_lookup(lut, (uint32_t)(buf >> 32), K);
    uint32_t len = e & 31u;
    const bool need = act && (len > n || (len == 0u && n < kMaxCodeLen));
    const uint64_t m = __ballot(need);
    if (m) {
      if (need) {
        const uint64_t idx = P + (uint64_t)__popcll(m & grp_below);
        uint32_t w = 0;
        if (idx < nw) w = d.words[wb + idx];
        else flags |= kFOverrun;
        buf |= (uint64_t)w << (32u - n);
        n += 32u;
        e = lut_lookup(lut, (uint32_t)(buf >> 32), K);
        len = e & 31u;
      }
      P += (uint64_t)__popcll(m & grp_mask);
    }
    if (act) {
      if (len == 0u) {
        flags |= kFBadCode;
        len = 1u;
      }
      buf <<= len;
      n -= len;
      const uint64_t k = sym0 + ((uint64_t)t << LOG2W) + j;
      if (MODE == kModeU8) {
        static_cast<uint8_t *>(d.out)[k] = (uint8_t)(e >> 8);
      } else if (MODE == kModeBf16) {
        static_cast<uint16_t *>(d.out)[k] = (uint16_t)(e >> 16);
      } else {
        const float v = __uint_as_float(e & 0xFFFF0000u);
#pragma unroll
        for (int bi = 0; bi < BATCH; ++bi) {
          if (bi < (int)a.batch) {
            const float xv = __uint_as_float((uint32_t)d.x[(uint64_t)bi * d.cols + col] << 16);
            acc[bi] = fmaf(v, xv, acc[bi]);
          }
        }
      }
    }
    if (MODE == kModeGemv) {
      col += W;
      if (col >= d.cols) {   // uniform: every chunk starts a row and W divides cols
        col -= d.cols;
#pragma unroll
        for (int bi = 0; bi < BATCH; ++bi) {
          float v = acc[bi];
#pragma unroll
          for (uint32_t off = W >> 1; off >= 1u; off >>= 1) v += __shfl_xor(v, (int)off, 64);
          if (act && j == 0u && bi < (int)a.batch) static_cast<float *>(d.out)[(uint64_t)bi * d.rows + row] = v;
          acc[bi] = 0.f;
        }
        ++row;
      }
    }
  }
  if (chunk_ok) {
    if (P < nw) flags |= kFUnderrun;
    if (buf != 0) flags |= kFPadding;
  }
  if (flags) atomicOr(d.status, flags);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static bool pow2_lanes(uint32_t w) { return w >= 1 && w <= 64 && (w & (w - 1)) == 0; }

static uint32_t log2u(uint32_t w) {
  uint32_t l = 0;
  while ((1u << l) < w) ++l;
  return l;
}

static entro_status check_tensor(const entro_tensor &t) {
  if (!pow2_lanes(t.lanes)) return ENTRO_E_FORMAT;
  if (t.chunk_symbols == 0 || t.chunk_symbols % t.lanes || t.chunk_symbols > kMaxChunk) return ENTRO_E_FORMAT;
  if (t.sym_bits != 4 && t.sym_bits != 8) return ENTRO_E_FORMAT;
  if (t.max_len < 1 || t.max_len > kMaxCodeLen) return ENTRO_E_FORMAT;
  if (t.n_symbols == 0) return ENTRO_OK;
  if (!t.d_lut || !t.d_words || !t.d_chunk_bit_off) return ENTRO_E_INVAL;
  const uint64_t nc = (t.n_symbols + t.chunk_symbols - 1) / t.chunk_symbols;
  if (nc > 0xFFFFFFFFull) return ENTRO_E_UNSUPPORTED;
  return ENTRO_OK;
}

template <int MODE, int BATCH>
static void launch_w(uint32_t log2w, uint32_t blocks, const LaunchArgs &a, hipStream_t s) {
  switch (log2w) {
#define ENTRO_CASE(L) \
  case L: hipLaunchKernelGGL((ecw_decode_kernel<MODE, L, BATCH>), dim3(blocks), dim3(kBlockThreads), 0, s, a); break;
    ENTRO_CASE(0) ENTRO_CASE(1) ENTRO_CASE(2) ENTRO_CASE(3) ENTRO_CASE(4) ENTRO_CASE(5) ENTRO_CASE(6)
#undef ENTRO_CASE
  }
}

// Validate everything, then enqueue launches of up to 32 tensors that share
// a lane count.
static entro_status run(int mode, const entro_tensor *t, size_t n, void *const *outs,
                        const entro_gemv_item *g, uint32_t batch, uint32_t *d_status, hipStream_t s) {
  if (n == 0) return ENTRO_OK;
  if (!t || !d_status) return ENTRO_E_INVAL;
  if (mode == kModeGemv) {
    if (!g || batch < 1 || batch > 8) return ENTRO_E_INVAL;
  } else if (!outs) {
    return ENTRO_E_INVAL;
  }
  for (size_t i = 0; i < n; ++i) {
    entro_status st = check_tensor(t[i]);
    if (st != ENTRO_OK) return st;
    if (mode == kModeGemv) {
      const entro_gemv_item &it = g[i];
      if ((uint64_t)it.rows * it.cols != t[i].n_symbols) return ENTRO_E_INVAL;
      if (t[i].n_symbols == 0) continue;
      if (!it.d_x || !it.d_y) return ENTRO_E_INVAL;
      if (it.cols % t[i].lanes || t[i].chunk_symbols % it.cols) return ENTRO_E_FORMAT;
    } else if (t[i].n_symbols && !outs[i]) {
      return ENTRO_E_INVAL;
    }
  }
  size_t i = 0;
  while (i < n) {
    LaunchArgs a;
    std::memset(&a, 0, sizeof a);
    a.batch = batch;
    uint32_t blocks = 0;
    uint32_t log2w = 0;
    uint32_t k = 0;
    for (; i < n && k < (uint32_t)kMaxTensorsPerLaunch; ++i) {
      const entro_tensor &x = t[i];
      if (x.n_symbols == 0) continue;
      const uint32_t lw = log2u(x.lanes);
      if (k == 0) log2w = lw;
      else if (lw != log2w) break;
      TensorArg &d = a.t[k];
      d.lut = static_cast<const uint32_t *>(x.d_lut);
      d.words = x.d_words;
      d.offs = x.d_chunk_bit_off;
      d.status = d_status + i;
      d.n_words = x.n_words;
      d.n_symbols = x.n_symbols;
      d.chunk = x.chunk_symbols;
      d.n_chunks = (uint32_t)((x.n_symbols + x.chunk_symbols - 1) / x.chunk_symbols);
      d.expect_hdr = (x.sym_bits << 8) | (x.max_len << 16);
      d.lut_words = (uint32_t)std::min<uint64_t>(x.lut_bytes / 4, kLutHeaderWords + kLutMaxEntries);
      if (mode == kModeGemv) {
        d.out = g[i].d_y;
        d.x = g[i].d_x;
        d.rows = g[i].rows;
        d.cols = g[i].cols;
      } else {
        d.out = outs[i];
      }
      const uint64_t chunks_per_wave = 64u >> lw;
      const uint64_t wave_tasks = (d.n_chunks + chunks_per_wave - 1) / chunks_per_wave;
      const uint64_t nb = (wave_tasks + kWavesPerBlock - 1) / kWavesPerBlock;
      if ((uint64_t)blocks + nb > 0x7FFFFFFFull) return ENTRO_E_UNSUPPORTED;
      a.block_begin[k] = blocks;
      blocks += (uint32_t)nb;
      ++k;
    }
    if (k == 0) continue;
    a.n_tensors = k;
    for (uint32_t r = k; r <= (uint32_t)kMaxTensorsPerLaunch; ++r) a.block_begin[r] = blocks;
    if (mode == kModeU8) launch_w<kModeU8, 1>(log2w, blocks, a, s);
    else if (mode == kModeBf16) launch_w<kModeBf16, 1>(log2w, blocks, a, s);
    else if (batch == 1) launch_w<kModeGemv, 1>(log2w, blocks, a, s);
    else launch_w<kModeGemv, 8>(log2w, blocks, a, s);
    if (hipGetLastError() != hipSuccess) return ENTRO_E_HIP;
  }
  return ENTRO_OK;
}

}  // namespace entro

using namespace entro;

extern "C" entro_status entro_decode(const entro_tensor *t, size_t n, uint8_t *const *d_out,
                                     uint32_t *d_status, hipStream_t stream) {
  return run(kModeU8, t, n, reinterpret_cast<void *const *>(d_out), nullptr, 1, d_status, stream);
}

extern "C" entro_status entro_decode_dequant(const entro_tensor *t, size_t n, uint16_t *const *d_out_bf16,
                                             uint32_t *d_status, hipStream_t stream) {
  return run(kModeBf16, t, n, reinterpret_cast<void *const *>(d_out_bf16), nullptr, 1, d_status, stream);
}

extern "C" entro_status entro_decode_gemv(const entro_tensor *t, size_t n, const entro_gemv_item *g,
                                          uint32_t batch, uint32_t *d_status, hipStream_t stream) {
  return run(kModeGemv, t, n, nullptr, g, batch, d_status, stream);
}
