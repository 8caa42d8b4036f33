// HIP kernels (gfx950) and the device entry points of the C ABI:
// entro_decode, entro_decode_dequant, entro_decode_gemv.
//
// Method: EntroLLM splits Huffman-coded weights into independent chunks that
// are decoded in parallel (gist.science technical summary, Methodology
// item 3); LazyWeights codes them in interleaved lanes and decodes them on
// demand so that only coded bytes cross the memory bus (abstract).  Here one
// wavefront (64 lanes) decodes 64 / W chunks of W lanes each, in lockstep:
//
//   per step t, every lane
//     1. looks up the next K bits of its bit buffer in the table held in LDS
//        (a second level for codes longer than K);
//     2. needs a word iff that codeword is longer than its loaded bits (an
//        entry without codeword counts as longer than any loaded count below
//        31, so a partial peek into unused code space also fetches);
//     3. the lanes needing a word take consecutive words of their chunk: word
//        index = chunk word pointer + number of lower lanes of the same chunk
//        needing one, a prefix count over the wavefront's ballot mask
//        (v_mbcnt);
//     4. after a refill the lookup is repeated; the codeword is consumed and
//        the result emitted: code byte, bf16 value, or an FMA into the GEMV
//        accumulators.
//   Writes of one step are contiguous: lane j of a chunk emits code t*W + j.
//
// Two paths share that step:
//   * staged: the workgroup is persistent and walks block tasks; a wavefront
//     copies all words of its task (64/W consecutive chunks, contiguous in
//     memory) into its LDS area with 16-byte loads that write LDS directly,
//     then decodes from LDS.  The bit buffer is two 32-bit registers, left-aligned; refill and
//     consume are v_alignbit / shift / or; the loop keeps word pointers and
//     output addresses in scalar registers.
//   * generic: any task (ragged last chunk, words beyond the staging area,
//     malformed offsets): reads words straight from global memory with
//     bounds checks and reports every fault.
//
// Table entries as held in LDS (converted from the host table on staging):
//   [4:0] (32 - len) mod 32 (the v_alignbit shift that consumes the codeword)
//   [7]   second-level pointer ([12:8] subtable index bits, [31:16] base)
//   [15:8] len (1..16; 31 = no codeword)
//   [31:16] bf16 value (dequant / GEMV) or [23:16] code value (decode)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <type_traits>
#include <vector>

#include "entro.h"
#include "entro_device.h"
#include "entro_internal.h"

namespace entro {

// Word pointers into LDS are kept as 32-bit LDS byte addresses (scalar
// registers): lds_word reads word idx after address a, lds_adv advances a by
// c words with one s_lshl2_add_u32 (which also writes SCC, so SCC is
// declared clobbered).
__device__ __forceinline__ uint32_t lds_word(uint32_t a, uint32_t idx) {
  return *(lds_u32 *)(uintptr_t)(a + (idx << 2));
}

__device__ __forceinline__ uint32_t lds_adv(uint32_t a, uint32_t c) {
  uint32_t r;
  asm("s_lshl2_add_u32 %0, %1, %2" : "=s"(r) : "s"(__builtin_amdgcn_readfirstlane(c)),
      "s"(__builtin_amdgcn_readfirstlane(a)) : "scc");
  return r;
}

template <int MODE>
__device__ __forceinline__ uint32_t kernel_entry(uint32_t h) {
  if (h & kEntryPointer) return h;
  uint32_t len = h & 31u;
  if (len == 0u) len = kInvalidLen;
  const uint32_t val = (MODE == kModeU8) ? (((h >> 8) & 0xFFu) << 16) : (h & 0xFFFF0000u);
  return ((32u - len) & 31u) | (len << 8) | val;
}

__device__ __forceinline__ uint32_t entry_len(uint32_t e) { return (e >> 8) & 0xFFu; }

// Lanes whose codeword is longer than their loaded bits: one SDWA compare of
// the entry's length byte against n, written straight to a lane mask.
__device__ __forceinline__ uint64_t need_mask(uint32_t e, uint32_t n) {
  uint64_t m;
  asm volatile("v_cmp_gt_u32_sdwa %0, %1, %2 src0_sel:BYTE_1 src1_sel:DWORD" : "=s"(m) : "v"(e), "v"(n));
  return m;
}

// n - (length byte of e), one SDWA subtract
__device__ __forceinline__ uint32_t sub_len(uint32_t n, uint32_t e) {
  uint32_t r;
  asm("v_sub_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
      : "=v"(r) : "v"(n), "v"(e));
  return r;
}

// lanes whose two codewords (length bytes of a and b) are longer than n
__device__ __forceinline__ uint32_t pair_len(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:BYTE_1"
      : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ uint64_t gt_mask(uint32_t a, uint32_t n) {
  uint64_t m;
  asm volatile("v_cmp_gt_u32 %0, %1, %2" : "=s"(m) : "v"(a), "v"(n));
  return m;
}

// scalar & vector, kept as one v_and (not folded into a select)
__device__ __forceinline__ uint32_t and_sv(uint32_t s, uint32_t v) {
  uint32_t r;
  asm("v_and_b32 %0, %1, %2" : "=v"(r) : "s"(s), "v"(v));
  return r;
}

// Wavefront issue priority (0..3).  Among wavefronts of equal priority the
// sequencer serves the oldest first, so without this the last-dispatched
// wavefronts of a SIMD finish their (equal) share of the work long after the
// first ones and the CU idles at the end.  The decode loops lower a
// wavefront's priority as it gets through its work, so that the ones behind
// catch up and all finish together.
__device__ __forceinline__ void set_prio(uint32_t p) {
  switch (p) {
    case 3: __builtin_amdgcn_s_setprio(3); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0); break;
  }
}

// Lanes whose first-level entry is a second-level pointer (byte 0 > 127).
__device__ __forceinline__ uint64_t pointer_mask(uint32_t e) {
  uint64_t m;
  asm volatile("v_cmp_lt_u32_sdwa %0, %1, %2 src0_sel:DWORD src1_sel:BYTE_0" : "=s"(m) : "v"(127u), "v"(e));
  return m;
}

// Entry for the next codeword at the top of hi: first level indexed by the
// top K bits; a pointer entry sends the lanes that hit it (rare when K is
// chosen as in entro_lut_build) to the subtable indexed by the next bits.
__device__ __forceinline__ uint32_t lookup(const uint32_t *lut, uint32_t hi, uint32_t K) {
  uint32_t e = lut[hi >> (32u - K)];
  const uint64_t pm = pointer_mask(e);
  if (pm) {
    if (__builtin_amdgcn_inverse_ballot_w64(pm)) {
      const uint32_t sb = (e >> 8) & 31u;
      const uint32_t i2 = (hi << K) >> (32u - sb);
      e = lut[((e >> 16) + i2) & (kLutMaxEntries - 1u)];
    }
  }
  return e;
}

template <int MODE, int CP>
__device__ __forceinline__ void emit(void *base, uint64_t k, uint32_t e) {
  if (CP == kStoreCached) {
    if (MODE == kModeU8) static_cast<uint8_t *>(base)[k] = (uint8_t)(e >> 16);
    else static_cast<uint16_t *>(base)[k] = (uint16_t)(e >> 16);
  } else if (MODE == kModeU8) {
    __builtin_nontemporal_store((uint8_t)(e >> 16), static_cast<uint8_t *>(base) + k);
  } else {
    __builtin_nontemporal_store((uint16_t)(e >> 16), static_cast<uint16_t *>(base) + k);
  }
}

// ---------------------------------------------------------------------------
// generic path: one wavefront task, words read from global memory, all checks
// ---------------------------------------------------------------------------
template <int MODE, int LOG2W, int BATCH, int CP>
__device__ void task_generic(const TensorArg &d, const uint32_t *lut, uint32_t K, uint64_t task, uint32_t batch,
                             uint32_t l_min) {
  constexpr uint32_t W = 1u << LOG2W;
  constexpr uint32_t G = 64u / W;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t grp = lane >> LOG2W;
  const uint32_t j = lane & (W - 1u);
  const uint64_t grp_mask = (W == 64u) ? ~0ull : (((1ull << (W & 63u)) - 1ull) << (grp * W));
  const uint64_t grp_below = grp_mask & ((1ull << lane) - 1ull);
  const uint32_t *__restrict__ words = d.words;
  const uint64_t n_words = d.n_words, n_symbols = d.n_symbols;
  const uint32_t chunk = d.chunk, cols = d.cols, rows = d.rows;
  const uint32_t D = d.refill_steps;

  const uint64_t c = task * G + grp;
  uint32_t flags = 0;
  bool chunk_ok = c < d.n_chunks;
  uint64_t wb = 0, nw = 0;
  uint32_t cc = 0;
  if (chunk_ok) {
    const uint64_t o0 = d.offs[c], o1 = d.offs[c + 1];
    if ((o0 & 31u) || (o1 & 31u) || o1 < o0 || (o1 >> 5) > n_words) {
      flags |= kFOffsets;
      chunk_ok = false;
    } else {
      wb = o0 >> 5;
      nw = (o1 - o0) >> 5;
      cc = (uint32_t)min((uint64_t)chunk, n_symbols - c * chunk);
    }
  }
  const uint32_t my_steps = (chunk_ok && j < cc) ? ((cc - j + W - 1u) >> LOG2W) : 0u;
  const uint32_t steps = chunk >> LOG2W;
  const uint64_t sym0 = c * chunk;

  uint64_t buf = 0;      // loaded, unconsumed bits, first bit at bit 63
  uint32_t n = 0;        // how many
  uint64_t P = 0;        // words of the chunk taken so far
  float acc[BATCH];
#pragma unroll
  for (int i = 0; i < BATCH; ++i) acc[i] = 0.f;
  uint32_t col = j;
  uint64_t row = 0;
  if (MODE == kModeGemv) row = sym0 / cols;

  for (uint32_t t0 = 0; t0 < steps; t0 += D) {
    // bits this lane's codewords of steps t0 .. t0+D-1 need (peeked with the
    // bits beyond n read as zeros: a code that fits is read exactly, one that
    // does not still shows a length above n)
    const bool act = t0 < my_steps;
    uint32_t e = lookup(lut, (uint32_t)(buf >> 32), K);
    uint32_t need_bits = entry_len(e);
    if (D == 2 && t0 + 1 < my_steps && need_bits <= 31u) {
      const uint32_t eb = lookup(lut, (uint32_t)((buf << need_bits) >> 32), K);
      need_bits += entry_len(eb);
    }
    // refilling ahead: while the lane has codes_left * l_min >= 32, a word
    // whenever fewer than 32 bits are loaded
    const bool early = d.ahead && act && (uint64_t)(my_steps - t0) * l_min >= 32u;
    const bool need = early ? n < 32u : (act && need_bits > n);
    const uint64_t m = __ballot(need);
    if (m) {
      if (need) {
        const uint64_t idx = P + (uint64_t)__popcll(m & grp_below);
        uint32_t w = 0;
        if (idx < nw) w = words[wb + idx];
        else flags |= kFOverrun;
        if (n > 32u) flags |= kFBadCode;   // only a malformed stream gets here with n > 32
        else buf |= (uint64_t)w << (32u - n);
        n += 32u;
      }
      P += (uint64_t)__popcll(m & grp_mask);
    }
    for (uint32_t dt = 0; dt < D; ++dt) {
      const uint32_t t = t0 + dt;
      if (t >= steps) break;
      const bool a = t < my_steps;
      e = lookup(lut, (uint32_t)(buf >> 32), K);
      uint32_t len = entry_len(e);
      if (a) {
        if (len > kMaxCodeLen || len > n) {
          flags |= kFBadCode;
          len = min(n, 31u);
        }
        buf = len >= 64u ? 0ull : buf << len;
        n -= len;
        if (MODE == kModeGemv) {
          const float v = __uint_as_float(e & 0xFFFF0000u);
#pragma unroll
          for (int bi = 0; bi < BATCH; ++bi) {
            if (bi < (int)batch) {
              const float xv = __uint_as_float((uint32_t)d.x[(uint64_t)bi * cols + col] << 16);
              acc[bi] = fmaf(v, xv, acc[bi]);
            }
          }
        } else {
          emit<MODE, CP>(d.out, sym0 + ((uint64_t)t << LOG2W) + j, e);
        }
      }
      if (MODE == kModeGemv) {
        col += W;
        if (col >= cols) {   // uniform: every chunk starts a row and W divides cols
          col -= cols;
#pragma unroll
          for (int bi = 0; bi < BATCH; ++bi) {
            float v = acc[bi];
#pragma unroll
            for (uint32_t off = W >> 1; off >= 1u; off >>= 1) v += __shfl_xor(v, (int)off, 64);
            if (a && j == 0u && bi < (int)batch) static_cast<float *>(d.out)[(uint64_t)bi * rows + row] = v;
            acc[bi] = 0.f;
          }
          ++row;
        }
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
// staged path: the decode loop over words held in LDS
// ---------------------------------------------------------------------------

// Each loop below decodes one full task from LDS.  Scalar bookkeeping is
// kept to a minimum (the CU's single scalar unit is shared by all of its
// wavefronts): one exec-mask branch per step for the refill, word pointers
// advanced by the mask's popcount, the output offset doubling as the loop
// counter.  Word pointers are not clamped: only a malformed stream moves them
// past its chunk, its LDS reads then return data of another area (LDS
// addressing cannot fault) and the end-of-chunk check flags the overrun,
// because a pointer never decreases.

// W = 64: one chunk per wavefront; word pointer in a scalar register.
template <int MODE, typename OutT>
__device__ __forceinline__ uint32_t loop64(const uint32_t *lut, uint32_t K, const uint32_t *sw, uint32_t nw,
                                           uint32_t steps, __amdgpu_buffer_rsrc_t outr, uint32_t lane) {
  const uint32_t voff = lane * (uint32_t)sizeof(OutT);
  const uint32_t send = steps * 64u * (uint32_t)sizeof(OutT);
  uint32_t hi = 0, lo = 0, n = 0, P = 0;
  for (uint32_t soff = 0; soff != send; soff += 64u * (uint32_t)sizeof(OutT)) {
    uint32_t e = lookup(lut, hi, K);
    const uint64_t m = need_mask(e, n);
    if (__builtin_amdgcn_inverse_ballot_w64(m)) {
      const uint32_t idx =
          __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      const uint32_t w = sw[P + idx];
      // fewer than 32 bits are loaded here, so lo is empty
      hi |= w >> n;
      lo = __builtin_amdgcn_alignbit(w, 0u, n);
      n += 32u;
      e = lookup(lut, hi, K);
    }
    P += (uint32_t)__popcll(m);
    const uint32_t nhi = __builtin_amdgcn_alignbit(hi, lo, e);
    lo = __builtin_amdgcn_alignbit(lo, 0u, e);
    hi = nhi;
    n = sub_len(n, e);
    store_out<OutT>(outr, voff, soff, e);
  }
  uint32_t flags = 0;
  if (P != nw) flags |= P < nw ? kFUnderrun : kFOverrun;
  if (hi | lo) flags |= kFPadding;
  return flags;
}

// W = 32: two chunks per wavefront.  Lanes 0-31 take words from chunk 0 at
// base P0, lanes 32-63 from chunk 1; D = (chunk 1 start - chunk 0 start) +
// P1 - P0 is kept so that one v_mbcnt pair, with addend D - popcount(lower
// half) in the upper half, gives every lane its word index relative to P0.
template <int MODE, typename OutT>
__device__ __forceinline__ uint32_t loop32(const uint32_t *lut, uint32_t K, const uint32_t *sw, uint32_t dcs,
                                           uint32_t nw0, uint32_t nw1, uint32_t steps, __amdgpu_buffer_rsrc_t outr,
                                           uint32_t lane_off, uint32_t lane) {
  const uint32_t upper = lane >= 32u ? ~0u : 0u;
  const uint32_t voff = lane_off * (uint32_t)sizeof(OutT);
  const uint32_t send = steps * 32u * (uint32_t)sizeof(OutT);
  uint32_t hi = 0, lo = 0, n = 0, P0 = 0, D = dcs;
  for (uint32_t soff = 0; soff != send; soff += 32u * (uint32_t)sizeof(OutT)) {
    uint32_t e = lookup(lut, hi, K);
    const uint64_t m = need_mask(e, n);
    const uint32_t mlo = (uint32_t)m, mhi = (uint32_t)(m >> 32);
    const uint32_t clo = (uint32_t)__popc(mlo);
    if (__builtin_amdgcn_inverse_ballot_w64(m)) {
      const uint32_t idx = __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, and_sv(D - clo, upper)));
      const uint32_t w = sw[P0 + idx];
      hi |= w >> n;
      lo = __builtin_amdgcn_alignbit(w, 0u, n);
      n += 32u;
      e = lookup(lut, hi, K);
    }
    P0 += clo;
    D += (uint32_t)__popc(mhi) - clo;
    const uint32_t nhi = __builtin_amdgcn_alignbit(hi, lo, e);
    lo = __builtin_amdgcn_alignbit(lo, 0u, e);
    hi = nhi;
    n = sub_len(n, e);
    store_out<OutT>(outr, voff, soff, e);
  }
  const uint32_t P1 = D - dcs + P0;
  const uint32_t P = upper ? P1 : P0, nw = upper ? nw1 : nw0;
  uint32_t flags = 0;
  if (P != nw) flags |= P < nw ? kFUnderrun : kFOverrun;
  if (hi | lo) flags |= kFPadding;
  return flags;
}

// W <= 16: per-lane word pointers, group masks.
template <int MODE, int LOG2W, typename OutT>
__device__ __forceinline__ uint32_t loop_small(const uint32_t *lut, uint32_t K, const uint32_t *stage,
                                               uint32_t cs, uint32_t nw, uint32_t steps,
                                               __amdgpu_buffer_rsrc_t outr, uint32_t lane_off, uint32_t lane) {
  constexpr uint32_t W = 1u << LOG2W;
  const uint32_t voff = lane_off * (uint32_t)sizeof(OutT);
  const uint32_t send = steps * W * (uint32_t)sizeof(OutT);
  const uint32_t grp = lane >> LOG2W;
  const uint64_t grp_mask = ((1ull << (W & 63u)) - 1ull) << (grp * W);
  const uint64_t grp_below = grp_mask & ((1ull << lane) - 1ull);
  uint32_t hi = 0, lo = 0, n = 0, P = 0;
  for (uint32_t soff = 0; soff != send; soff += W * (uint32_t)sizeof(OutT)) {
    uint32_t e = lookup(lut, hi, K);
    const uint64_t m = need_mask(e, n);
    if (__builtin_amdgcn_inverse_ballot_w64(m)) {
      const uint32_t w = stage[cs + P + (uint32_t)__popcll(m & grp_below)];
      hi |= w >> n;
      lo = __builtin_amdgcn_alignbit(w, 0u, n);
      n += 32u;
      e = lookup(lut, hi, K);
    }
    P += (uint32_t)__popcll(m & grp_mask);
    const uint32_t nhi = __builtin_amdgcn_alignbit(hi, lo, e);
    lo = __builtin_amdgcn_alignbit(lo, 0u, e);
    hi = nhi;
    n = sub_len(n, e);
    store_out<OutT>(outr, voff, soff, e);
  }
  uint32_t flags = 0;
  if (P != nw) flags |= P < nw ? kFUnderrun : kFOverrun;
  if (hi | lo) flags |= kFPadding;
  return flags;
}

// Pair loops (refill decision every two steps).  Per pair: look up the
// codeword A at the top of the buffer and B right after it; the lanes whose
// A+B is longer than their loaded bits take one word (32 bits always cover
// two codes of at most 16 bits) and look both up again; then A and B are
// consumed with one shift by their summed length (the alignbit shift fields
// of the two entries add up to (32 - lenA - lenB) mod 32) and written with
// one store per lane (store_pair; two stores for W = 1, where neighbouring
// lanes belong to different chunks).  An odd last step is a group of one.
template <int MODE, bool PACK, typename OutT>
__device__ __forceinline__ void consume_pair(uint32_t &hi, uint32_t &lo, uint32_t &n, uint32_t eA, uint32_t eB,
                                             uint32_t lab, __amdgpu_buffer_rsrc_t outr, uint32_t voff,
                                             uint32_t soff, uint32_t boff, uint32_t sel) {
  const uint32_t sab = eA + eB;
  const uint32_t nhi = __builtin_amdgcn_alignbit(hi, lo, sab);
  lo = __builtin_amdgcn_alignbit(lo, 0u, sab);
  hi = nhi;
  n -= lab;
  if (PACK) {
    store_pair<MODE, OutT::cp>(outr, voff, soff, pack_ab<MODE>(eA, eB), sel);
  } else {
    store_out<OutT>(outr, voff, soff, eA);
    store_out<OutT>(outr, voff, soff + boff, eB);
  }
}

// Early phase with code-table lookups (codes up to 16 bits): A is looked up
// in the bits loaded before the fetch, in flight together with the word;
// lanes whose A reaches past those bits look it up again, and B is looked
// up in the merged buffer (at least 32 bits hold both codes).
template <int MODE>
__device__ __forceinline__ void early_cpair64(const uint32_t *lut, uint32_t K, uint32_t &hi, uint32_t &lo,
                                              uint32_t &n, uint32_t &pa, uint32_t &eA, uint32_t &eB) {
  const uint64_t m = gt_mask(32u, n);
  uint32_t a = lookup(lut, hi, K);
  const uint32_t n0 = n;
  if (__builtin_amdgcn_inverse_ballot_w64(m)) {
    const uint32_t idx =
        __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    const uint32_t w = lds_word(pa, idx);
    hi |= w >> n;
    lo = __builtin_amdgcn_alignbit(w, 0u, n);
    n += 32u;
  }
  pa = lds_adv(pa, (uint32_t)__popcll(m));
  const uint64_t bad = need_mask(a, n0);
  if (bad) {
    if (__builtin_amdgcn_inverse_ballot_w64(bad)) a = lookup(lut, hi, K);
  }
  eA = a;
  eB = lookup(lut, __builtin_amdgcn_alignbit(hi, lo, a), K);
}

template <int MODE>
__device__ __forceinline__ void early_cpair32(const uint32_t *lut, uint32_t K, uint32_t &hi, uint32_t &lo,
                                              uint32_t &n, uint32_t &pa, uint32_t &D, uint32_t upper,
                                              uint32_t &eA, uint32_t &eB) {
  const uint64_t m = gt_mask(32u, n);
  const uint32_t mlo = (uint32_t)m, mhi = (uint32_t)(m >> 32);
  const uint32_t clo = (uint32_t)__popc(mlo);
  uint32_t a = lookup(lut, hi, K);
  const uint32_t n0 = n;
  if (__builtin_amdgcn_inverse_ballot_w64(m)) {
    const uint32_t idx = __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, and_sv(D - clo, upper)));
    const uint32_t w = lds_word(pa, idx);
    hi |= w >> n;
    lo = __builtin_amdgcn_alignbit(w, 0u, n);
    n += 32u;
  }
  pa = lds_adv(pa, clo);
  D += (uint32_t)__popc(mhi) - clo;
  const uint64_t bad = need_mask(a, n0);
  if (bad) {
    if (__builtin_amdgcn_inverse_ballot_w64(bad)) a = lookup(lut, hi, K);
  }
  eA = a;
  eB = lookup(lut, __builtin_amdgcn_alignbit(hi, lo, a), K);
}

template <int MODE, typename OutT>
__device__ __forceinline__ uint32_t pairs64(const uint32_t *lut, uint32_t K, const uint32_t *sw, uint32_t nw,
                                            uint32_t steps, __amdgpu_buffer_rsrc_t outr, uint32_t lane,
                                            uint32_t early) {
  constexpr uint32_t B = 64u * (uint32_t)sizeof(OutT);   // bytes per step
  const uint32_t voff = lane * (uint32_t)sizeof(OutT);
  const uint32_t voffp = pair_voff(lane, lane, 64u, (uint32_t)sizeof(OutT));
  const uint32_t sel = pair_sel<MODE>(lane);
  const uint32_t send = (steps & ~1u) * B;
  uint32_t hi = 0, lo = 0, n = 0;
  uint32_t pa = lds_addr(sw);
  // pairs [0, early) in the early phase of a stream encoded refilling ahead
  uint32_t soff = 0;
  for (const uint32_t eoff = early * 2u * B; soff < eoff; soff += 2u * B) {
    uint32_t eA, eB;
    early_cpair64<MODE>(lut, K, hi, lo, n, pa, eA, eB);
    consume_pair<MODE, true, OutT>(hi, lo, n, eA, eB, pair_len(eA, eB), outr, voffp, soff, B, sel);
  }
  for (; soff != send; soff += 2u * B) {
    uint32_t eA = lookup(lut, hi, K);
    uint32_t eB = lookup(lut, __builtin_amdgcn_alignbit(hi, lo, eA), K);
    uint32_t lab = pair_len(eA, eB);
    const uint64_t m = gt_mask(lab, n);
    if (__builtin_amdgcn_inverse_ballot_w64(m)) {
      const uint32_t idx =
          __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      const uint32_t w = lds_word(pa, idx);
      hi |= w >> n;
      lo = __builtin_amdgcn_alignbit(w, 0u, n);
      n += 32u;
      eA = lookup(lut, hi, K);
      eB = lookup(lut, __builtin_amdgcn_alignbit(hi, lo, eA), K);
      lab = pair_len(eA, eB);
    }
    pa = lds_adv(pa, (uint32_t)__popcll(m));
    consume_pair<MODE, true, OutT>(hi, lo, n, eA, eB, lab, outr, voffp, soff, B, sel);
  }
  if (steps & 1u) {   // last step alone
    uint32_t e = lookup(lut, hi, K);
    const uint64_t m = need_mask(e, n);
    if (__builtin_amdgcn_inverse_ballot_w64(m)) {
      const uint32_t idx =
          __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      const uint32_t w = lds_word(pa, idx);
      hi |= w >> n;
      lo = __builtin_amdgcn_alignbit(w, 0u, n);
      n += 32u;
      e = lookup(lut, hi, K);
    }
    pa = lds_adv(pa, (uint32_t)__popcll(m));
    const uint32_t nhi = __builtin_amdgcn_alignbit(hi, lo, e);
    lo = __builtin_amdgcn_alignbit(lo, 0u, e);
    hi = nhi;
    n = sub_len(n, e);
    store_out<OutT>(outr, voff, send, e);
  }
  const uint32_t P = ((pa - lds_addr(sw)) >> 2);
  uint32_t flags = 0;
  if (P != nw) flags |= P < nw ? kFUnderrun : kFOverrun;
  if (hi | lo) flags |= kFPadding;
  return flags;
}

template <int MODE, typename OutT>
__device__ __forceinline__ uint32_t pairs32(const uint32_t *lut, uint32_t K, const uint32_t *sw, uint32_t dcs,
                                            uint32_t nw0, uint32_t nw1, uint32_t steps, __amdgpu_buffer_rsrc_t outr,
                                            uint32_t lane_off, uint32_t lane, uint32_t early) {
  constexpr uint32_t B = 32u * (uint32_t)sizeof(OutT);
  const uint32_t upper = lane >= 32u ? ~0u : 0u;
  const uint32_t voff = lane_off * (uint32_t)sizeof(OutT);
  const uint32_t voffp = pair_voff(lane_off, lane, 32u, (uint32_t)sizeof(OutT));
  const uint32_t sel = pair_sel<MODE>(lane);
  const uint32_t send = (steps & ~1u) * B;
  uint32_t hi = 0, lo = 0, n = 0, D = dcs;
  uint32_t pa = lds_addr(sw);
  // pairs [0, early) in the early phase of a stream encoded refilling ahead
  uint32_t soff = 0;
  for (const uint32_t eoff = early * 2u * B; soff < eoff; soff += 2u * B) {
    uint32_t eA, eB;
    early_cpair32<MODE>(lut, K, hi, lo, n, pa, D, upper, eA, eB);
    consume_pair<MODE, true, OutT>(hi, lo, n, eA, eB, pair_len(eA, eB), outr, voffp, soff, B, sel);
  }
  for (; soff != send; soff += 2u * B) {
    uint32_t eA = lookup(lut, hi, K);
    uint32_t eB = lookup(lut, __builtin_amdgcn_alignbit(hi, lo, eA), K);
    uint32_t lab = pair_len(eA, eB);
    const uint64_t m = gt_mask(lab, n);
    const uint32_t mlo = (uint32_t)m, mhi = (uint32_t)(m >> 32);
    const uint32_t clo = (uint32_t)__popc(mlo);
    if (__builtin_amdgcn_inverse_ballot_w64(m)) {
      const uint32_t idx = __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, and_sv(D - clo, upper)));
      const uint32_t w = lds_word(pa, idx);
      hi |= w >> n;
      lo = __builtin_amdgcn_alignbit(w, 0u, n);
      n += 32u;
      eA = lookup(lut, hi, K);
      eB = lookup(lut, __builtin_amdgcn_alignbit(hi, lo, eA), K);
      lab = pair_len(eA, eB);
    }
    pa = lds_adv(pa, clo);
    D += (uint32_t)__popc(mhi) - clo;
    consume_pair<MODE, true, OutT>(hi, lo, n, eA, eB, lab, outr, voffp, soff, B, sel);
  }
  if (steps & 1u) {
    uint32_t e = lookup(lut, hi, K);
    const uint64_t m = need_mask(e, n);
    const uint32_t mlo = (uint32_t)m, mhi = (uint32_t)(m >> 32);
    const uint32_t clo = (uint32_t)__popc(mlo);
    if (__builtin_amdgcn_inverse_ballot_w64(m)) {
      const uint32_t idx = __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, and_sv(D - clo, upper)));
      const uint32_t w = lds_word(pa, idx);
      hi |= w >> n;
      lo = __builtin_amdgcn_alignbit(w, 0u, n);
      n += 32u;
      e = lookup(lut, hi, K);
    }
    pa = lds_adv(pa, clo);
    D += (uint32_t)__popc(mhi) - clo;
    const uint32_t nhi = __builtin_amdgcn_alignbit(hi, lo, e);
    lo = __builtin_amdgcn_alignbit(lo, 0u, e);
    hi = nhi;
    n = sub_len(n, e);
    store_out<OutT>(outr, voff, send, e);
  }
  const uint32_t P0 = ((pa - lds_addr(sw)) >> 2);
  const uint32_t P1 = D - dcs + P0;
  const uint32_t P = upper ? P1 : P0, nw = upper ? nw1 : nw0;
  uint32_t flags = 0;
  if (P != nw) flags |= P < nw ? kFUnderrun : kFOverrun;
  if (hi | lo) flags |= kFPadding;
  return flags;
}

template <int MODE, int LOG2W, typename OutT>
__device__ __forceinline__ uint32_t pairs_small(const uint32_t *lut, uint32_t K, const uint32_t *stage,
                                                uint32_t cs, uint32_t nw, uint32_t steps,
                                                __amdgpu_buffer_rsrc_t outr, uint32_t lane_off, uint32_t lane) {
  constexpr uint32_t W = 1u << LOG2W;
  constexpr bool PACK = LOG2W > 0;
  constexpr uint32_t B = W * (uint32_t)sizeof(OutT);
  const uint32_t voff = lane_off * (uint32_t)sizeof(OutT);
  const uint32_t voffp = PACK ? pair_voff(lane_off, lane, W, (uint32_t)sizeof(OutT)) : voff;
  const uint32_t sel = pair_sel<MODE>(lane);
  const uint32_t grp = lane >> LOG2W;
  const uint64_t grp_mask = ((1ull << (W & 63u)) - 1ull) << (grp * W);
  const uint64_t grp_below = grp_mask & ((1ull << lane) - 1ull);
  uint32_t hi = 0, lo = 0, n = 0, P = 0;
  for (uint32_t t = 0; t < steps; t += 2u) {
    const bool two = t + 1u < steps;
    uint32_t eA = lookup(lut, hi, K);
    uint32_t eB = two ? lookup(lut, __builtin_amdgcn_alignbit(hi, lo, eA), K) : 0u;
    uint32_t lab = pair_len(eA, eB);
    const uint64_t m = gt_mask(lab, n);
    if (__builtin_amdgcn_inverse_ballot_w64(m)) {
      const uint32_t w = stage[cs + P + (uint32_t)__popcll(m & grp_below)];
      hi |= w >> n;
      lo = __builtin_amdgcn_alignbit(w, 0u, n);
      n += 32u;
      eA = lookup(lut, hi, K);
      eB = two ? lookup(lut, __builtin_amdgcn_alignbit(hi, lo, eA), K) : 0u;
      lab = pair_len(eA, eB);
    }
    P += (uint32_t)__popcll(m & grp_mask);
    if (two) {
      consume_pair<MODE, PACK, OutT>(hi, lo, n, eA, eB, lab, outr, PACK ? voffp : voff, t * B, B, sel);
    } else {
      const uint32_t nhi = __builtin_amdgcn_alignbit(hi, lo, eA);
      lo = __builtin_amdgcn_alignbit(lo, 0u, eA);
      hi = nhi;
      n = sub_len(n, eA);
      store_out<OutT>(outr, voff, t * B, eA);
    }
  }
  uint32_t flags = 0;
  if (P != nw) flags |= P < nw ? kFUnderrun : kFOverrun;
  if (hi | lo) flags |= kFPadding;
  return flags;
}

// Two-code table, built in LDS from the code table when a 4-bit tensor is
// decoded in pairs: entry i (the next PB stream bits, PB = kPairBits or
// kPairBitsWide) holds, in its first word, the pair's two output values
// packed as by pack_ab and, in the second, the pair's summed length in byte 1
// and its alignbit shift in bits [4:0], so that one 8-byte read gives a whole
// pair.  Indices whose A and B do not both fit in PB bits carry
// kPairFallback in byte 0 (length 0); lanes that hit one look the two codes
// up in the code table instead.
__device__ __forceinline__ uint32_t pair_word(uint32_t lab) { return (lab << 8) | ((32u - lab) & 31u); }

template <int MODE, uint32_t PB = kPairBits>
__device__ u32x2 build_pair_entry(const uint32_t *lut, uint32_t K, uint32_t i) {
  const uint32_t hi = i << (32u - PB);
  const uint32_t eA = lookup(lut, hi, K);
  const uint32_t lA = entry_len(eA);
  u32x2 r;
  r.x = 0u;
  r.y = kPairFallback | 0xFF00u;   // length byte above any loaded count
  if (lA <= PB) {
    const uint32_t eB = lookup(lut, hi << lA, K);
    const uint32_t lB = entry_len(eB);
    if (lA + lB <= PB) {
      r.x = pack_ab<MODE>(eA, eB);
      r.y = pair_word(lA + lB);
    }
  }
  return r;
}

template <int MODE, uint32_t PB = kPairBits>
__device__ __forceinline__ u32x2 pair_lookup(const uint32_t *lut, uint32_t K, uint32_t hi, uint32_t lo) {
  u32x2 e2 = *(lds_u32x2 *)(uintptr_t)((hi >> (32u - PB)) << 3);   // table at LDS address 0
  const uint64_t fb = pointer_mask(e2.y);
  if (fb) {
    if (__builtin_amdgcn_inverse_ballot_w64(fb)) {
      const uint32_t eA = lookup(lut, hi, K);
      const uint32_t eB = lookup(lut, __builtin_amdgcn_alignbit(hi, lo, eA), K);
      e2.x = pack_ab<MODE>(eA, eB);
      e2.y = pair_word(pair_len(eA, eB));
    }
  }
  return e2;
}

// Pairs of the early phase of a stream encoded refilling ahead (see entro.h):
// a lane takes a word exactly when it holds fewer than 32 bits, so the fetch
// is decided before the lookup and both LDS reads are in flight together.
// The pair is looked up in the bits loaded before the fetch; the lanes whose
// pair reaches past them (or that hit a table miss, length byte 0xFF) look it
// up again in the merged buffer.
__device__ __forceinline__ uint32_t early_pairs(uint32_t ahead, uint32_t steps, uint32_t l_min) {
  if (!ahead) return 0u;
  const uint32_t need = (32u + l_min - 1u) / l_min;   // early while codes_left >= need
  return steps >= need ? (steps - need) / 2u + 1u : 0u;
}

template <int MODE>
__device__ __forceinline__ u32x2 early_pair64(const uint32_t *lut, uint32_t K, uint32_t &hi, uint32_t &lo,
                                              uint32_t &n, uint32_t &pa) {
  const uint64_t m = gt_mask(32u, n);
  u32x2 e2 = *(lds_u32x2 *)(uintptr_t)((hi >> (32u - kPairBits)) << 3);
  const uint32_t n0 = n;
  if (__builtin_amdgcn_inverse_ballot_w64(m)) {
    const uint32_t idx =
        __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    const uint32_t w = lds_word(pa, idx);
    hi |= w >> n;
    lo = __builtin_amdgcn_alignbit(w, 0u, n);
    n += 32u;
  }
  pa = lds_adv(pa, (uint32_t)__popcll(m));
  const uint64_t bad = need_mask(e2.y, n0);
  if (bad) {
    if (__builtin_amdgcn_inverse_ballot_w64(bad)) e2 = pair_lookup<MODE>(lut, K, hi, lo);
  }
  return e2;
}

template <int MODE>
__device__ __forceinline__ u32x2 early_pair32(const uint32_t *lut, uint32_t K, uint32_t &hi, uint32_t &lo,
                                              uint32_t &n, uint32_t &pa, uint32_t &D, uint32_t upper) {
  const uint64_t m = gt_mask(32u, n);
  const uint32_t mlo = (uint32_t)m, mhi = (uint32_t)(m >> 32);
  const uint32_t clo = (uint32_t)__popc(mlo);
  u32x2 e2 = *(lds_u32x2 *)(uintptr_t)((hi >> (32u - kPairBits)) << 3);
  const uint32_t n0 = n;
  if (__builtin_amdgcn_inverse_ballot_w64(m)) {
    const uint32_t idx = __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, and_sv(D - clo, upper)));
    const uint32_t w = lds_word(pa, idx);
    hi |= w >> n;
    lo = __builtin_amdgcn_alignbit(w, 0u, n);
    n += 32u;
  }
  pa = lds_adv(pa, clo);
  D += (uint32_t)__popc(mhi) - clo;
  const uint64_t bad = need_mask(e2.y, n0);
  if (bad) {
    if (__builtin_amdgcn_inverse_ballot_w64(bad)) e2 = pair_lookup<MODE>(lut, K, hi, lo);
  }
  return e2;
}

// W = 64 / W = 32 pair loops reading the two-code table.
template <int MODE, typename OutT>
__device__ __forceinline__ uint32_t tab_pairs64(const uint32_t *lut, uint32_t K, const uint32_t *sw, uint32_t nw, uint32_t steps,
                                                __amdgpu_buffer_rsrc_t outr, uint32_t lane, uint32_t prio,
                                                uint32_t early) {
  constexpr uint32_t B = 64u * (uint32_t)sizeof(OutT);
  const uint32_t voff = lane * (uint32_t)sizeof(OutT);
  const uint32_t voffp = pair_voff(lane, lane, 64u, (uint32_t)sizeof(OutT));
  const uint32_t sel = pair_sel<MODE>(lane);
  const uint32_t send = (steps & ~1u) * B;
  uint32_t hi = 0, lo = 0, n = 0;
  uint32_t pa = lds_addr(sw);
  // first half of the pairs at priority prio, second half one lower
  const uint32_t mid = send / (4u * B) * (2u * B);
  // pairs [0, early) in the early phase of a stream encoded refilling ahead
  const uint32_t eoff = early * 2u * B;
  uint32_t soff = 0;
  for (uint32_t h = 0; h < 2u; ++h) {
    set_prio(h ? (prio ? prio - 1u : 0u) : prio);
    const uint32_t stop = h ? send : mid;
    for (const uint32_t estop = min(stop, eoff); soff < estop; soff += 2u * B) {
      const u32x2 e2 = early_pair64<MODE>(lut, K, hi, lo, n, pa);
      const uint32_t nhi = __builtin_amdgcn_alignbit(hi, lo, e2.y);
      lo = __builtin_amdgcn_alignbit(lo, 0u, e2.y);
      hi = nhi;
      n = sub_len(n, e2.y);
      store_pair<MODE, OutT::cp>(outr, voffp, soff, e2.x, sel);
    }
    for (; soff != stop; soff += 2u * B) {
      u32x2 e2 = pair_lookup<MODE>(lut, K, hi, lo);
      const uint64_t m = need_mask(e2.y, n);
      if (__builtin_amdgcn_inverse_ballot_w64(m)) {
        const uint32_t idx =
            __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        const uint32_t w = lds_word(pa, idx);
        hi |= w >> n;
        lo = __builtin_amdgcn_alignbit(w, 0u, n);
        n += 32u;
        e2 = pair_lookup<MODE>(lut, K, hi, lo);
      }
      pa = lds_adv(pa, (uint32_t)__popcll(m));
      const uint32_t nhi = __builtin_amdgcn_alignbit(hi, lo, e2.y);
      lo = __builtin_amdgcn_alignbit(lo, 0u, e2.y);
      hi = nhi;
      n = sub_len(n, e2.y);
      store_pair<MODE, OutT::cp>(outr, voffp, soff, e2.x, sel);
    }
  }
  if (steps & 1u) {   // last step alone
    uint32_t e = lookup(lut, hi, K);
    const uint64_t m = need_mask(e, n);
    if (__builtin_amdgcn_inverse_ballot_w64(m)) {
      const uint32_t idx =
          __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      const uint32_t w = lds_word(pa, idx);
      hi |= w >> n;
      lo = __builtin_amdgcn_alignbit(w, 0u, n);
      n += 32u;
      e = lookup(lut, hi, K);
    }
    pa = lds_adv(pa, (uint32_t)__popcll(m));
    const uint32_t nhi = __builtin_amdgcn_alignbit(hi, lo, e);
    lo = __builtin_amdgcn_alignbit(lo, 0u, e);
    hi = nhi;
    n = sub_len(n, e);
    store_out<OutT>(outr, voff, send, e);
  }
  const uint32_t P = ((pa - lds_addr(sw)) >> 2);
  uint32_t flags = 0;
  if (P != nw) flags |= P < nw ? kFUnderrun : kFOverrun;
  if (hi | lo) flags |= kFPadding;
  return flags;
}

template <int MODE, typename OutT>
__device__ __forceinline__ uint32_t tab_pairs32(const uint32_t *lut, uint32_t K, const uint32_t *sw, uint32_t dcs, uint32_t nw0, uint32_t nw1,
                                                uint32_t steps, __amdgpu_buffer_rsrc_t outr, uint32_t lane_off,
                                                uint32_t lane, uint32_t prio, uint32_t early) {
  constexpr uint32_t B = 32u * (uint32_t)sizeof(OutT);
  const uint32_t upper = lane >= 32u ? ~0u : 0u;
  const uint32_t voff = lane_off * (uint32_t)sizeof(OutT);
  const uint32_t voffp = pair_voff(lane_off, lane, 32u, (uint32_t)sizeof(OutT));
  const uint32_t sel = pair_sel<MODE>(lane);
  const uint32_t send = (steps & ~1u) * B;
  uint32_t hi = 0, lo = 0, n = 0, D = dcs;
  uint32_t pa = lds_addr(sw);
  // first half of the pairs at priority prio, second half one lower
  const uint32_t mid = send / (4u * B) * (2u * B);
  // pairs [0, early) in the early phase of a stream encoded refilling ahead
  const uint32_t eoff = early * 2u * B;
  uint32_t soff = 0;
  for (uint32_t h = 0; h < 2u; ++h) {
    set_prio(h ? (prio ? prio - 1u : 0u) : prio);
    const uint32_t stop = h ? send : mid;
    for (const uint32_t estop = min(stop, eoff); soff < estop; soff += 2u * B) {
      const u32x2 e2 = early_pair32<MODE>(lut, K, hi, lo, n, pa, D, upper);
      const uint32_t nhi = __builtin_amdgcn_alignbit(hi, lo, e2.y);
      lo = __builtin_amdgcn_alignbit(lo, 0u, e2.y);
      hi = nhi;
      n = sub_len(n, e2.y);
      store_pair<MODE, OutT::cp>(outr, voffp, soff, e2.x, sel);
    }
    for (; soff != stop; soff += 2u * B) {
      u32x2 e2 = pair_lookup<MODE>(lut, K, hi, lo);
      const uint64_t m = need_mask(e2.y, n);
      const uint32_t mlo = (uint32_t)m, mhi = (uint32_t)(m >> 32);
      const uint32_t clo = (uint32_t)__popc(mlo);
      if (__builtin_amdgcn_inverse_ballot_w64(m)) {
        const uint32_t idx = __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, and_sv(D - clo, upper)));
        const uint32_t w = lds_word(pa, idx);
        hi |= w >> n;
        lo = __builtin_amdgcn_alignbit(w, 0u, n);
        n += 32u;
        e2 = pair_lookup<MODE>(lut, K, hi, lo);
      }
      pa = lds_adv(pa, clo);
      D += (uint32_t)__popc(mhi) - clo;
      const uint32_t nhi = __builtin_amdgcn_alignbit(hi, lo, e2.y);
      lo = __builtin_amdgcn_alignbit(lo, 0u, e2.y);
      hi = nhi;
      n = sub_len(n, e2.y);
      store_pair<MODE, OutT::cp>(outr, voffp, soff, e2.x, sel);
    }
  }
  if (steps & 1u) {
    uint32_t e = lookup(lut, hi, K);
    const uint64_t m = need_mask(e, n);
    const uint32_t mlo = (uint32_t)m, mhi = (uint32_t)(m >> 32);
    const uint32_t clo = (uint32_t)__popc(mlo);
    if (__builtin_amdgcn_inverse_ballot_w64(m)) {
      const uint32_t idx = __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, and_sv(D - clo, upper)));
      const uint32_t w = lds_word(pa, idx);
      hi |= w >> n;
      lo = __builtin_amdgcn_alignbit(w, 0u, n);
      n += 32u;
      e = lookup(lut, hi, K);
    }
    pa = lds_adv(pa, clo);
    D += (uint32_t)__popc(mhi) - clo;
    const uint32_t nhi = __builtin_amdgcn_alignbit(hi, lo, e);
    lo = __builtin_amdgcn_alignbit(lo, 0u, e);
    hi = nhi;
    n = sub_len(n, e);
    store_out<OutT>(outr, voff, send, e);
  }
  const uint32_t P0 = ((pa - lds_addr(sw)) >> 2);
  const uint32_t P1 = D - dcs + P0;
  const uint32_t P = upper ? P1 : P0, nw = upper ? nw1 : nw0;
  uint32_t flags = 0;
  if (P != nw) flags |= P < nw ? kFUnderrun : kFOverrun;
  if (hi | lo) flags |= kFPadding;
  return flags;
}

// Fused GEMV from LDS (W = 64: a wavefront decodes one chunk of whole rows;
// 4-bit codes decoded in pairs through the two-code table).  Lane j meets
// columns j, j+64, ... of every row, so for pair q of a row it needs
// x[b][128q + j] and x[b][128q + 64 + j]: the workgroup stages x with those
// two values packed in one dword per batch slot (layout in stage_x), and one
// v_dot2_f32_bf16 multiplies them with the pair's two packed bf16 weights and
// accumulates in fp32.  At a row end the 64 partial sums are added with DPP
// and lane 63 writes y.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t w2, uint32_t x2, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2), __builtin_bit_cast(bf16x2, x2), acc, false);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_amdgcn_update_dpp(0.f, v, CTRL, ROW_MASK, 0xF, false);
}

// Sum over the 64 lanes, left in lane 63 (quad swaps, half-row and row
// mirrors, then the row broadcasts of lanes 15 and 31).
__device__ __forceinline__ float wave_sum63(float v) {
  v = dpp_add<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
  v = dpp_add<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
  v = dpp_add<0x141, 0xF>(v);   // row_half_mirror
  v = dpp_add<0x140, 0xF>(v);   // row_mirror
  v = dpp_add<0x142, 0xA>(v);   // row_bcast:15 into rows 1, 3
  v = dpp_add<0x143, 0xC>(v);   // row_bcast:31 into rows 2, 3
  return v;
}

// Activation slots staged per workgroup: one (BATCH = 1) or eight (batches
// 2..8, unused slots zero).
template <int BATCH>
struct XSlots { static constexpr uint32_t n = BATCH == 1 ? 1u : 8u; };

// x[b][cols] (bf16, global) -> LDS for the pairs [q0, q0 + np) of a row.
// One slot: dword (q - q0)*64 + j holds x[128q + j] | x[128q + 64 + j] << 16.
// Eight slots: 16-byte unit (2(q - q0) + h)*64 + j holds that dword for
// b = 4h .. 4h+3, so a lane reads its four slots with one conflict-free
// 16-byte read.  This copy reads x two bytes at a time and works at any
// alignment of x.
template <int BATCH>
__device__ void stage_x(uint32_t *xl, const uint16_t *x, uint32_t cols, uint32_t batch, uint32_t q0, uint32_t np) {
  const uint32_t units = np * 64u;
  for (uint32_t s = threadIdx.x; s < units; s += kBlockThreads) {
    const uint32_t q = s >> 6, j = s & 63u, c = (q0 + q) * 128u + j;
    if (BATCH == 1) {
      xl[s] = (uint32_t)x[c] | ((uint32_t)x[c + 64u] << 16);
    } else {
#pragma unroll
      for (uint32_t h = 0; h < 2u; ++h) {
        u32x4 v;
#pragma unroll
        for (uint32_t i = 0; i < 4u; ++i) {
          const uint32_t b = 4u * h + i;
          v[i] = b < batch ? ((uint32_t)x[(uint64_t)b * cols + c] | ((uint32_t)x[(uint64_t)b * cols + c + 64u] << 16)) : 0u;
        }
        reinterpret_cast<u32x4 *>(xl)[(2u * q + h) * 64u + j] = v;
      }
    }
  }
}

// The same layout from a 16-byte aligned x (its rows then are too, cols
// being a multiple of 128), in two halves so that the loads are in flight
// while the workgroup does other work: x_load issues them into registers,
// x_store writes the LDS layout.  Item s is eight consecutive columns of one
// batch row in both halves of a 128-column block: columns 8g .. 8g + 7 and
// 64 + 8g .. 64 + 8g + 7 (g = s & 7) of block q = s / (8 SB), slot
// b = (s >> 3) % SB.  A thread holds at most kXItems items.
constexpr uint32_t kXItems = 2;
static_assert(kGemvXMaxBytes / 32u <= kXItems * kBlockThreads, "staged x: items per thread");
static_assert(kGemvSlicePairs * 64u <= kXItems * kBlockThreads, "x slice: items per thread");

struct XRegs {
  u32x4 lo[kXItems], hi[kXItems];
};

__device__ __forceinline__ bool x_vec_ok(const uint16_t *x) { return ((uintptr_t)x & 15u) == 0u; }

template <int BATCH>
__device__ __forceinline__ void x_load(XRegs &r, const uint16_t *x, uint32_t cols, uint32_t batch, uint32_t q0,
                                       uint32_t np) {
  constexpr uint32_t SB = XSlots<BATCH>::n;
  const uint32_t items = np * 8u * SB;
#pragma unroll
  for (uint32_t k = 0; k < kXItems; ++k) {
    const uint32_t s = threadIdx.x + k * kBlockThreads;
    const uint32_t g = s & 7u, b = (s >> 3) % SB, q = s / (8u * SB);
    u32x4 va = {0u, 0u, 0u, 0u}, vb = va;
    if (s < items && b < batch) {
      const u32x4 *p = reinterpret_cast<const u32x4 *>(x + (uint64_t)b * cols + (q0 + q) * 128u + 8u * g);
      va = p[0];
      vb = p[8];   // 64 columns on
    }
    r.lo[k] = va;
    r.hi[k] = vb;
  }
}

template <int BATCH>
__device__ __forceinline__ void x_store(uint32_t *xl, const XRegs &r, uint32_t np) {
  constexpr uint32_t SB = XSlots<BATCH>::n;
  const uint32_t items = np * 8u * SB;
#pragma unroll
  for (uint32_t k = 0; k < kXItems; ++k) {
    const uint32_t s = threadIdx.x + k * kBlockThreads;
    if (s >= items) continue;
    const uint32_t g = s & 7u, b = (s >> 3) % SB, q = s / (8u * SB);
    // dword for column 8g + m of the block: x[.. + 8g + m] | x[.. + 64 + 8g + m] << 16
    uint32_t w[8];
#pragma unroll
    for (uint32_t m = 0; m < 4u; ++m) {
      w[2u * m] = (r.lo[k][m] & 0xFFFFu) | (r.hi[k][m] << 16);
      w[2u * m + 1u] = (r.lo[k][m] >> 16) | (r.hi[k][m] & 0xFFFF0000u);
    }
    if (SB == 1) {
      u32x4 *dst = reinterpret_cast<u32x4 *>(xl + q * 64u + 8u * g);
      dst[0] = u32x4{w[0], w[1], w[2], w[3]};
      dst[1] = u32x4{w[4], w[5], w[6], w[7]};
    } else {
      uint32_t *dst = xl + ((2u * q + (b >> 2)) * 64u + 8u * g) * 4u + (b & 3u);
#pragma unroll
      for (uint32_t m = 0; m < 8u; ++m) dst[4u * m] = w[m];
    }
  }
}

// Decode state of one GEMV wavefront (W = 64, one chunk of whole rows).
template <int BATCH>
struct GemvLane {
  uint32_t hi, lo, n, pa, kk;   // bit buffer, loaded bits, word address, pair index in the chunk
  float acc[XSlots<BATCH>::n];
};

// One pair of the row: decode (early phase of refilling ahead for kk < early,
// else on demand), then one v_dot2_f32_bf16 per batch slot with the x pair at
// xp (staged as in stage_x).
template <int BATCH>
__device__ __forceinline__ void gemv_pair(GemvLane<BATCH> &g, const uint32_t *lut, uint32_t K, uint32_t early,
                                          const uint32_t *xp) {
  constexpr uint32_t SB = XSlots<BATCH>::n;
  // the x pair first: its LDS reads do not depend on the decode and land
  // while the table lookups do
  uint32_t x1s = 0u;
  u32x4 x0, x1;
  if (SB == 1) {
    x1s = xp[0];
  } else {
    x0 = *reinterpret_cast<const u32x4 *>(xp);
    x1 = *reinterpret_cast<const u32x4 *>(xp + 256);
  }
  u32x2 e2;
  if (g.kk < early) {
    e2 = early_pair64<kModeGemv>(lut, K, g.hi, g.lo, g.n, g.pa);
  } else {
    e2 = pair_lookup<kModeGemv>(lut, K, g.hi, g.lo);
    const uint64_t m = need_mask(e2.y, g.n);
    if (__builtin_amdgcn_inverse_ballot_w64(m)) {
      const uint32_t idx =
          __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      const uint32_t w = lds_word(g.pa, idx);
      g.hi |= w >> g.n;
      g.lo = __builtin_amdgcn_alignbit(w, 0u, g.n);
      g.n += 32u;
      e2 = pair_lookup<kModeGemv>(lut, K, g.hi, g.lo);
    }
    g.pa = lds_adv(g.pa, (uint32_t)__popcll(m));
  }
  ++g.kk;
  const uint32_t nhi = __builtin_amdgcn_alignbit(g.hi, g.lo, e2.y);
  g.lo = __builtin_amdgcn_alignbit(g.lo, 0u, e2.y);
  g.hi = nhi;
  g.n = sub_len(g.n, e2.y);
  if (SB == 1) {
    g.acc[0] = dot2(e2.x, x1s, g.acc[0]);
  } else {
#pragma unroll
    for (uint32_t i = 0; i < 4u; ++i) {
      g.acc[i] = dot2(e2.x, x0[i], g.acc[i]);
      g.acc[4u + i] = dot2(e2.x, x1[i], g.acc[4u + i]);
    }
  }
}

// Row end: the 64 partial sums of every slot added, y written by lane 63.
template <int BATCH>
__device__ __forceinline__ void gemv_row_end(GemvLane<BATCH> &g, float *y, uint64_t row, uint32_t rows,
                                             uint32_t batch, uint32_t lane) {
  constexpr uint32_t SB = XSlots<BATCH>::n;
#pragma unroll
  for (uint32_t b = 0; b < SB; ++b) g.acc[b] = wave_sum63(g.acc[b]);
  if (lane == 63u) {
#pragma unroll
    for (uint32_t b = 0; b < SB; ++b)
      if (b < batch) y[(uint64_t)b * rows + row] = g.acc[b];
  }
#pragma unroll
  for (uint32_t b = 0; b < SB; ++b) g.acc[b] = 0.f;
}

template <int BATCH>
__device__ __forceinline__ uint32_t gemv_end_flags(const GemvLane<BATCH> &g, uint32_t pa0, uint32_t nw) {
  const uint32_t P = (g.pa - pa0) >> 2;
  uint32_t flags = 0;
  if (P != nw) flags |= P < nw ? kFUnderrun : kFOverrun;
  if (g.hi | g.lo) flags |= kFPadding;
  return flags;
}

// A chunk of nrows whole rows with the whole of x staged in LDS.
template <int BATCH>
__device__ __forceinline__ uint32_t gemv_rows64(const uint32_t *lut, uint32_t K, const uint32_t *sw, uint32_t nw,
                                                const uint32_t *xl, uint32_t cols, uint32_t nrows,
                                                float *y, uint64_t row0, uint32_t rows, uint32_t batch,
                                                uint32_t lane, uint32_t early) {
  constexpr uint32_t SB = XSlots<BATCH>::n;
  const uint32_t pairs_per_row = cols >> 7;
  GemvLane<BATCH> g;
  g.hi = g.lo = g.n = g.kk = 0u;
  g.pa = lds_addr(sw);
#pragma unroll
  for (uint32_t b = 0; b < SB; ++b) g.acc[b] = 0.f;
  for (uint32_t r = 0; r < nrows; ++r) {
    const uint32_t *xp = xl + lane * (SB == 1 ? 1u : 4u);
    for (uint32_t q = 0; q < pairs_per_row; ++q, xp += 64u * SB) gemv_pair<BATCH>(g, lut, K, early, xp);
    gemv_row_end<BATCH>(g, y, row0 + r, rows, batch, lane);
  }
  return gemv_end_flags<BATCH>(g, lds_addr(sw), nw);
}

// Eight batch slots whose x does not fit in LDS: the workgroup's wavefronts
// walk their rows in lockstep over slices of kGemvSlicePairs pairs (128
// columns each); between workgroup barriers all threads stage the next
// slice of x into one of two buffers while the other is read.  Called by
// every wavefront of the workgroup for one block task; those without a
// staged full chunk (have == false) only take part in the barriers and
// loads.
template <int BATCH>
__device__ uint32_t gemv_sliced64(const TensorArg &d, const uint32_t *lut, uint32_t K, bool have,
                                  const uint32_t *sw, uint32_t nw, uint32_t *xb, uint64_t row0, uint32_t batch,
                                  uint32_t lane, uint32_t early) {
  constexpr uint32_t SB = XSlots<BATCH>::n;
  constexpr uint32_t S = kGemvSlicePairs;
  constexpr uint32_t BUF = S * 64u * SB;   // words per slice buffer
  const uint32_t cols = d.cols, nrows = d.chunk / d.cols;
  const uint32_t ppr = cols >> 7;
  const uint32_t nsl = (ppr + S - 1u) / S;
  const uint32_t total = nrows * nsl;
  const uint16_t *x = d.x;
  float *y = static_cast<float *>(d.out);
  GemvLane<BATCH> g;
  g.hi = g.lo = g.n = g.kk = 0u;
  g.pa = lds_addr(sw);
#pragma unroll
  for (uint32_t b = 0; b < SB; ++b) g.acc[b] = 0.f;
  // with x 16-byte aligned, the loads of slice gi + 2 are issued before the
  // decode of slice gi + 1 and written to LDS after it
  const bool vec = x_vec_ok(x);
  XRegs xr;
  const uint32_t s1 = 1u % nsl;
  if (vec) {
    XRegs x1;
    x_load<BATCH>(xr, x, cols, batch, 0u, min(S, ppr));
    if (total > 1u) x_load<BATCH>(x1, x, cols, batch, s1 * S, min(S, ppr - s1 * S));
    x_store<BATCH>(xb, xr, min(S, ppr));
    if (total > 1u) x_store<BATCH>(xb + BUF, x1, min(S, ppr - s1 * S));
    if (total > 2u) {
      const uint32_t s2 = 2u % nsl;
      x_load<BATCH>(xr, x, cols, batch, s2 * S, min(S, ppr - s2 * S));
    }
  } else {
    stage_x<BATCH>(xb, x, cols, batch, 0u, min(S, ppr));
    if (total > 1u) stage_x<BATCH>(xb + BUF, x, cols, batch, s1 * S, min(S, ppr - s1 * S));
  }
  __syncthreads();
  for (uint32_t gi = 0; gi < total; ++gi) {
    const uint32_t r = gi / nsl, sl = gi - r * nsl;
    const uint32_t q0 = sl * S, q1 = min(q0 + S, ppr);
    const uint32_t *buf = xb + (gi & 1u) * BUF;
    if (have) {
      const uint32_t *xp = buf + lane * (SB == 1 ? 1u : 4u);
      for (uint32_t q = q0; q < q1; ++q, xp += 64u * SB) gemv_pair<BATCH>(g, lut, K, early, xp);
      if (q1 == ppr) gemv_row_end<BATCH>(g, y, row0 + r, d.rows, batch, lane);
    }
    __syncthreads();
    if (gi + 2u < total) {
      const uint32_t s2 = (gi + 2u) % nsl;
      if (vec) {
        x_store<BATCH>(xb + (gi & 1u) * BUF, xr, min(S, ppr - s2 * S));
        if (gi + 3u < total) {
          const uint32_t s3 = (gi + 3u) % nsl;
          x_load<BATCH>(xr, x, cols, batch, s3 * S, min(S, ppr - s3 * S));
        }
      } else {
        stage_x<BATCH>(xb + (gi & 1u) * BUF, x, cols, batch, s2 * S, min(S, ppr - s2 * S));
      }
    }
  }
  return have ? gemv_end_flags<BATCH>(g, lds_addr(sw), nw) : 0u;
}

// ---------------------------------------------------------------------------
// Fused GEMV, streamed: W = 64 chunks of whole rows, 4-bit codes decoded in
// pairs through a two-code table of kPairBitsWide index bits, 128 | cols.
//
// A workgroup takes a contiguous share of the launch's chunks and splits the
// part of it that lies in one tensor into kWaves contiguous ranges, one per
// wavefront.  A wavefront's chunks are consecutive, so their words form one
// run of the stream, which it streams through a ring of kRingBlocks blocks in
// its LDS area (copies with 16-byte loads that write LDS directly).  Block k
// of the run (words [k B, (k + 1) B) from the run's block-aligned base) sits
// in ring slot k mod kRingBlocks.  When the word pointer P enters block k,
// slot k - 1 is free (all its words lie below P) and block k + 3 is copied
// into it; a step reads words [P, P + 64), within blocks k and k + 1, so the
// two newest copies may stay in flight (s_waitcnt vmcnt(2); vector-memory
// loads complete in order).  The buffer resource ends at the run's last
// word, so copies past it read zeros without touching memory.  No other
// vector-memory access happens while a run streams: the rows' y values are
// collected in registers and stored at most every 64 rows.
// ---------------------------------------------------------------------------

// The run of one wavefront: the buffer resource over its words (from the
// block-aligned base on), the word pointer P as a byte offset from the base,
// and the chunks' end offsets (lane i: byte offset of the end of chunk cb + i from the base, for
// the 64 chunks from chunk c64 on).
struct Run {
  __amdgpu_buffer_rsrc_t r;
  uint64_t base;     // first word of block 0 (stream word index)
  uint32_t p4;       // byte offset of P from the base
  uint32_t klast;    // the run's last block
  uint32_t bytes;    // the run's bytes from the base (the buffer resource's range)
  uint32_t ends;     // per lane: end of chunk c64 + lane (byte offset from the base)
};

// Copy block k of the run into its ring slot.  A ring of 2^RL words holds
// four blocks of 2^RL bytes: with RL = 10 one 16-byte copy per lane (64 lanes
// x 16 bytes), with RL = 9 two 4-byte copies per lane (2 x 64 lanes x 4
// bytes), with RL = 8 one 4-byte copy per lane, so that every lane takes part
// in every copy.  Every copy
// instruction reads memory: a block past the run's end is never read, and
// its slot receives the run's last block again instead; likewise the second
// half of the last block, where it lies wholly past the run's end, is
// replaced by the first.  (The waits count copies in flight and rely on
// copies completing in the order they were issued; a copy wholly outside
// the buffer resource reads no memory and can complete ahead of earlier
// ones.)  The copy's LDS write does not pass through the LDS instruction
// queue, so it can land before an LDS read of the slot that was issued
// earlier (the chunk's first fetch reads the block being left when the copy
// is issued); the wavefront's LDS reads are waited for first.
template <uint32_t RL>
__device__ __forceinline__ void ring_copy(const Run &R, uint32_t ring_base, uint32_t k, uint32_t lane) {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  asm volatile("" ::: "memory");
  const uint32_t dst = ring_base + ((k << RL) & ((4u << RL) - 1u));
  const uint32_t src = min(k, R.klast) << RL;
  static_assert(RL >= 8u && RL <= 10u, "ring blocks of 64, 128 or 256 words");
  if (RL == 10) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(R.r, (lds_void *)(uintptr_t)rfl(dst), 16, lane * 16u, rfl(src), 0, 0);
  } else if (RL == 8) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(R.r, (lds_void *)(uintptr_t)rfl(dst), 4, lane * 4u, rfl(src), 0, 0);
  } else {
    const uint32_t src2 = src + 256u < R.bytes ? src + 256u : src;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(R.r, (lds_void *)(uintptr_t)rfl(dst), 4, lane * 4u, rfl(src), 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(R.r, (lds_void *)(uintptr_t)rfl(dst + 256u), 4, lane * 4u, rfl(src2),
                                             0, 0);
  }
}

// Copy instructions per block
template <uint32_t RL>
struct RingCopies { static constexpr uint32_t n = RL == 9 ? 2u : 1u; };

// Wait until at most two blocks' copies are in flight (every block up to the
// one after P's has landed), then keep later LDS reads below the wait.
template <uint32_t RL>
__device__ __forceinline__ void ring_wait2() {
  if (RingCopies<RL>::n == 1) __builtin_amdgcn_s_waitcnt(0x0F72);   // vmcnt(2)
  else __builtin_amdgcn_s_waitcnt(0x0F74);                          // vmcnt(4)
  asm volatile("" ::: "memory");
}

// End offsets of chunks [c, min(c + 64, ce)) relative to the run's base, one
// per lane (a vector load, so that no scalar load is pending in the decode
// loop); lanes past ce hold the last one.  False if any is malformed (not a
// multiple of 32 bits, below the run's start, past the words).
__device__ __forceinline__ bool load_ends(const TensorArg &d, const Run &R, uint32_t c, uint32_t ce,
                                          uint64_t o_start, uint32_t lane, uint32_t &ends) {
  const uint32_t i = min(c + 1u + lane, ce);
  const uint64_t o = d.offs[i];
  const bool bad = (o & 31u) || o < o_start || (o >> 5) > d.n_words;
  ends = (uint32_t)((o >> 5) - R.base) * 4u;
  return __ballot(bad) == 0ull;
}

// Start the run of chunks [cb, ce) (cb < ce): the copies of its first NFILL
// blocks (the rest of the ring: ring_fill_rest).  False if the offsets are
// malformed; then no copy is issued (the buffer resource would be empty, and
// a copy that reads no memory can complete out of order), and the run is not
// decoded.
// run_begin takes the run's bounding offsets o0 = offs[cb], o1 = offs[ce],
// read beforehand.
template <uint32_t RL, uint32_t NFILL = kRingBlocks>
__device__ __forceinline__ bool run_begin(const TensorArg &d, uint32_t cb, uint32_t ce, uint64_t o0, uint64_t o1,
                                          uint32_t ring_base, uint32_t lane, Run &R) {
  constexpr uint32_t log2r = RL;
  const bool ok = !((o0 & 31u) || (o1 & 31u) || o1 < o0 || (o1 >> 5) > d.n_words);
  const uint32_t log2b = log2r - 2u;
  const uint64_t s0 = o0 >> 5, s1 = o1 >> 5;
  R.base = ok ? (s0 >> log2b) << log2b : 0u;
  const uint32_t bytes = ok ? (uint32_t)(s1 - R.base) * 4u : 0u;   // the host keeps streams below 4 GiB
  R.klast = rfl(bytes ? (bytes - 1u) >> log2r : 0u);
  R.bytes = rfl(bytes);
  R.r = __builtin_amdgcn_make_buffer_rsrc((void *)(d.words + R.base), (short)0, (int)bytes, 0x00020000);
  if (bytes) {
#pragma unroll
    for (uint32_t k = 0; k < NFILL; ++k) ring_copy<RL>(R, ring_base, k, lane);
  }
  // the end offsets after the copies, so that their load does not delay them
  const bool ends_ok = load_ends(d, R, cb, ce, o0, lane, R.ends);
  R.p4 = rfl((uint32_t)(s0 - R.base) * 4u);
  return ok && ends_ok;
}

template <uint32_t RL, uint32_t NFILL = kRingBlocks>
__device__ __forceinline__ bool run_start(const TensorArg &d, uint32_t cb, uint32_t ce, uint32_t ring_base,
                                          uint32_t lane, Run &R) {
  const __attribute__((address_space(4))) uint64_t *co =
      (const __attribute__((address_space(4))) uint64_t *)(uintptr_t)d.offs;
  return run_begin<RL, NFILL>(d, cb, ce, co[cb], co[ce], ring_base, lane, R);
}

// The ring's blocks NFILL.. of a run started with run_start<RL, NFILL>.
template <uint32_t RL, uint32_t NFILL>
__device__ __forceinline__ void ring_fill_rest(const Run &R, uint32_t ring_base, uint32_t lane) {
  if (R.bytes) {
#pragma unroll
    for (uint32_t k = NFILL; k < kRingBlocks; ++k) ring_copy<RL>(R, ring_base, k, lane);
  }
}

// After P moved from byte offset p_old on (by at most 256 bytes, less than a
// block): on entering a new block k, copy block k + 3 into the freed slot.
// The block index is P's, so the ring needs no state of its own.
template <uint32_t RL>
__device__ __forceinline__ void ring_advance(const Run &R, uint32_t p_old, uint32_t ring_base, uint32_t lane) {
  if ((p_old ^ R.p4) >> RL) {
    ring_copy<RL>(R, ring_base, (R.p4 >> RL) + (kRingBlocks - 1u), lane);
    ring_wait2<RL>();
  }
}

// P += 4 * (lanes of m), on the scalar unit
__device__ __forceinline__ void p4_add(uint32_t &p4, uint64_t m) {
  uint32_t r;
  asm("s_lshl2_add_u32 %0, %1, %2" : "=s"(r) : "s"((uint32_t)__popcll(m)), "s"(rfl(p4)) : "scc");
  p4 = r;
}

// Lanes of mask m take the next words of the run: word P + (lower lanes of m)
// from the ring (ring_v: the ring's LDS byte address, a multiple of its size,
// in a vector register), merged into the bit buffer at its end.
__device__ __forceinline__ void ring_fetch(uint64_t m, uint32_t &hi, uint32_t &lo, uint32_t &n, uint32_t p4,
                                           uint32_t ring_v, uint32_t rmask4) {
  const uint32_t idx = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  uint32_t a;
  asm("v_lshl_add_u32 %0, %1, 2, %2\n\tv_and_or_b32 %0, %0, %3, %4"
      : "=&v"(a) : "v"(idx), "s"(p4), "s"(rmask4), "v"(ring_v));
  const uint32_t w = *(lds_u32 *)(uintptr_t)a;
  hi |= w >> n;
  lo = __builtin_amdgcn_alignbit(w, 0u, n);
  n += 32u;
}

template <bool NOFB>
__device__ __forceinline__ u32x2 wide_pair(const uint32_t *lut, uint32_t K, uint32_t hi, uint32_t lo) {
  if (NOFB) return *(lds_u32x2 *)(uintptr_t)((hi >> (32u - kPairBitsWide)) << 3);
  return pair_lookup<kModeGemv, kPairBitsWide>(lut, K, hi, lo);
}

// One pair of steps of a run's chunk, in the early phase of a stream encoded
// refilling ahead (fetch iff fewer than 32 bits are held, decided before the
// lookup, so that the word and the pair are read together) or on demand.
// With NOFB every index of the two-code table holds a whole pair of at most
// 12 bits (codes of at most 6 bits); in the early phase at least 32 - 12 = 20
// bits are held before each pair (32 after the chunk's first word), so the
// lookup made before the fetch is exact.
template <bool EARLY, bool NOFB>
__device__ __forceinline__ u32x2 stream_pair(const uint32_t *lut, uint32_t K, uint32_t &hi, uint32_t &lo,
                                             uint32_t &n, uint32_t &p4, uint32_t ring_v, uint32_t rmask4) {
  u32x2 e2;
  if (EARLY) {
    const uint64_t m = gt_mask(32u, n);
    e2 = *(lds_u32x2 *)(uintptr_t)((hi >> (32u - kPairBitsWide)) << 3);
    const uint32_t n0 = n;
    if (__builtin_amdgcn_inverse_ballot_w64(m)) ring_fetch(m, hi, lo, n, p4, ring_v, rmask4);
    p4_add(p4, m);
    if (!NOFB) {
      const uint64_t bad = need_mask(e2.y, n0);
      if (bad) {
        if (__builtin_amdgcn_inverse_ballot_w64(bad)) e2 = wide_pair<false>(lut, K, hi, lo);
      }
    }
  } else {
    e2 = wide_pair<NOFB>(lut, K, hi, lo);
    const uint64_t m = need_mask(e2.y, n);
    if (__builtin_amdgcn_inverse_ballot_w64(m)) {
      ring_fetch(m, hi, lo, n, p4, ring_v, rmask4);
      e2 = wide_pair<NOFB>(lut, K, hi, lo);
    }
    p4_add(p4, m);
  }
  const uint32_t nhi = __builtin_amdgcn_alignbit(hi, lo, e2.y);
  lo = __builtin_amdgcn_alignbit(lo, 0u, e2.y);
  hi = nhi;
  n = sub_len(n, e2.y);
  return e2;
}

// Pairs [q0, q1) of a row: decode, one v_dot2_f32_bf16 per batch slot with
// the staged x pair, and the ring kept ahead.
template <int BATCH, bool EARLY, bool NOFB, uint32_t RL>
__device__ __forceinline__ void stream_pairs(const uint32_t *lut, uint32_t K, uint32_t q0, uint32_t q1,
                                             const uint32_t *xl, uint32_t lane, float *acc, uint32_t &hi,
                                             uint32_t &lo, uint32_t &n, Run &R, uint32_t ring_base,
                                             uint32_t ring_v, uint32_t rmask4) {
  constexpr uint32_t SB = XSlots<BATCH>::n;
  const uint32_t *xp = xl + lane * (SB == 1 ? 1u : 4u) + q0 * 64u * SB;
  for (uint32_t q = q0; q < q1; ++q, xp += 64u * SB) {
    uint32_t x1s = 0u;
    u32x4 x0, x1;
    if (SB == 1) {
      x1s = xp[0];
    } else {
      x0 = *reinterpret_cast<const u32x4 *>(xp);
      x1 = *reinterpret_cast<const u32x4 *>(xp + 256);
    }
    const uint32_t p_old = R.p4;
    const u32x2 e2 = stream_pair<EARLY, NOFB>(lut, K, hi, lo, n, R.p4, ring_v, rmask4);
    if (SB == 1) {
      acc[0] = dot2(e2.x, x1s, acc[0]);
    } else {
#pragma unroll
      for (uint32_t i = 0; i < 4u; ++i) {
        acc[i] = dot2(e2.x, x0[i], acc[i]);
        acc[4u + i] = dot2(e2.x, x1[i], acc[4u + i]);
      }
    }
    ring_advance<RL>(R, p_old, ring_base, lane);
  }
}

// Decode the run's chunks [cb, ce) (each of d.chunk / cols whole rows) and
// write y of their rows; returns the stream flags.
template <int BATCH, bool NOFB, uint32_t RL>
__device__ uint32_t stream_run(const TensorArg &d, const uint32_t *lut, uint32_t K, uint32_t l_min, Run &R,
                               uint32_t cb, uint32_t ce, const uint32_t *xl, uint32_t batch, uint32_t lane,
                               uint32_t ring_base) {
  constexpr uint32_t log2r = RL;
  constexpr uint32_t SB = XSlots<BATCH>::n;
  const uint32_t cols = d.cols, ppr = cols >> 7, rpc = d.chunk / cols, rows = d.rows;
  uint32_t ring_v;   // the ring's address in a vector register (an operand of v_and_or_b32)
  asm volatile("v_mov_b32 %0, %1" : "=v"(ring_v) : "s"(ring_base));
  const uint32_t rmask4 = rfl((4u << log2r) - 1u);
  float *y = static_cast<float *>(d.out);
  uint32_t flags = 0;
  uint64_t yrow0 = (uint64_t)cb * rpc;   // first row of the y values held
  uint32_t ycnt = 0;
  float yv[SB];
#pragma unroll
  for (uint32_t b = 0; b < SB; ++b) yv[b] = 0.f;
  ring_wait2<RL>();   // blocks 0 and 1 of the run
  // A run of several rows takes issue priority 1 for its first half and 0
  // for the rest: among wavefronts of equal priority the oldest is served
  // first, so without this the ones that started last finish last.
  const uint32_t run_rows =
      ce > cb ? (uint32_t)(min((uint64_t)ce * rpc, (uint64_t)rows) - (uint64_t)cb * rpc) : 0u;
  if (run_rows > 1u) set_prio(1u);
  uint32_t rows_done = 0;
  for (uint32_t c = cb; c < ce; ++c) {
    if (c != cb && ((c - cb) & 63u) == 0u) {   // the next 64 chunk ends
      const uint64_t o_start = R.base * 32u + R.p4 * 8u;
      if (!load_ends(d, R, c, ce, o_start, lane, R.ends)) {
        flags |= kFOffsets;
        break;
      }
    }
    const uint32_t end4 = __builtin_amdgcn_readlane(R.ends, (int)((c - cb) & 63u));
    // rows of this chunk (the last chunk of a tensor may hold fewer) and the
    // pairs of its early phase
    const uint32_t nr = (uint32_t)min((uint64_t)rpc, (uint64_t)rows - (uint64_t)c * rpc);
    const uint32_t early_n = rfl(early_pairs(d.ahead, nr * (cols >> 6), l_min));
    // the chunk's first decision point: every lane takes one word (both
    // refill rules agree there: no bits are held)
    uint32_t hi = 0, lo = 0, n = 0;
    ring_fetch(~0ull, hi, lo, n, R.p4, ring_v, rmask4);
    const uint32_t p_old = R.p4;
    R.p4 = rfl(R.p4 + 256u);
    ring_advance<RL>(R, p_old, ring_base, lane);
    uint32_t kk = 0;   // pairs of the chunk done
    for (uint32_t r = 0; r < nr; ++r, kk += ppr) {
      float acc[SB];
#pragma unroll
      for (uint32_t b = 0; b < SB; ++b) acc[b] = 0.f;
      const uint32_t qe = early_n > kk ? min(early_n - kk, ppr) : 0u;
      if (run_rows > 1u && rows_done == (run_rows >> 1)) set_prio(0u);
      ++rows_done;
      stream_pairs<BATCH, true, NOFB, RL>(lut, K, 0u, qe, xl, lane, acc, hi, lo, n, R, ring_base, ring_v, rmask4);
      stream_pairs<BATCH, false, NOFB, RL>(lut, K, qe, ppr, xl, lane, acc, hi, lo, n, R, ring_base, ring_v, rmask4);
      // row end: the row's sums (lane 63 after the reduction) go to lane ycnt
#pragma unroll
      for (uint32_t b = 0; b < SB; ++b) {
        const float s =
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_sum63(acc[b])), 63));
        yv[b] = lane == ycnt ? s : yv[b];
      }
      if (++ycnt == 64u) {
#pragma unroll
        for (uint32_t b = 0; b < SB; ++b)
          if (b < batch) y[(uint64_t)b * rows + yrow0 + lane] = yv[b];
        yrow0 += 64u;
        ycnt = 0;
      }
    }
    if (R.p4 != end4) flags |= R.p4 < end4 ? kFUnderrun : kFOverrun;
    if (hi | lo) flags |= kFPadding;
    if (R.p4 != end4) break;   // malformed: the rest of the run is not decoded
  }
  if (ycnt) {
#pragma unroll
    for (uint32_t b = 0; b < SB; ++b)
      if (b < batch && lane < ycnt) y[(uint64_t)b * rows + yrow0 + lane] = yv[b];
  }
  return flags;
}

// The tensor whose workgroups include workgroup b, that tensor's workgroup
// count nwg, and b's index bl among them (from the host's per-workgroup
// table).
__device__ __forceinline__ uint32_t wg_tensor(const StreamArgs &a, uint32_t b, uint32_t &nwg, uint32_t &bl) {
  const uint32_t info = (a.wg_info_w[b >> 1] >> ((b & 1u) * 16u)) & 0xFFFFu;
  const uint32_t tw = info >> 12;
  nwg = (a.wg_count_w[tw >> 1] >> ((tw & 1u) * 16u)) & 0xFFFFu;
  bl = info & 0xFFFu;
  return tw;
}

// The host-built two-code table of a tensor into LDS [0, 32 KiB): wavefront
// w copies bytes [2 KiB w, 2 KiB (w + 1)) with two 16-byte copies per lane.
__device__ __forceinline__ void ptab_copy(const uint32_t *plut, uint32_t wave, uint32_t lane) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(plut + kPairLutHeaderWords), (short)0, (int)(8u << kPairBitsWide), 0x00020000);
  const uint32_t b = wave * 2048u;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(uintptr_t)rfl(b), 16, lane * 16u, rfl(b), 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(uintptr_t)rfl(b + 1024u), 16, lane * 16u,
                                           rfl(b + 1024u), 0, 0);
}
static_assert((8u << kPairBitsWide) == 2048u * kWaves, "two-code table copy: 2 KiB per wavefront");

template <int BATCH, uint32_t RL>
__device__ __forceinline__ void gemv_stream(const StreamArgs &a) {
  constexpr uint32_t SB = XSlots<BATCH>::n;
  // dynamic LDS: the two-code table (kPairBitsWide index bits, at LDS address
  // 0), the code table (lut_cap entries), the staged activations (x_words),
  // the table-state word, then one ring per wavefront
  // Setup in four dependent rounds, each issued before anything waits on it
  // (kernel argument reads stay in the first block, ahead of every branch):
  // the workgroup split and the LDS layout; the tensor's fields and chunk
  // range; its table headers, run offsets, activations and table entries;
  // the ring's and the two-code table's copies.
  const uint32_t lut_cap = a.lut_cap, flag_word = a.flag_word, ring_off = a.ring_off, batch = a.batch;
  const uint32_t b = blockIdx.x;
  uint32_t nwg, bl;
  const uint32_t tw = wg_tensor(a, b, nwg, bl);
  const TensorArg d = a.t[tw];
  const uint32_t n_t = a.chunk_begin[tw + 1] - a.chunk_begin[tw];
  u32x2 *ptab = reinterpret_cast<u32x2 *>(dyn_lds);
  uint32_t *lut = reinterpret_cast<uint32_t *>(dyn_lds) + (2u << kPairBitsWide);
  uint32_t *xl = lut + lut_cap;
  uint32_t *state = reinterpret_cast<uint32_t *>(dyn_lds) + flag_word;
  const uint32_t wave = rfl(threadIdx.x >> 6);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t ring_base = rfl(lds_addr(dyn_lds) + ring_off + (wave << (RL + 2u)));
  // the workgroup's share, an even part of one tensor's chunks (the host
  // gives every tensor its own workgroups, each at least one chunk)
  const uint32_t c0 = bl * (n_t / nwg) + min(bl, n_t % nwg);   // chunks of tensor tw
  const uint32_t len = n_t / nwg + (bl < n_t % nwg ? 1u : 0u);
  {
    const uint32_t cb = c0 + (wave * len) / kWaves, ce = c0 + ((wave + 1u) * len) / kWaves;
    // the headers of both tables (in place of a missing or short table, the
    // first 16 bytes of the chunk offsets are read and ignored)
    const bool hv = d.lut_words >= kLutHeaderWords;
    const bool pt = d.plut != nullptr;
    const uint32_t *const offs32 = reinterpret_cast<const uint32_t *>(d.offs);
    const u32x4 hh = *(const __attribute__((address_space(4))) u32x4 *)(uintptr_t)(hv ? d.lut : offs32);
    const u32x4 ph = *(const __attribute__((address_space(4))) u32x4 *)(uintptr_t)(pt ? d.plut : offs32);
    const uint32_t h0 = hh[0], h1 = hh[1], hne = hh[2], hl1 = hh[3];
    const uint32_t p0 = ph[0], p1 = ph[1], p2 = ph[2];
    const __attribute__((address_space(4))) uint64_t *co =
        (const __attribute__((address_space(4))) uint64_t *)(uintptr_t)d.offs;
    const uint64_t o0 = co[cb], o1 = co[ce];   // the run's bounds (cb == ce reads one twice)
    if (!lds_at_zero()) {   // the two-code table is addressed from LDS address 0
      if (threadIdx.x == 0) atomicOr(d.status, kFLut);
      return;
    }
    // the two-code table's copy (nothing reads that LDS yet), activations
    // and table entries into registers (written to LDS after the barrier),
    // all in flight while the run's bounds arrive
    if (pt) ptab_copy(d.plut, wave, lane);
    const bool x_vec = x_vec_ok(d.x);
    XRegs xr;
    if (x_vec) x_load<BATCH>(xr, d.x, d.cols, batch, 0u, d.cols >> 7);
    const uint32_t ne_fetch = min(lut_cap, d.lut_words > kLutHeaderWords ? d.lut_words - kLutHeaderWords : 0u);
    const uint32_t nv = ((uintptr_t)d.lut & 15u) == 0u ? ne_fetch >> 2 : 0u;
    u32x4 lv = {0u, 0u, 0u, 0u};
    if (threadIdx.x < nv) lv = reinterpret_cast<const u32x4 *>(d.lut + kLutHeaderWords)[threadIdx.x];
    // blocks 0 and 1 of the run now, 2 and 3 after the barriers: the copies
    // that every wavefront waits for at the barrier are half the ring
    Run R;
    const bool have = cb < ce;
    const bool run_ok = have && run_begin<RL, 2u>(d, cb, ce, o0, o1, ring_base, lane, R);
    // The table entries, the activations and the table-state word go to LDS
    // before the workgroup's one set-up barrier: nothing reads them before
    // it, and the direct-to-LDS copies in flight (two-code table, rings)
    // write other LDS.
    if (threadIdx.x == 0) *state = 0u;
    if (threadIdx.x < nv)
      reinterpret_cast<u32x4 *>(lut)[threadIdx.x] =
          u32x4{kernel_entry<kModeGemv>(lv[0]), kernel_entry<kModeGemv>(lv[1]), kernel_entry<kModeGemv>(lv[2]),
                kernel_entry<kModeGemv>(lv[3])};
    for (uint32_t i = 4u * nv + threadIdx.x; i < ne_fetch; i += kBlockThreads)
      lut[i] = kernel_entry<kModeGemv>(d.lut[kLutHeaderWords + i]);
    if (x_vec) x_store<BATCH>(xl, xr, d.cols >> 7);
    else stage_x<BATCH>(xl, d.x, d.cols, batch, 0u, d.cols >> 7);
    uint32_t k = 0;
    if (hv) {
      const uint32_t kk = h1 & 0xFFu, lmin = h1 >> 24;
      if (h0 == kLutMagic && (h1 & 0x00FFFF00u) == d.expect_hdr && kk >= 1 && kk <= kSingleLevelMax &&
          hl1 == (1u << kk) && hne >= hl1 && hne <= lut_cap && hne <= d.lut_words - kLutHeaderWords &&
          lmin >= 1u && lmin <= kMaxCodeLen)
        k = kk | (lmin << 24);
    }
    if (pt && (p0 != kPairLutMagic || p2 != h1)) k = 0u;   // not this code's two-code table
    k = rfl(k);
    if (!k && threadIdx.x == 0) atomicOr(d.status, kFLut);
    const uint32_t K = k & 0xFFu, l_min = k >> 24;
    __syncthreads();
    // two-code table (unless copied); does any index miss a whole pair?
    bool nofb = (p1 & kPairLutWhole) != 0u;
    if (!pt) {
      bool miss = false;
      if (K) {
        for (uint32_t i = threadIdx.x; i < (1u << kPairBitsWide); i += kBlockThreads) {
          const u32x2 e = build_pair_entry<kModeGemv, kPairBitsWide>(lut, K, i);
          ptab[i] = e;
          miss |= (e.y & kPairFallback) != 0u;
        }
      }
      if (__ballot(miss) && lane == 0) atomicOr(state, 1u);
      __syncthreads();
      nofb = rfl(*state) == 0u;
    }
    if (!K) {
      wait_lds_copy();   // the run's first copies land before the workgroup ends
      return;
    }
    uint32_t flags = 0;
    if (have && !run_ok) {
      flags = kFOffsets;
    } else if (run_ok) {
      ring_fill_rest<RL, 2u>(R, ring_base, lane);
      flags = nofb ? stream_run<BATCH, true, RL>(d, lut, K, l_min, R, cb, ce, xl, batch, lane, ring_base)
                   : stream_run<BATCH, false, RL>(d, lut, K, l_min, R, cb, ce, xl, batch, lane, ring_base);
    }
    if (flags && lane == 0) atomicOr(d.status, flags);
  }
  // copies past the run's end may still be in flight into the ring
  wait_lds_copy();
  (void)SB;
}

// Batch 1: two 16-wave workgroups share a CU where the LDS allows it, which
// takes at most 64 SGPRs and 64 VGPRs per wavefront (8 wavefronts per SIMD).
// Batch 8: its activations leave room for one workgroup per CU; no budget.
template <uint32_t RL>
__global__ __launch_bounds__(kBlockThreads) __attribute__((amdgpu_num_sgpr(kKernelSgprs), amdgpu_waves_per_eu(8)))
void ecw_gemv_stream_kernel(const StreamArgs a) {
  gemv_stream<1, RL>(a);
}

template <uint32_t RL>
__global__ __launch_bounds__(kBlockThreads) void ecw_gemv8_stream_kernel(const StreamArgs a) {
  gemv_stream<8, RL>(a);
}

// Where a staged task's words sit in its LDS area: chunk of lane group g
// starts at word cs (al = 16-byte alignment shift of the first chunk) and
// has nw words.
struct Staged {
  uint32_t al, cs, nw;
};

// Start copying the words of wavefront task `task` (64 / W consecutive
// chunks) into the wavefront's LDS area; false (nothing usable staged) if the
// offsets are malformed or the words do not fit.  The copy is in flight on
// return: wait_lds_copy() before reading it (stage_task does both).
template <int LOG2W>
__device__ bool stage_task_issue(const TensorArg &d, uint64_t task, uint32_t *stage, uint32_t stage_words,
                                 Staged &st) {
  constexpr uint32_t W = 1u << LOG2W;
  constexpr uint32_t G = 64u / W;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t grp = lane >> LOG2W;
  const uint64_t c0 = task * G;
  const uint64_t n_words = d.n_words;
  (void)W;

  // offsets of the task's G + 1 chunk boundaries
  uint64_t o_first, o_last, og, og1;
  if constexpr (G <= 2) {
    // at most three, the same for every lane: scalar loads (read through the
    // constant address space, which the offsets are for the kernel).  Their
    // wait counter is not the vector-memory one, so waiting for them does not
    // also wait for the stores of the wavefront's previous task.
    const __attribute__((address_space(4))) uint64_t *co =
        (const __attribute__((address_space(4))) uint64_t *)(uintptr_t)d.offs;
    const uint64_t oA = co[c0], oB = co[c0 + 1u], oC = G == 2 ? co[c0 + 2u] : oB;
    const bool bad = (oA & 31u) || (oB & 31u) || oB < oA || (oB >> 5) > n_words ||
                     (G == 2 && ((oC & 31u) || oC < oB || (oC >> 5) > n_words));
    if (bad) return false;
    o_first = oA;
    o_last = G == 2 ? oC : oB;
    og = grp ? oB : oA;
    og1 = grp ? oC : oB;
  } else {
    // lane l < G holds the start of chunk c0 + l, the end of the task is
    // loaded once for all lanes
    const uint64_t o = d.offs[c0 + min(lane, G - 1u)];
    o_last = rfl64(d.offs[c0 + G]);
    const uint64_t o_down = __shfl_down(o, 1, 64);
    const uint64_t o_next = lane + 1u < G ? o_down : o_last;
    const bool bad = lane < G && ((o & 31u) || (o_next & 31u) || o_next < o || (o_next >> 5) > n_words);
    if (__ballot(bad)) return false;
    o_first = rfl64(__shfl(o, 0, 64));
    og = __shfl(o, (int)grp, 64);
    og1 = __shfl(o_next, (int)grp, 64);
  }
  const uint64_t task_words = (o_last - o_first) >> 5;
  if (task_words + 3u > stage_words) return false;

  // stage the task's words, 16 bytes per lane per load straight into LDS,
  // from a 16-byte aligned start; bytes past the tensor's words land as zero
  const uint64_t w_first = o_first >> 5;
  const uint32_t al = (uint32_t)(w_first & 3u);
  const uint64_t base_al = w_first - al;
  const uint64_t bytes_left = (n_words - base_al) * 4u;
  const uint32_t nrec = (uint32_t)min(bytes_left, (uint64_t)0xFFFFFFF0u);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)(d.words + base_al), (short)0, (int)nrec, 0x00020000);
  const uint32_t nvec = (uint32_t)((al + task_words + 3u) >> 2);
  lds_copy16(rsrc, rfl(lds_addr(stage)), rfl(nvec), lane);

  const uint32_t cs = al + (uint32_t)((og - o_first) >> 5);
  const uint32_t nw = (uint32_t)((og1 - og) >> 5);
  st.al = al;
  st.cs = cs;
  st.nw = nw;
  return true;
}

template <int LOG2W>
__device__ bool stage_task(const TensorArg &d, uint64_t task, uint32_t *stage, uint32_t stage_words, Staged &st) {
  const bool ok = stage_task_issue<LOG2W>(d, task, stage, stage_words, st);
  wait_lds_copy();
  return ok;
}

template <int MODE, int LOG2W, int BATCH, int CP>
__device__ bool task_staged(const TensorArg &d, const uint32_t *lut, uint32_t K, const u32x2 *ptab,
                            uint64_t task, uint32_t *stage, uint32_t stage_words, uint32_t prio,
                            const uint32_t *xl, uint32_t batch, uint32_t l_min, int pre, const Staged &pst) {
  constexpr uint32_t W = 1u << LOG2W;
  constexpr uint32_t G = 64u / W;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t grp = lane >> LOG2W;
  const uint32_t j = lane & (W - 1u);
  const uint64_t c0 = task * G;

  // the staging may have been issued before the table switch (pre >= 0)
  Staged st = pst;
  if (pre < 0) {
    if (!stage_task<LOG2W>(d, task, stage, stage_words, st)) return false;
  } else {
    wait_lds_copy();
    if (!pre) return false;
  }
  const uint32_t al = st.al, cs = st.cs, nw = st.nw;
  if constexpr (MODE == kModeGemv) {
    // one chunk (LOG2W == 6) of d.chunk / cols whole rows
    const uint32_t nrows = d.chunk / d.cols;
    const uint32_t flags = gemv_rows64<BATCH>(lut, K, stage + al, rfl(nw), xl, d.cols, nrows,
                                              static_cast<float *>(d.out), c0 * nrows, d.rows, batch, lane,
                                              rfl(early_pairs(d.ahead, d.chunk >> 6, l_min)));
    if (flags) atomicOr(d.status, flags);
    return true;
  } else {
  const uint32_t steps = d.chunk >> LOG2W;
  typedef OutElem<typename std::conditional<MODE == kModeU8, uint8_t, uint16_t>::type, CP> OutT;
  // output of the task: G full chunks from chunk c0 on
  OutT *outp = static_cast<OutT *>(d.out) + c0 * d.chunk;
  const uint32_t out_bytes = (uint32_t)min((uint64_t)G * d.chunk * sizeof(OutT), (uint64_t)0xFFFFFFF0u);
  const __amdgpu_buffer_rsrc_t outr = __builtin_amdgcn_make_buffer_rsrc((void *)outp, (short)0, (int)out_bytes, 0x00020000);
  const uint32_t lane_off = grp * d.chunk + j;
  uint32_t flags;
  const bool pairs = d.refill_steps == 2u;
  if (LOG2W == 6) {
    if (pairs && ptab)
      flags = tab_pairs64<MODE, OutT>(lut, K, stage + al, rfl(nw), steps, outr, lane, prio,
                                      rfl(early_pairs(d.ahead, steps, l_min)));
    else if (pairs)
      flags = pairs64<MODE, OutT>(lut, K, stage + al, rfl(nw), steps, outr, lane,
                                  rfl(early_pairs(d.ahead, steps, l_min)));
    else flags = loop64<MODE, OutT>(lut, K, stage + al, rfl(nw), steps, outr, lane);
  } else if (LOG2W == 5) {
    const uint32_t cs0 = rfl(__shfl(cs, 0, 64)), cs1 = rfl(__shfl(cs, 32, 64));
    const uint32_t nw0 = rfl(__shfl(nw, 0, 64)), nw1 = rfl(__shfl(nw, 32, 64));
    if (pairs && ptab)
      flags = tab_pairs32<MODE, OutT>(lut, K, stage + cs0, cs1 - cs0, nw0, nw1, steps, outr, lane_off, lane, prio,
                                      rfl(early_pairs(d.ahead, steps, l_min)));
    else if (pairs)
      flags = pairs32<MODE, OutT>(lut, K, stage + cs0, cs1 - cs0, nw0, nw1, steps, outr, lane_off, lane,
                                  rfl(early_pairs(d.ahead, steps, l_min)));
    else
      flags = loop32<MODE, OutT>(lut, K, stage + cs0, cs1 - cs0, nw0, nw1, steps, outr, lane_off, lane);
  } else {
    flags = pairs ? pairs_small<MODE, LOG2W, OutT>(lut, K, stage, cs, nw, steps, outr, lane_off, lane)
                  : loop_small<MODE, LOG2W, OutT>(lut, K, stage, cs, nw, steps, outr, lane_off, lane);
  }
  if (flags) atomicOr(d.status, flags);
  return true;
  }
}

// ---------------------------------------------------------------------------
// kernel: persistent workgroups over block tasks
// ---------------------------------------------------------------------------
// Residency: on gfx950 a wavefront's scalar-register allocation limits how
// many wavefronts a SIMD holds well before the 8-wave cap (two 16-wave
// workgroups of this kernel share a CU at 62 SGPRs, only one at 87; the
// occupancy query does not see this).  The budget below keeps two workgroups
// per CU; the few values it pushes out are per-task setup, reloaded from
// VGPR lanes outside the decode loops.
template <int MODE, int LOG2W, int BATCH, int CP>
__global__ __launch_bounds__(kBlockThreads) __attribute__((amdgpu_num_sgpr(kKernelSgprs))) void ecw_kernel(
    const LaunchArgs a) {
  constexpr uint32_t G = 64u >> LOG2W;
  // dynamic LDS: the two-code table if any (first, so that its address is a
  // constant), the code table (lut_cap entries, a multiple of 4), the staged
  // activations of the GEMV (x_words), then one 16-byte aligned staging area
  // per wavefront
  u32x2 *ptab_area = reinterpret_cast<u32x2 *>(dyn_lds);
  uint32_t *lut = reinterpret_cast<uint32_t *>(dyn_lds) + (a.pair_bits ? 2u << a.pair_bits : 0u);
  uint32_t *xl = lut + a.lut_cap;
  const uint32_t wave = rfl(threadIdx.x >> 6);
  const uint32_t stage_words = a.stage_words;
  uint32_t *stage = xl + a.x_words + wave * (stage_words + kStageSlack);
  const u32x2 *ptab = nullptr;
  bool x_staged = false, x_sliced = false;
  // The workgroup's tasks: [g0, g1) of the launch's task space (the first
  // tasks_r workgroups take one more than tasks_q), walked in rounds of up to
  // kWaves tasks that stay within one tensor; wavefront w takes the w-th task
  // of a round.  Workgroups thus differ by at most one task, and within one
  // the wavefronts of each SIMD (w mod 4) share the tasks evenly.
  const uint32_t b = blockIdx.x;
  const uint32_t g0 = b * a.tasks_q + min(b, a.tasks_r);
  const uint32_t g1 = g0 + a.tasks_q + (b < a.tasks_r ? 1u : 0u);
  uint32_t cur = 0xFFFFFFFFu;
  uint32_t K = 0, l_min = 1;
  uint32_t ti = 0, round = 0;
  for (uint32_t g = g0; g < g1; ++round) {
    while (ti + 1 < a.n_tensors && a.task_begin[ti + 1] <= g) ++ti;
    const TensorArg &d = a.t[ti];
    const uint32_t n_here = min(min(g1, a.task_begin[ti + 1]) - g, (uint32_t)kWaves);
    const uint64_t task = (uint64_t)(g - a.task_begin[ti]) + wave;   // within the tensor
    const bool mine = wave < n_here;
    g += n_here;
    // On a table switch, start staging this wavefront's task first: its loads
    // are in flight while the workgroup fetches and builds the tables (the
    // staging area is the wavefront's own; if the task later takes another
    // path the copy is simply not used, and copies land in issue order).
    int pre = -1;
    Staged pst{0u, 0u, 0u};
    if (ti != cur && stage_words) {
      const bool sliced = MODE == kModeGemv && BATCH != 1 && a.x_slice &&
                          (uint64_t)(d.cols >> 1) * XSlots<BATCH>::n > a.x_words;
      const bool full = mine && (task + 1) * G <= d.n_chunks && (task + 1) * G * (uint64_t)d.chunk <= d.n_symbols;
      if (full && !sliced) pre = stage_task_issue<LOG2W>(d, task, stage, stage_words, pst) ? 1 : 0;
    }
    if (ti != cur) {
      // The table switch issues its loads before the workgroup barrier, after
      // the staging above (whose copy should not queue behind them; issued
      // ahead of it, they were slower), and writes LDS after it: the activations of a GEMV tensor that may take
      // the LDS path (W = 64, pairs, an even number of steps per row, all of
      // x within its area) from an aligned x, the table's entries (16 bytes
      // per thread from an aligned table, whose header is 16 bytes) and its
      // header.  Every wavefront checks the header itself, and the entries
      // are fetched together with it, as many as the caller's table holds (at
      // most the launch's table capacity): a table whose header fails the
      // checks is then not used.
      const bool x_fit = MODE == kModeGemv && LOG2W == 6 && a.pair_bits && stage_words && (d.cols & 127u) == 0u &&
                         (uint64_t)(d.cols >> 1) * XSlots<BATCH>::n <= a.x_words;
      const bool x_vec = x_fit && x_vec_ok(d.x);
      XRegs xr;
      if (x_vec) x_load<BATCH>(xr, d.x, d.cols, a.batch, 0u, d.cols >> 7);
      static_assert(kLutMaxEntries / 4u <= (uint32_t)kBlockThreads, "table fetch: one 16-byte load per thread");
      const uint32_t ne_fetch = min(a.lut_cap, d.lut_words > kLutHeaderWords ? d.lut_words - kLutHeaderWords : 0u);
      const uint32_t nv = ((uintptr_t)d.lut & 15u) == 0u ? ne_fetch >> 2 : 0u;
      u32x4 lv = {0u, 0u, 0u, 0u};
      uint32_t h0 = 0, h1 = 0, hne = 0, hl1 = 0;
      auto fetch_table = [&]() {
        if (threadIdx.x < nv) lv = reinterpret_cast<const u32x4 *>(d.lut + kLutHeaderWords)[threadIdx.x];
        if (d.lut_words >= kLutHeaderWords) h0 = d.lut[0], h1 = d.lut[1], hne = d.lut[2], hl1 = d.lut[3];
      };
      // with eight batch slots the activations' loads fill this window
      // already: the table follows the barrier there (measured faster)
      if (BATCH == 1) fetch_table();
      __syncthreads();
      if (BATCH != 1) fetch_table();
      if (threadIdx.x < nv)
        reinterpret_cast<u32x4 *>(lut)[threadIdx.x] =
            u32x4{kernel_entry<MODE>(lv[0]), kernel_entry<MODE>(lv[1]), kernel_entry<MODE>(lv[2]), kernel_entry<MODE>(lv[3])};
      for (uint32_t i = 4u * nv + threadIdx.x; i < ne_fetch; i += kBlockThreads)
        lut[i] = kernel_entry<MODE>(d.lut[kLutHeaderWords + i]);
      if (x_vec) x_store<BATCH>(xl, xr, d.cols >> 7);
      uint32_t k = 0;
      if (d.lut_words >= kLutHeaderWords) {
        const uint32_t ne = hne, l1 = hl1;
        const uint32_t kk = h1 & 0xFFu;
        const uint32_t lmin = h1 >> 24;
        if (h0 == kLutMagic && (h1 & 0x00FFFF00u) == d.expect_hdr && kk >= 1 && kk <= kSingleLevelMax &&
            l1 == (1u << kk) && ne >= l1 && ne <= a.lut_cap && ne <= d.lut_words - kLutHeaderWords &&
            lmin >= 1u && lmin <= kMaxCodeLen)
          k = kk | (ne << 8) | (lmin << 24);
      }
      k = rfl(k);
      if (!k && threadIdx.x == 0) atomicOr(d.status, kFLut);
      K = k & 0xFFu;
      l_min = k >> 24;
      cur = ti;
      __syncthreads();
      // two-code table for 4-bit tensors decoded in pairs
      ptab = nullptr;
      if (a.pair_bits && K && d.refill_steps == 2u && ((d.expect_hdr >> 8) & 0xFFu) == 4u && lds_at_zero()) {
        for (uint32_t i = threadIdx.x; i < (1u << kPairBits); i += kBlockThreads)
          ptab_area[i] = build_pair_entry<MODE>(lut, K, i);
        ptab = ptab_area;
      }
      // activations of a GEMV tensor that the LDS path takes (W = 64, pairs,
      // two-code table, an even number of steps per row): all of x if it
      // fits its area, else slices of it (eight batch slots)
      x_staged = x_sliced = false;
      if (MODE == kModeGemv && LOG2W == 6 && ptab && stage_words && (d.cols & 127u) == 0u) {
        if (x_fit) {
          if (!x_vec) stage_x<BATCH>(xl, d.x, d.cols, a.batch, 0u, d.cols >> 7);
          x_staged = true;
        } else if (BATCH != 1 && a.x_slice) {
          x_sliced = true;
        }
      }
      __syncthreads();
    }
    if (!K) continue;
    if (MODE == kModeGemv && x_sliced) {
      // every wavefront of the workgroup takes part in the sliced walk
      const bool full = mine && (task + 1) * G <= d.n_chunks && (task + 1) * G * (uint64_t)d.chunk <= d.n_symbols;
      Staged st{0u, 0u, 0u};
      const bool have = full && stage_task<LOG2W>(d, task, stage, stage_words, st);
      const uint32_t flags =
          gemv_sliced64<BATCH>(d, lut, K, have, stage + st.al, rfl(st.nw), xl, task * (d.chunk / d.cols), a.batch,
                               threadIdx.x & 63u, rfl(early_pairs(d.ahead, d.chunk >> 6, l_min)));
      if (flags) atomicOr(d.status, flags);
      if (mine && !have) task_generic<MODE, LOG2W, BATCH, CP>(d, lut, K, task, a.batch, l_min);
      continue;
    }
    if (!mine) continue;
    bool done = false;
    // streams encoded refilling ahead: the pair loops for W = 32, 64
    const bool ahead_ok = !d.ahead || (d.refill_steps == 2u && LOG2W >= 5);
    if (stage_words && (MODE != kModeGemv || x_staged) && ahead_ok) {
      const bool full = (task + 1) * G <= d.n_chunks && (task + 1) * G * (uint64_t)d.chunk <= d.n_symbols;
      // priority 3, 2 over the wavefront's first task, 1, 0 over the second
      const uint32_t prio = round == 0u ? 3u : (round == 1u ? 1u : 0u);
      if (full)
        done = task_staged<MODE, LOG2W, BATCH, CP>(d, lut, K, ptab, task, stage, stage_words, prio, xl, a.batch, l_min,
                                                   pre, pst);
    }
    if (!done) task_generic<MODE, LOG2W, BATCH, CP>(d, lut, K, task, a.batch, l_min);
  }
  // a copy issued ahead for a task that took another path may still be in
  // flight: let it land while the workgroup's LDS is still its own
  wait_lds_copy();
}

// Workgroup barrier over LDS only: this wavefront's LDS accesses have
// completed (lgkmcnt(0)), and its vector-memory operations in flight (ring
// and x copies) stay in flight, unlike __syncthreads(), whose fence waits
// for them all.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Matrix-core operand types and the slice write shared by the decode + GEMM
// and batched GEMV kernels.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// The pair's two bf16 weights of every lane into slice row `row` (byte
// address): neighbouring lanes swap values (as for the packed decode
// outputs), so an even lane writes columns j, j+1 and an odd lane columns
// 64 + j - 1, 64 + j, one dword each.
__device__ __forceinline__ void gemm_put(uint32_t row_addr, uint32_t lane, uint32_t ab) {
  const uint32_t nb = (uint32_t)__builtin_amdgcn_mov_dpp((int)ab, 0xB1, 0xF, 0xF, false);
  const uint32_t v = __builtin_amdgcn_perm(nb, ab, pair_sel<kModeGemv>(lane));
  const uint32_t col = (lane & ~1u) + (lane & 1u) * 64u;
  *(__attribute__((address_space(3))) uint32_t *)(uintptr_t)(row_addr + col * 2u) = v;
}

// ---------------------------------------------------------------------------
// Fused GEMV of 2..8 activation rows on the matrix cores: the streamed layout
// (W = 64, 4-bit codes, refill every two steps) with one row per chunk,
// 512 | cols and cols >= 1024.
//
// A workgroup takes whole tiles of 16 consecutive rows.  Over the T tiles of
// its share that lie in one tensor, wavefront w takes the T consecutive rows
// [16 T' + w T, ...) of that range, one contiguous run of the stream that it
// streams through its ring exactly as the batch-1 kernel does; at step r the
// r-th rows of the 16 wavefronts form a tile.  The wavefronts advance in
// lockstep by slices of four pair steps (512 columns):
// - decode: wavefront m writes each pair it decodes, as the lane holds it
//   (the bf16 weights of columns 128q + j and 128q + 64 + j in one dword),
//   into row m of an LDS tile of 16 rows x 256 dwords (two such tiles);
// - barrier;
// - multiply: wavefront w takes dwords [16w, 16w + 16) of every tile row,
//   i.e. 32 columns, as the A operand of v_mfma_f32_16x16x32_bf16 and the
//   same columns of x, paired the same way, as B (token n in column n,
//   tokens >= batch zero), accumulating 16 rows x 16 tokens in fp32.
// At a row end the 16 wavefronts' partial tiles go to LDS and, after the next
// barrier, wavefront m adds the 16 partials of its own row; the sums of up to
// 64 rows wait in registers (lane i: the wavefront's i-th row) before their
// store.  x streams through LDS as well: three buffers of one 512-column
// slice per token, which wavefront n (< batch) fills for token n two slices
// ahead with 16-byte copies that write LDS directly.  Every weight is decoded
// once; the matrix cores do every multiplication.
// ---------------------------------------------------------------------------
constexpr uint32_t kTileRowBytes = 1040;   // one A row: 256 dwords, then 16 bytes that skew the banks
constexpr uint32_t kTileXBytes = 1056;     // one token's x slice: 512 bf16, then 32 bytes that skew the banks
constexpr uint32_t kTileXBufs = 3;
constexpr uint32_t kTileLog2Ring = 9;

typedef __attribute__((address_space(3))) uint32_t lds_w32;
typedef __attribute__((address_space(3))) u32x4 lds_w32x4;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

// s_waitcnt vmcnt(n) for a wavefront-uniform n (above 15: vmcnt(15), which
// waits for more than asked)
__device__ __forceinline__ void wait_vm(uint32_t n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    case 13: __builtin_amdgcn_s_waitcnt(0x0F7D); break;
    case 14: __builtin_amdgcn_s_waitcnt(0x0F7E); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F7F); break;
  }
  asm volatile("" ::: "memory");
}

// Pairs [q0, q1) of the slice: decode, write to the wavefront's tile row
// (arow: its LDS byte address plus 4 lane), keep the ring ahead; ops counts
// the copy instructions issued.
template <bool EARLY, bool NOFB, uint32_t RL>
__device__ __forceinline__ void tile_pairs(const uint32_t *lut, uint32_t K, uint32_t q0, uint32_t q1, uint32_t arow,
                                           uint32_t &hi, uint32_t &lo, uint32_t &n, Run &R, uint32_t ring_base,
                                           uint32_t ring_v, uint32_t rmask4, uint32_t lane, uint32_t &ops) {
  for (uint32_t q = q0; q < q1; ++q) {
    const uint32_t p_old = R.p4;
    const u32x2 e2 = stream_pair<EARLY, NOFB>(lut, K, hi, lo, n, R.p4, ring_v, rmask4);
    *(lds_w32 *)(uintptr_t)(arow + 256u * q) = e2.x;
    if ((p_old ^ R.p4) >> RL) {
      ring_copy<RL>(R, ring_base, (R.p4 >> RL) + (kRingBlocks - 1u), lane);
      ring_wait2<RL>();
      ops += RingCopies<RL>::n;
    }
  }
}

// The 512 columns of slice sl of token tok's activations into LDS (x_lds:
// that token's place in the buffer), one 16-byte copy per lane.
__device__ __forceinline__ void tile_x_copy(__amdgpu_buffer_rsrc_t xr, uint32_t x_lds, uint32_t cols, uint32_t tok,
                                            uint32_t sl, uint32_t lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void *)(uintptr_t)rfl(x_lds), 16, lane * 16u,
                                           rfl(tok * cols * 2u + sl * 1024u), 0, 0);
}

// One slice's product for wavefront w: A = dwords [16w, 16w + 16) of the 16
// tile rows (lane: row lane mod 16, dwords 16w + 4 (lane / 16) .. + 3), B =
// the same columns of x for token lane mod 16 (zero past the batch), paired
// as the weights are: dword i holds columns c + i and c + 64 + i.
__device__ __forceinline__ f32x4 tile_mma(uint32_t a_lds, uint32_t x_lds, uint32_t wave, uint32_t lane,
                                          uint32_t batch, f32x4 acc) {
  const uint32_t m = lane & 15u, g = lane >> 4;
  const u32x4 av = *(lds_u32x4 *)(uintptr_t)(a_lds + m * kTileRowBytes + 4u * (16u * wave + 4u * g));
  u32x4 bv = {0u, 0u, 0u, 0u};
  if (m < batch) {
    const uint32_t c = 128u * (wave >> 2) + 16u * (wave & 3u) + 4u * g;   // column within the slice
    const u32x2 lo = *(lds_u32x2 *)(uintptr_t)(x_lds + m * kTileXBytes + 2u * c);
    const u32x2 hi = *(lds_u32x2 *)(uintptr_t)(x_lds + m * kTileXBytes + 2u * (c + 64u));
    bv[0] = (lo.x & 0xFFFFu) | (hi.x << 16);
    bv[1] = (lo.x >> 16) | (hi.x & 0xFFFF0000u);
    bv[2] = (lo.y & 0xFFFFu) | (hi.y << 16);
    bv[3] = (lo.y >> 16) | (hi.y & 0xFFFF0000u);
  }
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), acc,
                                                 0, 0, 0);
}

// Wavefront w's rows [cb, ce) (ce - cb <= T, possibly none) in lockstep with
// the workgroup's T rows per wavefront; returns the stream flags.  live: the
// run started (cb < ce and valid offsets).
template <bool NOFB, uint32_t RL>
__device__ uint32_t tile_run(const TensorArg &d, const uint32_t *lut, uint32_t K, uint32_t l_min, Run &R, bool live,
                             uint32_t cb, uint32_t ce, uint32_t T, uint32_t batch, uint32_t wave, uint32_t lane,
                             uint32_t ring_base, uint32_t a_lds, uint32_t x_lds, uint32_t red_lds) {
  const uint32_t cols = d.cols, spr = cols >> 9, rows = d.rows;
  const uint32_t nsl = T * spr;
  const uint32_t xbuf = batch * kTileXBytes;
  uint32_t ring_v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(ring_v) : "s"(ring_base));
  const uint32_t rmask4 = rfl((4u << RL) - 1u);
  const uint32_t early_n = rfl(early_pairs(d.ahead, cols >> 6, l_min));
  float *y = static_cast<float *>(d.out);
  // x: wavefront `wave` < batch copies token `wave`; o_a (o_b) counts the
  // vector-memory instructions issued after the oldest (newest) copy in flight
  const bool xw = wave < batch;
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void *)d.x, (short)0, (int)(batch * cols * 2u), 0x00020000);
  uint32_t o_a = 0, o_b = 0, nx = 0;
  if (xw) {
    tile_x_copy(xr, x_lds + wave * kTileXBytes, cols, wave, 0u, lane);
    ++nx;
    if (nsl > 1u) {
      tile_x_copy(xr, x_lds + xbuf + wave * kTileXBytes, cols, wave, 1u % spr, lane);
      ++nx;
      o_a = 1u;
    }
  }
  if (live) wait_vm(2u * RingCopies<RL>::n + nx);   // blocks 0 and 1 of the run have landed
  uint32_t flags = 0;
  bool dead = !live;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  uint32_t hi = 0, lo = 0, n = 0, end4 = 0;
  uint32_t ycnt = 0;
  uint64_t yrow0 = cb;
  float yv[8];
#pragma unroll
  for (uint32_t b = 0; b < 8u; ++b) yv[b] = 0.f;
  bool pend = false, pend_row = false, row_live = false;
  // the 16 partial sums of this wavefront's row (lane n: token n) into lane
  // ycnt's registers, and the store of every 64 rows
  auto take_row = [&](bool store) {
    float s = 0.f;
    if (lane < batch) {
      const uint32_t src = red_lds + (16u * (wave >> 2) + lane) * 16u + 4u * (wave & 3u);
#pragma unroll
      for (uint32_t v = 0; v < (uint32_t)kWaves; ++v) s += __builtin_bit_cast(float, *(lds_u32 *)(uintptr_t)(src + v * 1024u));
    }
    if (!store) return;
#pragma unroll
    for (uint32_t b = 0; b < 8u; ++b) {
      const float sb = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), (int)b));
      yv[b] = lane == ycnt ? sb : yv[b];
    }
    if (++ycnt == 64u) {
#pragma unroll
      for (uint32_t b = 0; b < 8u; ++b)
        if (b < batch) y[(uint64_t)b * rows + yrow0 + lane] = yv[b];
      yrow0 += 64u;
      ycnt = 0;
    }
  };
  uint32_t r = 0, sl = 0;
  for (uint32_t t = 0; t < nsl; ++t) {
    const uint32_t arow = a_lds + (t & 1u) * (16u * kTileRowBytes) + wave * kTileRowBytes + 4u * lane;
    if (sl == 0u) {
      row_live = !dead && cb + r < ce;
      if (row_live && r != 0u && (r & 63u) == 0u) {   // the next 64 rows' end offsets
        const uint64_t o_start = R.base * 32u + R.p4 * 8u;
        if (!load_ends(d, R, cb + r, ce, o_start, lane, R.ends)) {
          flags |= kFOffsets;
          dead = true, row_live = false;
        }
      }
    }
    if (row_live) {
      if (sl == 0u) {
        end4 = __builtin_amdgcn_readlane(R.ends, (int)(r & 63u));
        hi = 0, lo = 0, n = 0;
        ring_fetch(~0ull, hi, lo, n, R.p4, ring_v, rmask4);
        const uint32_t p_old = R.p4;
        R.p4 = rfl(R.p4 + 256u);
        if ((p_old ^ R.p4) >> RL) {
          ring_copy<RL>(R, ring_base, (R.p4 >> RL) + (kRingBlocks - 1u), lane);
          ring_wait2<RL>();
          o_a += RingCopies<RL>::n, o_b += RingCopies<RL>::n;
        }
      }
      const uint32_t q0 = 4u * sl;
      const uint32_t qe = early_n > q0 ? min(early_n - q0, 4u) : 0u;
      uint32_t ops = 0;
      tile_pairs<true, NOFB, RL>(lut, K, 0u, qe, arow, hi, lo, n, R, ring_base, ring_v, rmask4, lane, ops);
      tile_pairs<false, NOFB, RL>(lut, K, qe, 4u, arow, hi, lo, n, R, ring_base, ring_v, rmask4, lane, ops);
      o_a += ops, o_b += ops;
      if (sl == spr - 1u) {
        if (R.p4 != end4) flags |= R.p4 < end4 ? kFUnderrun : kFOverrun;
        if (hi | lo) flags |= kFPadding;
        if (R.p4 != end4) dead = true;   // malformed: the rest of the run is not decoded
      }
    } else {
#pragma unroll
      for (uint32_t q = 0; q < 4u; ++q) *(lds_w32 *)(uintptr_t)(arow + 256u * q) = 0u;
    }
    if (xw) wait_vm(o_a);   // this slice's x has landed
    lds_barrier();
    o_a = o_b, o_b = 0;
    if (xw && t + 2u < nsl) {
      tile_x_copy(xr, x_lds + ((t + 2u) % kTileXBufs) * xbuf + wave * kTileXBytes, cols, wave, (t + 2u) % spr, lane);
      o_a += 1u;
    }
    if (pend) {
      take_row(pend_row);
      pend = false;
    }
    acc = tile_mma(a_lds + (t & 1u) * (16u * kTileRowBytes), x_lds + (t % kTileXBufs) * xbuf, wave, lane, batch, acc);
    if (++sl == spr) {
      *(lds_w32x4 *)(uintptr_t)(red_lds + (wave * 64u + lane) * 16u) = __builtin_bit_cast(u32x4, acc);
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      pend = true, pend_row = row_live;
      sl = 0, ++r;
    }
  }
  lds_barrier();
  if (pend) take_row(pend_row);
  if (ycnt) {
#pragma unroll
    for (uint32_t b = 0; b < 8u; ++b)
      if (b < batch && lane < ycnt) y[(uint64_t)b * rows + yrow0 + lane] = yv[b];
  }
  return flags;
}

template <uint32_t RL>
__global__ __launch_bounds__(kBlockThreads) void ecw_gemv_tile_kernel(const StreamArgs a) {
  // Setup in dependent rounds, each issued before anything waits on it, as
  // in the streamed kernel.  Dynamic LDS: the two-code table (at LDS address
  // 0), the code table (lut_cap entries), the table-state word, the two A
  // tiles, the x buffers, the partial sums of a row end, then one ring per
  // wavefront.
  const uint32_t lut_cap = a.lut_cap, flag_word = a.flag_word, ring_off = a.ring_off, batch = a.batch;
  const uint32_t tile_a_off = a.tile_a_off, tile_x_off = a.tile_x_off, tile_red_off = a.tile_red_off;
  const uint32_t b = blockIdx.x;
  uint32_t nwg, bl;
  const uint32_t tw = wg_tensor(a, b, nwg, bl);
  const TensorArg d = a.t[tw];
  const uint32_t n_t = a.chunk_begin[tw + 1] - a.chunk_begin[tw];   // tiles of 16 rows
  u32x2 *ptab = reinterpret_cast<u32x2 *>(dyn_lds);
  uint32_t *lut = reinterpret_cast<uint32_t *>(dyn_lds) + (2u << kPairBitsWide);
  uint32_t *state = reinterpret_cast<uint32_t *>(dyn_lds) + flag_word;
  const uint32_t wave = rfl(threadIdx.x >> 6);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t lds0 = lds_addr(dyn_lds);
  const uint32_t ring_base = rfl(lds0 + ring_off + (wave << (RL + 2u)));
  const uint32_t a_lds = rfl(lds0 + tile_a_off), x_lds = rfl(lds0 + tile_x_off), red_lds = rfl(lds0 + tile_red_off);
  // the workgroup's tiles [t0, t0 + T), an even part of tensor tw's; wavefront
  // w takes rows r0 + w T .. of them
  const uint32_t t0 = bl * (n_t / nwg) + min(bl, n_t % nwg);
  const uint32_t T = n_t / nwg + (bl < n_t % nwg ? 1u : 0u);
  const uint32_t r0 = t0 * 16u;
  const uint32_t r1 = min(r0 + 16u * T, d.n_chunks);
  const uint32_t cb = min(r0 + wave * T, r1), ce = min(cb + T, r1);
  {
    // the headers of both tables (in place of a missing or short table, the
    // first 16 bytes of the chunk offsets are read and ignored), the run's
    // bounds
    const bool hv = d.lut_words >= kLutHeaderWords;
    const bool pt = d.plut != nullptr;
    const uint32_t *const offs32 = reinterpret_cast<const uint32_t *>(d.offs);
    const u32x4 hh = *(const __attribute__((address_space(4))) u32x4 *)(uintptr_t)(hv ? d.lut : offs32);
    const u32x4 ph = *(const __attribute__((address_space(4))) u32x4 *)(uintptr_t)(pt ? d.plut : offs32);
    const uint32_t h0 = hh[0], h1 = hh[1], hne = hh[2], hl1 = hh[3];
    const uint32_t p0 = ph[0], p1 = ph[1], p2 = ph[2];
    const __attribute__((address_space(4))) uint64_t *co =
        (const __attribute__((address_space(4))) uint64_t *)(uintptr_t)d.offs;
    const uint64_t o0 = co[cb], o1 = co[ce];
    if (!lds_at_zero()) {   // the two-code table is addressed from LDS address 0
      if (threadIdx.x == 0) atomicOr(d.status, kFLut);
      return;
    }
    // the two-code table's copy (nothing reads that LDS yet) and the table
    // entries into registers, in flight while the run's bounds arrive
    if (pt) ptab_copy(d.plut, wave, lane);
    const uint32_t ne_fetch = min(lut_cap, d.lut_words > kLutHeaderWords ? d.lut_words - kLutHeaderWords : 0u);
    const uint32_t nv = ((uintptr_t)d.lut & 15u) == 0u ? ne_fetch >> 2 : 0u;
    u32x4 lv = {0u, 0u, 0u, 0u};
    if (threadIdx.x < nv) lv = reinterpret_cast<const u32x4 *>(d.lut + kLutHeaderWords)[threadIdx.x];
    Run R;
    const bool have = cb < ce;
    const bool run_ok = have && run_begin<RL>(d, cb, ce, o0, o1, ring_base, lane, R);
    // table entries and the table-state word before the one set-up barrier,
    // as in the streamed kernel
    if (threadIdx.x == 0) *state = 0u;
    if (threadIdx.x < nv)
      reinterpret_cast<u32x4 *>(lut)[threadIdx.x] =
          u32x4{kernel_entry<kModeGemv>(lv[0]), kernel_entry<kModeGemv>(lv[1]), kernel_entry<kModeGemv>(lv[2]),
                kernel_entry<kModeGemv>(lv[3])};
    for (uint32_t i = 4u * nv + threadIdx.x; i < ne_fetch; i += kBlockThreads)
      lut[i] = kernel_entry<kModeGemv>(d.lut[kLutHeaderWords + i]);
    uint32_t k = 0;
    if (hv) {
      const uint32_t kk = h1 & 0xFFu, lmin = h1 >> 24;
      if (h0 == kLutMagic && (h1 & 0x00FFFF00u) == d.expect_hdr && kk >= 1 && kk <= kSingleLevelMax &&
          hl1 == (1u << kk) && hne >= hl1 && hne <= lut_cap && hne <= d.lut_words - kLutHeaderWords &&
          lmin >= 1u && lmin <= kMaxCodeLen)
        k = kk | (lmin << 24);
    }
    if (pt && (p0 != kPairLutMagic || p2 != h1)) k = 0u;   // not this code's two-code table
    k = rfl(k);
    if (!k && threadIdx.x == 0) atomicOr(d.status, kFLut);
    const uint32_t K = k & 0xFFu, l_min = k >> 24;
    __syncthreads();
    // two-code table (unless copied); does any index miss a whole pair?
    bool nofb = (p1 & kPairLutWhole) != 0u;
    if (!pt) {
      bool miss = false;
      if (K) {
        for (uint32_t i = threadIdx.x; i < (1u << kPairBitsWide); i += kBlockThreads) {
          const u32x2 e = build_pair_entry<kModeGemv, kPairBitsWide>(lut, K, i);
          ptab[i] = e;
          miss |= (e.y & kPairFallback) != 0u;
        }
      }
      if (__ballot(miss) && lane == 0) atomicOr(state, 1u);
      __syncthreads();
      nofb = rfl(*state) == 0u;
    }
    if (!K) {
      wait_lds_copy();   // the run's first copies land before the workgroup ends
      return;
    }
    uint32_t flags = have && !run_ok ? kFOffsets : 0u;
    flags |= nofb ? tile_run<true, RL>(d, lut, K, l_min, R, run_ok, cb, ce, T, batch, wave, lane, ring_base, a_lds,
                                       x_lds, red_lds)
                  : tile_run<false, RL>(d, lut, K, l_min, R, run_ok, cb, ce, T, batch, wave, lane, ring_base, a_lds,
                                        x_lds, red_lds);
    if (flags && lane == 0) atomicOr(d.status, flags);
  }
  wait_lds_copy();
}

// ---------------------------------------------------------------------------
// decode + GEMM for prompts (y[t][o] = sum_k deq(W[o][k]) x[t][k], up to
// 256 tokens per launch: one 16-token group per wavefront)
//
// A workgroup owns tiles of 16 CH consecutive rows (CH = 1, 2 or 4).
// Wavefront w decodes rows w, 16 + w, ... of a tile (chains 0..CH-1), each
// streamed through a ring of four 64-word blocks in LDS, one pair of steps
// (128 columns) per chain and slice, into a double-buffered LDS slice of the
// tile's rows; after an LDS-only barrier it multiplies the slice on the
// matrix cores (v_mfma_f32_16x16x32_bf16: A = 16 rows x 32 columns of the
// slice, B = 32 columns x 16 tokens of x, fp32 accumulation) for its token
// group, with x operands loaded into registers a slice ahead and reused by
// the tile's CH 16-row blocks.  Every weight is decoded once per launch.
//
// Ring waits: a pair step reads at most 64 words, one block, so a chain
// enters at most one new block per slice.  After its step in every slice a
// chain copies the block three past P's into the slot of the block before
// P's (again, while P stays in one block: the same bytes), so the last copy
// of the block after P's was issued while P was two blocks back, at least
// two slices earlier.  Before decoding a slice the wavefront therefore waits
// only for the copies and x loads issued before the previous slice's.
// Every slice issues the same memory operations, CH copies and 4 NT x
// loads, whatever the data: the waits are constant and the compiler's own
// waits for the x operands count exactly.  A chain without a row (past the
// tensor's last row, or whose offsets were refused) copies the tensor's
// first offsets instead, which lie inside their buffer; a copy wholly
// outside its buffer could complete ahead of earlier loads.
// ---------------------------------------------------------------------------
constexpr uint32_t kGemmRingLog2 = 8;       // rings of 256 words, blocks of 64

// A tile of CH rows per wavefront (CH = 4: 64 rows; CH = 2: 32 rows).
template <int CH>
struct GemmTile {
  static constexpr uint32_t rows = (uint32_t)CH * kWaves;
  static constexpr uint32_t slice_bytes = rows * kGemmRowStride * 2u;
};

struct GemmChain {
  Run R;
  uint32_t hi, lo, n;
  uint32_t end4;
};

// One pair step of a chain whose two-code table holds whole pairs, as
// stream_pair<EARLY, true> computes it, without branches: every lane reads
// the ring word it would take and looks the pair up again, and the lanes
// that take a word keep the results.  Steps of several chains written one
// after another can then be interleaved.  (A lane that takes no word reads
// a word of its own ring: the index is masked to the ring.)
template <bool EARLY>
__device__ __forceinline__ uint32_t gemm_pair_nofb(uint32_t &hi, uint32_t &lo, uint32_t &n, uint32_t &p4,
                                                   uint32_t ring_v, uint32_t rmask4) {
  u32x2 e2 = *(lds_u32x2 *)(uintptr_t)((hi >> (32u - kPairBitsWide)) << 3);
  const bool take = EARLY ? n < 32u : ((e2.y >> 8) & 0xFFu) > n;
  const uint64_t m = __builtin_amdgcn_ballot_w64(take);
  const uint32_t idx = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  uint32_t a;
  asm("v_lshl_add_u32 %0, %1, 2, %2\n\tv_and_or_b32 %0, %0, %3, %4"
      : "=&v"(a) : "v"(idx), "s"(p4), "s"(rmask4), "v"(ring_v));
  const uint32_t w = *(lds_u32 *)(uintptr_t)a;
  const uint32_t hi2 = hi | (w >> (n & 31u));
  const uint32_t lo2 = __builtin_amdgcn_alignbit(w, 0u, n);
  if (!EARLY) {   // the pair is looked up again with the word merged in
    const u32x2 e2b = *(lds_u32x2 *)(uintptr_t)((hi2 >> (32u - kPairBitsWide)) << 3);
    e2.x = take ? e2b.x : e2.x;
    e2.y = take ? e2b.y : e2.y;
  }
  hi = take ? hi2 : hi;
  lo = take ? lo2 : lo;
  n = take ? n + 32u : n;
  p4_add(p4, m);
  const uint32_t nhi = __builtin_amdgcn_alignbit(hi, lo, e2.y);
  lo = __builtin_amdgcn_alignbit(lo, 0u, e2.y);
  hi = nhi;
  n = sub_len(n, e2.y);
  return e2.x;
}

// x operands of slice q.  Every lane loads: a lane past the tokens reads the
// last token's row, and the products of those columns are not stored.
template <int NT>
__device__ __forceinline__ void gemm_b_load(u32x4 (&bo)[NT][4], const uint16_t *x, uint32_t cols, uint32_t n_tokens,
                                            uint32_t wave, uint32_t lane, uint32_t q) {
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const uint32_t tok = min((wave + (uint32_t)tt * (uint32_t)kWaves) * 16u + (lane & 15u), n_tokens - 1u);
    const u32x4 *p = reinterpret_cast<const u32x4 *>(x + (uint64_t)tok * cols + q * kGemmSliceCols + 8u * (lane >> 4));
#pragma unroll
    for (uint32_t ks = 0; ks < 4u; ++ks) bo[tt][ks] = p[ks * 4u];
  }
}

// The tile of rows [r0, r0 + 64) (rows < d.rows): decode, multiply, write y.
template <int NT, int CH, bool NOFB>
__device__ uint32_t gemm_tile(const TensorArg &d, const uint32_t *lut, uint32_t K, uint32_t l_min, uint32_t r0,
                              uint32_t n_tokens, uint32_t wave, uint32_t lane, uint32_t ring0, uint32_t slices) {
  const uint32_t cols = d.cols, rows = d.rows, q_n = cols / kGemmSliceCols;
  const uint32_t tok_groups = (n_tokens + 15u) >> 4;
  const uint32_t rmask4 = rfl((4u << kGemmRingLog2) - 1u);
  const uint32_t early_n = rfl(early_pairs(d.ahead, cols >> 6, l_min));
  uint32_t flags = 0;
  // the chains' runs (one row each) and their first four blocks
  GemmChain C[CH];
  bool live[CH];
  uint32_t ring_b[CH], ring_vv[CH];
#pragma unroll
  for (uint32_t c = 0; c < (uint32_t)CH; ++c) {
    const uint32_t row = r0 + 16u * c + wave;
    ring_b[c] = rfl(ring0 + c * (4u << kGemmRingLog2));
    asm volatile("v_mov_b32 %0, %1" : "=v"(ring_vv[c]) : "s"(ring_b[c]));
    live[c] = row < rows;
    C[c].hi = C[c].lo = C[c].n = 0u;
    C[c].end4 = 0u;
    if (live[c]) {
      const __attribute__((address_space(4))) uint64_t *co =
          (const __attribute__((address_space(4))) uint64_t *)(uintptr_t)d.offs;
      const bool ok = run_begin<kGemmRingLog2>(d, row, row + 1u, co[row], co[row + 1u], ring_b[c], lane, C[c].R);
      if (!ok) {
        flags |= kFOffsets;
        live[c] = false;
      } else {
        C[c].end4 = __builtin_amdgcn_readlane(C[c].R.ends, 0);
      }
    }
    if (!live[c]) {   // copies read the first 16 bytes of the offsets (two of them exist)
      C[c].R.r = __builtin_amdgcn_make_buffer_rsrc((void *)d.offs, (short)0, 16, 0x00020000);
      C[c].R.klast = 0u;
      C[c].R.bytes = 16u;
      C[c].R.p4 = 0u;
    }
  }
  wait_vm(0u);   // every ring's first four blocks
  // each row's first decision point: every lane takes one word
#pragma unroll
  for (uint32_t c = 0; c < (uint32_t)CH; ++c) {
    if (!live[c]) continue;
    ring_fetch(~0ull, C[c].hi, C[c].lo, C[c].n, C[c].R.p4, ring_vv[c], rmask4);
    const uint32_t p_old = C[c].R.p4;
    C[c].R.p4 = rfl(C[c].R.p4 + 256u);
    if ((p_old ^ C[c].R.p4) >> kGemmRingLog2)
      ring_copy<kGemmRingLog2>(C[c].R, ring_b[c], (C[c].R.p4 >> kGemmRingLog2) + (kRingBlocks - 1u), lane);
  }
  f32x4 acc[CH][NT];
#pragma unroll
  for (uint32_t c = 0; c < (uint32_t)CH; ++c)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[c][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Slice 0 is decoded before the loop; between two barriers a wavefront
  // then multiplies slice q - 1 and decodes slice q, in that order in half of
  // the wavefronts of each SIMD and in the other order in the rest, so that
  // each SIMD's matrix cores and vector ALUs run at once.  Right after its
  // products a wavefront loads the x operands of the next slice into the
  // same registers: a decode lies between those loads and their use, and the
  // wavefronts' loads are spread over the interval (loading two slices ahead
  // measured slower).  The last interval multiplies only.
  constexpr uint32_t kOps = (uint32_t)CH * RingCopies<kGemmRingLog2>::n + 4u * NT;   // per interval
  const bool decode_first = (wave & 4u) != 0u;
  auto decode = [&](uint32_t q) {
    const uint32_t buf = slices + (q & 1u) * GemmTile<CH>::slice_bytes;
    uint32_t ab[CH];
    if (NOFB) {   // every chain steps (one without a row decodes its own ring), without branches
      if (q < early_n) {
#pragma unroll
        for (uint32_t c = 0; c < (uint32_t)CH; ++c)
          ab[c] = gemm_pair_nofb<true>(C[c].hi, C[c].lo, C[c].n, C[c].R.p4, ring_vv[c], rmask4);
      } else {
#pragma unroll
        for (uint32_t c = 0; c < (uint32_t)CH; ++c)
          ab[c] = gemm_pair_nofb<false>(C[c].hi, C[c].lo, C[c].n, C[c].R.p4, ring_vv[c], rmask4);
      }
#pragma unroll
      for (uint32_t c = 0; c < (uint32_t)CH; ++c) ab[c] = live[c] ? ab[c] : 0u;
    } else if (q < early_n) {
#pragma unroll
      for (uint32_t c = 0; c < (uint32_t)CH; ++c)
        ab[c] = live[c] ? stream_pair<true, NOFB>(lut, K, C[c].hi, C[c].lo, C[c].n, C[c].R.p4, ring_vv[c], rmask4).x
                        : 0u;
    } else {
#pragma unroll
      for (uint32_t c = 0; c < (uint32_t)CH; ++c)
        ab[c] = live[c] ? stream_pair<false, NOFB>(lut, K, C[c].hi, C[c].lo, C[c].n, C[c].R.p4, ring_vv[c], rmask4).x
                        : 0u;
    }
#pragma unroll
    for (uint32_t c = 0; c < (uint32_t)CH; ++c) gemm_put(buf + (16u * c + wave) * kGemmRowStride * 2u, lane, ab[c]);
    // every chain copies the block three past P's, whether or not P entered a new block
#pragma unroll
    for (uint32_t c = 0; c < (uint32_t)CH; ++c)
      ring_copy<kGemmRingLog2>(C[c].R, ring_b[c], (C[c].R.p4 >> kGemmRingLog2) + (kRingBlocks - 1u), lane);
  };
  // A: rows 16c + lane mod 16 of the slice, columns 32 ks + 8 (lane / 16);
  // a k step's fragments are all read before its products
  auto multiply = [&](uint32_t q, const u32x4 (&b)[NT][4]) {
    const uint32_t a_addr = slices + (q & 1u) * GemmTile<CH>::slice_bytes +
                            ((lane & 15u) * kGemmRowStride + 8u * (lane >> 4)) * 2u;
    auto a_frag = [&](uint32_t c, uint32_t ks) {
      return __builtin_bit_cast(bf16x8, *(__attribute__((address_space(3))) const u32x4 *)(uintptr_t)(
                                            a_addr + 16u * c * kGemmRowStride * 2u + ks * 64u));
    };
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      if (wave + (uint32_t)tt * (uint32_t)kWaves >= tok_groups) continue;   // no tokens in this group
#pragma unroll
      for (uint32_t ks = 0; ks < 4u; ++ks) {
        bf16x8 av[CH];
#pragma unroll
        for (uint32_t c = 0; c < (uint32_t)CH; ++c) av[c] = a_frag(c, ks);
#pragma unroll
        for (uint32_t c = 0; c < (uint32_t)CH; ++c)
          acc[c][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[c], __builtin_bit_cast(bf16x8, b[tt][ks]), acc[c][tt],
                                                               0, 0, 0);
      }
    }
  };
  u32x4 bx[NT][4];
  gemm_b_load<NT>(bx, d.x, cols, n_tokens, wave, lane, 0u);
  decode(0u);
  lds_barrier();
  for (uint32_t q = 1; q < q_n; ++q) {
    wait_vm(kOps);   // copies and loads issued before the previous interval
    if (!decode_first) {
      multiply(q - 1u, bx);
      gemm_b_load<NT>(bx, d.x, cols, n_tokens, wave, lane, q);
    }
    decode(q);
    if (decode_first) {
      multiply(q - 1u, bx);
      gemm_b_load<NT>(bx, d.x, cols, n_tokens, wave, lane, q);
    }
    lds_barrier();
  }
  multiply(q_n - 1u, bx);
  // row ends
#pragma unroll
  for (uint32_t c = 0; c < (uint32_t)CH; ++c) {
    if (!live[c]) continue;
    if (C[c].R.p4 != C[c].end4) flags |= C[c].R.p4 < C[c].end4 ? kFUnderrun : kFOverrun;
    if (C[c].hi | C[c].lo) flags |= kFPadding;
  }
  // D of 16-row block c, token group g: lane holds rows 16c + 4 (lane / 16)
  // + v for token 16 g + lane mod 16
  float *y = static_cast<float *>(d.out);
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const uint32_t tok = (wave + (uint32_t)tt * (uint32_t)kWaves) * 16u + (lane & 15u);
    if (tok < n_tokens) {
#pragma unroll
      for (uint32_t c = 0; c < (uint32_t)CH; ++c)
#pragma unroll
        for (uint32_t v = 0; v < 4u; ++v) {
          const uint32_t o = r0 + 16u * c + 4u * (lane >> 4) + v;
          if (o < rows) y[(uint64_t)tok * rows + o] = acc[c][tt][v];
        }
    }
  }
  wait_lds_copy();   // copies past the rows' ends may still be in flight into the rings
  lds_barrier();     // every wavefront is done with both slices before the next tile writes them
  return flags;
}

// Four wavefronts per SIMD (one workgroup per CU), whatever the register
// count below 128.
template <int NT, int CH>
__global__ __launch_bounds__(kBlockThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void ecw_gemm_ring_kernel(
    const StreamArgs a) {
  // Set-up as in the matrix-core GEMV.  Dynamic LDS: the two-code table (at
  // LDS address 0), the code table (lut_cap entries), the table-state word,
  // the two 64-row slices, then four rings per wavefront.
  const uint32_t lut_cap = a.lut_cap, flag_word = a.flag_word, ring_off = a.ring_off, n_tokens = a.batch;
  const uint32_t slices_off = a.tile_a_off;
  const uint32_t b = blockIdx.x;
  uint32_t nwg, bl;
  const uint32_t tw = wg_tensor(a, b, nwg, bl);
  const TensorArg d = a.t[tw];
  const uint32_t n_t = a.chunk_begin[tw + 1] - a.chunk_begin[tw];   // tiles of 16 CH rows
  u32x2 *ptab = reinterpret_cast<u32x2 *>(dyn_lds);
  uint32_t *lut = reinterpret_cast<uint32_t *>(dyn_lds) + (2u << kPairBitsWide);
  uint32_t *state = reinterpret_cast<uint32_t *>(dyn_lds) + flag_word;
  const uint32_t wave = rfl(threadIdx.x >> 6);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t lds0 = lds_addr(dyn_lds);
  const uint32_t ring0 = rfl(lds0 + ring_off + wave * ((uint32_t)CH << (kGemmRingLog2 + 2u)));
  const uint32_t slices = rfl(lds0 + slices_off);
  const uint32_t t0 = bl * (n_t / nwg) + min(bl, n_t % nwg);
  const uint32_t T = n_t / nwg + (bl < n_t % nwg ? 1u : 0u);
  const bool hv = d.lut_words >= kLutHeaderWords;
  const bool pt = d.plut != nullptr;
  const uint32_t *const offs32 = reinterpret_cast<const uint32_t *>(d.offs);
  const u32x4 hh = *(const __attribute__((address_space(4))) u32x4 *)(uintptr_t)(hv ? d.lut : offs32);
  const u32x4 ph = *(const __attribute__((address_space(4))) u32x4 *)(uintptr_t)(pt ? d.plut : offs32);
  const uint32_t h0 = hh[0], h1 = hh[1], hne = hh[2], hl1 = hh[3];
  const uint32_t p0 = ph[0], p1 = ph[1], p2 = ph[2];
  if (!lds_at_zero()) {   // the two-code table is addressed from LDS address 0
    if (threadIdx.x == 0) atomicOr(d.status, kFLut);
    return;
  }
  if (pt) ptab_copy(d.plut, wave, lane);   // nothing reads that LDS yet
  const uint32_t ne_fetch = min(lut_cap, d.lut_words > kLutHeaderWords ? d.lut_words - kLutHeaderWords : 0u);
  const uint32_t nv = ((uintptr_t)d.lut & 15u) == 0u ? ne_fetch >> 2 : 0u;
  u32x4 lv = {0u, 0u, 0u, 0u};
  if (threadIdx.x < nv) lv = reinterpret_cast<const u32x4 *>(d.lut + kLutHeaderWords)[threadIdx.x];
  __syncthreads();
  if (threadIdx.x == 0) *state = 0u;
  if (threadIdx.x < nv)
    reinterpret_cast<u32x4 *>(lut)[threadIdx.x] =
        u32x4{kernel_entry<kModeGemv>(lv[0]), kernel_entry<kModeGemv>(lv[1]), kernel_entry<kModeGemv>(lv[2]),
              kernel_entry<kModeGemv>(lv[3])};
  for (uint32_t i = 4u * nv + threadIdx.x; i < ne_fetch; i += kBlockThreads)
    lut[i] = kernel_entry<kModeGemv>(d.lut[kLutHeaderWords + i]);
  uint32_t k = 0;
  if (hv) {
    const uint32_t kk = h1 & 0xFFu, lmin = h1 >> 24;
    if (h0 == kLutMagic && (h1 & 0x00FFFF00u) == d.expect_hdr && kk >= 1 && kk <= kSingleLevelMax &&
        hl1 == (1u << kk) && hne >= hl1 && hne <= lut_cap && hne <= d.lut_words - kLutHeaderWords &&
        lmin >= 1u && lmin <= kMaxCodeLen)
      k = kk | (lmin << 24);
  }
  if (pt && (p0 != kPairLutMagic || p2 != h1)) k = 0u;   // not this code's two-code table
  k = rfl(k);
  if (!k && threadIdx.x == 0) atomicOr(d.status, kFLut);
  const uint32_t K = k & 0xFFu, l_min = k >> 24;
  __syncthreads();
  bool nofb = (p1 & kPairLutWhole) != 0u;
  if (!pt) {
    bool miss = false;
    if (K) {
      for (uint32_t i = threadIdx.x; i < (1u << kPairBitsWide); i += kBlockThreads) {
        const u32x2 e = build_pair_entry<kModeGemv, kPairBitsWide>(lut, K, i);
        ptab[i] = e;
        miss |= (e.y & kPairFallback) != 0u;
      }
    }
    if (__ballot(miss) && lane == 0) atomicOr(state, 1u);
    __syncthreads();
    nofb = rfl(*state) == 0u;
  }
  if (!K) return;
  uint32_t flags = 0;
  for (uint32_t t = t0; t < t0 + T; ++t) {
    flags |= nofb ? gemm_tile<NT, CH, true>(d, lut, K, l_min, t * GemmTile<CH>::rows, n_tokens, wave, lane, ring0,
                                            slices)
                  : gemm_tile<NT, CH, false>(d, lut, K, l_min, t * GemmTile<CH>::rows, n_tokens, wave, lane, ring0,
                                             slices);
  }
  if (flags && lane == 0) atomicOr(d.status, flags);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

// Workgroup cap of every launch (entro_set_max_workgroups; 0: none).
static std::atomic<uint32_t> g_max_workgroups{0};

static uint64_t cap_grid(uint64_t grid) {
  const uint32_t cap = g_max_workgroups.load(std::memory_order_relaxed);
  return cap && grid > cap ? cap : grid;
}

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
  if (t.refill_steps > 2 || t.refill_ahead > 1 || t.out_cached > 1) return ENTRO_E_FORMAT;
  if (t.n_symbols == 0) return ENTRO_OK;
  if (!t.d_lut || !t.d_words || !t.d_chunk_bit_off) return ENTRO_E_INVAL;
  const uint64_t nc = (t.n_symbols + t.chunk_symbols - 1) / t.chunk_symbols;
  if (nc > 0xFFFFFFFFull) return ENTRO_E_UNSUPPORTED;
  return ENTRO_OK;
}

template <int MODE, int L, int BATCH, int CP>
static hipError_t launch_one(uint32_t total_tasks, LaunchArgs &a, size_t dyn, hipStream_t s) {
  auto kern = ecw_kernel<MODE, L, BATCH, CP>;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipGetLastError();
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kBlockThreads, dyn) != hipSuccess || per_cu < 1)
    per_cu = 1;
  // Plan with less LDS than the CU has: workgroups that fill it to the last
  // KiB are not all resident at once, and the persistent grid then runs in
  // two rounds.
  const int lds_fit = (int)((kLdsPerCu - kLdsPlanReserve) / (dyn + kStaticLds));
  if (lds_fit >= 1 && per_cu > lds_fit) per_cu = lds_fit;
  if (cus < 1) cus = 1;
  // k workgroups per CU on every CU, k the fewest that give each wavefront
  // a task (at most per_cu; fewer workgroups than CUs if there are fewer
  // tasks), the tasks spread over them evenly.  A second workgroup per CU
  // only when the first ones are full leaves room on the CUs for work on
  // other streams (decoding ahead of a consumer).
  const uint64_t k = std::min<uint64_t>((uint64_t)per_cu,
                                        (total_tasks + (uint64_t)kWaves * cus - 1) / ((uint64_t)kWaves * cus));
  const uint32_t grid = (uint32_t)cap_grid(std::min<uint64_t>((uint64_t)cus * std::max<uint64_t>(k, 1), total_tasks));
  a.tasks_q = total_tasks / grid;
  a.tasks_r = total_tasks % grid;
  // clear an error left by an earlier call (ours, such as a failed occupancy
  // query, or the caller's): the check below then sees this launch alone
  (void)hipGetLastError();
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlockThreads), dyn, s, a);
  return hipGetLastError();
}

template <int MODE, int BATCH, int CP>
static hipError_t launch_w(uint32_t log2w, uint32_t total_tasks, LaunchArgs &a, size_t dyn, hipStream_t s) {
  switch (log2w) {
    case 0: return launch_one<MODE, 0, BATCH, CP>(total_tasks, a, dyn, s);
    case 1: return launch_one<MODE, 1, BATCH, CP>(total_tasks, a, dyn, s);
    case 2: return launch_one<MODE, 2, BATCH, CP>(total_tasks, a, dyn, s);
    case 3: return launch_one<MODE, 3, BATCH, CP>(total_tasks, a, dyn, s);
    case 4: return launch_one<MODE, 4, BATCH, CP>(total_tasks, a, dyn, s);
    case 5: return launch_one<MODE, 5, BATCH, CP>(total_tasks, a, dyn, s);
    default: return launch_one<MODE, 6, BATCH, CP>(total_tasks, a, dyn, s);
  }
}

// Streamed GEMV launches (ecw_gemv_stream_kernel): tensors with 64 lanes,
// 4-bit codes, refill every two steps, 128 | cols, a stream below 4 GiB,
// and activations that fit the LDS block (eight batch slots when batch > 1).
// Rings of 1024 words (blocks of 64 lanes x 16 bytes), or of 512 words
// (blocks of 2 x 64 lanes x 4 bytes) where that lets two workgroups share a
// CU or is needed to fit at all.
constexpr uint32_t kStreamLog2Ring = 10;
constexpr uint32_t kStreamLog2RingSmall = 9;

// LDS bytes of a streamed launch (code table of lut_cap entries, x_words of
// activations, rings of 2^log2r words); sets the layout fields of a if given.
static size_t stream_lds_bytes(uint64_t lut_cap, uint64_t x_words, uint32_t log2r, StreamArgs *a = nullptr) {
  size_t dyn = ((size_t)8u << kPairBitsWide) + (size_t)lut_cap * 4u + (size_t)x_words * 4u;
  if (a) a->flag_word = (uint32_t)(dyn / 4u);
  dyn += 16u;
  const size_t ring_bytes = (size_t)4u << log2r;
  dyn = (dyn + ring_bytes - 1u) / ring_bytes * ring_bytes;
  if (a) a->ring_off = (uint32_t)dyn, a->log2_ring = log2r;
  return dyn + (size_t)kWaves * ring_bytes;
}

static bool stream_fits(uint64_t lut_cap, uint64_t x_words, uint32_t log2r = kStreamLog2RingSmall) {
  return stream_lds_bytes((lut_cap + 3) & ~3ull, (x_words + 3) & ~3ull, log2r) + kStaticLds <=
         kLdsPerCu - kLdsPlanReserve;
}

// Ring size of a launch: 512 words if that gives two workgroups per CU where
// 1024 give one, or if 1024 do not fit; else 1024.
static uint32_t stream_ring(uint64_t lut_cap, uint64_t x_words) {
  const size_t budget = kLdsPerCu - kLdsPlanReserve;
  const size_t big = stream_lds_bytes(lut_cap, x_words, kStreamLog2Ring) + kStaticLds;
  const size_t small = stream_lds_bytes(lut_cap, x_words, kStreamLog2RingSmall) + kStaticLds;
  if (big > budget) return kStreamLog2RingSmall;
  if (2u * big > budget && 2u * small <= budget) return kStreamLog2RingSmall;
  return kStreamLog2Ring;
}

static uint64_t stream_lut_entries(const entro_tensor &t) {
  const uint64_t w = std::min<uint64_t>(t.lut_bytes / 4, kLutHeaderWords + kLutMaxEntries);
  return w > kLutHeaderWords ? w - kLutHeaderWords : 0;
}

static uint64_t stream_x_words(const entro_gemv_item &g, uint32_t batch) {
  return (uint64_t)(g.cols >> 1) * (batch == 1 ? 1u : 8u);
}

static bool stream_ok(const entro_tensor &t, const entro_gemv_item &g, uint32_t batch) {
  if (t.n_symbols == 0 || t.lanes != 64u || t.sym_bits != 4u || t.refill_steps != 2u) return false;
  if (g.cols == 0 || (g.cols & 127u) || t.chunk_symbols % g.cols) return false;
  if (t.n_words >= (1ull << 30)) return false;
  const uint64_t xw = stream_x_words(g, batch);   // the activation staging moves at most kGemvXMaxBytes
  return xw * 4u <= kGemvXMaxBytes && stream_fits(stream_lut_entries(t), xw);
}

// The workgroups of a streamed or matrix-core launch, split by tensor, so
// that no workgroup's share straddles two tensors (a straddling workgroup
// decodes its two parts one after the other, each after a table switch,
// while the others decode one).  Tensor i gets floor(grid n_i / total)
// workgroups, at least one and at most its n_i chunks or tiles; the rest of
// the grid goes to the largest remainders.  The split stays within grid (the
// resident workgroups) unless there are more tensors than that.  Returns the
// launch's grid.
static uint32_t split_grid(StreamArgs &a, uint32_t total, uint64_t grid) {
  const uint32_t nt = a.n_tensors;
  grid = std::min<uint64_t>(grid, (uint64_t)(kMaxStreamWgs - kMaxStreamTensors));   // the workgroup table
  uint64_t w[kMaxStreamTensors], rem[kMaxStreamTensors], n[kMaxStreamTensors];
  uint64_t used = 0;
  for (uint32_t i = 0; i < nt; ++i) {
    n[i] = a.chunk_begin[i + 1] - a.chunk_begin[i];
    w[i] = std::max<uint64_t>(1, std::min<uint64_t>(n[i] * grid / total, n[i]));
    rem[i] = (n[i] * grid) % total;
    used += w[i];
  }
  while (used < grid) {   // the largest remainder among tensors with a chunk to spare
    int best = -1;
    for (uint32_t i = 0; i < nt; ++i)
      if (w[i] < n[i] && (best < 0 || rem[i] > rem[best])) best = (int)i;
    if (best < 0) break;
    ++w[best], ++used;
    rem[best] = 0;
  }
  uint32_t wb = 0;
  for (uint32_t i = 0; i < nt; ++i) {
    a.wg_count[i] = (uint16_t)w[i];
    for (uint32_t j = 0; j < (uint32_t)w[i]; ++j) a.wg_info[wb + j] = (uint16_t)(i << 12 | j);
    wb += (uint32_t)w[i];
  }
  return wb;
}

// How a GEMV tensor is launched: the matrix-core kernel, the streamed one,
// or (0) the staged or generic paths of ecw_kernel.
constexpr char kTakeStream = 1, kTakeTile = 2;

struct StreamPlan {
  StreamArgs a;
  size_t dyn;
  uint32_t total;
};

template <int BATCH>
static hipError_t launch_stream(StreamPlan &pl, hipStream_t s) {
  auto kern = BATCH == 1 ? (pl.a.log2_ring == kStreamLog2Ring ? ecw_gemv_stream_kernel<kStreamLog2Ring>
                                                              : ecw_gemv_stream_kernel<kStreamLog2RingSmall>)
                         : (pl.a.log2_ring == kStreamLog2Ring ? ecw_gemv8_stream_kernel<kStreamLog2Ring>
                                                              : ecw_gemv8_stream_kernel<kStreamLog2RingSmall>);
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipGetLastError();
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kBlockThreads, pl.dyn) != hipSuccess || per_cu < 1)
    per_cu = 1;
  const int lds_fit = (int)((kLdsPerCu - kLdsPlanReserve) / (pl.dyn + kStaticLds));
  if (lds_fit >= 1 && per_cu > lds_fit) per_cu = lds_fit;
  if (cus < 1) cus = 1;
  // as for the decode kernel: the fewest workgroups per CU that give every
  // wavefront a chunk, the chunks spread evenly
  const uint64_t k = std::min<uint64_t>((uint64_t)per_cu,
                                        (pl.total + (uint64_t)kWaves * cus - 1) / ((uint64_t)kWaves * cus));
  const uint32_t grid = split_grid(pl.a, pl.total,
                                  cap_grid(std::min<uint64_t>((uint64_t)cus * std::max<uint64_t>(k, 1), pl.total)));
  (void)hipGetLastError();
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlockThreads), pl.dyn, s, pl.a);
  return hipGetLastError();
}

// Plan the streamed launches of the tensors marked in `take` (groups of up to
// 32).
// The tensor arguments of a streamed or matrix-core GEMV launch.
static void stream_tensor_arg(TensorArg &d, const entro_tensor &x, const entro_gemv_item &gi, uint32_t *status,
                              uint64_t nc) {
  d.lut = static_cast<const uint32_t *>(x.d_lut);
  d.plut = (reinterpret_cast<uintptr_t>(x.d_pair_lut) & 15u) == 0u ? static_cast<const uint32_t *>(x.d_pair_lut)
                                                                    : nullptr;
  d.words = x.d_words;
  d.offs = x.d_chunk_bit_off;
  d.status = status;
  d.n_words = x.n_words;
  d.n_symbols = x.n_symbols;
  d.chunk = x.chunk_symbols;
  d.n_chunks = (uint32_t)nc;
  d.expect_hdr = (x.sym_bits << 8) | (x.max_len << 16);
  d.lut_words = (uint32_t)std::min<uint64_t>(x.lut_bytes / 4, kLutHeaderWords + kLutMaxEntries);
  d.refill_steps = 2u;
  d.ahead = x.refill_ahead;
  d.out = gi.d_y;
  d.x = gi.d_x;
  d.rows = gi.rows;
  d.cols = gi.cols;
  d.n_tasks = (uint32_t)nc;
}

static entro_status plan_stream(const entro_tensor *t, size_t n, const entro_gemv_item *g, uint32_t batch,
                                uint32_t *d_status, const std::vector<char> &take, std::vector<StreamPlan> &plans) {
  size_t i = 0;
  while (i < n) {
    plans.emplace_back();
    StreamPlan &pl = plans.back();
    std::memset(&pl, 0, sizeof pl);
    StreamArgs &a = pl.a;
    a.batch = batch;
    uint32_t total = 0, k = 0;
    uint64_t lut_need = 0, x_need = 0;
    for (; i < n && k < (uint32_t)kMaxStreamTensors; ++i) {
      if (take[i] != kTakeStream) continue;
      const entro_tensor &x = t[i];
      const uint64_t nc = (x.n_symbols + x.chunk_symbols - 1) / x.chunk_symbols;
      if ((uint64_t)total + nc > 0x7FFFFFFFull) break;
      // a tensor whose table or activations would overflow this launch's LDS
      // starts the next one (each fits alone: stream_ok)
      if (k && !stream_fits(std::max(lut_need, stream_lut_entries(x)), std::max(x_need, stream_x_words(g[i], batch))))
        break;
      stream_tensor_arg(a.t[k], x, g[i], d_status + i, nc);
      a.chunk_begin[k] = total;
      total += (uint32_t)nc;
      lut_need = std::max<uint64_t>(lut_need, stream_lut_entries(x));
      x_need = std::max<uint64_t>(x_need, stream_x_words(g[i], batch));
      ++k;
    }
    if (k == 0) {
      plans.pop_back();
      continue;
    }
    a.n_tensors = k;
    for (uint32_t r = k; r <= (uint32_t)kMaxStreamTensors; ++r) a.chunk_begin[r] = total;
    a.lut_cap = (uint32_t)((lut_need + 3) & ~3ull);
    a.x_words = (uint32_t)((x_need + 3) & ~3ull);
    pl.dyn = stream_lds_bytes(a.lut_cap, a.x_words, stream_ring(a.lut_cap, a.x_words), &a);
    if (pl.dyn + kStaticLds > kLdsPerCu - kLdsPlanReserve) return ENTRO_E_UNSUPPORTED;   // not reached (stream_ok)
    pl.total = total;
  }
  return ENTRO_OK;
}

// Matrix-core GEMV launches (ecw_gemv_tile_kernel): batch 2..8, tensors of
// the streamed layout with one row per chunk, 512 | cols, cols >= 1024, and x
// 16-byte aligned (its slices are copied 16 bytes a lane).

// LDS bytes of a matrix-core launch (code table of lut_cap entries); sets the
// layout fields of a if given.
static size_t tile_lds_bytes(uint64_t lut_cap, uint32_t batch, StreamArgs *a = nullptr) {
  size_t dyn = ((size_t)8u << kPairBitsWide) + (size_t)lut_cap * 4u;
  if (a) a->flag_word = (uint32_t)(dyn / 4u);
  dyn = (dyn + 16u + 15u) & ~(size_t)15u;
  if (a) a->tile_a_off = (uint32_t)dyn;
  dyn += 2u * 16u * kTileRowBytes;
  if (a) a->tile_x_off = (uint32_t)dyn;
  dyn += (size_t)kTileXBufs * batch * kTileXBytes;
  if (a) a->tile_red_off = (uint32_t)dyn;
  dyn += (size_t)kWaves * 64u * 16u;
  const size_t ring_bytes = (size_t)4u << kTileLog2Ring;
  dyn = (dyn + ring_bytes - 1u) / ring_bytes * ring_bytes;
  if (a) a->ring_off = (uint32_t)dyn, a->log2_ring = kTileLog2Ring;
  return dyn + (size_t)kWaves * ring_bytes;
}

static bool tile_fits(uint64_t lut_cap, uint32_t batch) {
  return tile_lds_bytes((lut_cap + 3) & ~3ull, batch) + kStaticLds <= kLdsPerCu - kLdsPlanReserve;
}

static bool tile_ok(const entro_tensor &t, const entro_gemv_item &g, uint32_t batch) {
  if (batch < 2u || batch > 8u) return false;
  if (t.n_symbols == 0 || t.lanes != 64u || t.sym_bits != 4u || t.refill_steps != 2u) return false;
  if (g.cols < 1024u || (g.cols & 511u) || t.chunk_symbols != g.cols) return false;
  if (t.n_words >= (1ull << 30) || (reinterpret_cast<uintptr_t>(g.d_x) & 15u)) return false;
  if ((uint64_t)batch * g.cols * 2u > 0x7FFFFFFFull) return false;
  return tile_fits(stream_lut_entries(t), batch);
}

static hipError_t launch_tile(StreamPlan &pl, hipStream_t s) {
  auto kern = ecw_gemv_tile_kernel<kTileLog2Ring>;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipGetLastError();
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kBlockThreads, pl.dyn) != hipSuccess || per_cu < 1)
    per_cu = 1;
  const int lds_fit = (int)((kLdsPerCu - kLdsPlanReserve) / (pl.dyn + kStaticLds));
  if (lds_fit >= 1 && per_cu > lds_fit) per_cu = lds_fit;
  if (cus < 1) cus = 1;
  // every workgroup resident at once, the tiles spread evenly
  const uint32_t grid =
      split_grid(pl.a, pl.total, cap_grid(std::min<uint64_t>((uint64_t)cus * (uint64_t)per_cu, pl.total)));
  (void)hipGetLastError();
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlockThreads), pl.dyn, s, pl.a);
  return hipGetLastError();
}

// Plan the matrix-core launches of the tensors marked in `take` (groups of up
// to kMaxStreamTensors; chunk_begin counts tiles of 16 rows).
static entro_status plan_tile(const entro_tensor *t, size_t n, const entro_gemv_item *g, uint32_t batch,
                              uint32_t *d_status, const std::vector<char> &take, std::vector<StreamPlan> &plans) {
  size_t i = 0;
  while (i < n) {
    plans.emplace_back();
    StreamPlan &pl = plans.back();
    std::memset(&pl, 0, sizeof pl);
    StreamArgs &a = pl.a;
    a.batch = batch;
    uint32_t total = 0, k = 0;
    uint64_t lut_need = 0;
    for (; i < n && k < (uint32_t)kMaxStreamTensors; ++i) {
      if (take[i] != kTakeTile) continue;
      const entro_tensor &x = t[i];
      const uint64_t nc = (x.n_symbols + x.chunk_symbols - 1) / x.chunk_symbols;
      const uint64_t tiles = (nc + 15u) / 16u;
      if ((uint64_t)total + tiles > 0x7FFFFFFFull) break;
      if (k && !tile_fits(std::max(lut_need, stream_lut_entries(x)), batch)) break;
      stream_tensor_arg(a.t[k], x, g[i], d_status + i, nc);
      a.chunk_begin[k] = total;
      total += (uint32_t)tiles;
      lut_need = std::max<uint64_t>(lut_need, stream_lut_entries(x));
      ++k;
    }
    if (k == 0) {
      plans.pop_back();
      continue;
    }
    a.n_tensors = k;
    for (uint32_t r = k; r <= (uint32_t)kMaxStreamTensors; ++r) a.chunk_begin[r] = total;
    a.lut_cap = (uint32_t)((lut_need + 3) & ~3ull);
    pl.dyn = tile_lds_bytes(a.lut_cap, batch, &a);
    if (pl.dyn + kStaticLds > kLdsPerCu - kLdsPlanReserve) return ENTRO_E_UNSUPPORTED;   // not reached (tile_ok)
    pl.total = total;
  }
  return ENTRO_OK;
}

// One planned launch: its arguments, dynamic LDS bytes and task count.
struct LaunchPlan {
  LaunchArgs a;
  size_t dyn;
  uint32_t total, log2w;
  bool cached;
};

// Validate everything and plan every launch (groups of up to 32 tensors that
// share a lane count and an output cache policy), then enqueue them: a call
// that fails validation or planning enqueues nothing.
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
    } else if (t[i].n_symbols) {
      // neighbouring lanes' outputs are stored together (2 or 4 bytes)
      const uintptr_t align = mode == kModeU8 ? 2u : 4u;
      if (!outs[i] || (reinterpret_cast<uintptr_t>(outs[i]) & (align - 1u))) return ENTRO_E_INVAL;
    }
  }
  // GEMV tensors of the streamed layout take the streamed kernel
  // (batch 2..8: where the activations do not fit the streamed kernel's LDS
  // block, the matrix-core kernel, which streams them in slices)
  std::vector<char> take(n, 0);
  std::vector<StreamPlan> splans, tplans;
  if (mode == kModeGemv) {
    bool any_s = false, any_t = false;
    for (size_t j = 0; j < n; ++j) {
      if (stream_ok(t[j], g[j], batch)) take[j] = kTakeStream, any_s = true;
      else if (tile_ok(t[j], g[j], batch)) take[j] = kTakeTile, any_t = true;
    }
    if (any_t) {
      const entro_status st = plan_tile(t, n, g, batch, d_status, take, tplans);
      if (st != ENTRO_OK) return st;
    }
    if (any_s) {
      const entro_status st = plan_stream(t, n, g, batch, d_status, take, splans);
      if (st != ENTRO_OK) return st;
    }
  }
  std::vector<LaunchPlan> plans;
  size_t i = 0;
  while (i < n) {
    plans.emplace_back();
    LaunchPlan &pl = plans.back();
    std::memset(&pl, 0, sizeof pl);
    LaunchArgs &a = pl.a;
    a.batch = batch;
    uint32_t total = 0, log2w = 0, k = 0;
    bool cached = false;   // output cache policy of the launch (GEMV: unused)
    uint64_t stage_need = 0, lut_need = 0, x_fit_words = 0;
    bool x_slices = false;
    bool stage_known = true, want_pairs = false;
    for (; i < n && k < (uint32_t)kMaxTensorsPerLaunch; ++i) {
      const entro_tensor &x = t[i];
      if (x.n_symbols == 0 || take[i]) continue;
      const uint32_t lw = log2u(x.lanes);
      const bool xc = mode != kModeGemv && x.out_cached;
      if (k == 0) log2w = lw, cached = xc;
      else if (lw != log2w || xc != cached) break;
      // the launch's task space stays below 2^31 tasks
      const uint64_t chunks_per_wave = 64u >> lw;
      const uint64_t tasks = ((x.n_symbols + x.chunk_symbols - 1) / x.chunk_symbols + chunks_per_wave - 1) / chunks_per_wave;
      if (tasks > 0x7FFFFFFFull) return ENTRO_E_UNSUPPORTED;
      if ((uint64_t)total + tasks > 0x7FFFFFFFull) break;
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
      d.refill_steps = x.refill_steps == 2u ? 2u : 1u;
      d.ahead = x.refill_ahead;
      if (d.refill_steps == 2u && x.sym_bits == 4u) want_pairs = true;
      if (mode == kModeGemv) {
        d.out = g[i].d_y;
        d.x = g[i].d_x;
        d.rows = g[i].rows;
        d.cols = g[i].cols;
        if ((d.cols & 127u) == 0u) {
          const uint64_t xw = (uint64_t)(d.cols >> 1) * (batch == 1 ? 1u : 8u);
          if (xw * 4u <= kGemvXMaxBytes) x_fit_words = std::max<uint64_t>(x_fit_words, xw);
          else if (batch != 1) x_slices = true;
        }
      } else {
        d.out = outs[i];
      }
      d.n_tasks = (uint32_t)tasks;
      a.task_begin[k] = total;
      total += (uint32_t)tasks;
      lut_need = std::max<uint64_t>(lut_need, d.lut_words > kLutHeaderWords ? d.lut_words - kLutHeaderWords : 0);
      if (x.max_chunk_words) stage_need = std::max<uint64_t>(stage_need, chunks_per_wave * x.max_chunk_words);
      else stage_known = false, stage_need = std::max<uint64_t>(stage_need, (x.n_words + tasks - 1) / tasks * 5 / 4 + 64);
      ++k;
    }
    if (k == 0) {
      plans.pop_back();
      continue;
    }
    a.n_tensors = k;
    for (uint32_t r = k; r <= (uint32_t)kMaxTensorsPerLaunch; ++r) a.task_begin[r] = total;
    (void)stage_known;
    // LDS: the largest table of the launch, then the staging areas (room for
    // the largest task plus 16-byte alignment), within 160 KiB
    a.lut_cap = (uint32_t)((lut_need + 3) & ~3ull);
    a.pair_bits = want_pairs ? kPairBits : 0u;
    size_t dyn = (size_t)a.lut_cap * 4u + (a.pair_bits ? (size_t)8u << a.pair_bits : 0u);
    // GEMV from LDS: W = 64 with pairs, and the launch's largest activation
    // block within kGemvXMaxBytes; otherwise every GEMV task takes the
    // generic path
    bool stage = mode != kModeGemv;
    if (mode == kModeGemv && log2w == 6 && want_pairs) {
      // x of every tensor that fits kGemvXMaxBytes, or two slice buffers
      // for those that do not (eight batch slots)
      const uint64_t slice_words = x_slices ? 2u * kGemvSlicePairs * 64u * 8u : 0u;
      const uint64_t x_words = std::max<uint64_t>(x_fit_words, slice_words);
      if (x_words) {
        a.x_words = (uint32_t)((x_words + 3u) & ~3ull);
        a.x_slice = x_slices ? 1u : 0u;
        dyn += (size_t)a.x_words * 4u;
        stage = true;
      }
    }
    if (stage) {
      const uint64_t cap = ((kLdsPerCu - kStaticLds) / 4u - dyn / 4u) / kWaves - kStageSlack;
      uint64_t sw = (stage_need + 3 + 3) & ~3ull;
      sw = std::max<uint64_t>(64, std::min<uint64_t>(sw, cap & ~3ull));
      a.stage_words = (uint32_t)sw;
      dyn += (size_t)kWaves * (sw + kStageSlack) * 4u;
    }
    pl.dyn = dyn;
    pl.total = total;
    pl.log2w = log2w;
    pl.cached = cached;
  }
  for (StreamPlan &tp : tplans)
    if (launch_tile(tp, s) != hipSuccess) return ENTRO_E_HIP;
  for (StreamPlan &sp : splans) {
    const hipError_t err = batch == 1 ? launch_stream<1>(sp, s) : launch_stream<8>(sp, s);
    if (err != hipSuccess) return ENTRO_E_HIP;
  }
  for (LaunchPlan &pl : plans) {
    hipError_t err;
    const uint32_t log2w = pl.log2w, total = pl.total;
    const size_t dyn = pl.dyn;
    LaunchArgs &a = pl.a;
    if (mode == kModeU8 && pl.cached) err = launch_w<kModeU8, 1, kStoreCached>(log2w, total, a, dyn, s);
    else if (mode == kModeU8) err = launch_w<kModeU8, 1, kStoreNT>(log2w, total, a, dyn, s);
    else if (mode == kModeBf16 && pl.cached) err = launch_w<kModeBf16, 1, kStoreCached>(log2w, total, a, dyn, s);
    else if (mode == kModeBf16) err = launch_w<kModeBf16, 1, kStoreNT>(log2w, total, a, dyn, s);
    else if (batch == 1) err = launch_w<kModeGemv, 1, kStoreNT>(log2w, total, a, dyn, s);
    else err = launch_w<kModeGemv, 8, kStoreNT>(log2w, total, a, dyn, s);
    if (err != hipSuccess) return ENTRO_E_HIP;
  }
  return ENTRO_OK;
}

// decode + GEMM (ecw_gemm_ring_kernel): tensors of the streamed layout (64
// lanes, 4-bit codes, refill every two steps, one row per chunk, 128 | cols,
// a stream below 4 GiB).  A launch takes at most kGemmRingMaxTokens tokens
// (one 16-token group per wavefront); longer prompts are split.
constexpr uint32_t kGemmRingMaxTokens = 16u * kWaves;

// LDS bytes of a launch of ch rows per wavefront (code table of lut_cap
// entries); sets the layout fields of a if given.
static size_t gemm_ring_lds_bytes(uint64_t lut_cap, uint32_t ch, StreamArgs *a = nullptr) {
  size_t dyn = ((size_t)8u << kPairBitsWide) + (size_t)lut_cap * 4u;
  if (a) a->flag_word = (uint32_t)(dyn / 4u);
  dyn = (dyn + 16u + 15u) & ~(size_t)15u;
  if (a) a->tile_a_off = (uint32_t)dyn;
  dyn += 2u * (size_t)ch * kWaves * kGemmRowStride * 2u;
  const size_t ring_bytes = (size_t)4u << kGemmRingLog2;
  dyn = (dyn + ring_bytes - 1u) / ring_bytes * ring_bytes;
  if (a) a->ring_off = (uint32_t)dyn, a->log2_ring = kGemmRingLog2;
  return dyn + (size_t)kWaves * ch * ring_bytes;
}

static bool gemm_ring_fits(uint64_t lut_entries, uint32_t ch = 4) {
  return gemm_ring_lds_bytes((lut_entries + 3) & ~3ull, ch) + kStaticLds <= kLdsPerCu - kLdsPlanReserve;
}


static entro_status plan_gemm_ring(const entro_tensor *t, size_t n, const entro_gemv_item *g, uint32_t n_tokens,
                                   uint32_t ch, uint32_t *d_status, std::vector<StreamPlan> &plans) {
  size_t i = 0;
  while (i < n) {
    plans.emplace_back();
    StreamPlan &pl = plans.back();
    std::memset(&pl, 0, sizeof pl);
    StreamArgs &a = pl.a;
    a.batch = n_tokens;
    uint32_t total = 0, k = 0;
    uint64_t lut_need = 0;
    for (; i < n && k < (uint32_t)kMaxStreamTensors; ++i) {
      const entro_tensor &x = t[i];
      if (x.n_symbols == 0) continue;
      const uint64_t nc = (x.n_symbols + x.chunk_symbols - 1) / x.chunk_symbols;
      const uint64_t tiles = (g[i].rows + 16u * ch - 1u) / (16u * ch);
      if ((uint64_t)total + tiles > 0x7FFFFFFFull) break;
      if (k && !gemm_ring_fits(std::max(lut_need, stream_lut_entries(x)), ch)) break;
      stream_tensor_arg(a.t[k], x, g[i], d_status + i, nc);
      a.chunk_begin[k] = total;
      total += (uint32_t)tiles;
      lut_need = std::max<uint64_t>(lut_need, stream_lut_entries(x));
      ++k;
    }
    if (k == 0) {
      plans.pop_back();
      continue;
    }
    a.n_tensors = k;
    for (uint32_t r = k; r <= (uint32_t)kMaxStreamTensors; ++r) a.chunk_begin[r] = total;
    a.lut_cap = (uint32_t)((lut_need + 3) & ~3ull);
    pl.dyn = gemm_ring_lds_bytes(a.lut_cap, ch, &a);
    if (pl.dyn + kStaticLds > kLdsPerCu - kLdsPlanReserve) return ENTRO_E_UNSUPPORTED;   // not reached (gemm_ring_ok)
    pl.total = total;
  }
  return ENTRO_OK;
}

static hipError_t launch_gemm_ring(StreamPlan &pl, uint32_t ch, hipStream_t s) {
  auto kern = ch == 4u ? ecw_gemm_ring_kernel<1, 4> : ch == 2u ? ecw_gemm_ring_kernel<1, 2> : ecw_gemm_ring_kernel<1, 1>;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipGetLastError();
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kBlockThreads, pl.dyn) != hipSuccess || per_cu < 1)
    per_cu = 1;
  const int lds_fit = (int)((kLdsPerCu - kLdsPlanReserve) / (pl.dyn + kStaticLds));
  if (lds_fit >= 1 && per_cu > lds_fit) per_cu = lds_fit;
  if (cus < 1) cus = 1;
  // every workgroup resident at once, the tiles spread evenly
  const uint32_t grid =
      split_grid(pl.a, pl.total, cap_grid(std::min<uint64_t>((uint64_t)cus * (uint64_t)per_cu, pl.total)));
  (void)hipGetLastError();
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlockThreads), pl.dyn, s, pl.a);
  return hipGetLastError();
}

static entro_status run_gemm(const entro_tensor *t, size_t n, const entro_gemv_item *g, uint32_t n_tokens,
                             uint32_t *d_status, hipStream_t s) {
  if (n == 0) return ENTRO_OK;
  if (!t || !g || !d_status || n_tokens < 1 || n_tokens > kGemmMaxTokens) return ENTRO_E_INVAL;
  for (size_t i = 0; i < n; ++i) {
    const entro_status st = check_tensor(t[i]);
    if (st != ENTRO_OK) return st;
    const entro_gemv_item &it = g[i];
    if ((uint64_t)it.rows * it.cols != t[i].n_symbols) return ENTRO_E_INVAL;
    if (t[i].n_symbols == 0) continue;
    if (!it.d_x || !it.d_y || (reinterpret_cast<uintptr_t>(it.d_x) & 15u)) return ENTRO_E_INVAL;
    if (it.cols % kGemmSliceCols || t[i].chunk_symbols != it.cols) return ENTRO_E_FORMAT;
    if (t[i].lanes != 64u || t[i].sym_bits != 4u || t[i].refill_steps != 2u) return ENTRO_E_UNSUPPORTED;
  }
  // Tile height: 64 rows where the call has a 64-row tile for every CU, 32
  // where its 32-row tiles fill three quarters of the CUs, else 16 (on a
  // Mistral-shaped layer: gate/up, q/k/v and o/down respectively, each the
  // fastest of the three at 1 to 256 tokens); lower if the tables do not
  // fit the LDS beside the taller tiles.
  uint64_t tiles64 = 0, tiles32 = 0, lut_need = 0;
  for (size_t i = 0; i < n; ++i) {
    if (t[i].n_symbols == 0) continue;
    if (t[i].n_words >= (1ull << 30)) return ENTRO_E_UNSUPPORTED;
    tiles64 += (g[i].rows + 63u) / 64u;
    tiles32 += (g[i].rows + 31u) / 32u;
    lut_need = std::max<uint64_t>(lut_need, stream_lut_entries(t[i]));
  }
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  uint32_t ch = tiles64 >= (uint64_t)cus ? 4u : 4u * tiles32 >= 3u * (uint64_t)cus ? 2u : 1u;
  while (ch > 1u && !gemm_ring_fits(lut_need, ch)) ch >>= 1;
  if (!gemm_ring_fits(lut_need, ch)) return ENTRO_E_UNSUPPORTED;   // not reached: tables hold at most 4096 entries
  // every launch planned before any is enqueued; prompts of more than
  // kGemmRingMaxTokens tokens in parts of that many, each with its own x and
  // y rows
  std::vector<StreamPlan> plans;
  std::vector<entro_gemv_item> part(n);
  for (uint32_t t0 = 0; t0 < n_tokens; t0 += kGemmRingMaxTokens) {
    const uint32_t nt = std::min(n_tokens - t0, kGemmRingMaxTokens);
    for (size_t i = 0; i < n; ++i) {
      part[i] = g[i];
      if (t[i].n_symbols == 0) continue;
      part[i].d_x = static_cast<const uint16_t *>(g[i].d_x) + (size_t)t0 * g[i].cols;
      part[i].d_y = static_cast<float *>(g[i].d_y) + (size_t)t0 * g[i].rows;
    }
    const entro_status st = plan_gemm_ring(t, n, part.data(), nt, ch, d_status, plans);
    if (st != ENTRO_OK) return st;
  }
  for (auto &pl : plans)
    if (launch_gemm_ring(pl, ch, s) != hipSuccess) return ENTRO_E_HIP;
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

extern "C" entro_status entro_decode_gemm(const entro_tensor *t, size_t n, const entro_gemv_item *g,
                                          uint32_t n_tokens, uint32_t *d_status, hipStream_t stream) {
  return run_gemm(t, n, g, n_tokens, d_status, stream);
}

extern "C" uint32_t entro_set_max_workgroups(uint32_t n) { return g_max_workgroups.exchange(n); }
