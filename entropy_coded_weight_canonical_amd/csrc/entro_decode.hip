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
#include <cstring>
#include <type_traits>

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
// decoded in pairs: entry i (the next kPairBits stream bits) holds, in its
// first word, the pair's two output values packed as by pack_ab and, in the
// second, the pair's summed length in byte 1 and its alignbit shift in bits
// [4:0], so that one 8-byte read gives a whole pair.  Indices whose A and B
// do not both fit in kPairBits bits carry kPairFallback in byte 0 (length 0);
// lanes that hit one look the two codes up in the code table instead.
__device__ __forceinline__ uint32_t pair_word(uint32_t lab) { return (lab << 8) | ((32u - lab) & 31u); }

template <int MODE>
__device__ u32x2 build_pair_entry(const uint32_t *lut, uint32_t K, uint32_t i) {
  const uint32_t hi = i << (32u - kPairBits);
  const uint32_t eA = lookup(lut, hi, K);
  const uint32_t lA = entry_len(eA);
  u32x2 r;
  r.x = 0u;
  r.y = kPairFallback | 0xFF00u;   // length byte above any loaded count
  if (lA <= kPairBits) {
    const uint32_t eB = lookup(lut, hi << lA, K);
    const uint32_t lB = entry_len(eB);
    if (lA + lB <= kPairBits) {
      r.x = pack_ab<MODE>(eA, eB);
      r.y = pair_word(lA + lB);
    }
  }
  return r;
}

template <int MODE>
__device__ __forceinline__ u32x2 pair_lookup(const uint32_t *lut, uint32_t K, uint32_t hi, uint32_t lo) {
  u32x2 e2 = *(lds_u32x2 *)(uintptr_t)((hi >> (32u - kPairBits)) << 3);   // table at LDS address 0
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

// ---------------------------------------------------------------------------
// decode + GEMM (prefill, n_tokens up to kGemmMaxTokens):
//   y[t][o] = sum_k deq(W[o][k]) * x[t][k]
// A workgroup owns kWaves consecutive rows of one matrix; wavefront w
// decodes row w of the tile (its chunk: one row, W = 64, 4-bit codes in
// pairs through the two-code table).  Each pair of steps gives a lane the
// weights of columns 128q + j and 128q + 64 + j; the wavefronts write them
// (packed like the decode outputs) into one of two LDS slices of
// kWaves x 128 bf16, and after a workgroup barrier every wavefront that owns
// 16-token groups multiplies the slice with them on the matrix cores
// (v_mfma_f32_16x16x32_bf16: A = 16 rows x 32 columns of the slice,
// B = 32 columns x 16 tokens of x, fp32 accumulation), while the next pair
// is decoded into the other slice.  Every weight is decoded once.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Decode the next pair of steps of a GEMM row (no arithmetic on it).
__device__ __forceinline__ u32x2 gemm_pair(GemvLane<1> &g, const uint32_t *lut, uint32_t K, uint32_t early) {
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
  return e2;
}

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

// 16 consecutive bytes of x (8 bf16) as an MFMA operand; zero past the tokens.
__device__ __forceinline__ bf16x8 gemm_x8(const uint16_t *x, uint32_t cols, uint32_t tok, uint32_t n_tokens,
                                          uint32_t col) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (tok < n_tokens) v = *reinterpret_cast<const u32x4 *>(x + (uint64_t)tok * cols + col);
  return __builtin_bit_cast(bf16x8, v);
}

// Activations of one slice (the tile's 128 columns of every token) staged in
// LDS for prompts of at most kGemmXlTokens tokens: 16-byte units, unit u =
// token u / 16, columns 8 (u % 16) .. +7; two units per thread at most.
struct XSliceRegs { u32x4 v[2]; };

__device__ __forceinline__ void gemm_x_load(XSliceRegs &r, const uint16_t *x, uint32_t cols, uint32_t n_tokens,
                                            uint32_t units, uint32_t col0) {
#pragma unroll
  for (uint32_t h = 0; h < 2u; ++h) {
    const uint32_t u = threadIdx.x + h * kBlockThreads;
    const uint32_t tok = u >> 4;
    r.v[h] = u32x4{0u, 0u, 0u, 0u};
    if (u < units && tok < n_tokens)
      r.v[h] = *reinterpret_cast<const u32x4 *>(x + (uint64_t)tok * cols + col0 + 8u * (u & 15u));
  }
}

__device__ __forceinline__ void gemm_x_store(const XSliceRegs &r, uint32_t xs_addr, uint32_t units) {
#pragma unroll
  for (uint32_t h = 0; h < 2u; ++h) {
    const uint32_t u = threadIdx.x + h * kBlockThreads;
    if (u < units)
      *(__attribute__((address_space(3))) u32x4 *)(uintptr_t)(xs_addr + ((u >> 4) * kGemmRowStride + 8u * (u & 15u)) * 2u) =
          r.v[h];
  }
}

template <int NT, bool XL>
__global__ __launch_bounds__(kBlockThreads) __attribute__((amdgpu_num_sgpr(kKernelSgprs))) void ecw_gemm_kernel(
    const GemmArgs a) {
  // dynamic LDS: two-code table (at 0), code table, the two weight slices,
  // the table state word, one staging area per wavefront
  u32x2 *ptab_area = reinterpret_cast<u32x2 *>(dyn_lds);
  uint32_t *lut = reinterpret_cast<uint32_t *>(dyn_lds) + (2u << kPairBits);
  const uint32_t slices = lds_addr(dyn_lds) + a.slice_byte;
  const uint32_t xslices = slices + 2u * kGemmSliceBytes;   // two activation slices (XL)
  if (!lds_at_zero()) {   // the two-code table is addressed from LDS address 0
    if (threadIdx.x == 0)
      for (uint32_t i = 0; i < a.n_tensors; ++i) atomicOr(a.t[i].status, kFLut);
    return;
  }
  uint32_t &lut_state = reinterpret_cast<uint32_t *>(dyn_lds)[a.state_word];
  const uint32_t wave = rfl(threadIdx.x >> 6);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t stage_words = a.stage_words;
  uint32_t *stage = reinterpret_cast<uint32_t *>(dyn_lds) + a.state_word + 4u + wave * (stage_words + kStageSlack);
  const uint32_t tok_groups = (a.n_tokens + 15u) >> 4;
  const uint32_t t0 = blockIdx.x * a.tiles_per_block;
  const uint32_t t1 = min(t0 + a.tiles_per_block, a.total_tiles);
  uint32_t cur = 0xFFFFFFFFu;
  uint32_t K = 0, l_min = 1;
  for (uint32_t tile = t0; tile < t1; ++tile) {
    uint32_t ti = 0;
    while (ti + 1 < a.n_tensors && a.tile_begin[ti + 1] <= tile) ++ti;
    const TensorArg &d = a.t[ti];
    if (ti != cur) {
      __syncthreads();
      if (threadIdx.x == 0) {
        uint32_t k = 0;
        if (d.lut_words >= kLutHeaderWords) {
          const uint32_t h0 = d.lut[0], h1 = d.lut[1], ne = d.lut[2], l1 = d.lut[3];
          const uint32_t kk = h1 & 0xFFu;
          const uint32_t lmin = h1 >> 24;
          if (h0 == kLutMagic && (h1 & 0x00FFFF00u) == d.expect_hdr && kk >= 1 && kk <= kSingleLevelMax &&
              l1 == (1u << kk) && ne >= l1 && ne <= a.lut_cap && ne <= d.lut_words - kLutHeaderWords &&
              lmin >= 1u && lmin <= kMaxCodeLen)
            k = kk | (ne << 8) | (lmin << 24);
        }
        if (!k) atomicOr(d.status, kFLut);
        lut_state = k;
      }
      __syncthreads();
      const uint32_t ne = (lut_state >> 8) & 0xFFFFu;
      for (uint32_t i = threadIdx.x; i < ne; i += kBlockThreads) lut[i] = kernel_entry<kModeGemv>(d.lut[kLutHeaderWords + i]);
      K = rfl(lut_state & 0xFFu);
      l_min = rfl(lut_state >> 24);
      cur = ti;
      __syncthreads();
      if (K)
        for (uint32_t i = threadIdx.x; i < (1u << kPairBits); i += kBlockThreads)
          ptab_area[i] = build_pair_entry<kModeGemv>(lut, K, i);
      __syncthreads();
    }
    if (!K) continue;
    const uint32_t r0 = (tile - a.tile_begin[ti]) * (uint32_t)kWaves;
    const uint32_t row = r0 + wave;
    const uint32_t cols = d.cols, rows = d.rows;
    // this wavefront's row: chunk `row` (the host requires one row per chunk)
    Staged st{0u, 0u, 0u};
    const bool mine = row < rows;
    const bool have = mine && stage_task<6>(d, row, stage, stage_words, st);
    if (mine && !have && lane == 0u) atomicOr(d.status, kFOffsets);
    GemvLane<1> g;
    g.hi = g.lo = g.n = g.kk = 0u;
    g.pa = lds_addr(stage + st.al);
    const uint32_t early = rfl(early_pairs(d.ahead, cols >> 6, l_min));
    const uint32_t q_n = cols / kGemmSliceCols;
    const uint32_t my_row_addr = slices + wave * kGemmRowStride * 2u;
    f32x4 acc[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // A operand: row lane % 16 of the slice, columns 8 * (lane / 16) + 32 ks
    const uint32_t a_addr = slices + ((lane & 15u) * kGemmRowStride + 8u * (lane >> 4)) * 2u;
    // staged activations (XL): B operand of group grp from token row
    // grp * 16 + lane % 16 of the x slice, same column pattern as A
    const uint32_t xunits = tok_groups * 256u;
    const uint32_t b_addr = xslices + ((lane & 15u) * kGemmRowStride + 8u * (lane >> 4)) * 2u;
    XSliceRegs xr;
    if (XL) {
      gemm_x_load(xr, d.x, cols, a.n_tokens, xunits, 0u);
      gemm_x_store(xr, xslices, xunits);
    }
    if (have) gemm_put(my_row_addr, lane, gemm_pair(g, lut, K, early).x);
    __syncthreads();
    for (uint32_t q = 0; q < q_n; ++q) {
      const uint32_t buf = (q & 1u) * kGemmSliceBytes;
      const bool next = q + 1u < q_n;
      if (XL && next) gemm_x_load(xr, d.x, cols, a.n_tokens, xunits, (q + 1u) * kGemmSliceCols);
      if (have && next) gemm_put(my_row_addr + (kGemmSliceBytes - buf), lane, gemm_pair(g, lut, K, early).x);
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const uint32_t grp = wave + (uint32_t)tt * (uint32_t)kWaves;
        if (grp < tok_groups) {
          const uint32_t tok = grp * 16u + (lane & 15u);
#pragma unroll
          for (uint32_t ks = 0; ks < 4u; ++ks) {
            const bf16x8 av = __builtin_bit_cast(
                bf16x8, *(__attribute__((address_space(3))) const u32x4 *)(uintptr_t)(a_addr + buf + ks * 64u));
            bf16x8 bv;
            if (XL)
              bv = __builtin_bit_cast(bf16x8, *(__attribute__((address_space(3))) const u32x4 *)(uintptr_t)(
                                                  b_addr + (q & 1u) * a.xslice_bytes + grp * 16u * kGemmRowStride * 2u +
                                                  ks * 64u));
            else
              bv = gemm_x8(d.x, cols, tok, a.n_tokens, q * kGemmSliceCols + ks * 32u + 8u * (lane >> 4));
            acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[tt], 0, 0, 0);
          }
        }
      }
      if (XL && next) gemm_x_store(xr, xslices + ((q + 1u) & 1u) * a.xslice_bytes, xunits);
      __syncthreads();
    }
    if (have) {
      const uint32_t flags = gemv_end_flags<1>(g, lds_addr(stage + st.al), rfl(st.nw));
      if (flags && lane == 0u) atomicOr(d.status, flags);
    }
    // D of group grp: lane holds rows r0 + 4 (lane / 16) + v for token grp * 16 + lane % 16
    float *y = static_cast<float *>(d.out);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const uint32_t grp = wave + (uint32_t)tt * (uint32_t)kWaves;
      const uint32_t tok = grp * 16u + (lane & 15u);
      if (grp < tok_groups && tok < a.n_tokens) {
#pragma unroll
        for (uint32_t v = 0; v < 4u; ++v) {
          const uint32_t o = r0 + 4u * (lane >> 4) + v;
          if (o < rows) y[(uint64_t)tok * rows + o] = acc[tt][v];
        }
      }
    }
  }
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
  const uint32_t grid = (uint32_t)std::min<uint64_t>((uint64_t)cus * std::max<uint64_t>(k, 1), total_tasks);
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

// Validate everything, then enqueue launches of up to 32 tensors that share
// a lane count and an output cache policy.
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
  size_t i = 0;
  while (i < n) {
    LaunchArgs a;
    std::memset(&a, 0, sizeof a);
    a.batch = batch;
    uint32_t total = 0, log2w = 0, k = 0;
    bool cached = false;   // output cache policy of the launch (GEMV: unused)
    uint64_t stage_need = 0, lut_need = 0, x_fit_words = 0;
    bool x_slices = false;
    bool stage_known = true, want_pairs = false;
    for (; i < n && k < (uint32_t)kMaxTensorsPerLaunch; ++i) {
      const entro_tensor &x = t[i];
      if (x.n_symbols == 0) continue;
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
    if (k == 0) continue;
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
    hipError_t err;
    if (mode == kModeU8 && cached) err = launch_w<kModeU8, 1, kStoreCached>(log2w, total, a, dyn, s);
    else if (mode == kModeU8) err = launch_w<kModeU8, 1, kStoreNT>(log2w, total, a, dyn, s);
    else if (mode == kModeBf16 && cached) err = launch_w<kModeBf16, 1, kStoreCached>(log2w, total, a, dyn, s);
    else if (mode == kModeBf16) err = launch_w<kModeBf16, 1, kStoreNT>(log2w, total, a, dyn, s);
    else if (batch == 1) err = launch_w<kModeGemv, 1, kStoreNT>(log2w, total, a, dyn, s);
    else err = launch_w<kModeGemv, 8, kStoreNT>(log2w, total, a, dyn, s);
    if (err != hipSuccess) return ENTRO_E_HIP;
  }
  return ENTRO_OK;
}

static hipError_t launch_gemm(GemmArgs &a, size_t dyn, hipStream_t s) {
  auto kern = a.xslice_bytes ? ecw_gemm_kernel<1, true>
                             : (a.n_tokens <= 16u * (uint32_t)kWaves ? ecw_gemm_kernel<1, false> : ecw_gemm_kernel<2, false>);
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipGetLastError();
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kBlockThreads, dyn) != hipSuccess || per_cu < 1)
    per_cu = 1;
  const int lds_fit = (int)((kLdsPerCu - kLdsPlanReserve) / (dyn + kStaticLds));
  if (lds_fit >= 1 && per_cu > lds_fit) per_cu = lds_fit;
  if (cus < 1) cus = 1;
  const uint64_t slots = (uint64_t)cus * (uint64_t)per_cu;
  const uint32_t per_block = (uint32_t)((a.total_tiles + slots - 1) / slots);
  a.tiles_per_block = per_block < 1 ? 1 : per_block;
  const uint32_t grid = (a.total_tiles + a.tiles_per_block - 1) / a.tiles_per_block;
  // clear an error left by an earlier call (ours, such as a failed occupancy
  // query, or the caller's): the check below then sees this launch alone
  (void)hipGetLastError();
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlockThreads), dyn, s, a);
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
    if (t[i].lanes != 64u || t[i].sym_bits != 4u || t[i].refill_steps != 2u || t[i].max_chunk_words == 0u)
      return ENTRO_E_UNSUPPORTED;
  }
  size_t i = 0;
  while (i < n) {
    GemmArgs a;
    std::memset(&a, 0, sizeof a);
    a.n_tokens = n_tokens;
    uint32_t total = 0, k = 0;
    uint64_t stage_need = 0, lut_need = 0;
    for (; i < n && k < (uint32_t)kMaxTensorsPerLaunch; ++i) {
      const entro_tensor &x = t[i];
      if (x.n_symbols == 0) continue;
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
      d.refill_steps = 2u;
      d.ahead = x.refill_ahead;
      d.out = g[i].d_y;
      d.x = g[i].d_x;
      d.rows = g[i].rows;
      d.cols = g[i].cols;
      d.n_tasks = d.n_chunks;
      const uint64_t tiles = (d.rows + kWaves - 1) / kWaves;
      if ((uint64_t)total + tiles > 0x7FFFFFFFull) return ENTRO_E_UNSUPPORTED;
      a.tile_begin[k] = total;
      total += (uint32_t)tiles;
      lut_need = std::max<uint64_t>(lut_need, d.lut_words > kLutHeaderWords ? d.lut_words - kLutHeaderWords : 0);
      stage_need = std::max<uint64_t>(stage_need, x.max_chunk_words);
      ++k;
    }
    if (k == 0) continue;
    a.n_tensors = k;
    a.total_tiles = total;
    for (uint32_t r = k; r <= (uint32_t)kMaxTensorsPerLaunch; ++r) a.tile_begin[r] = total;
    // LDS: two-code table, code table, two weight slices, state word, then
    // one staging area per wavefront (the largest row plus alignment)
    a.lut_cap = (uint32_t)((lut_need + 3) & ~3ull);
    size_t dyn = ((size_t)8u << kPairBits) + (size_t)a.lut_cap * 4u;
    dyn = (dyn + 15u) & ~(size_t)15u;
    a.slice_byte = (uint32_t)dyn;
    dyn += 2u * kGemmSliceBytes;
    // short prompts: the activations of each slice staged in LDS as well
    const uint32_t tok_pad = (n_tokens + 15u) & ~15u;
    if (n_tokens <= kGemmXlTokens) {
      a.xslice_bytes = tok_pad * kGemmRowStride * 2u;
      dyn += 2u * (size_t)a.xslice_bytes;
    }
    a.state_word = (uint32_t)(dyn / 4u);
    dyn += 16u;
    const uint64_t sw = (stage_need + 3 + 3) & ~3ull;
    const uint64_t cap = ((kLdsPerCu - kStaticLds) / 4u - dyn / 4u) / kWaves - kStageSlack;
    if (sw > cap) return ENTRO_E_UNSUPPORTED;
    a.stage_words = (uint32_t)sw;
    dyn += (size_t)kWaves * (sw + kStageSlack) * 4u;
    if (launch_gemm(a, dyn, s) != hipSuccess) return ENTRO_E_HIP;
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

extern "C" entro_status entro_decode_gemm(const entro_tensor *t, size_t n, const entro_gemv_item *g,
                                          uint32_t n_tokens, uint32_t *d_status, hipStream_t stream) {
  return run_gemm(t, n, g, n_tokens, d_status, stream);
}
