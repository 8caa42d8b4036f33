// HIP kernel (gfx950) and device entry points of the interleaved rANS
// decoder: entro_rans_decode, entro_rans_decode_dequant.  The stream layout
// (ECR v1) and the host encoder are in entro_rans.h / entro_rans.cpp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <type_traits>

#include "entro.h"
#include "entro_device.h"
#include "entro_internal.h"
#include "entro_rans.h"

namespace entro {

// ---------------------------------------------------------------------------
// interleaved rANS (ECR v1, layout in entro_rans.h): decode to codes or bf16
// One wavefront decodes 64 / W chunks (W = 32 or 64) in lockstep, one code
// per step: the slot table (4096 entries of 8 bytes, at LDS address 0)
// gives the code's output value, frequency f and the slot's offset in the
// code's range; x = f (x >> 12) + offset; lanes whose state fell below 2^16
// take the next 16-bit unit of their chunk (wavefront prefix count, as for
// the Huffman words).  Two steps are stored packed per lane (store_pair).
// ---------------------------------------------------------------------------
constexpr uint32_t kRansMagic = 0x31524345u;   // "ECR1"
constexpr uint32_t kRansSlots = 4096u;
constexpr uint32_t kRansL = 1u << 16;

struct RansArg {
  const uint32_t *table;     // header + slots
  const uint16_t *units;
  const uint64_t *offs;      // unit offsets of the chunks
  void *out;
  uint32_t *status;
  uint64_t n_units;
  uint64_t n_symbols;
  uint32_t n_chunks;
  uint32_t chunk;
  uint32_t sym_bits;
  uint32_t table_words;
  uint32_t n_tasks;
};

// Tasks as for the Huffman decoder: the launch's task space is the tensors'
// wavefront tasks one after another; workgroup b takes tasks_q of them (one
// more if b < tasks_r) from task b * tasks_q + min(b, tasks_r) on.
struct RansLaunch {
  RansArg t[kMaxTensorsPerLaunch];
  uint32_t task_begin[kMaxTensorsPerLaunch + 1];   // first task of each tensor (then the total)
  uint32_t n_tensors;
  uint32_t tasks_q;
  uint32_t tasks_r;
  uint32_t stage_units;      // staging units per wavefront (a multiple of 8)
  uint32_t state_word;       // LDS word of the table state
};

template <int MODE>
__device__ __forceinline__ uint32_t rans_entry(uint32_t x) {
  return MODE == kModeU8 ? ((x & 0xFFu) << 16) : (x & 0xFFFF0000u);
}

// One step of every active lane: returns the code's output value (bits
// [31:16]) and advances x and the unit pointers (LDS byte addresses of the
// two chunk halves' next units for W = 32, one for W = 64).
template <int LOG2W>
__device__ __forceinline__ uint32_t rans_step(uint32_t &x, uint32_t &pu0, uint32_t &pu1, uint32_t upper, bool act) {
  const u32x2 e = *(lds_u32x2 *)(uintptr_t)((x & (kRansSlots - 1u)) << 3);
  uint32_t nx = (e.y & 0xFFFFu) * (x >> 12) + (e.y >> 16);
  if (!act) nx = x;
  const uint64_t m = __ballot(act && nx < kRansL);
  if (__builtin_amdgcn_inverse_ballot_w64(m)) {
    const uint32_t mlo = (uint32_t)m, mhi = (uint32_t)(m >> 32);
    uint32_t addr;
    if (LOG2W == 6) {
      addr = pu0 + 2u * __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, 0u));
    } else {
      const uint32_t below = upper ? __builtin_amdgcn_mbcnt_hi(mhi, 0u) : __builtin_amdgcn_mbcnt_lo(mlo, 0u);
      addr = (upper ? pu1 : pu0) + 2u * below;
    }
    const uint32_t u = *(__attribute__((address_space(3))) const uint16_t *)(uintptr_t)addr;
    nx = (nx << 16) | u;
  }
  x = nx;
  if (LOG2W == 6) {
    pu0 += 2u * (uint32_t)__popcll(m);
  } else {
    pu0 += 2u * (uint32_t)__popc((uint32_t)m);
    pu1 += 2u * (uint32_t)__popc((uint32_t)(m >> 32));
  }
  return e.x;
}

template <int MODE, int LOG2W>
__global__ __launch_bounds__(kBlockThreads) __attribute__((amdgpu_num_sgpr(kKernelSgprs))) void ecr_kernel(
    const RansLaunch a) {
  constexpr uint32_t W = 1u << LOG2W;
  constexpr uint32_t G = 64u >> LOG2W;
  typedef OutElem<typename std::conditional<MODE == kModeU8, uint8_t, uint16_t>::type, kStoreNT> OutT;
  u32x2 *tab = reinterpret_cast<u32x2 *>(dyn_lds);
  uint32_t &state = reinterpret_cast<uint32_t *>(dyn_lds)[a.state_word];
  const uint32_t wave = rfl(threadIdx.x >> 6);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t grp = lane >> LOG2W;
  const uint32_t j = lane & (W - 1u);
  uint16_t *stage = reinterpret_cast<uint16_t *>(reinterpret_cast<uint32_t *>(dyn_lds) + a.state_word + 4u) +
                    (size_t)wave * (a.stage_units + 8u);
  if (!lds_at_zero()) {   // the slot table is addressed from LDS address 0
    if (threadIdx.x == 0)
      for (uint32_t i = 0; i < a.n_tensors; ++i) atomicOr(a.t[i].status, kFLut);
    return;
  }
  // rounds of up to kWaves tasks within one tensor; wavefront w takes the
  // w-th task of a round
  const uint32_t b = blockIdx.x;
  const uint32_t g0 = b * a.tasks_q + min(b, a.tasks_r);
  const uint32_t g1 = g0 + a.tasks_q + (b < a.tasks_r ? 1u : 0u);
  uint32_t cur = 0xFFFFFFFFu;
  uint32_t ok = 0, ti = 0;
  for (uint32_t g = g0; g < g1;) {
    while (ti + 1 < a.n_tensors && a.task_begin[ti + 1] <= g) ++ti;
    const RansArg &d = a.t[ti];
    const uint32_t n_here = min(min(g1, a.task_begin[ti + 1]) - g, (uint32_t)kWaves);
    const uint64_t task = (uint64_t)(g - a.task_begin[ti]) + wave;   // within the tensor
    const bool mine = wave < n_here;
    g += n_here;
    if (ti != cur) {
      __syncthreads();
      if (threadIdx.x == 0) {
        uint32_t k = 0;
        if (d.table_words >= 4u + 2u * kRansSlots && d.table[0] == kRansMagic &&
            d.table[1] == (d.sym_bits | (12u << 8)) && d.table[2] == kRansSlots)
          k = 1;
        if (!k) atomicOr(d.status, kFLut);
        state = k;
      }
      __syncthreads();
      ok = rfl(state);
      if (ok)
        for (uint32_t i = threadIdx.x; i < kRansSlots; i += kBlockThreads) {
          u32x2 e;
          e.x = rans_entry<MODE>(d.table[4u + 2u * i]);
          e.y = d.table[4u + 2u * i + 1u];
          tab[i] = e;
        }
      cur = ti;
      __syncthreads();
    }
    if (!ok || !mine) continue;
    // chunk offsets of the task: lane l < G holds chunk c0 + l's start
    const uint64_t c0 = task * G;
    const uint32_t nck = (uint32_t)min((uint64_t)G, (uint64_t)d.n_chunks - c0);
    const uint64_t o = d.offs[c0 + min(lane, nck - 1u)];
    const uint64_t o_last = rfl64(d.offs[c0 + nck]);
    const uint64_t o_down = __shfl_down(o, 1, 64);
    const uint64_t o_next = lane + 1u < nck ? o_down : o_last;
    const uint64_t o_first = rfl64(__shfl(o, 0, 64));
    const bool badoff = lane < nck && (o_next < o || o_next > d.n_units || o_next - o < 2u * W);
    const uint64_t task_units = o_last - o_first;
    if (__ballot(badoff) || o_last < o_first || task_units + 8u > a.stage_units) {
      if (lane == 0) atomicOr(d.status, kFOffsets);
      continue;
    }
    // stage the units (16-byte loads straight into LDS from a 16-byte aligned
    // start; past the tensor's units lands as zero)
    const uint32_t al = (uint32_t)(o_first & 7u);
    const uint64_t base_al = o_first - al;
    const uint64_t bytes_left = (d.n_units - base_al) * 2u;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(d.units + base_al), (short)0, (int)min(bytes_left, (uint64_t)0xFFFFFFF0u), 0x00020000);
    const uint32_t nvec = (uint32_t)((al + task_units + 7u) >> 3);
    lds_copy16(rsrc, rfl(lds_addr(stage)), rfl(nvec), lane);
    wait_lds_copy();
    // the range check works per dword: with an odd unit count the tensor's
    // last unit shares its dword with the end of the range and landed as
    // zero above, so it is fetched alone, after the copy has landed
    if ((d.n_units & 1u) && o_last == d.n_units && lane == 0u) {
      const uint32_t li = (uint32_t)(d.n_units - 1u - base_al);
      stage[li] = __builtin_amdgcn_raw_buffer_load_b16(rsrc, (int)(2u * li), 0, 0);
    }
    asm volatile("" ::: "memory");
    // this lane's chunk: units [cs, cs + nu) of the staging area
    const uint64_t og = __shfl(o, (int)min(grp, nck - 1u), 64), og1 = __shfl(o_next, (int)min(grp, nck - 1u), 64);
    const uint32_t cs = al + (uint32_t)(og - o_first);
    const uint32_t nu = (uint32_t)(og1 - og);
    const bool live = grp < nck;
    const uint64_t chunk0 = c0 + (live ? grp : 0u);
    const uint32_t cc = live ? (uint32_t)min((uint64_t)d.chunk, d.n_symbols - chunk0 * d.chunk) : 0u;
    const uint32_t steps = rfl((uint32_t)min((uint64_t)d.chunk, d.n_symbols - c0 * d.chunk) / W + 1u);
    const uint32_t sbase = lds_addr(stage);
    uint32_t x = live ? ((uint32_t)stage[cs + 2u * j] | ((uint32_t)stage[cs + 2u * j + 1u] << 16)) : kRansL;
    // unit pointers (LDS byte addresses) of the two halves' chunks
    const uint32_t cs0 = rfl(__shfl(cs, 0, 64));
    const uint32_t cs1 = rfl(__shfl(cs, 63, 64));
    uint32_t pu0 = sbase + 2u * (cs0 + 2u * W), pu1 = sbase + 2u * (cs1 + 2u * W);
    const uint32_t upper = lane >= 32u ? 1u : 0u;
    OutT *outp = reinterpret_cast<OutT *>(rfl64(reinterpret_cast<uint64_t>(static_cast<OutT *>(d.out) + c0 * d.chunk)));
    const uint32_t out_bytes = rfl((uint32_t)min((uint64_t)nck * d.chunk * sizeof(OutT), (uint64_t)0xFFFFFFF0u));
    // stores of this task's chunks only (a short last chunk is written by
    // the masked loop below)
    const __amdgpu_buffer_rsrc_t outr = __builtin_amdgcn_make_buffer_rsrc((void *)outp, (short)0, (int)out_bytes, 0x00020000);
    const uint32_t lane_off = grp * d.chunk + j;
    constexpr uint32_t B = W * (uint32_t)sizeof(OutT);
    const uint32_t voffp = pair_voff(lane_off, lane, W, (uint32_t)sizeof(OutT));
    const uint32_t sel = pair_sel<MODE>(lane);
    const bool full = rfl(nck == G && (c0 + G) * (uint64_t)d.chunk <= d.n_symbols ? 1u : 0u);
    if (full) {
      const uint32_t sfull = d.chunk >> LOG2W;
      uint32_t t = 0;
      for (; t + 2u <= sfull; t += 2u) {
        const uint32_t eA = rans_step<LOG2W>(x, pu0, pu1, upper, true);
        const uint32_t eB = rans_step<LOG2W>(x, pu0, pu1, upper, true);
        store_pair<MODE, kStoreNT>(outr, voffp, t * B, pack_ab<MODE>(eA, eB), sel);
      }
      if (t < sfull) store_out<OutT>(outr, lane_off * (uint32_t)sizeof(OutT), rfl(t * B),
                                     rans_step<LOG2W>(x, pu0, pu1, upper, true));
    } else {
      for (uint32_t t = 0; t < steps; ++t) {
        const bool act = live && t * W + j < cc;
        const uint32_t e = rans_step<LOG2W>(x, pu0, pu1, upper, act);
        // inactive lanes store past the buffer's range: the bounds check drops them
        store_out<OutT>(outr, act ? lane_off * (uint32_t)sizeof(OutT) : 0x80000000u, rfl(t * B), e);
      }
    }
    // every lane ends in state L; each chunk's units are used exactly
    const uint32_t used = ((upper && LOG2W == 5 ? pu1 : pu0) - sbase) / 2u - cs;
    uint32_t flags = 0;
    if (live && used != nu) flags |= used < nu ? kFUnderrun : kFOverrun;
    if (live && x != kRansL) flags |= kFPadding;
    uint32_t all = flags;
    for (int s = 32; s >= 1; s >>= 1) all |= (uint32_t)__shfl_xor((int)all, s, 64);
    if (all && lane == 0u) atomicOr(d.status, all);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static entro_status run_rans(int mode, const entro_rans_tensor *t, size_t n, void *const *outs, uint32_t *d_status,
                             hipStream_t s) {
  if (n == 0) return ENTRO_OK;
  if (!t || !outs || !d_status) return ENTRO_E_INVAL;
  for (size_t i = 0; i < n; ++i) {
    const entro_rans_tensor &x = t[i];
    if (x.lanes != 32u && x.lanes != 64u) return ENTRO_E_FORMAT;
    if (x.chunk_symbols == 0 || x.chunk_symbols % x.lanes || x.chunk_symbols > kMaxChunk) return ENTRO_E_FORMAT;
    if (x.sym_bits != 4 && x.sym_bits != 8) return ENTRO_E_FORMAT;
    if (x.n_symbols == 0) continue;
    if (!x.d_table || !x.d_units || !x.d_chunk_unit_off || !outs[i]) return ENTRO_E_INVAL;
    const uintptr_t align = mode == kModeU8 ? 2u : 4u;
    if (reinterpret_cast<uintptr_t>(outs[i]) & (align - 1u)) return ENTRO_E_INVAL;
    if ((x.n_symbols + x.chunk_symbols - 1) / x.chunk_symbols > 0xFFFFFFFFull) return ENTRO_E_UNSUPPORTED;
  }
  size_t i = 0;
  while (i < n) {
    RansLaunch a;
    std::memset(&a, 0, sizeof a);
    uint32_t total = 0, k = 0, lanes = 0;
    uint64_t stage_need = 0;
    for (; i < n && k < (uint32_t)kMaxTensorsPerLaunch; ++i) {
      const entro_rans_tensor &x = t[i];
      if (x.n_symbols == 0) continue;
      if (k == 0) lanes = x.lanes;
      else if (x.lanes != lanes) break;
      // the launch's task space stays below 2^31 tasks
      const uint64_t tasks = ((x.n_symbols + x.chunk_symbols - 1) / x.chunk_symbols + 64u / x.lanes - 1) / (64u / x.lanes);
      if (tasks > 0x7FFFFFFFull) return ENTRO_E_UNSUPPORTED;
      if ((uint64_t)total + tasks > 0x7FFFFFFFull) break;
      RansArg &d = a.t[k];
      d.table = static_cast<const uint32_t *>(x.d_table);
      d.units = x.d_units;
      d.offs = x.d_chunk_unit_off;
      d.out = outs[i];
      d.status = d_status + i;
      d.n_units = x.n_units;
      d.n_symbols = x.n_symbols;
      d.chunk = x.chunk_symbols;
      d.n_chunks = (uint32_t)((x.n_symbols + x.chunk_symbols - 1) / x.chunk_symbols);
      d.sym_bits = x.sym_bits;
      d.table_words = (uint32_t)(entro_rans_table_bytes() / 4u);
      const uint32_t g = 64u / x.lanes;
      d.n_tasks = (d.n_chunks + g - 1) / g;
      a.task_begin[k] = total;
      total += d.n_tasks;
      const uint64_t mcu = x.max_chunk_units ? x.max_chunk_units : (x.n_units + d.n_chunks - 1) / d.n_chunks * 2u;
      stage_need = std::max<uint64_t>(stage_need, (uint64_t)g * mcu);
      ++k;
    }
    if (k == 0) continue;
    a.n_tensors = k;
    for (uint32_t r = k; r <= (uint32_t)kMaxTensorsPerLaunch; ++r) a.task_begin[r] = total;
    // LDS: the slot table (32 KiB, at 0), the state word, then one staging
    // area per wavefront (the largest task plus alignment)
    size_t dyn = (size_t)kRansSlots * 8u;
    a.state_word = (uint32_t)(dyn / 4u);
    dyn += 16u;
    const uint64_t su = (stage_need + 8u + 7u) & ~7ull;
    const uint64_t cap = ((kLdsPerCu - kStaticLds - dyn) / 2u) / kWaves - 8u;
    if (su > cap) return ENTRO_E_UNSUPPORTED;
    a.stage_units = (uint32_t)su;
    dyn += (size_t)kWaves * (su + 8u) * 2u;
    auto kern = mode == kModeU8 ? (lanes == 64u ? ecr_kernel<kModeU8, 6> : ecr_kernel<kModeU8, 5>)
                                : (lanes == 64u ? ecr_kernel<kModeBf16, 6> : ecr_kernel<kModeBf16, 5>);
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return ENTRO_E_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kBlockThreads, dyn) != hipSuccess || per_cu < 1)
      per_cu = 1;
    const int lds_fit = (int)((kLdsPerCu - kLdsPlanReserve) / (dyn + kStaticLds));
    if (lds_fit >= 1 && per_cu > lds_fit) per_cu = lds_fit;
    if (cus < 1) cus = 1;
    // one workgroup per slot (fewer if there are fewer tasks), the tasks
    // spread over them evenly
    const uint64_t slots = (uint64_t)cus * (uint64_t)per_cu;
    const uint32_t grid = (uint32_t)std::min<uint64_t>(slots, total);
    a.tasks_q = total / grid;
    a.tasks_r = total % grid;
    // clear an error left by an earlier call (ours, such as a failed occupancy
    // query, or the caller's): the check below then sees this launch alone
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlockThreads), dyn, s, a);
    if (hipGetLastError() != hipSuccess) return ENTRO_E_HIP;
  }
  return ENTRO_OK;
}

}  // namespace entro

using namespace entro;

extern "C" entro_status entro_rans_decode(const entro_rans_tensor *t, size_t n, uint8_t *const *d_out,
                                          uint32_t *d_status, hipStream_t stream) {
  return run_rans(kModeU8, t, n, reinterpret_cast<void *const *>(d_out), d_status, stream);
}

extern "C" entro_status entro_rans_decode_dequant(const entro_rans_tensor *t, size_t n, uint16_t *const *d_out_bf16,
                                                  uint32_t *d_status, hipStream_t stream) {
  return run_rans(kModeBf16, t, n, reinterpret_cast<void *const *>(d_out_bf16), d_status, stream);
}
