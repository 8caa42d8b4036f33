// Constants and launch descriptors shared by the host code and the HIP
// kernels of the library (not part of the public ABI).
#pragma once

#include <stdint.h>

namespace entro {

constexpr uint32_t kLutMagic = 0x31574345u;   // "ECW1", little-endian
constexpr uint32_t kLutHeaderWords = 4;
constexpr uint32_t kLutMaxEntries = 4096;     // 16 KiB of LDS per workgroup
constexpr uint32_t kMaxCodeLen = 16;
constexpr uint32_t kSingleLevelMax = 12;      // codes up to 12 bits: one level
constexpr uint32_t kFirstLevelBits = 11;      // longer codes: at most an 11-bit first level
constexpr uint32_t kFirstLevelMin = 5;        // narrowest first level considered
constexpr uint32_t kEntryPointer = 0x80u;
constexpr uint32_t kMaxChunk = 1u << 20;
constexpr uint32_t kInvalidLen = 31u;         // length field of an entry without codeword

// status bits (mirror ENTRO_F_* of entro.h)
constexpr uint32_t kFOverrun = 0x01u, kFUnderrun = 0x02u, kFBadCode = 0x04u,
                   kFPadding = 0x08u, kFOffsets = 0x10u, kFLut = 0x20u;

enum Mode : int { kModeU8 = 0, kModeBf16 = 1, kModeGemv = 2 };

// One tensor of a launch.
struct TensorArg {
  const uint32_t *lut;     // header + entries
  const uint32_t *plut;    // host-built two-code table (header + entries) or null
  const uint32_t *words;
  const uint64_t *offs;
  void *out;               // u8 / bf16 codes, or fp32 y for the GEMV
  const uint16_t *x;       // GEMV activations, bf16 [batch][cols]
  uint32_t *status;
  uint64_t n_words;
  uint64_t n_symbols;
  uint32_t n_chunks;
  uint32_t chunk;
  uint32_t rows, cols;     // GEMV shape
  uint32_t expect_hdr;     // sym_bits << 8 | max_len << 16 (header word 1 without K)
  uint32_t lut_words;      // readable uint32 words at lut
  uint32_t n_tasks;        // wavefront tasks: ceil(n_chunks / chunks per wavefront)
  uint32_t refill_steps;   // steps per refill decision (1 or 2)
  uint32_t ahead;          // 1: refill ahead while codes_left * l_min >= 32
};

constexpr int kMaxTensorsPerLaunch = 32;
constexpr int kWaves = 16;                      // wavefronts per workgroup
constexpr int kBlockThreads = 64 * kWaves;
constexpr uint32_t kLdsPerCu = 160u * 1024u;     // gfx950
constexpr uint32_t kGemvXMaxBytes = 64u * 1024u; // largest activation block staged in LDS
constexpr uint32_t kGemvSlicePairs = 8;          // pairs of steps (1024 columns) per activation slice
constexpr int kKernelSgprs = 64;                 // scalar registers per wavefront (residency)
constexpr uint32_t kLdsPlanReserve = 4u * 1024u; // kept free when sizing the persistent grid
constexpr uint32_t kStaticLds = 256u;            // margin for static LDS (the kernel declares none)
// Cache policy of the decoded outputs: non-temporal (nt), the hint that the
// data will not be reused.  Each output is written once and never read back
// by the kernel, and the hint keeps the output stream from being retained
// in the caches (measured on the 4096x4096 4-bit to bf16 workload: 131 ->
// 115 us per launch).
constexpr int kStoreNT = 2;
// Ordinary stores, for outputs that a consumer reads right after the decode
// (decode-ahead staging, entro_tensor.out_cached): they stay in L2 and the
// last-level cache instead of going out to HBM first.
constexpr int kStoreCached = 0;
constexpr uint32_t kStageSlack = 72;            // words after each wavefront's staging area (reads of a well-formed stream stay within 64 words past its chunk)

// A wavefront task is 64 / lanes consecutive chunks.  The tasks of the
// launch's tensors, one after another, form its task space; workgroup b
// takes tasks_q of them (one more if b < tasks_r), from task
// b * tasks_q + min(b, tasks_r) on.
struct LaunchArgs {
  TensorArg t[kMaxTensorsPerLaunch];
  uint32_t task_begin[kMaxTensorsPerLaunch + 1];   // first task of each tensor (then the total)
  uint32_t n_tensors;
  uint32_t batch;                                  // GEMV rows of x / y
  uint32_t tasks_q;
  uint32_t tasks_r;
  uint32_t stage_words;                            // staging words per wavefront (0: none)
  uint32_t lut_cap;                                // table entries reserved in LDS
  uint32_t pair_bits;                              // index bits of the two-code table (0: none)
  uint32_t x_words;                                // LDS words of staged GEMV activations (0: none)
  uint32_t x_slice;                                // 1: activations too large for x_words go in slices
};

// Decode + GEMM (prefill): a workgroup owns tiles of 16, 32 or 64 weight
// rows (one chunk each), decoded two steps (128 columns) at a time into one
// of two LDS slices, which the matrix cores multiply with the activations.
constexpr uint32_t kGemmMaxTokens = 512;
constexpr uint32_t kGemmSliceCols = 128;                       // columns per slice (one pair of steps)
constexpr uint32_t kGemmRowStride = kGemmSliceCols + 8;        // bf16 per slice row (padding: no bank conflicts)

// Streamed fused GEMV (W = 64, 4-bit codes in pairs, chunks of whole rows,
// 128 | cols): the launch's workgroups are split by tensor, and tensor i's
// wg_count[i] workgroups split its chunks (or tiles) into even parts, one
// per workgroup.  Each wavefront streams the words of its chunks through a
// ring of kRingBlocks blocks in LDS.
constexpr uint32_t kRingBlocks = 4;
constexpr int kMaxStreamTensors = 16;
constexpr uint32_t kMaxStreamWgs = 1024;   // at most 4096: wg_info keeps 12 bits of index

struct StreamArgs {
  TensorArg t[kMaxStreamTensors];
  uint32_t chunk_begin[kMaxStreamTensors + 1];  // first chunk of each tensor (then the total)
  // workgroup b works on tensor wg_info[b] >> 12 as its workgroup
  // wg_info[b] & 0xFFF of wg_count[that tensor]: one scalar load each (as
  // 32-bit words), so that a workgroup finds its share in two round trips
  union {
    uint16_t wg_count[kMaxStreamTensors];
    uint32_t wg_count_w[kMaxStreamTensors / 2];
  };
  union {
    uint16_t wg_info[kMaxStreamWgs];
    uint32_t wg_info_w[kMaxStreamWgs / 2];
  };
  uint32_t n_tensors;
  uint32_t batch;
  uint32_t lut_cap;        // code-table entries reserved in LDS (a multiple of 4)
  uint32_t x_words;        // LDS words of the staged activations
  uint32_t flag_word;      // LDS word index of the workgroup's table-state word
  uint32_t ring_off;       // LDS byte offset of the first ring (a multiple of the ring's bytes)
  uint32_t log2_ring;      // log2 of a ring's words (a block is a quarter of it)
  uint32_t tile_a_off;     // matrix-core GEMV: LDS byte offsets of the A tiles,
  uint32_t tile_x_off;     //   the x buffers
  uint32_t tile_red_off;   //   and the row-end partial sums
};
static_assert(sizeof(StreamArgs) <= 4096, "kernel arguments: at most 4 KiB");

constexpr uint32_t kPairBits = 10;                 // two-code table: 1024 entries of 8 bytes
constexpr uint32_t kPairBitsWide = 12;             // streamed GEMV: 4096 entries of 8 bytes
constexpr uint32_t kPairFallback = 0x80u;          // flag (byte 0 of the second word): no pair
constexpr uint32_t kPairLutMagic = 0x31504345u;    // "ECP1", little-endian
constexpr uint32_t kPairLutHeaderWords = 4;        // magic, flags, the code table's header word 1, 0
constexpr uint32_t kPairLutWhole = 1u;             // flags: every index holds a whole pair

}  // namespace entro
