/*
 * entro.h - C ABI of the entropy-coded weight library for MI355X (gfx950).
 *
 * The library decodes per-tensor quantized LLM weight codes (4-bit or 8-bit)
 * that were compressed with a length-limited canonical Huffman code laid out
 * in independent chunks of lane-interleaved 32-bit words, and optionally
 * dequantizes them to bf16 or multiplies them with activation vectors on the
 * fly.  Method: EntroLLM (arXiv 2505.02380) - tensor-level mixed quantization,
 * Huffman coding of the codes, chunks decoded in parallel; LazyWeights
 * (arXiv 2611.17108) - codes Huffman-coded in interleaved lanes and decoded on
 * demand so that memory moves only coded bytes.
 *
 * Stream layout ("ECW v1") for a tensor of N codes, chunk size C, lanes W:
 *   - the tensor is flattened row-major; chunk c holds codes [c*C, min((c+1)*C, N));
 *   - inside a chunk, code k belongs to lane k mod W and is decoded at step k / W;
 *   - each lane's codewords (canonical: codes of one length are consecutive in
 *     symbol order, shorter codes first, first code zero; MSB-first) are packed
 *     into 32-bit words, first bit in bit 31, the last word zero-padded;
 *   - refill decisions are taken every D steps (D = refill_steps, 1 or 2): at a
 *     step t with t mod D == 0 a lane takes its next word when its codewords of
 *     steps t .. t+D-1 are together longer than the number of loaded,
 *     unconsumed bits it holds (one word always suffices: codes are at most 16
 *     bits); words are stored in the order they are taken, lanes of one
 *     decision point in increasing lane order;
 *   - with refill_ahead, a lane that still has R codes to decode from step t
 *     on, with R * l_min >= 32 (l_min: the codebook's shortest code length),
 *     instead takes its next word at a decision point exactly when it holds
 *     fewer than 32 loaded bits; such a word always exists, so the word count
 *     is unchanged, and a decoder can fetch it before looking up codewords;
 *   - chunk_bit_off[c] = 32 * (words before chunk c); chunk_bit_off[n_chunks]
 *     = 32 * n_words.  Words are little-endian uint32.
 *   - A descriptor may also cover only the whole chunks c0 .. c1 - 1 of a
 *     stream: d_chunk_bit_off then points at entry c0 of the stream's offsets,
 *     n_symbols counts those chunks' codes, and d_words / n_words stay the
 *     whole stream's (the offsets remain bit positions in it).  This decodes
 *     a block of rows of a matrix whose chunks hold whole rows.
 *
 * Conventions
 *   - Pointers named d_* are DEVICE pointers (hipMalloc'd or torch CUDA/HIP
 *     tensors on the current device); all others are host pointers.  Every
 *     buffer is owned by the caller and only read (or written, for outputs)
 *     during the call or the work it enqueues.
 *   - Device entry points validate their host-side arguments synchronously
 *     and return a nonzero status before enqueuing anything.  They enqueue on
 *     the caller's stream (0 = the null stream) and return without waiting.
 *   - Problems found in the data itself (offsets, LUT header, the bitstream)
 *     are reported by OR-ing ENTRO_F_* bits into the caller-zeroed
 *     d_status[i] of tensor i; read it after synchronizing.  Kernels never
 *     read outside [d_words, d_words + n_words) or outside the chunk-offset
 *     array, and never abort.  Outputs of a flagged tensor are unspecified.
 *   - The library allocates no device memory and keeps no state between
 *     calls; calls on different streams may run concurrently.
 */
#ifndef ENTRO_H
#define ENTRO_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ENTRO_ABI_VERSION 1

typedef enum {
  ENTRO_OK = 0,
  ENTRO_E_INVAL = 1,        /* null pointer, bad size, inconsistent descriptor  */
  ENTRO_E_CODEBOOK = 2,     /* lengths over the cap, Kraft sum > 1, no symbols  */
  ENTRO_E_FORMAT = 3,       /* chunk/lane/shape parameters outside the layout   */
  ENTRO_E_UNSUPPORTED = 4,  /* valid but not handled (e.g. LUT larger than LDS) */
  ENTRO_E_HIP = 5           /* the HIP runtime reported an error                */
} entro_status;

/* Per-tensor data faults OR-ed into d_status[i] by the device entry points. */
#define ENTRO_F_OVERRUN 0x01u   /* a lane needed a word past its chunk's end     */
#define ENTRO_F_UNDERRUN 0x02u  /* a chunk ended with words left unused          */
#define ENTRO_F_BADCODE 0x04u   /* bits matched no codeword                       */
#define ENTRO_F_PADDING 0x08u   /* nonzero bits after a lane's last codeword      */
#define ENTRO_F_OFFSETS 0x10u   /* chunk offsets not ascending multiples of 32,
                                   or past n_words; such a chunk is skipped      */
#define ENTRO_F_LUT 0x20u       /* LUT header does not match the descriptor;
                                   the tensor is skipped                          */

/* A per-tensor codebook (host memory, read during the call only).
 * Defined by: EntroLLM - Huffman code built per layer/tensor from the value
 * frequencies of the quantized weights (gist.science technical summary,
 * Methodology item 2), tensor-level unsigned/asymmetric quantization (abstract).
 * dequantized value of code q: bf16 = RNE(f32(scale) * f32(q - zero_point)). */
typedef struct {
  uint32_t sym_bits;        /* 4 or 8: the alphabet is 2^sym_bits codes            */
  uint32_t max_len;         /* 1..16: cap on the code lengths used when encoding   */
  const uint8_t *code_len;  /* [1 << sym_bits] code lengths; 0 = code value absent */
  float scale;              /* per-tensor scale                                    */
  int32_t zero_point;       /* per-tensor zero point                               */
} entro_codebook;

/* One coded tensor as the device entry points read it. */
typedef struct {
  const void *d_lut;              /* entro_lut_build bytes, copied to the device by the caller */
  const uint32_t *d_words;        /* [n_words] ECW v1 stream                            */
  const uint64_t *d_chunk_bit_off;/* [n_chunks + 1], n_chunks = ceil(n_symbols / chunk) */
  uint64_t n_words;
  uint64_t n_symbols;             /* codes in the tensor; 0 = empty tensor (skipped)   */
  uint32_t chunk_symbols;         /* C >= 1, a multiple of lanes, <= 2^20               */
  uint32_t lanes;                 /* W in {1, 2, 4, 8, 16, 32, 64}                      */
  uint32_t sym_bits;              /* must equal the codebook the LUT was built from    */
  uint32_t max_len;               /* likewise                                           */
  uint64_t lut_bytes;             /* bytes readable at d_lut (entro_lut_bytes); a table
                                     whose header claims more is rejected (ENTRO_F_LUT) */
  uint32_t max_chunk_words;       /* words of the largest chunk, or 0 if unknown; sizes
                                     the on-chip staging (a chunk larger than stated is
                                     still decoded correctly, only more slowly)          */
  uint32_t refill_steps;          /* steps per refill decision the stream was encoded
                                     with: 1 or 2 (0 is read as 1)                       */
  uint32_t refill_ahead;          /* 1 if the stream was encoded refilling ahead, else 0 */
  uint32_t out_cached;            /* decode entry points: 0 streams the outputs past the
                                     caches (nothing reads them soon); 1 writes them with
                                     ordinary stores, so that a consumer right after the
                                     call (decode-ahead staging) finds them in L2 or the
                                     last-level cache.  Values only; the GEMV ignores it */
  const void *d_pair_lut;         /* optional, fused GEMV of 4-bit tensors: the two-code
                                     table entro_pair_lut_build made from this tensor's
                                     decode table, copied to the device 16-byte aligned;
                                     each workgroup then loads it instead of building it
                                     on chip.  NULL (or unaligned): built on chip.  A table
                                     whose header does not match the decode table sets
                                     ENTRO_F_LUT and the tensor is not decoded          */
} entro_tensor;

/* Operands of the fused GEMV for one tensor, read as a [rows][cols] row-major
 * matrix (rows = output features, cols = input features). */
typedef struct {
  uint32_t rows, cols;      /* rows * cols == n_symbols; cols % lanes == 0;
                               chunk_symbols % cols == 0 (chunks hold whole rows)   */
  const uint16_t *d_x;      /* bf16 activations [batch][cols]                        */
  float *d_y;               /* fp32 outputs [batch][rows], overwritten              */
} entro_gemv_item;

/* Size in bytes of the decode table built from cb (0 if cb is invalid).
 * The table holds a 16-byte header and 4-byte entries: one level indexed by
 * the next K stream bits and, for codes longer than K, second-level tables
 * indexed by the following bits.  K is the smallest width from 5 up (at most
 * 12, or 11 when longer codes exist) for which the codes longer than K have
 * an estimated probability (sum of 2^-length) of at most 2^-10, and for which
 * the table fits 4096 entries; a shorter first level means fewer LDS bank
 * conflicts and less LDS per workgroup.  The header also records the
 * shortest code length (which the refill-ahead layout depends on).  Each
 * entry carries the code length, the code value and its bf16 dequantized
 * value.  Defined by: canonical Huffman codes (reading of EntroLLM's Huffman
 * step, see the stream layout above) and the dequantization rule of
 * entro_codebook. */
size_t entro_lut_bytes(const entro_codebook *cb);

/* Build the decode table of cb into host_lut (cap bytes, 4-byte aligned).
 * Errors: ENTRO_E_INVAL (null pointers, cap too small), ENTRO_E_CODEBOOK
 * (a length > max_len, Kraft sum > 1, or no code value present),
 * ENTRO_E_FORMAT (sym_bits not 4/8, max_len not in 1..16),
 * ENTRO_E_UNSUPPORTED (table larger than 16 KiB of entries). */
entro_status entro_lut_build(const entro_codebook *cb, void *host_lut, size_t cap);

/* Size in bytes of a two-code table (entro_pair_lut_build): a 16-byte header
 * and 4096 entries of 8 bytes. */
size_t entro_pair_lut_bytes(void);

/* Build the two-code table of a 4-bit decode table (host_lut: lut_bytes of
 * entro_lut_build output) into host_out (cap bytes, 4-byte aligned).  Entry i
 * is indexed by the next 12 stream bits (MSB first): the bf16 values of the
 * two codewords those bits begin with, their summed length and the matching
 * shift, or a mark that the two codewords do not both lie within the 12 bits
 * (then the decoder looks them up one at a time).  The header records
 * whether every entry holds a whole pair and repeats the decode table's
 * header word that names the code (first-level width, alphabet, length cap,
 * shortest length).  The entry layout is the library's own; upload the bytes
 * as they are.  Defined by: the same canonical code and dequantization as
 * entro_lut_build; the pages leave the decoder's table structure open, and
 * two codewords per lookup is this library's design.  Errors:
 * ENTRO_E_INVAL (null pointers, cap too small, a malformed decode table),
 * ENTRO_E_UNSUPPORTED (not a 4-bit table). */
entro_status entro_pair_lut_build(const void *host_lut, size_t lut_bytes, void *host_out, size_t cap);

/* Decode n tensors to their codes: d_out[i] receives t[i].n_symbols bytes.
 * Defined by: EntroLLM's parallel decoding of independent chunks
 * (gist.science technical summary, Methodology item 3) and LazyWeights'
 * interleaved-lane Huffman decoding (abstract).  One wavefront decodes
 * 64 / lanes chunks in lockstep.  t and d_out are host arrays of n entries;
 * d_status is a device array of n uint32 that the caller zeroes first.
 * Each d_out[i] must be 2-byte aligned (outputs of neighbouring lanes are
 * written together); ENTRO_E_INVAL otherwise. */
entro_status entro_decode(const entro_tensor *t, size_t n, uint8_t *const *d_out,
                          uint32_t *d_status, hipStream_t stream);

/* Decode n tensors and dequantize: d_out_bf16[i] receives t[i].n_symbols bf16
 * values, RNE(f32(scale) * f32(q - zero_point)), the scale and zero point
 * being those the LUT was built with.  Defined by: EntroLLM's tensor-level
 * unsigned/asymmetric quantization (abstract; gist.science technical summary,
 * Methodology item 1) undone after decoding.  Each d_out_bf16[i] must be
 * 4-byte aligned; ENTRO_E_INVAL otherwise. */
entro_status entro_decode_dequant(const entro_tensor *t, size_t n, uint16_t *const *d_out_bf16,
                                  uint32_t *d_status, hipStream_t stream);

/* Fused decode + dequant + GEMV: for each tensor i,
 *   g[i].d_y[b][o] = sum_k deq(W_i[o][k]) * x_i[b][k]   for b < batch,
 * fp32 accumulation; the weights never reach memory in decoded form.
 * Defined by: LazyWeights' decode on demand, where memory moves only coded
 * bytes and the consuming matrix-vector work is unchanged (abstract);
 * EntroLLM's note that token generation is bandwidth-bound (gist.science
 * technical summary, Problem statement).  batch in 1..8; g is a host array
 * of n items. */
entro_status entro_decode_gemv(const entro_tensor *t, size_t n, const entro_gemv_item *g,
                               uint32_t batch, uint32_t *d_status, hipStream_t stream);

/* Fused decode + dequant + GEMM for prompt processing (n_tokens activations
 * at once): for each tensor i,
 *   g[i].d_y[t][o] = sum_k deq(W_i[o][k]) * x_i[t][k]   for t < n_tokens,
 * with every weight decoded once and the products on the matrix cores
 * (bf16 inputs, fp32 accumulation).  Defined by: EntroLLM's separate
 * pre-fill measurement of the coded uint4 model (gist.science technical
 * summary, Experimental results, inference-latency item) with LazyWeights'
 * decode on demand (abstract); the dense product is where matrix cores
 * belong.  n_tokens in
 * 1..512; d_x[i] is bf16 [n_tokens][cols], 16-byte aligned; d_y[i] is fp32
 * [n_tokens][rows], overwritten.  Layouts decoded here: 4-bit codes, 64
 * lanes, refill every two steps, one row per chunk (chunk_symbols == cols,
 * cols a multiple of 128), rows of any length (streamed through small
 * on-chip rings), a stream below 2^30 words; ENTRO_E_FORMAT or
 * ENTRO_E_UNSUPPORTED otherwise.  Prompts of more than 256 tokens run as
 * several launches, each decoding every weight again.  The tile height
 * (16, 32 or 64 rows) follows the call's row count against the GPU's CU
 * count and changes the results only in fp32 summation order.  Data faults
 * set d_status bits as for the other entry points. */
entro_status entro_decode_gemm(const entro_tensor *t, size_t n, const entro_gemv_item *g,
                               uint32_t n_tokens, uint32_t *d_status, hipStream_t stream);

/* Cap the workgroups of every later launch of this library in this process
 * (0, the default: no cap).  A launch then spreads its chunks, tasks or tiles
 * over at most n workgroups (the fused GEMV's streamed launches: at least one
 * per tensor), which leaves CUs free for work on other streams and gives
 * each wavefront a longer run; results do not depend on it.  A launch
 * setting, not part of the method; returns the previous cap. */
uint32_t entro_set_max_workgroups(uint32_t n);

/* Static English text for a status code. */
const char *entro_status_str(entro_status s);

#ifdef __cplusplus
}
#endif

#endif /* ENTRO_H */
