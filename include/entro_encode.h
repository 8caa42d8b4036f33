/*
 * entro_encode.h - offline (host-only) side of the entropy-coded weight
 * library: per-tensor quantization, optimal length-limited code lengths and
 * the ECW v1 stream encoder.  Everything here runs on the CPU, once per
 * tensor, before the device entry points of entro.h decode the result.
 *
 * Method: EntroLLM (arXiv 2505.02380) quantizes each tensor as a whole with
 * an unsigned or an asymmetric scheme chosen from the tensor's weight
 * distribution (abstract; gist.science technical summary, Methodology item 1),
 * then Huffman-codes the integer codes (item 2) in chunks that can be decoded
 * independently (item 3); LazyWeights (arXiv 2611.17108) codes them in
 * interleaved lanes (abstract).  The stream layout is described in entro.h.
 *
 * All pointers are host pointers owned by the caller.  Functions are
 * reentrant and allocate only transient host memory.
 */
#ifndef ENTRO_ENCODE_H
#define ENTRO_ENCODE_H

#include <stddef.h>
#include <stdint.h>

#include "entro.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ENTRO_Q_ASYMMETRIC = 0,  /* min-max affine: s = (max-min)/Q, zp = clamp(rint(-min/s))      */
  ENTRO_Q_UNSIGNED = 1,    /* symmetric range, unsigned codes: s = m/(2^(b-1)-1), zp = 2^(b-1) */
  ENTRO_Q_MIXED = 2        /* both; keep the lower code entropy, ties to asymmetric          */
} entro_qscheme;

/* Quantize n float32 weights to bits-bit codes (bits 4 or 8), one scale and
 * zero point for the whole tensor: q = clamp(rint(w / s) + zp, 0, 2^bits - 1),
 * computed in float64 with s rounded to float32 first; rint rounds half to
 * even.  For ENTRO_Q_UNSIGNED, clip > 0 replaces max|w| as the range end.
 * A tensor with max == min (or max|w| == 0) gets s = 1.  chosen (optional)
 * receives the scheme used.  Defined by: EntroLLM's tensor-level mixed
 * quantization (abstract; gist.science technical summary, Methodology item 1);
 * the formulas are readings, the pages print none.
 * Errors: ENTRO_E_INVAL (null pointers), ENTRO_E_FORMAT (bits, scheme). */
entro_status entro_quantize(const float *w, uint64_t n, uint32_t bits, entro_qscheme scheme,
                            float clip, uint8_t *q_out, float *scale_out, int32_t *zero_point_out,
                            entro_qscheme *chosen);

/* Optimal prefix-code lengths for the histogram of q (n codes < 2^bits) with
 * every length <= max_len (minimum sum of count * length; package-merge).
 * code_len_out receives 2^bits lengths, 0 for absent values; a tensor with a
 * single distinct value gets length 1.  Defined by: Huffman coding of the
 * quantized weights from their frequencies (gist.science technical summary,
 * Methodology item 2); the length cap is needed by the decode tables.
 * Errors: ENTRO_E_INVAL (null, n == 0, code out of range), ENTRO_E_FORMAT. */
entro_status entro_code_lengths(const uint8_t *q, uint64_t n, uint32_t bits, uint32_t max_len,
                                uint8_t *code_len_out);

/* Chunk offsets of the ECW v1 stream of q: chunk_bit_off receives
 * ceil(n / chunk) + 1 entries, n_words the total word count.
 * Errors: ENTRO_E_INVAL, ENTRO_E_FORMAT (lanes, chunk), ENTRO_E_CODEBOOK
 * (a code without codeword). */
entro_status entro_encode_layout(const uint8_t *q, uint64_t n, const uint8_t *code_len, uint32_t bits,
                                 uint32_t chunk, uint32_t lanes, uint64_t *chunk_bit_off,
                                 uint64_t *n_words);

/* Write the ECW v1 words of q (offsets from entro_encode_layout) using up to
 * `threads` host threads (0 = hardware concurrency).  refill_steps (1 or 2;
 * 0 means 1) is the number of steps per refill decision and refill_ahead
 * (0 or 1) selects refilling ahead, see entro.h; the decoder must be given
 * the same values.  With 2 steps, every code length must be at most 16
 * (always true for the codebooks of entro_code_lengths).  Refilling ahead
 * stores the same words in another order (offsets are unchanged). */
entro_status entro_encode(const uint8_t *q, uint64_t n, const uint8_t *code_len, uint32_t bits,
                          uint32_t chunk, uint32_t lanes, uint32_t refill_steps, uint32_t refill_ahead,
                          const uint64_t *chunk_bit_off, uint32_t *words, uint32_t threads);

#ifdef __cplusplus
}
#endif

#endif /* ENTRO_ENCODE_H */
