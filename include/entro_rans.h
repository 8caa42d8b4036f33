/*
 * entro_rans.h - the interleaved rANS variant of the coded-weight stream
 * ("ECR v1"): same quantized codes, same chunks and lanes as the Huffman
 * stream of entro.h, a range-ANS coder per lane instead of a prefix code.
 *
 * Defined by: LazyWeights' comparison of its Huffman decoder with an rANS
 * decoder in rate and area at equal throughput (LazyWeights abstract,
 * arXiv 2611.17108).  The pages fix no rANS parameters; the layout below is
 * this library's reading, built to mirror the Huffman stream so that the two
 * decoders can be compared on one GPU.
 *
 * Layout (ECR v1):
 *   - frequencies: the code histogram scaled to M = 4096 (entro_rans_freqs);
 *     cum[s] = sum of the frequencies of the codes below s;
 *   - coder: 32-bit state per lane, L = 2^16, 16-bit units.  Decoding a code
 *     from state x: slot = x mod M, s the code whose range [cum, cum + f)
 *     holds slot, x = f (x div M) + slot - cum, then x = x * 2^16 + (next
 *     unit) if x < L (one unit always suffices).  The encoder is the exact
 *     inverse, run backwards from x = L; every lane ends decoding at L;
 *   - chunks and lanes as in entro.h (code k of a chunk: lane k mod W,
 *     step k div W);
 *   - a chunk's 16-bit units: each lane's initial state (low half first,
 *     lanes in order), then the renormalization units in the order a
 *     lockstep decoder takes them (step by step, lanes of a step in
 *     increasing order); chunk_unit_off[c] = units before chunk c.
 *
 * Pointers named d_* are device pointers, the others host pointers, all
 * owned by the caller.  Status codes, d_status flags and stream semantics
 * are those of entro.h.
 */
#ifndef ENTRO_RANS_H
#define ENTRO_RANS_H

#include <stddef.h>
#include <stdint.h>

#include "entro.h"

#ifdef __cplusplus
extern "C" {
#endif

#define ENTRO_RANS_M_BITS 12

/* Scale a histogram of `alphabet` code values (2..256) to frequencies that
 * sum to 4096: every present value gets max(1, floor(4096 c / N)); while the
 * sum is below 4096 the value with the largest shortfall 4096 c / N - f gains
 * one (ties: lower value); while above, the largest frequency above 1 loses
 * one (ties: lower value).  Absent values get 0.  ENTRO_E_INVAL for null
 * pointers or an empty histogram, ENTRO_E_CODEBOOK for more than 4096
 * present values. */
entro_status entro_rans_freqs(const uint64_t *counts, uint32_t alphabet, uint32_t *freqs);

/* Bytes of the decode table (16-byte header + 4096 slots of 8 bytes). */
size_t entro_rans_table_bytes(void);

/* Decode table for frequencies freqs[1 << sym_bits] (summing to 4096) and the
 * dequantization bf16 = RNE(f32(scale) * f32(q - zero_point)): for every slot
 * the code, its bf16 value, its frequency and the slot's offset in the code's
 * range.  Errors: ENTRO_E_INVAL (null pointers, cap too small),
 * ENTRO_E_FORMAT (sym_bits not 4/8), ENTRO_E_CODEBOOK (frequencies not
 * summing to 4096). */
entro_status entro_rans_table_build(uint32_t sym_bits, const uint32_t *freqs, float scale, int32_t zero_point,
                                    void *host_table, size_t cap);

/* Encode n codes (q[i] < 2^sym_bits, each with a nonzero frequency) as ECR v1
 * with `chunk` codes per chunk and `lanes` lanes, on up to `threads` host
 * threads (0: all).  chunk_unit_off receives ceil(n / chunk) + 1 offsets;
 * *n_units the total; units (if not null) receives the units when cap_units
 * is large enough, else ENTRO_E_INVAL is returned with *n_units set.
 * Errors: ENTRO_E_INVAL, ENTRO_E_FORMAT (lanes not a power of two in 1..64,
 * chunk not a positive multiple of lanes), ENTRO_E_CODEBOOK (a code with
 * frequency 0, or frequencies not summing to 4096). */
entro_status entro_rans_encode(const uint8_t *q, uint64_t n, const uint32_t *freqs, uint32_t sym_bits,
                               uint32_t chunk, uint32_t lanes, uint64_t *chunk_unit_off, uint16_t *units,
                               uint64_t cap_units, uint64_t *n_units, uint32_t threads);

/* One rANS-coded tensor as the device entry points read it. */
typedef struct {
  const void *d_table;              /* entro_rans_table_build bytes, on the device        */
  const uint16_t *d_units;          /* [n_units] ECR v1 stream                            */
  const uint64_t *d_chunk_unit_off; /* [n_chunks + 1]                                      */
  uint64_t n_units;
  uint64_t n_symbols;               /* 0 = empty tensor (skipped)                          */
  uint32_t chunk_symbols;           /* C >= 1, a multiple of lanes, <= 2^20                */
  uint32_t lanes;                   /* W in {32, 64}                                       */
  uint32_t sym_bits;                /* 4 or 8                                              */
  uint32_t max_chunk_units;         /* units of the largest chunk (sizes the staging)      */
} entro_rans_tensor;

/* Decode n rANS-coded tensors to their codes (d_out[i]: n_symbols bytes,
 * 2-byte aligned) or to bf16 (d_out_bf16[i]: n_symbols values, 4-byte
 * aligned).  A wavefront decodes 64 / lanes chunks in lockstep, the slot
 * table in LDS.  d_status as in entro.h (ENTRO_F_OVERRUN / UNDERRUN: a chunk
 * needs more units than it has / leaves some unused; ENTRO_F_PADDING: a lane
 * does not end in state L; ENTRO_F_OFFSETS: bad chunk offsets or a chunk
 * larger than stated; ENTRO_F_LUT: table header mismatch).  Errors:
 * ENTRO_E_INVAL, ENTRO_E_FORMAT (lanes other than 32 or 64, chunk, sym_bits),
 * ENTRO_E_UNSUPPORTED (a chunk larger than the on-chip staging). */
entro_status entro_rans_decode(const entro_rans_tensor *t, size_t n, uint8_t *const *d_out, uint32_t *d_status,
                               hipStream_t stream);
entro_status entro_rans_decode_dequant(const entro_rans_tensor *t, size_t n, uint16_t *const *d_out_bf16,
                                       uint32_t *d_status, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ENTRO_RANS_H */
