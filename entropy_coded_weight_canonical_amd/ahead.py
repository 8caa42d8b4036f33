"""Decode-ahead streaming: coded weight matrices consumed by an unchanged
matrix-multiply kernel.

LazyWeights keeps the GPU's compute kernels unchanged and decodes the coded
weights on their way from DRAM, so that only coded bytes cross the memory bus
(LazyWeights abstract, arXiv 2611.17108).  The software analogue on one GPU:
while the stock kernel (``torch.mm``, hipBLASLt on ROCm) multiplies by one
block of rows of a matrix, the library decodes the next block to bf16 on a
side stream into one of ``depth`` staging buffers; events order the two
streams (the decode of block k + depth waits until the multiply of block k
has read its buffer, the multiply of block k until block k is decoded).

A block is a run of whole chunks: with row-aligned chunks (chunk a multiple
of the row length) a block of chunks is a block of rows, decoded through a
descriptor that covers only those chunks of the full stream.  Small blocks
keep the staging buffers cache-resident between the decode and the multiply;
``block_elems=None`` decodes whole matrices.  The staging decodes are issued
with ``out_cached`` set (ordinary stores instead of the streaming stores of a
standalone decode), so that the multiply finds the weights in L2 or the
last-level cache.

Every decode runs in the library's kernels (``decode_dequant``); this module
only orders launches on torch streams (all at the default priority).  A whole
``run`` can be captured in a HIP graph (``torch.cuda.graph``) and replayed.
"""
from __future__ import annotations

from typing import Sequence

from . import Tensor, decode_dequant


def chunk_range_view(desc: Tensor, c0: int, c1: int) -> Tensor:
    """Descriptor of chunks ``[c0, c1)`` of a coded tensor (same words, same
    table; offsets are positions in the full stream)."""
    chunk = int(desc.chunk_symbols)
    n = min(c1 * chunk, int(desc.n_symbols)) - c0 * chunk
    if not (0 <= c0 < c1) or n <= 0:
        raise ValueError("empty or out-of-range chunk range")
    return Tensor(desc.d_lut, desc.d_words, int(desc.d_chunk_bit_off) + 8 * c0, desc.n_words, n,
                  desc.chunk_symbols, desc.lanes, desc.sym_bits, desc.max_len, desc.lut_bytes,
                  desc.max_chunk_words, desc.refill_steps, desc.refill_ahead, desc.out_cached)


def _staging(desc: Tensor) -> Tensor:
    """The staged weights are read by the next matrix product right away:
    decode them with ordinary stores, which leave them in the caches."""
    desc.out_cached = 1
    return desc


class DecodeAhead:
    """A fixed sequence of coded matrices ``W_m`` (``rows_m x cols_m``, row-major
    ``[out][in]``) multiplied in order by inputs ``x_m`` with the stock kernel,
    each block of rows decoded to bf16 just ahead of its use."""

    def __init__(self, tensors: Sequence, shapes: Sequence[tuple[int, int]], depth: int = 2,
                 block_elems: int | None = None, device="cuda"):
        import torch

        if len(tensors) != len(shapes) or not tensors:
            raise ValueError("need one (rows, cols) shape per coded tensor, and at least one tensor")
        if depth < 2:
            raise ValueError("depth must be at least 2 (one buffer decoding while another is read)")
        self.tensors = list(tensors)
        self.shapes = [(int(r), int(c)) for r, c in shapes]
        # blocks: (matrix, first row, end row, descriptor)
        self.blocks = []
        for m, (t, (r, c)) in enumerate(zip(self.tensors, self.shapes)):
            d = t.desc
            if int(d.n_symbols) != r * c:
                raise ValueError(f"tensor of {d.n_symbols} symbols does not match shape {r}x{c}")
            chunk = int(d.chunk_symbols)
            n_chunks = -(-r * c // chunk)
            if block_elems is None or chunk % c or r * c <= block_elems:
                self.blocks.append((m, 0, r, _staging(chunk_range_view(d, 0, n_chunks))))
                continue
            rows_per_chunk = chunk // c
            per = max(1, int(block_elems) // chunk)
            for c0 in range(0, n_chunks, per):
                c1 = min(n_chunks, c0 + per)
                self.blocks.append((m, c0 * rows_per_chunk, min(r, c1 * rows_per_chunk),
                                    _staging(chunk_range_view(d, c0, c1))))
        self.depth = min(depth, len(self.blocks))
        elems = max((r1 - r0) * self.shapes[m][1] for m, r0, r1, _ in self.blocks)
        self.bufs = [torch.empty(elems, dtype=torch.bfloat16, device=device) for _ in range(self.depth)]
        self.status = torch.zeros(len(self.tensors), dtype=torch.int32, device=device)
        self.side = torch.cuda.Stream(device=device)
        self.ready = [torch.cuda.Event() for _ in range(self.depth)]
        self.free = [torch.cuda.Event() for _ in range(self.depth)]

    def _decode(self, k: int) -> None:
        m, _, _, desc = self.blocks[k]
        b = k % self.depth
        if k >= self.depth:
            self.side.wait_event(self.free[b])
        decode_dequant([desc], [self.bufs[b].data_ptr()], self.status.data_ptr() + 4 * m, stream=self.side)
        self.ready[b].record(self.side)

    def run(self, xs: Sequence) -> list:
        """``y_m = x_m W_m^T`` for every matrix in order, on the current stream;
        ``x_m`` is bf16 ``[batch, cols_m]``, ``y_m`` a bf16 ``[batch, rows_m]``
        view of a ``[rows_m, batch]`` result.

        Decode flags of matrix m are OR-ed into ``self.status[m]`` (cleared at
        the start of each run); read them after synchronizing.
        """
        import torch

        if len(xs) != len(self.tensors):
            raise ValueError("need one input per matrix")
        main = torch.cuda.current_stream()
        self.side.wait_stream(main)
        with torch.cuda.stream(self.side):
            self.status.zero_()
        for k in range(self.depth):
            self._decode(k)
        xts = [x.t().contiguous() for x in xs]
        yts = [torch.empty((r, x.shape[0]), dtype=torch.bfloat16, device=x.device)
               for (r, _), x in zip(self.shapes, xs)]
        for k, (m, r0, r1, _) in enumerate(self.blocks):
            b = k % self.depth
            c = self.shapes[m][1]
            main.wait_event(self.ready[b])
            torch.mm(self.bufs[b][: (r1 - r0) * c].view(r1 - r0, c), xts[m], out=yts[m][r0:r1])
            self.free[b].record(main)
            if k + self.depth < len(self.blocks):
                self._decode(k + self.depth)
        main.wait_stream(self.side)
        return [yt.t() for yt in yts]
