"""CPU oracle for entropy-coded weights — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct implementations of what the GPU path computes,
written from the descriptions of EntroLLM (arXiv 2505.02380) and LazyWeights
(arXiv 2611.17108).  Only the test-suite, the smoke check and the benchmark's
CPU-baseline leg may import or execute anything in this package; the product
library never does, and this package never imports the product library.

Modules
-------
quant      per-tensor quantizers (asymmetric / unsigned), mixed selection, entropy
huffman    optimal code lengths: heap Huffman and package-merge (length-limited)
canonical  canonical code assignment from code lengths
ecw        chunked, lane-interleaved stream: pure-Python encoder and a
           bit-serial canonical decoder (small inputs)
ccodec     the same encoder / decoder in plain C (``codec.c``) for full sizes
dequant    code -> fp32 -> bf16 (round to nearest even)
gemv       float64 GEMV on dequantized weights, and the error metric
rans       interleaved rANS coder of the same codes: frequency quantizer,
           encoder and lockstep decoder (small inputs)
groupwise  group-wise quantizer, for the tensor-level versus group-wise study
entropy_study  code entropy, Huffman mean length and side information of
           every workload under both quantizers

Parity status (what pins each function; see the tests named in each module):
every function listed above is pinned by tests that do not call it back
(brute force, closed forms, invariants, library routines, hand-derived
fixtures under ``tests/golden``).  No function here is "parity unpinned".
"""
