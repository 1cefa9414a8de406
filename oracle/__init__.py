"""Oracle: a plain, slow, CPU-only definition of the low-bit dequantize-and-multiply path.

TEST INFRASTRUCTURE ONLY. Nothing in the product may import, call or execute anything in
this package; only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may. It shares no code, tables or constants with the HIP library and does not
import it; the only module both sides use is ``workloads`` (seeded random draws).

What it defines, following the two source pages:
  * "二三五六位量化" (lpnh.cn, 2/3/5/6-bit quantization): section 2.1 (two-level scales:
    fp16 super-block scale, low-bit sub-block scales, 256-weight super-blocks), section 2.2
    (little-endian cross-byte bit packing: 8 x 3-bit codes in 3 bytes, 8 x 5-bit codes in
    5 bytes, 4 x 6-bit codes in 3 bytes), section 2.3 (the byte table: 84 / 110 / 176 / 210
    bytes per super-block, 5- and 6-bit codes split into a low-4-bit plane and a high-bit
    plane), section 3.3 (the scalar GEMV form (s*q + m)*x and its Sigma-x factorization),
    section 3.4 (the self-check table: pack/unpack round trip, dequant error below half a step);
  * "DBHOO-CIM" (pwwt.cn, CPU INT4 inference): section 2.1 and 3.1 (symmetric INT4,
    scale = max|w|/8, q = clamp(round(w/scale), -8, 7), groups of 32 along the input
    dimension), section 3.2 (two codes per byte, low nibble first, stored as unsigned 0..15),
    section 4.1 (fp32 scales in a separate array), section 4.4 (effective bandwidth = weight
    bytes / latency);
  * act-order weights ("二三五六位量化" sections 2.4 and 3.2, stage 3: columns quantized in
    a stored permuted order, restored at inference), in ``actorder``;
  * the 8-bit KV-cache group codec ("二三五六位量化" section 4.1: one fp16 scale per 32
    elements, about 1.06 bytes per element), in ``kvcache``;
  * format variants: INT4 groups of 16/64/128, asymmetric INT4 with a zero point
    ("二三五六位量化" section 2.1) and INT4 with fp16 group scales (section 2.1) in ``int4``;
    super-block formats with bf16 super-scales (section 2.3) in ``superblock`` / ``bf16``.

Readings taken where the pages are silent or garbled are listed in each module's docstring.
Floating point is fp64 throughout except where the pages fix another precision (the INT4
quantizer computes its scale and quotient in fp32, as the page's PyTorch code does).

Parity status: every function here is pinned by tests under ``tests/test_oracle_*.py``
(golden vectors hand-derived from the pages' printed semantics, the pages' byte table,
closed forms, invariants and brute force). The choice of super-block scales is the pages'
silence filled by a stated rule ("range-covering round-to-nearest"); the rule itself is
pinned by hand-worked examples, but no page prints a scale value to compare with.
"""
