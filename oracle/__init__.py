"""CPU oracle for batched paged-KV attention -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct float64 implementation of what the paged
attention path computes: the KV store by slot, the CSR page-table arithmetic,
per-request masked softmax attention with GQA, and the log-sum-exp merge of
split states.  It shares no code with the HIP library and imports nothing from
it.  Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import it; the product path never does.

Pinned functions (see tests/test_oracle_pins.py): every function here is pinned
against page-printed worked examples, library routines, closed forms or brute
force.  Window inclusivity, the LSE base and the padding-slot sentinel are
readings of the pages with no printed number to pin them ("parity unpinned" for
those three conventions; the arithmetic around them is pinned).
"""
from . import attention, codecs, metadata  # noqa: F401
