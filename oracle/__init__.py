"""CPU oracle for batched paged-KV attention -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct float64 implementation of what the paged
attention path computes: the KV store by slot, the CSR page-table arithmetic,
per-request masked softmax attention with GQA, and the log-sum-exp merge of
split states.  It shares no code with the HIP library and imports nothing from
it.  Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import it; the product path never does.

Pinned functions (see tests/test_oracle_pins.py and
tests/test_generated_cache_pins.py): every function here is pinned against
page-printed worked examples, library routines, closed forms or brute force.
The window rule follows the masks formula the pages print (keys t >= p - w) and
the natural-log LSE follows their merge formula, both checked by tests that
encode them independently; the negative padding slot of a slot mapping is an
interface convention with nothing to compute.
"""
from . import attention, codecs, metadata  # noqa: F401
