"""fp64 CPU oracle of the IndexMem / MomentKV hot path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never calls it, and it shares no code with the
GPU library: this package imports nothing but NumPy.

Sources (cited by page title and section throughout):
  [IM]   "IndexMem - learned KV-cache eviction with latent memory", technical summary
         (gist.science, arXiv 2605.25475; Japanese and Italian editions), section 2
         "Method": A (learnable indexer), B (latent memory), and its formula for o.
  [MKV]  "MOMENTKV" technical summary (gist.science, arXiv 2606.01563), Method parts
         1 (moment statistics), 2 (first-order approximation, displayed equation),
         3 (moment-informed eviction, displayed equation) and 4 (normalization-
         corrected inference, displayed equation).
  [ASM]  "Context Memorization for Efficient Long Context Generation" technical
         summary (gist.science, arXiv 2605.18226), Method: the attention state (a, Z)
         and its online-softmax merge.

Where the pages leave a step open the plainest reading is taken; every such reading
is named in the docstring of the function that takes it ("Reading: ...").

Parity status: every public function is pinned by tests/test_oracle_pins.py and
tests/test_oracle_golden.py against closed forms, textbook special cases, brute
force on tiny inputs or hand-computed fixtures; none is "parity unpinned".
"""
from . import asm, chunked, indexmem, moment_stream, momentkv, streaming  # noqa: F401
