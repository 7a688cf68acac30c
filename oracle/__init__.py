"""Reference oracle for exact scaled dot-product attention and paged-KV decode.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: it is used by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``, and by nothing else.  It shares
no code with the HIP library under ``paged_attention_attn_amd/``; the only
module both sides use is ``workloads`` (seeded input generators, which hold
none of the method's arithmetic).

Every function computes the plain definition in float64 with NumPy: explicit
scores, a max-shifted softmax over the whole visible key range of each row,
then the probability-weighted sum of values.  There is no online softmax, no
tiling and no split-KV merge here.

Parity status: every public function has a pin in ``tests/oracle_pins.py``
(run by ``tests/test_oracle_pins.py``, which also plants mistakes in the
helpers and checks that some pin catches each one):

* ``attention``: closed forms (Q = 0, identical V rows, causal row 0), a
  brute-force ``math.fsum`` loop, torch's CPU float64 SDPA, GQA against
  repeated KV heads, key permutation, and a separate tile-by-tile online
  model of the recurrence; ``softmax_probs``: rows sum to 1.
* ``attention_rows``, ``attention_window_rows``, ``attention_fp8_rows``: equal
  to the selected rows of the full functions.
* ``attention_window``: brute force, torch SDPA with a loop-built mask,
  window 1, window 1 with one global token.
* ``paged_gather``, ``paged_decode``: the pages' block-table example
  (``tests/golden/``), decode = last row of causal prefill, L = 1, L = 0,
  page-permutation invariance; the ``seqs=`` subset equals the full call's
  rows in order.
* ``paged_append``, ``paged_prefill``: torch SDPA over context + chunk, the
  block-table example with an appended chunk, one-token chunk = decode,
  no-context chunk = causal prefill, two chunks = one, brute force; the
  ``seqs=`` subset equals the full call's rows in order.
* ``e4m3_bits_to_f64``, ``attention_fp8``, ``paged_decode_fp8``: torch's
  ``float8_e4m3fn`` decoding of all 256 codes and hand-decoded codes, torch
  SDPA over torch-decoded inputs, the scales entering linearly, FP8 decode =
  the bf16 decode of the same values, the ``seqs=`` subset.
* ``bf16_bits_to_f64``: hand-decoded bit patterns.

No function here is "parity unpinned".
"""

from .exact import (  # noqa: F401
    attention,
    attention_fp8,
    attention_fp8_rows,
    attention_rows,
    attention_window,
    attention_window_rows,
    paged_append,
    paged_decode,
    paged_decode_fp8,
    paged_gather,
    paged_prefill,
    softmax_probs,
    bf16_bits_to_f64,
    e4m3_bits_to_f64,
)
