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

Parity status: every public function is pinned by ``tests/test_oracle_pins.py``
(closed forms, invariants, a brute-force ``math.fsum`` implementation, the
CPU float64 ``torch.nn.functional.scaled_dot_product_attention`` library
routine and the block-table worked example in ``tests/golden/``).  No function
here is "parity unpinned".
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
