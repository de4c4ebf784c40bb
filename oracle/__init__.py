"""CPU fp64 oracle for exact attention.

TEST INFRASTRUCTURE ONLY. The only code allowed to import, call or execute
anything in this package is: ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``. The library (``exact_attention_amd``)
never imports it, and the oracle imports nothing from the library: the two share
no kernels, helpers, tables or constants. Only the seeded input generators in
``workloads`` serve both sides.

What it computes is the plain definition of attention, in float64, on the same
bf16 / e4m3-rounded input bits the GPU reads:

    O = softmax(scale * Q K^T) V,   lse = log(sum_j exp(scale * q_i . k_j))

(stated as exact attention in "FlashAttention: not less compute, less data
movement", section 01; the tiled/online method reaches the same result up to
rounding order, section 02 there), and its gradients with respect to Q, K and V
for a given output gradient dO (``attention_backward``: the five products of
the backward in "Low-precision FlashAttention-4: end-to-end block-scaled
attention for Blackwell", section 2.2, evaluated on full score rows). Every function here evaluates full score
rows with a two-pass softmax; none of them use the streaming recurrence except
``online_softmax_row``, which restates that recurrence so the pins can compare
the two formulations.

Parity status: every function is pinned by a CPU test in
``tests/test_oracle_pins.py`` (worked example, closed forms, brute force at
50 digits, invariants) except where marked "parity unpinned" below.
"""
from .attention import (  # noqa: F401
    bf16_to_f64,
    e4m3_to_f64,
    e5m2_to_f64,
    e8m0_to_f64,
    dequant_mx,
    allowed_keys,
    attention,
    attention_rows,
    attention_varlen,
    gather_pages,
    decode_paged,
    decode_paged_heads,
    online_softmax_row,
    lse_combine,
    attention_backward,
)
