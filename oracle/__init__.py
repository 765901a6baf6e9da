"""Plain, slow, fp64 CPU oracle for paged MQA logits.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call, link or execute anything under
``oracle/``.  Only the tests, the smoke check and the CPU-baseline leg of the
benchmark use it.

What it computes is the scoring step of a sparse-attention indexer described
on the page "[flashinfer] Blackwell 아키텍처를 위한 고성능 Paged MQA Logits 커널
도입" (introduction: ReLU of each head's score against a paged KV token,
weighted per head and summed over heads), with the formula

    logits[r, t] = sum_h w[r, h] * ReLU(scale_t * q[r, h, :] . k_t)

for t below the row's causal limit, and -inf elsewhere.

Modules
-------
formats       exact e4m3fn / e2m1 / e8m0 decoders built from the bit fields
reference     the fp64 definition for the fp8 and MXFP4 variants
exact         rational (fractions.Fraction) brute force for tiny inputs
schedule_ref  the persistent-worker partition: linear scan and binary search
quantize      the cache producer: fp8 and MXFP4 quantize-and-append
topk          top-k token selection over rows of logits

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against something other than itself (library casts, brute force, closed
forms, invariants).  No function is "parity unpinned".
"""
