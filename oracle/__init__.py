"""Float64 CPU oracle for decode attention over a low-rank-compressed KV cache.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package. The HIP library never imports it and shares no code, header, table or
helper with it; the two meet only at the seeded inputs of ``synth``.

Everything is numpy float64 except the int4 codec, which reproduces the fixed
fp32 / fp16 steps of the quantiser on purpose (see ``codec``).

Modules and what pins each one (tests/test_oracle_*.py):

* ``prep``       offline weight preparation: truncated SVD factoring, G-LRD
                 grouping, Walsh-Hadamard fold, value/key fusion.
                 Pinned by Eckart-Young closed forms, full-rank equivalence,
                 the fusion identities and Hadamard orthogonality.
* ``rope``       rotate-half rotary embedding. Pinned by norm preservation,
                 relative-position invariance and the explicit inverse.
* ``codec``      symmetric int4, groups of 32, fp16 scales. Pinned by
                 hand-built tie cases, the error bound and amax -> +-7.
* ``attn``       textbook softmax attention, the reconstruct-with-RoPE and
                 absorbed-query decode paths, chunked online softmax.
                 Pinned by dense attention at full rank, brute-force loops and
                 chunk-count independence.
* ``paged``      page states, truncated-SVD / Gram-eigen / Jacobi page factors,
                 hybrid dense+factored attention. Pinned by the closed-form
                 page states against a token-by-token replay, Eckart-Young
                 optimality, the storage-ratio formula and dense equivalence.
* ``accounting`` KV-cache and latent byte counts. Pinned by the sizes the pages
                 print for Qwen3-32B and Llama-3.1-8B.
* ``brute``      pure-Python loop versions for tiny shapes.

Every function above has at least one such pin. The pages print no worked
numeric example of an attention output or of an int4 code, so those values are
pinned by the identities, closed forms, special cases and brute force listed
above rather than by stored printed numbers.
"""
