"""CPU oracle for SANTA stochastic sparse decode-step attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The GPU library never links it, the Python binding never imports
it, and there is no CPU fallback that routes through it.

The oracle is a plain, slow, obviously correct fp64 NumPy implementation of
what the method computes, written from the abstract "Stochastic Sparse
Attention for Memory-Bound Inference" (arXiv 2605.01910; both versions of the
abstract) plus the readings of what that abstract leaves open, each stated in
the docstring of the function that depends on it.  It shares no code, tables
or constants with the HIP path; the only thing both sides share is the seeded
input generator module
``stochastic_sparse_decode_amd.workloads``, which contains none of the
method's arithmetic.

Modules
-------
philox   Philox4x32-10 counter-based generator (Salmon et al., SC'11) and the
         uniform stream layout used by the sampler.
santa    scores, softmax distribution, stratum points, inverse-CDF search,
         gather-average estimate, dense attention and the Bernoulli qK^T mode.
moments  exact first and second moments of the three estimators.
fp8      exact decoding of the OCP E4M3 bytes of the fp8 key cache.
parity   index-parity bookkeeping: which index differences a CDF boundary
         within the tolerance band excuses.

Parity status: every function here is pinned by a ``-m "not gpu"`` test
against something other than itself (known-answer vectors, a library
routine, closed forms, brute-force enumeration or fine-grid integration).
"""

from . import fp8, moments, parity, philox, santa  # noqa: F401
