"""CPU oracle for response-replay attention.  TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 NumPy implementations of what the HIP library computes.  Only the
test suite, the package entry point's smoke check and the benchmark's CPU-baseline leg
may import it; the product path never does.  It shares no code with the HIP path: the
only thing both sides see are the seeded input arrays, which callers pass in already
widened to fp64.

Modules
  dense   exact attention of replayed response rows over a stop-gradient resident
          prompt KV plus the response's own causal KV; response-only backward; per-chunk
          softmax-statistics partials and their exact merge; full-sequence gradients
          (the prompt-side term the response-only contract drops); serial accumulation.
  sparse  latent-page variant: fp64 index scores, per-query top-k selection with ties
          broken toward the lower position, attention over the selected latent rows
          plus the causal response rows, response-only backward.

Parity pins: every function is checked in tests/test_oracle_*.py against something
other than itself (torch's CPU fp64 scaled_dot_product_attention and autograd, finite
differences, closed forms, brute-force enumeration, hand-derived fixtures under
tests/golden/).  No function here is "parity unpinned".
"""
from . import dense, lastkv, sparse  # noqa: F401
