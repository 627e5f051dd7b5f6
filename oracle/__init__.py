"""CPU fp64 oracle of the Kimi K3 LatentMoE layer forward.

TEST INFRASTRUCTURE. This package is the slow, plain definition the GPU path is
checked against. Only the tests, the smoke check and the benchmark's CPU
baseline may import it; the library and its Python binding never do, and it
shares no code with them.

What it follows: the Kimi K3 course, lesson 6 "LatentMoE" -- the layer of
"show me the actual equation" (eq. 11: routed experts in latent space, p-weighted
combine, RMSNorm, up-projection, plus full-width shared experts) and the router
of eq. 13 (sigmoid scores, bias-steered top-k, weights renormalised over the
selected set from the unbiased scores).

Precision: every value is an fp64 number. Weights and quantised activations are
decoded exactly (MX codes times power-of-two scales are exact in fp64); the
quantisation points named by the workloads (bf16 rounding or MXFP8 encoding of
activations) are applied where the layer's definition places them.

Parity pins live in tests/ (run with -m "not gpu"). Functions without such a pin
say "parity unpinned" in their docstring; at present there are none.
"""
from . import mx, layer  # noqa: F401
