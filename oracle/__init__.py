"""CPU oracle for the Averis mean-residual split FP4 linear (fwd + dgrad hot path).

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow reference that the
HIP library is checked against.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the product path never does.
It shares no code with the HIP path: no kernels, headers, tables or helpers.

Sources (cited by title and section throughout; no line numbers):

* [Lighthouse] -- the "Lighthouse" blog review of "The Curse and Blessing of
  Mean Bias in FP4-Quantized LLM Training" (dongdongbear.github.io).
  §2.1 defines the activation matrix X (l tokens x m hidden) and its column
  mean over tokens, mu_X = (1/l) 1^T X, and the three-part decomposition
  X = 1 mu^T + U_k S_k V_k^T + X_tail.  §2.2 "Averis 方法" gives the forward
  Y = 1(mean_q W_q) + X_R,q W_q with mean_q = Q4(mu_X), X_R,q = Q4(X - 1 mu_X),
  the backward dX = 1(mean_q,D W_q^T) + D_R,q W_q^T (same split on the output
  gradient D), and the cost note (two reduces, two subtractions).  §3.1 fixes
  the format: W4A4G4, E2M1 NVFP4 elements, stochastic rounding by default.
  §1.1 says the block scale is set by the block's largest magnitude.
* [Abstract] -- the arXiv abstract (v2) of the same paper: Averis separates the
  mean with reductions and elementwise subtractions before FP4 quantization;
  vanilla NVFP4 is the comparison arm.
* [Gist] -- the gist.science technical summary of the same paper, §2 "Il
  Metodo Proposto: Averis": X_R = X - 1 mu_X^T, mean and residual quantized
  independently, forward and backward recomposed from the two parts.
* [NVFP4-outliers] -- abstract of "Dissecting Outlier Dynamics in LLM NVFP4
  Pretraining": NVFP4 uses hierarchical (two-level) microscaling.

Where the pages leave a step open (the exact NVFP4 two-level scale recipe, the
rounding of every FP32 intermediate, the SR bit budget, the RNG counter
layout, the precision of the mean), the oracle takes one stated reading; each
is listed in the module that implements it.

Parity status: every function here is pinned by a `-m "not gpu"` test against
something other than itself (closed forms, invariants, torch's E4M3 cast,
rocRAND's Philox4x32-10, brute force on tiny inputs).  None is unpinned.
"""

from . import philox, formats, averis  # noqa: F401
