"""CPU oracle for the fused FP8 ReLU^2 MLP path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
``cpu_baseline`` leg of the benchmark may import this package.  The product
(the HIP library and its Python binding) never imports, links or calls it, and
this package imports nothing from the product.

Everything here is plain numpy in float64 with every rounding written out:

* ``formats``  -- bf16 / fp32 / OCP e4m3 number formats (decode, round-to-
  nearest-even encode, saturation).
* ``mlp``      -- the method: up-projection + ReLU^2 + delayed-scale e4m3
  quantisation + partial amax, FP8 down-projection against a transposed
  fp8 W2 cache, the bf16 backward that rebuilds relu(pre) as sqrt(post),
  the weight cast-transpose, amax reduction and the FP8 linear used for the
  attention projections.
* ``stack``    -- the layer stack around the block (RMSNorm, residual, SGD).
* ``ce``       -- the fused softcapped cross-entropy over a language-model
  head (loss, logit gradient, dX, dW).

Parity pins: every function is checked in ``tests/test_oracle_*.py`` against
something other than itself (the OCP e4m3 code points, torch's independent
CPU casts, brute-force loops, closed forms, finite differences and a lossless
special case).  Nothing in this package is "parity unpinned".
"""
from . import ce, formats, mlp, stack  # noqa: F401
