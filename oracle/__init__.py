"""fp64 CPU oracle for skip-softmax (BLASST) attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import this package. The product path (the C-ABI library and its Python
binding) never imports, links or calls anything here, and this package never
imports the product path: the two share no code. Both may consume inputs from
the `synth` generator, which holds no attention arithmetic.

Contents:
  skip_softmax  -- the tile loop of the method, step by step (sequential form),
                   its prefix-max fast form, the multi-threshold calibration
                   counter and the textbook dense attention definition.
  calibration   -- log2 threshold conversion, the log-space exponential fit,
                   threshold resolution with its priority rules.
  gating        -- flow-schedule timesteps, the disabled_until_timestep
                   cutoff and per-layer ignore / override patterns.

Parity status of every function is stated in its docstring ("pinned by ..."
or "parity unpinned").
"""
from . import calibration, gating, skip_softmax  # noqa: F401
