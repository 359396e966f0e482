"""Timestep and layer gating of skip-softmax attention, written from the pages.

TEST INFRASTRUCTURE ONLY (see the package header): never called by the product.

Sources (web pages, cited by title and section):
* TensorRT-LLM docs "VisualGen Sparse Attention (Beta)":
  - section "Checkpoint Config": disabled_until_timestep is a normalized
    [0, 1] cutoff. Skip-softmax is off while the timestep is >= the cutoff and
    on once it drops below. Ignore entries are fnmatch patterns that match
    full module names and component-relative names.
  - section "User Configuration": a direct threshold_scale_factor takes
    precedence over target_sparsity; checkpoint ignore patterns always
    disable matching layers.
  - section "Mapping disabled_until_timestep to Actual Denoising Steps":
    dense_steps = count(t[i] >= cutoff). For the 40-step flow schedule with
    1,000 training timesteps and flow shift 3 it prints the unshifted sigma
    s[i], the shifted sigma and a table of cutoff -> dense steps.
  - section on CUDA graphs: per-token timesteps reduce to their largest live
    value.
* TensorRT-LLM pull request "Add SkipSoftmax sparse attention support for
  visual generation", section "Use Cases", case 1d: per-layer overrides map
  fnmatch patterns to a threshold_scale_factor, where 0 means dense.

Readings where the pages are silent (each is listed in the design notes):
* The normalized runtime timestep is t[i] = (1 - 1/T) * shifted_sigma[i],
  with T the number of training timesteps. The pages do not print the
  conversion. Two other readings fail the printed table:
  - t = shifted_sigma gives 11 dense steps at cutoff 0.90, not 10;
  - t = shifted_sigma also gives 1 dense step at cutoff 1.00, not 0.
  This reading reproduces every printed row, and the printed t[13] ~ 0.861.
* A component-relative name is the module name without its first dotted
  component ("transformer.blocks.0.attn1" -> "blocks.0.attn1").
* When several override patterns match, the first one in the given order
  wins.
* A missing cutoff (None) never disables. A cutoff of 0.0 disables at every
  timestep in [0, 1].
"""
from __future__ import annotations

import fnmatch
from typing import Optional, Sequence, Tuple

import numpy as np

# Rules reported by gate_layer, same meaning as the library's.
RULE_BASE = 0       # base threshold applies
RULE_TIMESTEP = 1   # dense: timestep at or above the cutoff
RULE_IGNORED = 2    # dense: layer matches an ignore pattern
RULE_OVERRIDE = 3   # a per-layer override applies (its value may be 0 = dense)


def flow_timesteps(n_steps: int, num_train_timesteps: int = 1000, flow_shift: float = 3.0) -> np.ndarray:
    """Normalized runtime timesteps of an n-step flow-matching schedule.

    Follows "Mapping disabled_until_timestep to Actual Denoising Steps":
    - s[i] = 1 - i * (1 - 1/T) / n;
    - shifted = shift * s / (1 + (shift - 1) * s);
    - t[i] = (1 - 1/T) * shifted[i] (the conversion reading above).
    The page prints shifted = 3 s / (1 + 2 s), which is this formula at
    shift 3.
    Pinned by the printed 40-step table and the printed t[13] (tests).
    """
    T = float(num_train_timesteps)
    i = np.arange(n_steps, dtype=np.float64)
    s = 1.0 - i * (1.0 - 1.0 / T) / n_steps
    shifted = flow_shift * s / (1.0 + (flow_shift - 1.0) * s)
    return (1.0 - 1.0 / T) * shifted


def dense_steps(t: Sequence[float], cutoff: Optional[float]) -> int:
    """Number of schedule entries with t >= cutoff (equality is dense)."""
    if cutoff is None:
        return 0
    return int(sum(1 for x in t if x >= cutoff))


def _names(layer: str) -> Tuple[str, ...]:
    rel = layer.split(".", 1)[1] if "." in layer else None
    return (layer,) if rel is None else (layer, rel)


def layer_matches(layer: str, pattern: str) -> bool:
    """fnmatch (case-sensitive) against the full or component-relative name."""
    return any(fnmatch.fnmatchcase(n, pattern) for n in _names(layer))


def gate_layer(layer: str, timesteps: Sequence[float], base_scale_factor: float,
               cutoff: Optional[float] = None, ignore: Sequence[str] = (),
               overrides: Sequence[Tuple[str, float]] = ()) -> Tuple[int, float]:
    """Effective threshold_scale_factor of one attention layer at one forward.

    The forward's timestep is the largest entry of `timesteps` (per-token
    timesteps reduce to their largest live value). Rules, in order:
    1. dense (sf = 0) while that timestep >= cutoff;
    2. dense when the layer matches an ignore pattern;
    3. the first matching override's value (0 = dense);
    4. otherwise base_scale_factor.
    Returns (rule, scale_factor).
    Pinned by the pages' matching example and the documented rule order
    (tests).
    """
    t = max(float(x) for x in timesteps)
    if cutoff is not None and t >= cutoff:
        return RULE_TIMESTEP, 0.0
    if any(layer_matches(layer, p) for p in ignore):
        return RULE_IGNORED, 0.0
    for pattern, value in overrides:
        if layer_matches(layer, pattern):
            return RULE_OVERRIDE, float(value)
    return RULE_BASE, float(base_scale_factor)
