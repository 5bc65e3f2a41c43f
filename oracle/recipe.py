"""Recipe defaults and validation.

Oracle module (test infrastructure only; see the package docstring).

From "BitDecoding-FP4 evaluation/config.py":

* RECIPE turns on the two-term query, underflow-aware probability scaling
  with c = 8 and tau = "calibrate", and key smoothing, Hadamard rotation and
  adaptive block-scale search for keys;
* ``recipe_additional_config`` maps that to key scale mode four_six (amax6
  when the search is off), value and query amax6, two query terms (one when
  the dual residual is off) and rotation hadamard (none when off);
* ``probability_environment``: with the scaling off, P takes mode amax6; the
  multiplier c takes the values 1 and 8; an uncalibrated tau is refused
  outside calibration, a calibrated one lies in [0, 448];
* KV_MODES ``bitdecoding-nvfp4`` keeps a 16-token BF16 sink and names a key
  scale geometry, ``local`` unless overridden;
  ``bitdecoding-mxfp4`` uses mxfp4_search with the same sink, two query terms
  and Hadamard rotation.

Here tau = NaN stands for "calibrate".
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

from . import quant as Q


# key scale geometries ("BitDecoding-FP4 evaluation/config.py", KV_MODES
# bitdecoding-nvfp4 key_scale_geometry, default "local"; "kv-landlords
# scripts/quant_ab.py", SCHEMES: keys quantized per "channel" as against per
# "headdim"). local: an NVFP4 key block is 16 consecutive channels of one
# token (the head-dim blocks every other tensor uses); channel: 16 consecutive
# tokens of one channel, inside one frozen page.
LOCAL = "local"
CHANNEL = "channel"


class RecipeError(ValueError):
    pass


class UncalibratedError(RecipeError):
    pass


@dataclass(frozen=True)
class Recipe:
    sink_tokens: int = 16
    rotation: bool = True
    key_smoothing: bool = True
    scale_mode_k: str = Q.FOUR_SIX
    scale_mode_v: str = Q.AMAX6
    scale_mode_q: str = Q.AMAX6
    scale_mode_p: str = Q.AMAX2_OR_AMAX6
    query_terms: int = 2
    c: int = 8
    tau: float = float("nan")
    rotate_v: bool = False          # recipe variant: values rotated as keys are, output rotated back
    p_running_max: bool = False     # recipe variant: P of each 16-token block against the running maximum
    key_scale_geometry: str = "local"   # "local": K blocks of 16 channels of one token; "channel": 16 tokens of one channel

    def with_(self, **kw) -> "Recipe":
        return replace(self, **kw)


def nvfp4_default() -> Recipe:
    """The bitdecoding-nvfp4 recipe, tau still to be calibrated."""
    return Recipe()


def mxfp4_default() -> Recipe:
    """The bitdecoding-mxfp4 recipe, tau still to be calibrated."""
    return Recipe(scale_mode_k=Q.MXFP4_SEARCH, scale_mode_v=Q.MXFP4_SEARCH,
                  scale_mode_q=Q.MXFP4_SEARCH)


def _tau_problem(tau):
    """None for a usable amax2_or_amax6 threshold; else the error to raise.
    NaN stands for a threshold not yet calibrated; a calibrated one is a
    finite number inside the E4M3 range."""
    if isinstance(tau, float) and math.isnan(tau):
        return UncalibratedError("tau is NaN: calibrate it before decoding")
    if isinstance(tau, bool) or not isinstance(tau, (int, float)) or not math.isfinite(tau):
        return RecipeError(f"tau = {tau!r} is not a finite number")
    if tau < 0 or tau > 448:
        return RecipeError(f"tau = {tau!r} lies outside [0, 448]")
    return None


def validate(r: Recipe) -> None:
    """Raise RecipeError / UncalibratedError for recipes the method refuses.

    The constraints on P follow "BitDecoding-FP4 evaluation/config.py",
    probability_environment: with amax2_or_amax6, tau must be calibrated and
    lie in [0, 448]; c is 1 or 8 for every quantized P mode. The P mode is
    checked first, then tau, then c."""
    if r.scale_mode_p not in (Q.AMAX2_OR_AMAX6, Q.AMAX6, Q.NONE):
        raise RecipeError(f"bad probability scale mode {r.scale_mode_p!r}")
    if r.scale_mode_p == Q.AMAX2_OR_AMAX6:
        err = _tau_problem(r.tau)
        if err is not None:
            raise err
    if r.scale_mode_p != Q.NONE and r.c not in (1, 8):
        raise RecipeError(f"c = {r.c!r}: P is multiplied by 1 or 8 before quantization")
    if r.query_terms not in (1, 2):
        raise RecipeError("query_terms is 1 or 2")
    if r.sink_tokens < 0 or r.sink_tokens >= 128 or r.sink_tokens % 16:
        raise RecipeError("sink_tokens is a multiple of 16 in [0, 112]")
    if r.key_scale_geometry not in (LOCAL, CHANNEL):
        raise RecipeError(f"bad key scale geometry {r.key_scale_geometry!r}")
    if r.key_scale_geometry == CHANNEL and r.scale_mode_k not in (Q.FOUR_SIX, Q.AMAX6):
        raise RecipeError("the channel key geometry takes NVFP4 key blocks (four_six or amax6)")
    for m, ok in ((r.scale_mode_k, (Q.FOUR_SIX, Q.AMAX6, Q.MXFP4_SEARCH, Q.NONE)),
                  (r.scale_mode_v, (Q.AMAX6, Q.MXFP4_SEARCH, Q.NONE)),
                  (r.scale_mode_q, (Q.AMAX6, Q.MXFP4_SEARCH, Q.NONE))):
        if m not in ok:
            raise RecipeError(f"bad scale mode {m!r}")
