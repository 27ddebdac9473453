"""Shared helpers of the GPU tests (device transfer, cached inputs, metrics)."""
import functools
import sys

import numpy as np
import torch

from synth import inputs as si

# Tolerances.  bf16: max|gpu - ref| / max|ref| <= 2e-2 for attention outputs,
# logits and written K/V (the stated bound).  f32 storage: 1e-4 (fp32
# operands and accumulation over at most a few thousand terms; rounding is
# ~1e-6).
TOL = {"bf16": 2e-2, "f32": 1e-4}


def token_gap(dtype, logit_rms):
    """Per-row top-2 gap above which the greedy token is decided.

    Each logit of a row is held to TOL times the row's rms; two logits that
    each move by at most that much cannot swap order across a gap larger than
    twice it.  Rows below the gap are near-ties that rounding in the storage
    precision may legitimately break either way."""
    return 2.0 * TOL[dtype] * np.asarray(logit_rms)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_to_f64(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def bits(t):
    """Raw bit patterns of a device tensor as a numpy array."""
    t = t.detach().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy().view(np.uint32)
    return t.cpu().numpy()


@functools.lru_cache(maxsize=2)
def gptoss_weights():
    return si.drafter_weights(si.GPTOSS_DIMS, 1)
