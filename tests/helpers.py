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

# Greedy tokens must equal the oracle's wherever its top-2 logit gap exceeds
# GAP: the stated 1e-2 for bf16; for f32 storage (operands and accumulation
# in fp32, logit errors ~1e-6) a tighter 1e-4.
GAP = {"bf16": 1e-2, "f32": 1e-4}


def kernel_top2_ok(tokens, logits):
    """Each token is one of the two largest of the kernel's own logits of its
    row (the LM head scores those two again in fp32 and keeps the larger)."""
    z = np.asarray(logits)
    second = np.partition(z, -2, axis=1)[:, -2] if z.shape[1] > 1 else np.full(z.shape[0], -np.inf)
    zt = z[np.arange(z.shape[0]), np.asarray(tokens)]
    return bool(np.all(zt >= second))


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
