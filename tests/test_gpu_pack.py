"""pe_pack_weight: bit-exact against the packed layout as the header defines it."""
import numpy as np
import pytest
import torch

from drafter_pe_build_amd import _lib as L
from drafter_pe_build_amd.step import to_device
from helpers import say

pytestmark = pytest.mark.gpu


def packed_reference(w_bytes, N, row_bytes):
    """Row block b, 64-byte step s: 1 KB at (b*S + s)*1024; slice l = bytes
    [16*(l//16), +16) of step s of row 16b + l%16 (zero rows past N)."""
    Np = (N + 15) // 16 * 16
    S = row_bytes // 64
    src = np.zeros((Np, row_bytes), np.uint8)
    src[:N] = w_bytes.reshape(N, row_bytes)
    out = np.zeros((Np // 16, S, 64, 16), np.uint8)
    for l in range(64):
        rows = np.arange(Np // 16) * 16 + (l % 16)
        for s in range(S):
            out[:, s, l, :] = src[rows, s * 64 + (l // 16) * 16: s * 64 + (l // 16) * 16 + 16]
    return out.reshape(-1)


@pytest.mark.parametrize("dtype,N,K", [("bf16", 48, 64), ("bf16", 37, 2880), ("f32", 21, 48), ("f32", 16, 256),
                                       ("bf16", 1000, 128)])
def test_pack_bit_exact(dtype, N, K):
    say("pack %s N=%d K=%d" % (dtype, N, K))
    g = np.random.default_rng(N * K)
    if dtype == "bf16":
        w = g.integers(0, 1 << 16, (N, K), dtype=np.uint16)
        t = to_device(w, "cuda")
    else:
        w = g.standard_normal((N, K)).astype(np.float32)
        t = to_device(w, "cuda")
    out = L.pe_pack_weight(t)
    torch.cuda.synchronize()
    ref = packed_reference(w.view(np.uint8), N, w.view(np.uint8).shape[1])
    got = out.cpu().numpy()
    assert got.shape == ref.shape
    np.testing.assert_array_equal(got, ref)
