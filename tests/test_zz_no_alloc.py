"""GPU check of pe_lm_head_argmax_noalloc (the LM head with the library's
fixed device array as workspace) against pe_lm_head_argmax with a caller
workspace: the same kernels, so tokens and logits must be equal bit for bit.
Two calls in a row on the same array, the second smaller than the first
(the large-batch kernel first, then the weight-streaming kernel), and a
third back on a large batch, so stale contents of the array would show.
"""
import numpy as np
import pytest
import torch

from drafter_pe_build_amd import _lib as L
from drafter_pe_build_amd.step import to_device
from helpers import say
from synth import inputs as si

pytestmark = pytest.mark.gpu


def _head(dims, seed):
    W = si.drafter_weights(dims, seed, random_gains=True,
                           skip=("embed", "w_fc", "w_qkv", "w_o", "w_gate", "w_up", "w_down", "h_shared"))
    cd = L.dims_struct(dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.ffn, dims.vocab,
                       dims.mask_token_id, dims.eps, dims.dtype)
    cw = L.weights_struct(dict(w_lm=L.pe_pack_weight(to_device(W["w_lm"], "cuda")),
                               final_gain=to_device(W["final_gain"], "cuda")))
    return cd, cw


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_point(dtype):
    dims = si.DrafterDims(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=64, ffn=512, vocab=30011, dtype=dtype)
    cd, cw = _head(dims, 70)
    g = np.random.default_rng(71)
    for n in (300, 7, 129):   # large-batch kernel, then the weight stream, then large again
        say("noalloc %s n=%d" % (dtype, n))
        x = torch.from_numpy(g.standard_normal((n, dims.hidden)).astype(np.float32)).cuda()
        tok_ref = torch.empty(n, dtype=torch.int32, device="cuda")
        lg_ref = torch.empty((n, dims.vocab), dtype=torch.float32, device="cuda")
        L.pe_lm_head_argmax(cd, cw, n, x, tok_ref, lg_ref)
        tok = torch.full((n,), -7, dtype=torch.int32, device="cuda")
        lg = torch.full((n, dims.vocab), float("nan"), dtype=torch.float32, device="cuda")
        L.pe_lm_head_argmax_noalloc(cd, cw, n, x, tok, lg)
        tok2 = torch.full((n,), -7, dtype=torch.int32, device="cuda")
        L.pe_lm_head_argmax_noalloc(cd, cw, n, x, tok2)          # without logits
        torch.cuda.synchronize()
        assert torch.equal(tok, tok_ref) and torch.equal(tok2, tok_ref)
        assert torch.equal(lg, lg_ref)
        assert int(tok.min()) >= 0 and int(tok.max()) < dims.vocab


def test_noalloc_refuses_oversized_batch_on_gpu():
    dims = si.DrafterDims(hidden=2880, n_q_heads=64, n_kv_heads=8, head_dim=64, ffn=8192, vocab=201088,
                          dtype="bf16")
    cd = L.dims_struct(dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.ffn, dims.vocab,
                       dims.mask_token_id, dims.eps, dims.dtype)
    w = L.PeWeights()
    dummy = torch.zeros(64, dtype=torch.float32, device="cuda")
    w.w_lm = L.ptr(dummy)
    w.final_gain = L.ptr(dummy)
    x = torch.zeros((598, 2880), dtype=torch.float32, device="cuda")
    tok = torch.empty(598, dtype=torch.int32, device="cuda")
    with pytest.raises(L.PeError) as e:
        L.pe_lm_head_argmax_noalloc(cd, w, 598, x, tok)
    assert e.value.code == 2
