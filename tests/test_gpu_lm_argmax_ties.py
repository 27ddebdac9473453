"""GPU check of the LM head's tie rule (the greedy token is the lowest index
of the maximum logit) on exact ties.

One row of W_lm is made the largest logit of every batch row (positive
activations and gains, a constant positive weight row) and copied to several
other indices: in the same 16-row weight block, in other blocks (other
workgroups and partials of the fixed-order reduce) and in the ragged tail of
the vocabulary.  Copies of a row give bit-identical logits, so the token must
be the lowest copy on every path: the weight stream (M <= 16), the tiled
kernel and the large-M bf16 kernel.  The oracle, given the same weights,
takes the same first maximum.
"""
import numpy as np
import pytest
import torch

from drafter_pe_build_amd import _lib as L
from drafter_pe_build_amd.step import to_device
from helpers import say
from oracle import drafter as od
from synth import inputs as si

pytestmark = pytest.mark.gpu

VOCAB = 3001


def _weights(dims, seed, copies):
    W = si.drafter_weights(dims, seed, random_gains=True,
                           skip=("embed", "w_fc", "w_qkv", "w_o", "w_gate", "w_up", "w_down", "h_shared"))
    w = W["w_lm"].copy()
    # 0.5 in the storage type: bf16 bits 0x3f00, or f32
    top = np.full(dims.hidden, 0x3F00, dtype=w.dtype) if dims.dtype == "bf16" else np.full(dims.hidden, 0.5, w.dtype)
    for j in copies:
        w[j] = top
    W["w_lm"] = w
    return W


@pytest.mark.parametrize("dtype,n", [("bf16", 7), ("f32", 16), ("bf16", 40), ("f32", 150), ("bf16", 300)])
@pytest.mark.parametrize("copies", [(2500, 1800, 17, 1801), (3000, 2999)])
def test_ties_take_the_lowest_index(dtype, n, copies):
    dims = si.DrafterDims(hidden=128, n_q_heads=2, n_kv_heads=1, head_dim=64, ffn=128, vocab=VOCAB, dtype=dtype)
    W = _weights(dims, 60 + n, copies)
    g = np.random.default_rng(61 + n)
    x = (np.abs(g.standard_normal((n, dims.hidden))) + 0.1).astype(np.float32)
    want = min(copies)
    say("ties %s n=%d copies=%s -> %d" % (dtype, n, copies, want))

    ref_tok, ref_gap, _, _ = od.lm_head_argmax(x, W["final_gain"], W["w_lm"], dims.eps, dtype=dtype,
                                               keep_logits=False)
    assert np.all(ref_tok == want) and np.all(ref_gap == 0.0)

    cd = L.dims_struct(dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.ffn, dims.vocab,
                       dims.mask_token_id, dims.eps, dims.dtype)
    cw = L.weights_struct(dict(w_lm=L.pe_pack_weight(to_device(W["w_lm"], "cuda")),
                               final_gain=to_device(W["final_gain"], "cuda")))
    xd = torch.from_numpy(x).cuda()
    tok = torch.empty(n, dtype=torch.int32, device="cuda")
    logits = torch.empty((n, dims.vocab), dtype=torch.float32, device="cuda")
    L.pe_lm_head_argmax(cd, cw, n, xd, tok, logits)
    torch.cuda.synchronize()
    z = logits.cpu().numpy()
    cols = list(copies)
    # the copies tie bit for bit and hold the maximum of every row
    assert np.all(z[:, cols] == z[:, [want]])
    assert np.all(z[:, want] == z.max(axis=1))
    assert np.all(tok.cpu().numpy() == want)
    # without logits (the streaming paths keep no row of them)
    tok2 = torch.empty(n, dtype=torch.int32, device="cuda")
    L.pe_lm_head_argmax(cd, cw, n, xd, tok2)
    torch.cuda.synchronize()
    assert torch.equal(tok, tok2)
