"""GPU check of the LM head's precision paths against the fp64 oracle.

"P-EAGLE: parallel speculative decoding in vLLM", "Step 2: parallel
drafting": the LM head turns every draft row into its greedy token.  With
bf16 weights and up to 8 rows (the single-request decode step), the kernel
multiplies the normalised row as two bf16 parts, the rounded row and its
remainder, so its logits match the unrounded row's to about 2^-17 relative
(plus fp32 accumulation), far inside the stated 2e-2; with more rows the
operand is the rounded row (errors near 2^-9 relative) and the two leading
candidates are scored again in fp32.  Both must give the oracle's token
wherever its top-2 gap exceeds the stated 1e-2; on the hi + lo path the
logits themselves must be that precise, which also shows the path runs.
"""
import numpy as np
import pytest
import torch

from drafter_pe_build_amd import _lib as L
from drafter_pe_build_amd.step import to_device
from helpers import GAP, TOL, say
from oracle import drafter as od
from synth import inputs as si

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,hidden,vocab", [(1, 2880, 5003), (7, 2880, 12011), (8, 1024, 4099), (9, 2880, 5003),
                                            (16, 512, 2053)])
def test_lm_head_logits_and_tokens(n, hidden, vocab):
    dims = si.DrafterDims(hidden=hidden, n_q_heads=2, n_kv_heads=1, head_dim=64, ffn=128, vocab=vocab, dtype="bf16")
    W = si.drafter_weights(dims, 70 + n, random_gains=True,
                           skip=("embed", "w_fc", "w_qkv", "w_o", "w_gate", "w_up", "w_down", "h_shared"))
    g = np.random.default_rng(71 + n)
    x = (g.standard_normal((n, hidden)) * 3.0).astype(np.float32)
    exact = n <= 8
    say("lm head n=%d hidden=%d vocab=%d (%s)" % (n, hidden, vocab, "hi + lo operand" if exact else "re-score"))

    ref_tok, ref_gap, ref_z, _ = od.lm_head_argmax(x, W["final_gain"], W["w_lm"], dims.eps, dtype="bf16")
    cd = L.dims_struct(dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.ffn, dims.vocab,
                       dims.mask_token_id, dims.eps, dims.dtype)
    cw = L.weights_struct(dict(w_lm=L.pe_pack_weight(to_device(W["w_lm"], "cuda")),
                               final_gain=to_device(W["final_gain"], "cuda")))
    xd = torch.from_numpy(x).cuda()
    tok = torch.empty(n, dtype=torch.int32, device="cuda")
    logits = torch.empty((n, vocab), dtype=torch.float32, device="cuda")
    L.pe_lm_head_argmax(cd, cw, n, xd, tok, logits)
    tok2 = torch.empty(n, dtype=torch.int32, device="cuda")
    L.pe_lm_head_argmax(cd, cw, n, xd, tok2)
    torch.cuda.synchronize()
    z = logits.cpu().numpy().astype(np.float64)
    err = np.max(np.abs(z - ref_z)) / np.max(np.abs(ref_z))
    say("  max |dz| / max |z| = %.3e" % err)
    # hi + lo operand: the remainder of each rounded element is carried, so
    # the logits are fp32-accurate; the rounded operand alone is not
    assert err <= (1e-4 if exact else TOL["bf16"])
    t = tok.cpu().numpy()
    assert np.array_equal(t, tok2.cpu().numpy())
    sel = ref_gap > GAP["bf16"]
    say("  tokens compared where the oracle gap exceeds %.0e: %d of %d" % (GAP["bf16"], int(sel.sum()), n))
    assert np.array_equal(t[sel], ref_tok[sel])
    if exact:  # the largest of its own logits, exactly (no second scoring)
        assert np.all(z[np.arange(n), t] == z.max(axis=1))
