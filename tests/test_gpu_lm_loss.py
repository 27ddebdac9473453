"""GPU parity of pe_lm_head_loss (log-sum-exp and cross-entropy of the LM
head without materialising logits) against oracle.drafter.lm_head_loss.

Cases cover the three LM-head paths: the weight stream for M <= 16 rows
(bf16 and f32), the tiled kernel (17..127 rows, and f32 at any size) and the
large-M bf16 kernel on operand-layout rows (two row tiles, a ragged tail);
targets include ignored rows (-1 and >= vocab).  Full-size: the c=1 shape
(7 rows, vocab 201,088) in full and a training-sized batch (2,022 rows) on a
sample of rows, with a workspace far below the logits' size.  Results repeat
bit for bit.
"""
import numpy as np
import pytest
import torch

from drafter_pe_build_amd import _lib as L
from drafter_pe_build_amd.step import to_device
from helpers import TOL, say
from oracle import drafter as od
from oracle import metrics as om
from synth import inputs as si

pytestmark = pytest.mark.gpu


def _case(dims, n, seed):
    W = si.drafter_weights(dims, seed, random_gains=True,
                           skip=("embed", "w_fc", "w_qkv", "w_o", "w_gate", "w_up", "w_down", "h_shared"))
    g = np.random.default_rng(seed)
    x = g.standard_normal((n, dims.hidden)).astype(np.float32)
    t = g.integers(0, dims.vocab, n).astype(np.int32)
    if n > 3:
        t[1] = -1
        t[n // 2] = dims.vocab + 5
    return W, x, t


def _run(dims, W, x, t, dev=None):
    n = x.shape[0]
    cd = L.dims_struct(dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.ffn, dims.vocab,
                       dims.mask_token_id, dims.eps, dims.dtype)
    if dev is None:
        dev = dict(w_lm=L.pe_pack_weight(to_device(W["w_lm"], "cuda")), final_gain=to_device(W["final_gain"], "cuda"))
    cw = L.weights_struct(dev)
    xd = torch.from_numpy(x).cuda()
    td = torch.from_numpy(t).cuda()
    lse = torch.empty(n, dtype=torch.float32, device="cuda")
    loss = torch.empty(n, dtype=torch.float32, device="cuda")
    L.pe_lm_head_loss(cd, cw, n, xd, td, lse, loss)
    torch.cuda.synchronize()
    return lse, loss, dev, (cd, cw, xd, td)


def _check(name, dims, W, x, t, lse, loss, rows=None):
    rows = np.arange(x.shape[0]) if rows is None else rows
    ref_lse, ref_loss = od.lm_head_loss(x[rows], W["final_gain"], W["w_lm"], dims.eps, t[rows], dtype=dims.dtype)
    tol = TOL[dims.dtype]
    g_lse = lse.cpu().numpy().astype(np.float64)[rows]
    g_loss = loss.cpu().numpy().astype(np.float64)[rows]
    e1 = om.relerr(g_lse, ref_lse)
    e2 = om.relerr(g_loss, ref_loss)
    say("  [%s] lse relerr %.3g  loss relerr %.3g  (%d rows)" % (name, e1, e2, len(rows)))
    assert e1 <= tol and e2 <= tol
    ign = (t[rows] < 0) | (t[rows] >= dims.vocab)
    assert np.all(g_loss[ign] == 0.0)


@pytest.mark.parametrize("dtype,n", [("bf16", 7), ("f32", 16), ("bf16", 40), ("f32", 150), ("bf16", 300)])
def test_small_vocab_paths(dtype, n):
    dims = si.DrafterDims(hidden=128, n_q_heads=2, n_kv_heads=1, head_dim=64, ffn=128, vocab=3001, dtype=dtype)
    W, x, t = _case(dims, n, 40 + n)
    say("loss %s n=%d vocab=%d" % (dtype, n, dims.vocab))
    lse, loss, dev, args = _run(dims, W, x, t)
    _check("%s n=%d" % (dtype, n), dims, W, x, t, lse, loss)
    lse2, loss2, _, _ = _run(dims, W, x, t, dev)
    assert torch.equal(lse, lse2) and torch.equal(loss, loss2)


def test_full_vocab_decode_shape():
    dims = si.GPTOSS_DIMS
    W, x, t = _case(dims, 7, 47)
    say("loss full vocab n=7")
    lse, loss, _, _ = _run(dims, W, x, t)
    _check("vocab 201088 n=7", dims, W, x, t, lse, loss)


def test_training_sized_batch_sampled():
    dims = si.GPTOSS_DIMS
    n = 2022
    W, x, t = _case(dims, n, 48)
    cd = L.dims_struct(dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.ffn, dims.vocab,
                       dims.mask_token_id, dims.eps, dims.dtype)
    ws = L.pe_lm_head_loss_workspace(cd, n)
    say("loss full vocab n=%d, workspace %.1f MB (logits would be %.1f GB)" % (n, ws / 1e6, n * dims.vocab * 4 / 1e9))
    assert ws * 20 < n * dims.vocab * 4        # per-tile partials, not logits
    lse, loss, _, _ = _run(dims, W, x, t)
    rows = np.unique(np.concatenate([[0, 1, n // 2, n - 1], np.random.default_rng(4).choice(n, 28, replace=False)]))
    _check("vocab 201088 n=%d sampled" % n, dims, W, x, t, lse, loss, rows)
