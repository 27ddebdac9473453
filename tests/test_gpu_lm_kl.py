"""GPU parity of pe_lm_head_kl (KL loss of the LM head against a top-k target
distribution, without materialising logits) against
oracle.drafter.lm_head_kl_topk.

Cases cover the three LM-head paths that produce the log-sum-exp (the weight
stream for M <= 16 rows, the tiled kernel, the large-M bf16 kernel) in bf16
and f32, k from 1 to 64, and pairs that add nothing (ids -1 and >= vocab, a
zero and a NaN probability, a row with no valid pair).  Full-size: the c=1
shape (7 rows, vocab 201,088) in full and the 7,794-row training batch at
k = 32 on a sample of rows.  Results repeat bit for bit, and reading the
target rows from the row-major LM head (w_lm_rows) gives the same bits as
gathering them from the packed one: each lane sums the same chunks in the
same order either way.
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


def _case(dims, n, k, seed):
    W = si.drafter_weights(dims, seed, random_gains=True,
                           skip=("embed", "w_fc", "w_qkv", "w_o", "w_gate", "w_up", "w_down", "h_shared"))
    g = np.random.default_rng(seed)
    x = g.standard_normal((n, dims.hidden)).astype(np.float32)
    ids, p = si.kl_targets(n, dims.vocab, k, seed)
    if n > 3 and k > 2:
        ids[1, 0] = -1
        ids[2, 1] = dims.vocab + 3
        p[n // 2, 0] = 0.0
        p[n // 2, 1] = np.nan
        ids[n - 1, :] = -1                      # nothing to add: kl = 0
    return W, x, ids, p


def _run(dims, W, x, ids, p, dev=None, rows=False):
    n, k = ids.shape
    cd = L.dims_struct(dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.ffn, dims.vocab,
                       dims.mask_token_id, dims.eps, dims.dtype)
    if dev is None:
        dev = dict(w_lm=L.pe_pack_weight(to_device(W["w_lm"], "cuda")), final_gain=to_device(W["final_gain"], "cuda"))
    cw = L.weights_struct(dev)
    w_rows = None
    if rows:
        w_rows = dev.get("w_lm_rows")
        if w_rows is None:
            w_rows = dev["w_lm_rows"] = to_device(W["w_lm"], "cuda")
    xd = torch.from_numpy(x).cuda()
    idd = torch.from_numpy(ids).cuda()
    pd = torch.from_numpy(p).cuda()
    lse = torch.empty(n, dtype=torch.float32, device="cuda")
    kl = torch.empty(n, dtype=torch.float32, device="cuda")
    L.pe_lm_head_kl(cd, cw, n, xd, k, idd, pd, kl, lse, w_lm_rows=w_rows)
    torch.cuda.synchronize()
    return lse, kl, dev


def _check(name, dims, W, x, ids, p, lse, kl, rows=None):
    rows = np.arange(x.shape[0]) if rows is None else rows
    pp = np.where(np.isnan(p), 0.0, p)           # NaN: not positive, adds nothing (as p = 0)
    ref_lse, ref_kl = od.lm_head_kl_topk(x[rows], W["final_gain"], W["w_lm"], dims.eps, ids[rows], pp[rows],
                                         dtype=dims.dtype)
    tol = TOL[dims.dtype]
    g_lse = lse.cpu().numpy().astype(np.float64)[rows]
    g_kl = kl.cpu().numpy().astype(np.float64)[rows]
    e1 = om.relerr(g_lse, ref_lse)
    e2 = om.relerr(g_kl, ref_kl)
    say("  [%s] lse relerr %.3g  kl relerr %.3g  max|dkl| %.3g  (%d rows)"
        % (name, e1, e2, np.max(np.abs(g_kl - ref_kl)), len(rows)))
    assert e1 <= tol and e2 <= tol
    empty = np.all((ids[rows] < 0) | (ids[rows] >= dims.vocab) | ~(pp[rows] > 0), axis=1)
    assert np.all(g_kl[empty] == 0.0)


@pytest.mark.parametrize("dtype,n,k", [("bf16", 7, 1), ("f32", 16, 5), ("bf16", 40, 33), ("f32", 150, 9),
                                       ("bf16", 300, 64)])
def test_small_vocab_paths(dtype, n, k):
    dims = si.DrafterDims(hidden=128, n_q_heads=2, n_kv_heads=1, head_dim=64, ffn=128, vocab=3001, dtype=dtype)
    W, x, ids, p = _case(dims, n, k, 60 + n)
    say("kl %s n=%d k=%d vocab=%d" % (dtype, n, k, dims.vocab))
    lse, kl, dev = _run(dims, W, x, ids, p)
    _check("%s n=%d k=%d" % (dtype, n, k), dims, W, x, ids, p, lse, kl)
    lse2, kl2, _ = _run(dims, W, x, ids, p, dev)
    assert torch.equal(lse, lse2) and torch.equal(kl, kl2)
    lse3, kl3, _ = _run(dims, W, x, ids, p, dev, rows=True)
    assert torch.equal(lse, lse3) and torch.equal(kl, kl3)


def test_ragged_hidden_rounds():
    # hidden 2,880 bf16: 360 chunks of 8, padded to two rounds of 256 chunks;
    # f32 at 1,040: 260 chunks of 4 (one chunk into the second round)
    for dtype, hidden in (("bf16", 2880), ("f32", 1040)):
        dims = si.DrafterDims(hidden=hidden, n_q_heads=2, n_kv_heads=1, head_dim=64, ffn=128, vocab=1000, dtype=dtype)
        W, x, ids, p = _case(dims, 24, 17, 70)
        say("kl %s hidden=%d" % (dtype, hidden))
        lse, kl, dev = _run(dims, W, x, ids, p)
        _check("%s hidden=%d" % (dtype, hidden), dims, W, x, ids, p, lse, kl)
        lse2, kl2, _ = _run(dims, W, x, ids, p, dev, rows=True)
        assert torch.equal(lse, lse2) and torch.equal(kl, kl2)


def test_full_vocab_decode_shape():
    dims = si.GPTOSS_DIMS
    W, x, ids, p = _case(dims, 7, 64, 71)
    say("kl full vocab n=7 k=64")
    lse, kl, _ = _run(dims, W, x, ids, p)
    _check("vocab 201088 n=7 k=64", dims, W, x, ids, p, lse, kl)


def test_training_sized_batch_sampled():
    dims = si.GPTOSS_DIMS
    n, k = 7794, 32
    W, x, ids, p = _case(dims, n, k, 72)
    say("kl full vocab n=%d k=%d" % (n, k))
    lse, kl, dev = _run(dims, W, x, ids, p)
    lse2, kl2, _ = _run(dims, W, x, ids, p, dev, rows=True)
    assert torch.equal(lse, lse2) and torch.equal(kl, kl2)
    del dev
    rows = np.unique(np.concatenate([[0, 1, 2, n // 2, n - 2, n - 1],
                                     np.random.default_rng(5).choice(n, 26, replace=False)]))
    _check("vocab 201088 n=%d k=%d sampled" % (n, k), dims, W, x, ids, p, lse, kl, rows)
