"""GPU parity of pe_draft_attention_backward against oracle.cod.attention_backward.

The forward runs on the GPU (pe_draft_attention, its bf16 output and f32
log-sum-exp feed the backward); gradients are compared in fp64 with the
oracle's per-query formulas.  Small layouts: every dq, dk, dv, and a pass in
query chunks (dk, dv accumulated) against one call over all rows.  The
training-shaped N=4096 COD layout: dq on sampled queries, dk and dv on key
rows whose full set of viewing queries is small enough for the oracle
(late original positions and chain rows).  An empty chunk is a no-op.
"""
import numpy as np
import pytest
import torch

from drafter_pe_build_amd import _lib as L
from drafter_pe_build_amd.step import to_device
from helpers import TOL, dev_to_f64, say
from oracle import cod as oc
from oracle import drafter as od
from oracle import metrics as om
from synth import inputs as si

pytestmark = pytest.mark.gpu


def _upload(Lay, seed):
    T = Lay["T"]
    Hq, Hkv, Dh = Lay["heads"]
    dout = si.to_storage(np.random.default_rng(seed).standard_normal((T, Hq, Dh)).astype(np.float32), "bf16")
    D = dict(q=to_device(Lay["q"], "cuda"), k=to_device(Lay["k"], "cuda"), v=to_device(Lay["v"], "cuda"),
             dout=to_device(dout, "cuda"), start=to_device(Lay["start"].astype(np.int32), "cuda"),
             depth=to_device(Lay["depth"].astype(np.int32), "cuda"),
             parent=to_device(Lay["parent"].astype(np.int32), "cuda"),
             goff=to_device(Lay["group_off"].astype(np.int32), "cuda"),
             self_row=to_device(np.arange(T, dtype=np.int32), "cuda"),
             base=torch.zeros(1, dtype=torch.int32, device="cuda"))
    return D, dout


def _forward(D, Lay):
    T = Lay["T"]
    Hq, Hkv, Dh = Lay["heads"]
    out = torch.empty((T, Hq, Dh), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    a = L.attn_args(num_q=T, num_seg=1, q_per_seg=T, num_kv_rows=T, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=Dh,
                    scale=1.0 / np.sqrt(Dh), dtype=L.PE_BF16, q=D["q"], q_row_stride=Hq * Dh, k=D["k"], v=D["v"],
                    seg_kv_base=D["base"], q_start=D["start"], q_depth=D["depth"], q_self_row=D["self_row"],
                    kv_parent=D["parent"], max_prefix=Lay["N"], out=out, lse=lse,
                    max_depth=max(1, int(Lay["depth"].max())))
    L.pe_draft_attention(a, "cuda")
    return out, lse


def _backward(D, Lay, out, lse, chunks):
    T = Lay["T"]
    Hq, Hkv, Dh = Lay["heads"]
    dq = torch.empty((T, Hq, Dh), dtype=torch.float32, device="cuda")
    dk = torch.zeros((T, Hkv, Dh), dtype=torch.float32, device="cuda")
    dv = torch.zeros((T, Hkv, Dh), dtype=torch.float32, device="cuda")
    for c0, c1 in chunks:
        a = L.attn_bwd_args(num_rows=T, n_pos=Lay["N"], n_groups=len(Lay["group_off"]) - 1, n_q_heads=Hq,
                            n_kv_heads=Hkv, head_dim=Dh, scale=1.0 / np.sqrt(Dh), dtype=L.PE_BF16,
                            group_off=D["goff"], start=D["start"], depth=D["depth"], q=D["q"], k=D["k"], v=D["v"],
                            out=out, dout=D["dout"], lse=lse, q_begin=c0, q_end=c1, dq=dq[c0:c1], dk=dk, dv=dv)
        L.pe_draft_attention_backward(a, "cuda")
    torch.cuda.synchronize()
    return dq, dk, dv


def _oracle(Lay, dout, queries):
    f = lambda a: od.to_f64(a, "bf16")
    q = f(Lay["q"])
    return oc.attention_backward(q, f(Lay["k"]), f(Lay["v"]), Lay["start"], Lay["depth"], f(dout)[queries], queries)


@pytest.mark.parametrize("heads,N,D,keep,loss", [
    ((8, 2, 128), 150, 5, 0.7, 0.5),
    ((32, 8, 128), 130, 8, 1.0, 1.0),
    ((16, 4, 64), 200, 4, 0.8, 0.7),
    ((4, 4, 64), 170, 3, 0.9, 1.0),      # G = 1: 128 queries per tile
    ((64, 1, 128), 90, 4, 0.8, 1.0),     # G = 64: 2 queries per tile
])
def test_backward_small_layouts(heads, N, D, keep, loss):
    Lay = si.cod_case(N, D, keep, loss, 27, heads=heads, dtype="bf16")
    T = Lay["T"]
    name = "bwd N=%d D=%d heads=%s T=%d" % (N, D, heads, T)
    say(name)
    Dv, dout = _upload(Lay, 28)
    out, lse = _forward(Dv, Lay)
    dq, dk, dv = _backward(Dv, Lay, out, lse, [(0, T)])
    rq, rk, rv = _oracle(Lay, dout, np.arange(T))
    tol = TOL["bf16"]
    for nm, g_, r_ in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        e = om.relerr(dev_to_f64(g_), r_)
        say("  %s relerr %.3g" % (nm, e))
        assert e <= tol, nm
    # chunks (ragged, not aligned to the workgroup's query count): dq per
    # chunk and the accumulated dk, dv agree with the single call
    cut = [0, T // 3 + 5, 2 * T // 3 - 7, T]
    dq2, dk2, dv2 = _backward(Dv, Lay, out, lse, list(zip(cut[:-1], cut[1:])))
    for nm, a_, b_ in (("dq", dq2, dq), ("dk", dk2, dk), ("dv", dv2, dv)):
        e = om.relerr(dev_to_f64(a_), dev_to_f64(b_))
        say("  chunked %s vs single call relerr %.3g" % (nm, e))
        assert e <= 1e-5, nm


def test_backward_training_shape_n4096():
    Lay = si.cod_config(3)
    T, N = Lay["T"], Lay["N"]
    say("bwd COD N=4096 T=%d" % T)
    Dv, dout = _upload(Lay, 29)
    out, lse = _forward(Dv, Lay)
    dq, dk, dv = _backward(Dv, Lay, out, lse, [(0, T)])
    tol = TOL["bf16"]
    go = Lay["group_off"]
    start, depth = Lay["start"], Lay["depth"]
    D = len(go) - 1
    # key rows checked in full: every chain row of the deepest group (each is
    # seen by itself only) and the last 64 original positions (seen by the
    # queries starting there); their viewers plus a dq sample (32 queries of
    # each depth group and 64 at random) go through the oracle in one call
    deep = np.arange(go[D - 1], go[D])
    late = np.arange(N - 64, N)
    viewers = np.nonzero(start >= N - 64)[0]
    dq_rows = set(np.random.default_rng(5).choice(T, 64, replace=False).tolist())
    for e in range(D):
        dq_rows.update(np.linspace(go[e], go[e + 1] - 1, 32).astype(int).tolist())
    qs = np.array(sorted(set(deep.tolist()) | set(viewers.tolist()) | dq_rows))
    say("  oracle backward over %d queries" % len(qs))
    rq, rk, rv = _oracle(Lay, dout, qs)
    pos = {int(t): n for n, t in enumerate(qs)}
    dqr = np.array(sorted(dq_rows))
    e = om.relerr(dev_to_f64(dq)[dqr], rq[[pos[int(t)] for t in dqr]])
    say("  dq relerr %.3g (%d queries)" % (e, len(dqr)))
    assert e <= tol
    gk, gv = dev_to_f64(dk), dev_to_f64(dv)
    for name, rows in (("depth-%d chain rows" % (D - 1), deep), ("last 64 positions", late)):
        # every viewer of these rows is among the oracle's queries
        for j in rows[:: max(1, len(rows) // 8)]:
            vis = oc.visible(start, depth, np.array([start[j]]), np.array([depth[j]]))
            assert set(np.nonzero(vis)[0].tolist()) <= set(qs.tolist())
        ek = om.relerr(gk[rows], rk[rows])
        ev = om.relerr(gv[rows], rv[rows])
        say("  %s (%d rows): dk relerr %.3g dv relerr %.3g" % (name, len(rows), ek, ev))
        assert ek <= tol and ev <= tol
    # identities over every row: the probabilities of a query sum to one, so
    # sum_j dV[j] is the sum of dout over the queries of each kv head's group,
    # and dS sums to zero over a query's keys, so sum_j dK[j] = 0
    Hq, Hkv, Dh = Lay["heads"]
    G = Hq // Hkv
    dsum = dev_to_f64(Dv["dout"]).reshape(T, Hkv, G, Dh).sum(axis=(0, 2))
    e = om.relerr(gv.sum(axis=0), dsum)
    say("  sum of dV over all rows vs sum of dout: relerr %.3g" % e)
    assert e <= tol
    ek0 = np.abs(gk.sum(axis=0)).max() / np.abs(gk).sum(axis=0).max()
    say("  |sum of dK over all rows| / sum |dK|: %.3g" % ek0)
    assert ek0 <= tol


def test_backward_empty_chunk_is_noop():
    Lay = si.cod_case(64, 3, 0.7, 0.5, 30, heads=(8, 2, 128), dtype="bf16")
    Dv, _ = _upload(Lay, 31)
    out, lse = _forward(Dv, Lay)
    T = Lay["T"]
    dk = torch.full((T, 2, 128), 7.0, dtype=torch.float32, device="cuda")
    dv = torch.full((T, 2, 128), 7.0, dtype=torch.float32, device="cuda")
    a = L.attn_bwd_args(num_rows=T, n_pos=64, n_groups=3, n_q_heads=8, n_kv_heads=2, head_dim=128,
                        scale=1.0 / np.sqrt(128), dtype=L.PE_BF16, group_off=Dv["goff"], start=Dv["start"],
                        depth=Dv["depth"], q=Dv["q"], k=Dv["k"], v=Dv["v"], out=out, dout=Dv["dout"], lse=lse,
                        q_begin=10, q_end=10, dq=None, dk=dk, dv=dv)
    L.pe_draft_attention_backward(a, "cuda")
    torch.cuda.synchronize()
    assert bool((dk == 7.0).all()) and bool((dv == 7.0).all())


def test_backward_repeats_bit_for_bit():
    """No atomics and fixed-order reduces: two calls on the same inputs (an
    N=1,024 layout; every key tile's query tiles are shared by four dK/dV
    workgroups whose partial sums are added in order) give the same bits."""
    Lay = si.cod_case(1024, 5, 0.7, 0.5, 31, heads=(32, 8, 128), dtype="bf16")
    T = Lay["T"]
    say("bwd repeat N=1024 T=%d" % T)
    Dv, _ = _upload(Lay, 32)
    out, lse = _forward(Dv, Lay)
    a = _backward(Dv, Lay, out, lse, [(0, T)])
    b = _backward(Dv, Lay, out, lse, [(0, T)])
    for nm, x, y in zip(("dq", "dk", "dv"), a, b):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32)), nm
