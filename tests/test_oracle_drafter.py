"""Pins of the oracle's RMSNorm, fc fusion, decoder layer and LM-head argmax.

RMSNorm: its closed form (unit-gain output has RMS sqrt(ms/(ms+eps))), scale
invariance, and torch.nn.functional.rms_norm in fp64.  Layer: a composition
of torch fp64 CPU ops (rms_norm, linear, scaled_dot_product_attention with a
boolean mask and GQA, silu).  Argmax: numpy's first maximum, including ties
across the oracle's vocabulary slices.  LM-head loss: torch's logsumexp and
cross_entropy (ignore_index) in fp64 over slices that do not divide V, log V
for equal logits, and direct summation on a two-token vocabulary.  Top-k KL
loss: torch's kl_div of the log-softmax (a full target in shuffled order and
a sparse top-k target scattered into the vocabulary), the cross-entropy for a
one-hot target, zero for the drafter's own distribution, sum p log p + log V
for equal logits, and ignored pairs (p = 0, ids outside the vocabulary).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import batch as ob
from oracle import drafter as od
from synth import inputs as si


def test_rmsnorm_closed_form_and_scale_invariance():
    g = np.random.default_rng(0)
    x = g.standard_normal((5, 96)) * 0.7
    eps = 1e-6
    y = od.rmsnorm(x, np.ones(96), eps)
    ms = np.mean(x * x, axis=1)
    rms_y = np.sqrt(np.mean(y * y, axis=1))
    np.testing.assert_allclose(rms_y, np.sqrt(ms / (ms + eps)), rtol=1e-12)
    y3 = od.rmsnorm(3.0 * x, np.ones(96), eps)
    assert np.max(np.abs(y3 - y)) < 1e-5


def test_rmsnorm_matches_torch():
    g = np.random.default_rng(1)
    x = g.standard_normal((7, 128))
    w = g.uniform(0.5, 1.5, 128)
    ref = F.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(w), eps=1e-6).numpy()
    np.testing.assert_allclose(od.rmsnorm(x, w, 1e-6), ref, rtol=1e-12, atol=1e-14)


def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x4049], np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(od.bf16_to_f64(bits), ref)


def _tiny_case(seed=3, R=3, K=3, dtype="f32"):
    dims = si.DrafterDims(hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, ffn=96,
                          vocab=300, dtype=dtype)
    W = si.drafter_weights(dims, seed, random_gains=True)
    c = si.decode_case(dims, seed, R, K, W=[4, 0, 5][:R], kv_len=[3, 7, 0][:R], n_rej=[1, 0, 2][:R])
    b = ob.build_draft_batch(K, dims.mask_token_id, c["cu_window"], c["n_rej"], c["kv_len"],
                             c["kv_base"], c["window_ids"], c["window_pos"], c["window_hrow"],
                             c["new_token"], c["ctx_hrow"], c["target_hidden"], W["h_shared"])
    return dims, W, c, b


def _torch_layer_reference(dims, W, c, b):
    """The same layer assembled from torch fp64 ops, one request at a time."""
    T = torch.float64
    d, Hq, Hkv, Dh = dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    w = {k: torch.from_numpy(od.to_f64(W[k], dims.dtype)) for k in
         ("w_fc", "w_qkv", "w_o", "w_gate", "w_up", "w_down", "embed", "w_lm")}
    g = {k: torch.from_numpy(np.asarray(W[k], np.float64)) for k in
         ("stream_gain", "attn_gain", "mlp_gain", "final_gain")}
    hid = torch.from_numpy(od.to_f64(b["draft_hidden"], dims.dtype))
    u = torch.cat([F.rms_norm(hid[:, s], (d,), g["stream_gain"][s], eps=dims.eps) for s in range(3)], 1)
    x0 = F.embedding(torch.from_numpy(b["draft_ids"].astype(np.int64)), w["embed"]) + F.linear(u, w["w_fc"])
    kc = torch.from_numpy(od.to_f64(c["k_cache"].view(np.uint16) if dims.dtype == "bf16" else c["k_cache"], dims.dtype)).clone()
    vc = torch.from_numpy(od.to_f64(c["v_cache"].view(np.uint16) if dims.dtype == "bf16" else c["v_cache"], dims.dtype)).clone()
    live = torch.from_numpy(b["rejected"] == 0)
    a = F.rms_norm(x0, (d,), g["attn_gain"], eps=dims.eps)
    qkv = F.linear(a, w["w_qkv"])
    q = qkv[:, :Hq * Dh].reshape(-1, Hq, Dh)
    k = qkv[:, Hq * Dh:(Hq + Hkv) * Dh].reshape(-1, Hkv, Dh)
    v = qkv[:, (Hq + Hkv) * Dh:].reshape(-1, Hkv, Dh)
    sl = torch.from_numpy(b["slot_mapping"].astype(np.int64))
    kc[sl[live]] = k[live]
    vc[sl[live]] = v[live]
    kc = torch.nan_to_num(kc, nan=0.0)   # unwritten rows are masked out below
    vc = torch.nan_to_num(vc, nan=0.0)
    o = torch.zeros(len(x0), Hq, Dh, dtype=T)
    for r in range(c["R"]):
        rows = [t for t in range(b["T"]) if b["req_of_row"][t] == r and b["rejected"][t] == 0]
        base = int(c["kv_base"][r])
        cap = (int(c["kv_base"][r + 1]) if r + 1 < c["R"] else c["kv_rows"]) - base
        pos = torch.tensor([int(b["draft_pos"][t]) for t in rows])
        mask = torch.arange(cap)[None, :] <= pos[:, None]
        qq = q[rows].permute(1, 0, 2)[None]
        kk = kc[base:base + cap].permute(1, 0, 2)[None]
        vv = vc[base:base + cap].permute(1, 0, 2)[None]
        oo = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask[None, None], enable_gqa=True)
        o[rows] = oo[0].permute(1, 0, 2)
    x1 = x0 + F.linear(o.reshape(-1, Hq * Dh), w["w_o"])
    bb = F.rms_norm(x1, (d,), g["mlp_gain"], eps=dims.eps)
    x2 = x1 + F.linear(F.silu(F.linear(bb, w["w_gate"])) * F.linear(bb, w["w_up"]), w["w_down"])
    qr = torch.from_numpy(b["query_rows"].astype(np.int64))
    f = F.rms_norm(x2[qr], (d,), g["final_gain"], eps=dims.eps)
    z = F.linear(f, w["w_lm"])
    return x0.numpy(), x2.numpy(), z.numpy(), kc.numpy(), live.numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_matches_torch_composition(dtype):
    dims, W, c, b = _tiny_case(dtype=dtype)
    res = od.drafter_forward(dims, W, b, c["kv_base"], c["k_cache"], c["v_cache"])
    x0, x2, z, kc, live = _torch_layer_reference(dims, W, c, b)
    np.testing.assert_allclose(res["x0"][live], x0[live], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(res["x_query"], x2[b["query_rows"]], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(res["logits"], z, rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(res["tokens"], np.argmax(z, axis=1))
    written = b["slot_mapping"][live]
    np.testing.assert_allclose(res["k_cache"][written], kc[written], rtol=1e-12, atol=1e-13)


def test_sentinel_rows_untouched_and_unread():
    dims, W, c, b = _tiny_case(dtype="bf16")
    res = od.drafter_forward(dims, W, b, c["kv_base"], c["k_cache"], c["v_cache"])
    assert np.all(np.isfinite(res["x_query"]))   # no query read a sentinel row
    live = b["slot_mapping"][b["rejected"] == 0]
    untouched = np.setdiff1d(np.arange(c["kv_rows"]), live)
    cached = np.concatenate([np.arange(c["kv_base"][r], c["kv_base"][r] + c["kv_len"][r]) for r in range(c["R"])])
    sentinel_rows = np.setdiff1d(untouched, cached)
    assert len(sentinel_rows) == int(np.sum(c["n_rej"]))
    assert np.all(np.isnan(res["k_cache"][sentinel_rows]))


def test_argmax_ties_and_slices():
    """Integer logits (x = +-1 so RMSNorm with eps=0 is exact, integer W_lm)
    give exact ties, many of them across the oracle's vocabulary slices."""
    g = np.random.default_rng(4)
    d, V = 8, 700
    w = g.integers(-3, 4, (V, d)).astype(np.float64)
    x = g.choice([-1.0, 1.0], (6, d))
    tok, gap, logits, rms = od.lm_head_argmax(x, np.ones(d), w, 0.0, dtype="f64", chunk=128)
    z = x @ w.T
    np.testing.assert_array_equal(logits, z)
    np.testing.assert_allclose(rms, np.sqrt(np.mean(z * z, axis=1)), rtol=1e-14)
    np.testing.assert_array_equal(tok, np.argmax(z, axis=1))     # first maximum
    srt = np.sort(z, axis=1)
    np.testing.assert_array_equal(gap, srt[:, -1] - srt[:, -2])
    assert np.any(gap == 0.0)
    for i in range(len(x)):
        assert tok[i] == np.nonzero(z[i] == z[i].max())[0][0]


def test_lm_head_loss_against_torch_cross_entropy():
    g = np.random.default_rng(31)
    n, d, V = 9, 24, 1000
    x = g.standard_normal((n, d))
    gain = g.uniform(0.5, 1.5, d)
    w = g.standard_normal((V, d)) * 0.5
    targets = g.integers(0, V, n)
    targets[3] = -1                                      # an ignored row
    lse, loss = od.lm_head_loss(x, gain, w, 1e-6, targets, chunk=300)   # slices that do not divide V
    f = od.rmsnorm(x, gain, 1e-6)
    z = torch.from_numpy(f @ w.T)
    ref_lse = torch.logsumexp(z, dim=1).numpy()
    ref = torch.nn.functional.cross_entropy(z, torch.from_numpy(targets), ignore_index=-1, reduction="none").numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13)
    np.testing.assert_allclose(loss, ref, rtol=1e-12, atol=1e-13)
    assert loss[3] == 0.0
    # a target past the vocabulary has no logit: an ignored row like -1
    t2 = targets.copy()
    t2[5] = V + 2
    _, loss2 = od.lm_head_loss(x, gain, w, 1e-6, t2, chunk=300)
    assert loss2[5] == 0.0 and np.array_equal(np.delete(loss2, 5), np.delete(loss, 5))


def test_lm_head_loss_closed_forms():
    # equal logits: lse = log V and every target costs log V
    n, d, V = 4, 8, 777
    x = np.random.default_rng(1).standard_normal((n, d))
    lse, loss = od.lm_head_loss(x, np.ones(d), np.zeros((V, d)), 1e-6, [0, 5, 776, 300], chunk=128)
    np.testing.assert_allclose(lse, np.log(V), rtol=1e-15)
    np.testing.assert_allclose(loss, np.log(V), rtol=1e-15)
    # two tokens: direct summation without a shift
    w = np.array([[1.0, 0.0], [0.0, 2.0]])
    xx = np.array([[3.0, 4.0]])
    f = xx / np.sqrt(np.mean(xx ** 2) + 1e-6)
    lse, loss = od.lm_head_loss(xx, np.ones(2), w, 1e-6, [1], chunk=1)
    z = np.array([f[0, 0], 2 * f[0, 1]])
    assert abs(lse[0] - np.log(np.exp(z[0]) + np.exp(z[1]))) < 1e-14
    assert abs(loss[0] - (lse[0] - z[1])) < 1e-14


def _kl_case(seed, n=6, d=16, V=500):
    g = np.random.default_rng(seed)
    x = g.standard_normal((n, d))
    gain = g.uniform(0.5, 1.5, d)
    w = g.standard_normal((V, d)) * 0.5
    return x, gain, w


def test_lm_head_kl_against_torch_kl_div():
    # a full target distribution over the whole vocabulary (k = V, in shuffled
    # order): torch's kl_div of the log-softmax in fp64
    x, gain, w = _kl_case(41)
    n, V = x.shape[0], w.shape[0]
    g = np.random.default_rng(42)
    logits_t = g.standard_normal((n, V)) * 2.0
    p = np.exp(logits_t - logits_t.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    perm = np.stack([g.permutation(V) for _ in range(n)])
    ids = perm
    probs = np.take_along_axis(p, perm, axis=1)
    lse, kl = od.lm_head_kl_topk(x, gain, w, 1e-6, ids, probs, chunk=128)
    z = torch.from_numpy(od.rmsnorm(x, gain, 1e-6) @ w.T)
    ref = F.kl_div(F.log_softmax(z, dim=1), torch.from_numpy(p), reduction="none").sum(1).numpy()
    np.testing.assert_allclose(kl, ref, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(z, 1).numpy(), rtol=1e-13)


def test_lm_head_kl_topk_against_torch_kl_div_sparse():
    # a top-k target (zero mass elsewhere): torch's kl_div over the dense
    # vocabulary with the k probabilities scattered in, zeros contributing 0
    x, gain, w = _kl_case(43)
    n, V, k = x.shape[0], w.shape[0], 7
    g = np.random.default_rng(44)
    ids = np.stack([g.choice(V, k, replace=False) for _ in range(n)])
    probs = g.dirichlet(np.ones(k), n)
    _, kl = od.lm_head_kl_topk(x, gain, w, 1e-6, ids, probs, chunk=77)
    dense = np.zeros((n, V))
    np.put_along_axis(dense, ids, probs, axis=1)
    z = torch.from_numpy(od.rmsnorm(x, gain, 1e-6) @ w.T)
    ref = F.kl_div(F.log_softmax(z, dim=1), torch.from_numpy(dense), reduction="none").sum(1).numpy()
    np.testing.assert_allclose(kl, ref, rtol=1e-11, atol=1e-13)
    assert np.all(kl > 0)                               # Gibbs: p differs from q


def test_lm_head_kl_special_cases():
    x, gain, w = _kl_case(45)
    n, V = x.shape[0], w.shape[0]
    # one-hot target: the cross-entropy of that token
    t = np.random.default_rng(46).integers(0, V, n)
    _, kl = od.lm_head_kl_topk(x, gain, w, 1e-6, t[:, None], np.ones((n, 1)), chunk=64)
    _, ce = od.lm_head_loss(x, gain, w, 1e-6, t, chunk=64)
    np.testing.assert_allclose(kl, ce, rtol=1e-13)
    # the drafter's own distribution as the target: KL = 0
    z = od.rmsnorm(x, gain, 1e-6) @ w.T
    q = np.exp(z - z.max(1, keepdims=True))
    q /= q.sum(1, keepdims=True)
    ids = np.tile(np.arange(V), (n, 1))
    _, kl0 = od.lm_head_kl_topk(x, gain, w, 1e-6, ids, q, chunk=64)
    assert np.max(np.abs(kl0)) < 1e-12
    # equal logits: KL = sum p log p + log V
    p = np.array([[0.5, 0.25, 0.25], [1.0, 0.0, 0.0]])
    _, klu = od.lm_head_kl_topk(x[:2], gain, np.zeros((V, x.shape[1])), 1e-6, [[3, 9, 400], [7, 8, 9]], p)
    np.testing.assert_allclose(klu, [np.log(V) - 1.5 * np.log(2.0), np.log(V)], rtol=1e-14)
    # zero-probability and out-of-vocabulary pairs add nothing; order is free
    ids = np.array([[5, 17, 200, -1, V, 31]])
    pr = np.array([[0.2, 0.3, 0.5, 0.7, 0.9, 0.0]])
    _, a = od.lm_head_kl_topk(x[:1], gain, w, 1e-6, ids, pr)
    _, b = od.lm_head_kl_topk(x[:1], gain, w, 1e-6, ids[:, [2, 0, 1]], pr[:, [2, 0, 1]])
    np.testing.assert_allclose(a, b, rtol=1e-14)
    # bf16 storage: the same as fp64 weights holding the decoded values
    wb = si.f32_to_bf16_bits(w.astype(np.float32))
    _, kb = od.lm_head_kl_topk(x[:1], gain, wb, 1e-6, ids, pr, dtype="bf16")
    _, kf = od.lm_head_kl_topk(x[:1], gain, od.bf16_to_f64(wb), 1e-6, ids, pr)
    np.testing.assert_array_equal(kb, kf)
