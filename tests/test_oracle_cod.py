"""Pins of the COD layout, visibility predicate and masked attention.

* Brute force on every tiny layout: the label predicate equals the key sets
  obtained from a prefix range plus a parent walk (the form the kernels use),
  and the generator's depth-major layout equals the oracle's own loop-built
  row labels.
* One depth reduces to plain causal attention (torch SDPA, is_causal=True).
* Attention through a dense T x T mask equals attention over the index sets.
* Chunked == unchunked, bit for bit; a chunking that drops cross-chunk keys
  does not.
* Position counts: T = N*K and the visible-pair count in closed form at keep
  1.0; the mean of T over seeds against N * sum_{n<D} p^n; the page's
  rounded 2.73 against the exact 2.7731; (N*K)^2 > 4e9 at N=8192, K=8.
* Q = 0 gives the mean of the visible V rows.
* Random anchors: a hand-worked layout with its key sets; the generator
  against the oracle's loop-built rows and parent chains; anchors on every
  loss-mask position reduce to the symmetric COD rows; the query and key
  counts against the page's (anchors x 2.73) x (anchors x 1.73 + N).
* StreamingLLM window: a hand-worked example, the per-query count in closed
  form, reduction to the plain predicate when the window spans the
  sequence, one depth against SDPA with a banded-plus-sink mask.
* Backward: fp64 torch autograd through SDPA with the dense mask, central
  finite differences, and query chunks whose key/value gradients sum to the
  unchunked ones.
"""
import itertools

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import cod as oc
from synth import inputs as si


def _layout(N, D, keep, loss_rate, seed, heads=(4, 2, 8), dtype="f32"):
    return si.cod_case(N, D, keep, loss_rate, seed, heads=heads, dtype=dtype)


def _index_sets(L):
    """Keys by prefix range over group 0 plus a walk up the parent links."""
    sets = []
    for t in range(L["T"]):
        s, d = int(L["start"][t]), int(L["depth"][t])
        keys = set(range(0, s + 1))            # group 0 row j holds start j
        r = t
        for _ in range(d):
            keys.add(r)
            r = int(L["parent"][r])
        assert r == -1 or d == 0
        sets.append(keys)
    return sets


def test_predicate_vs_index_sets_all_tiny_layouts():
    n_cases = 0
    for N in range(1, 6):
        for D in range(1, 5):
            for bits in itertools.product([False, True], repeat=N):
                for keep in (0.5, 1.0):
                    L = _layout(N, D, keep, 0.0, 11)
                    # overwrite the drawn loss mask with every pattern
                    L = _relayout(np.array(bits), L["U"], keep, D)
                    sets = _index_sets(L)
                    for t in range(L["T"]):
                        vis = oc.visible(L["start"][t], L["depth"][t], L["start"], L["depth"])
                        assert set(np.nonzero(vis)[0].tolist()) == sets[t]
                    n_cases += 1
    assert n_cases > 400


def _relayout(loss_mask, U, keep, D):
    """Rebuild a generator-format layout for a given loss mask, reusing U."""
    N = len(loss_mask)
    starts = [np.arange(N)]
    alive = loss_mask.copy()
    for e in range(1, D):
        alive = alive & (U[:, e - 1] < keep)
        starts.append(np.nonzero(alive)[0])
    off = np.concatenate([[0], np.cumsum([len(s) for s in starts])])
    start = np.concatenate(starts)
    depth = np.concatenate([np.full(len(s), e) for e, s in enumerate(starts)])
    parent = np.full(len(start), -1)
    for e in range(2, D):
        parent[off[e]:off[e + 1]] = off[e - 1] + np.searchsorted(starts[e - 1], starts[e])
    return dict(start=start, depth=depth, parent=parent, T=len(start))


@pytest.mark.parametrize("seed", range(6))
def test_generator_layout_matches_oracle_rows(seed):
    L = _layout(40, 5, 0.7, 0.5, seed)
    rows = oc.cod_rows(L["loss_mask"], L["U"], 0.7, 5)
    assert list(zip(L["start"].tolist(), L["depth"].tolist())) == rows
    sets = _index_sets(L)
    for t in range(L["T"]):
        vis = oc.visible(L["start"][t], L["depth"][t], L["start"], L["depth"])
        assert set(np.nonzero(vis)[0].tolist()) == sets[t]


def test_count_closed_form_per_query():
    L = _layout(300, 6, 0.6, 0.5, 9)
    cnt, _ = oc.index_stats(L["start"], L["depth"])
    np.testing.assert_array_equal(cnt, L["start"] + 1 + L["depth"])


def test_single_depth_is_causal_attention():
    g = np.random.default_rng(2)
    N, Hq, Hkv, Dh = 37, 4, 2, 16
    q = g.standard_normal((N, Hq, Dh))
    k = g.standard_normal((N, Hkv, Dh))
    v = g.standard_normal((N, Hkv, Dh))
    start = np.arange(N)
    depth = np.zeros(N, int)
    out, _ = oc.attention(q, k, v, start, depth)
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2)[None], torch.from_numpy(k).permute(1, 0, 2)[None],
        torch.from_numpy(v).permute(1, 0, 2)[None], is_causal=True, enable_gqa=True)
    np.testing.assert_allclose(out, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_dense_mask_attention_equals_index_attention():
    L = _layout(23, 4, 0.7, 0.6, 5)
    T = L["T"]
    g = np.random.default_rng(3)
    q = g.standard_normal((T, 4, 8))
    k = g.standard_normal((T, 2, 8))
    v = g.standard_normal((T, 2, 8))
    out, lse = oc.attention(q, k, v, L["start"], L["depth"])
    # dense T x T boolean mask built from the parent-walk sets, then SDPA
    sets = _index_sets(L)
    M = np.zeros((T, T), bool)
    for t, s in enumerate(sets):
        M[t, list(s)] = True
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2)[None], torch.from_numpy(k).permute(1, 0, 2)[None],
        torch.from_numpy(v).permute(1, 0, 2)[None], attn_mask=torch.from_numpy(M)[None, None],
        enable_gqa=True)
    np.testing.assert_allclose(out, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-14)
    # lse: log sum_k exp(s) from the dense scores
    s = np.einsum("thd,khd->thk", q, np.repeat(k, 2, axis=1)) / np.sqrt(8)
    s = np.where(M[:, None, :], s, -np.inf)
    np.testing.assert_allclose(lse, np.log(np.exp(s).sum(-1)), rtol=1e-12)


def test_chunked_equals_unchunked_bitwise():
    L = _layout(32, 4, 1.0, 1.0, 1)   # 4 groups of 32 rows, 8 chunks of 16
    T = L["T"]
    g = np.random.default_rng(8)
    q = g.standard_normal((T, 4, 8))
    k = g.standard_normal((T, 2, 8))
    v = g.standard_normal((T, 2, 8))
    a, la = oc.attention(q, k, v, L["start"], L["depth"])
    b, lb = oc.attention_chunked(q, k, v, L["start"], L["depth"], 16)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    # a partition that loses the keys of earlier chunks is not the same
    wrong = []
    for c0 in range(0, T, 16):
        sl = slice(c0, c0 + 16)
        o, _ = oc.attention(q[sl], k[sl], v[sl], L["start"][sl], L["depth"][sl])
        wrong.append(o)
    assert not np.allclose(np.concatenate(wrong), a)


def test_keep_one_counts_exact():
    N, K = 64, 8
    L = _layout(N, K, 1.0, 1.0, 0)
    assert L["T"] == N * K
    cnt, _ = oc.index_stats(L["start"], L["depth"])
    assert int(cnt.sum()) == K * N * (N + 1) // 2 + N * K * (K - 1) // 2


def test_long_sequence_counts():
    L = si.cod_config(4, draw_qkv=False)
    N, K = 8192, 8
    assert L["T"] == 65536
    assert (N * K) ** 2 == 4294967296 > 4e9
    # visible pairs from the per-query closed form (start + 1 + depth),
    # itself pinned by brute force above, against the summed formula
    pairs = int(np.sum(L["start"].astype(np.int64) + 1 + L["depth"]))
    assert pairs == K * N * (N + 1) // 2 + N * K * (K - 1) // 2 == 268697600


def test_position_count_statistics():
    p, D, N = 0.7, 5, 4096
    exact = sum(p ** n for n in range(D))
    assert abs(exact - 2.7731) < 1e-12
    assert abs(exact - 2.73) / exact < 0.016              # the page's rounded figure
    EL = sum(p ** e for e in range(1, D))
    EL2 = sum((2 * e - 1) * p ** e for e in range(1, D))
    var = EL2 - EL ** 2
    assert abs(var - 2.4218) < 1e-4
    Ts = [si.cod_case(N, D, p, 1.0, 1000 + s, draw_qkv=False)["T"] for s in range(200)]
    sigma = np.sqrt(N * var)
    assert abs(np.mean(Ts) - N * exact) < 4 * sigma / np.sqrt(200)
    # loss-mask-0.5 rule of the training-shaped case
    c3 = si.cod_config(3, draw_qkv=False)
    mean3 = N * (1 + 0.5 * EL)
    var3 = 0.5 * EL2 - (0.5 * EL) ** 2
    assert abs(mean3 - 7727.3) < 0.1
    assert abs(c3["T"] - mean3) < 4 * np.sqrt(N * var3)


def test_zero_query_gives_mean_of_visible_values():
    L = _layout(19, 3, 0.7, 0.7, 4)
    T = L["T"]
    g = np.random.default_rng(1)
    k = g.standard_normal((T, 2, 8))
    v = g.standard_normal((T, 2, 8))
    out, _ = oc.attention(np.zeros((T, 4, 8)), k, v, L["start"], L["depth"])
    for t in range(T):
        vis = oc.visible(L["start"][t], L["depth"][t], L["start"], L["depth"])
        mv = v[vis].mean(axis=0)
        np.testing.assert_allclose(out[t], np.repeat(mv, 2, axis=0), rtol=1e-12, atol=1e-14)


def test_mix64_reference_values():
    # SplitMix64 seeded with 0 yields these first outputs (states gamma, 2*gamma, ...)
    outs = oc.mix64(np.arange(3, dtype=np.uint64) * oc.GOLDEN_GAMMA)
    assert [hex(int(x)) for x in outs] == ["0xe220a8397b1dcdaf", "0x6e789e6aa1b965f4", "0x6c45d188009454f"]


def _mix64_int(x):
    """SplitMix64 output in Python integers (mod 2^64), written out apart from oc.mix64."""
    m = (1 << 64) - 1
    z = (x + 0x9E3779B97F4A7C15) & m
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
    return z ^ (z >> 31)


@pytest.mark.parametrize("seg_base,P", [(0, 0), (0, 5), (37, 0), (37, 12), (1000, 63), (123456, 64)])
def test_region_index_stats_pinned(seg_base, P):
    # A decode query at position P sees rows seg_base + 0..P of its region:
    # count P + 1, and the hash equals the predicate-based index_stats of a
    # one-depth layout (start j at row j, the same keys by the visibility
    # predicate) placed at row offset seg_base, and a Python-integer sum.
    cnt, hsh = oc.region_index_stats(seg_base, P)
    assert cnt == P + 1
    L = P + 3                                     # rows after P must stay invisible
    c2, h2 = oc.index_stats(np.arange(L), np.zeros(L, int), queries=[P], row_offset=seg_base)
    assert int(c2[0]) == cnt and h2[0] == hsh
    ref = sum(_mix64_int(seg_base + j) for j in range(P + 1)) & ((1 << 64) - 1)
    assert int(hsh) == ref


# ---- random anchors (max_anchors): a query subset against the full sequence

def test_anchor_rows_hand_example():
    # N = 8, loss mask at 1, 2, 4, 6; anchors 2 and 6; keep 0.5, 3 depths.
    # Anchor 2 draws (0.3, 0.4): depths 1 and 2; anchor 6 draws (0.2, 0.9):
    # depth 1 only.  Non-anchor rows draw 0 (they would survive if they
    # started chains, which they must not).
    loss = np.zeros(8, bool)
    loss[[1, 2, 4, 6]] = True
    U = np.zeros((8, 2))
    U[2] = (0.3, 0.4)
    U[6] = (0.2, 0.9)
    rows, queries = oc.anchor_rows(loss, [6, 2], U, 0.5, 3)
    assert rows == [(i, 0) for i in range(8)] + [(2, 1), (6, 1), (2, 2)]
    assert queries == [2, 6, 8, 9, 10]
    start = np.array([r[0] for r in rows])
    depth = np.array([r[1] for r in rows])
    keys = [set(np.nonzero(oc.visible(start[t], depth[t], start, depth))[0].tolist()) for t in queries]
    assert keys == [{0, 1, 2}, set(range(7)), {0, 1, 2, 8}, set(range(7)) | {9}, {0, 1, 2, 8, 10}]
    with pytest.raises(ValueError):
        oc.anchor_rows(loss, [3], U, 0.5, 3)   # 3 is not a loss-mask position


@pytest.mark.parametrize("seed", range(4))
def test_anchor_generator_matches_oracle_rows(seed):
    A = si.anchor_case(60, 5, 0.7, 0.5, 9, seed, heads=(4, 2, 8), dtype="f32")
    assert len(A["anchors"]) == 9 and all(A["loss_mask"][A["anchors"]])
    rows, queries = oc.anchor_rows(A["loss_mask"], A["anchors"], A["U"], 0.7, 5)
    assert list(zip(A["start"].tolist(), A["depth"].tolist())) == rows
    assert A["q_rows"].tolist() == queries
    # parent links walk each chain row back to depth 1 through its own start
    for t in range(A["N"], A["T"]):
        r, d = t, int(A["depth"][t])
        while d > 1:
            r = int(A["parent"][r])
            d -= 1
            assert (int(A["start"][r]), int(A["depth"][r])) == (int(A["start"][t]), d)
        assert int(A["parent"][r]) == -1


def test_anchors_on_every_loss_position_reduce_to_cod_rows():
    # with every loss-mask position an anchor, the key rows are the COD layout
    # of the symmetric case, and the queries are its chain rows plus the anchors
    A = _layout(50, 4, 0.7, 0.5, 3)
    anchors = np.nonzero(A["loss_mask"])[0]
    rows, queries = oc.anchor_rows(A["loss_mask"], anchors, A["U"], 0.7, 4)
    assert rows == oc.cod_rows(A["loss_mask"], A["U"], 0.7, 4)
    assert queries == sorted(anchors.tolist()) + list(range(50, len(rows)))


def test_anchor_shape_formula():
    # [RFC] "Proposed Change": (anchors x 2.73) queries against
    # (anchors x 1.73 + sequence length) keys at keep 0.7 and 4 speculative tokens
    p, D = 0.7, 5
    q_mult = sum(p ** n for n in range(D))
    k_mult = sum(p ** n for n in range(1, D))
    assert abs(q_mult - 2.7731) < 1e-12 and abs(k_mult - 1.7731) < 1e-12
    assert abs(q_mult - 2.73) / q_mult < 0.016 and abs(k_mult - 1.73) / k_mult < 0.025
    N, A = 2048, 256
    EL = k_mult
    var = sum((2 * e - 1) * p ** e for e in range(1, D)) - EL ** 2   # chain length variance
    nq = [si.anchor_case(N, D, p, 0.5, A, 2000 + s, draw_qkv=False)["num_q"] for s in range(100)]
    nk = [si.anchor_case(N, D, p, 0.5, A, 2000 + s, draw_qkv=False)["T"] for s in range(100)]
    tol = 4 * np.sqrt(A * var) / np.sqrt(100)
    assert abs(np.mean(nq) - A * q_mult) < tol
    assert abs(np.mean(nk) - (A * k_mult + N)) < tol
    # the 8K setting: 1024 anchors at keep 0.5 over 8 depths
    c = si.anchor_config(draw_qkv=False)
    assert c["N"] == 8192 and len(c["anchors"]) == 1024
    EL8 = sum(0.5 ** n for n in range(1, 8))
    var8 = sum((2 * e - 1) * 0.5 ** e for e in range(1, 8)) - EL8 ** 2
    assert abs(c["num_q"] - 1024 * (1 + EL8)) < 4 * np.sqrt(1024 * var8)


def test_query_ordered_q_matches_row_ordered_q():
    A = si.anchor_case(40, 4, 0.8, 0.6, 7, 11, heads=(4, 2, 8), dtype="f32", draw_qkv=False)
    T, qr = A["T"], A["q_rows"]
    g = np.random.default_rng(5)
    qfull = g.standard_normal((T, 4, 8))
    k = g.standard_normal((T, 2, 8))
    v = g.standard_normal((T, 2, 8))
    a, la = oc.attention(qfull, k, v, A["start"], A["depth"], qr)
    b, lb = oc.attention(qfull[qr], k, v, A["start"], A["depth"], qr, q_by_query=True)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


# ---- StreamingLLM window (sink + recent window over the depth-0 keys)

def test_window_hand_example():
    # N = 10, chains of start 7 to depth 2: rows 0..9 at depth 0, (7,1) = row 10, (7,2) = row 11
    start = np.array(list(range(10)) + [7, 7])
    depth = np.array([0] * 10 + [1, 2])
    keys = lambda t: set(np.nonzero(oc.visible(start[t], depth[t], start, depth, sink=2, window=3))[0].tolist())
    assert keys(7) == {0, 1, 5, 6, 7}
    assert keys(11) == {0, 1, 5, 6, 7, 10, 11}
    assert keys(3) == {0, 1, 2, 3}            # the window reaches back into the sink
    assert keys(0) == {0}


def test_window_count_closed_form_and_reduction():
    L = _layout(300, 5, 0.7, 0.5, 12)
    for sink, window in ((4, 16), (0, 1), (32, 64), (1, 300)):
        cnt, _ = oc.index_stats(L["start"], L["depth"], sink=sink, window=window)
        i = L["start"].astype(np.int64)
        lo = np.maximum(sink, i - window + 1)
        closed = np.minimum(sink, i + 1) + np.maximum(0, i - lo + 1) + L["depth"]
        np.testing.assert_array_equal(cnt, closed)
    # a window covering the whole sequence is the unwindowed predicate
    full, fh = oc.index_stats(L["start"], L["depth"])
    wide, wh = oc.index_stats(L["start"], L["depth"], sink=0, window=300)
    assert np.array_equal(full, wide) and np.array_equal(fh, wh)


def test_window_single_depth_is_banded_sdpa():
    g = np.random.default_rng(6)
    N, Hq, Hkv, Dh, sink, window = 45, 4, 2, 16, 3, 7
    q = g.standard_normal((N, Hq, Dh))
    k = g.standard_normal((N, Hkv, Dh))
    v = g.standard_normal((N, Hkv, Dh))
    out, _ = oc.attention(q, k, v, np.arange(N), np.zeros(N, int), sink=sink, window=window)
    ones = torch.ones(N, N, dtype=torch.bool)
    col = torch.arange(N)[None, :].expand(N, N)
    mask = torch.tril(ones) & (torch.triu(ones, diagonal=-(window - 1)) | (col < sink))
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2)[None], torch.from_numpy(k).permute(1, 0, 2)[None],
        torch.from_numpy(v).permute(1, 0, 2)[None], attn_mask=mask[None, None], enable_gqa=True)
    np.testing.assert_allclose(out, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


# ---- attention backward (the training side of the sequence partition)

def _grads_torch(q, k, v, start, depth, dout):
    """fp64 autograd through SDPA with the dense boolean mask of the predicate."""
    T = q.shape[0]
    M = np.zeros((T, T), bool)
    for t in range(T):
        M[t] = oc.visible(start[t], depth[t], start, depth)
    qt, kt, vt = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    o = F.scaled_dot_product_attention(qt.permute(1, 0, 2)[None], kt.permute(1, 0, 2)[None],
                                       vt.permute(1, 0, 2)[None], attn_mask=torch.from_numpy(M)[None, None],
                                       enable_gqa=True)[0].permute(1, 0, 2)
    (o * torch.from_numpy(dout)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def test_backward_matches_torch_autograd():
    L = _layout(21, 4, 0.7, 0.6, 13)
    T = L["T"]
    g = np.random.default_rng(14)
    q = g.standard_normal((T, 4, 8))
    k = g.standard_normal((T, 2, 8))
    v = g.standard_normal((T, 2, 8))
    dout = g.standard_normal((T, 4, 8))
    dq, dk, dv = oc.attention_backward(q, k, v, L["start"], L["depth"], dout)
    rq, rk, rv = _grads_torch(q, k, v, L["start"], L["depth"], dout)
    for a, b in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def test_backward_finite_differences():
    L = _layout(9, 3, 0.8, 1.0, 2)
    T = L["T"]
    g = np.random.default_rng(15)
    q = g.standard_normal((T, 2, 4))
    k = g.standard_normal((T, 1, 4))
    v = g.standard_normal((T, 1, 4))
    dout = g.standard_normal((T, 2, 4))
    dq, dk, dv = oc.attention_backward(q, k, v, L["start"], L["depth"], dout)
    loss = lambda q_, k_, v_: float(np.sum(oc.attention(q_, k_, v_, L["start"], L["depth"])[0] * dout))
    h = 1e-6
    for arr, grad, idx in ((q, dq, (3, 1, 2)), (k, dk, (0, 0, 1)), (v, dv, (2, 0, 3)), (k, dk, (T - 1, 0, 0))):
        a1 = arr.copy(); a1[idx] += h
        a2 = arr.copy(); a2[idx] -= h
        args1 = [q, k, v]; args2 = [q, k, v]
        which = 0 if arr is q else (1 if arr is k else 2)
        args1[which] = a1; args2[which] = a2
        fd = (loss(*args1) - loss(*args2)) / (2 * h)
        assert abs(fd - grad[idx]) < 1e-7 * max(1.0, abs(fd)), (idx, fd, grad[idx])


def test_backward_query_chunks_accumulate():
    # the key/value gradients of a chunked pass are the sums of the chunks'
    # contributions; each chunk's dq is its rows of the unchunked dq
    L = _layout(30, 4, 0.7, 1.0, 4)
    T = L["T"]
    g = np.random.default_rng(16)
    q = g.standard_normal((T, 4, 8))
    k = g.standard_normal((T, 2, 8))
    v = g.standard_normal((T, 2, 8))
    dout = g.standard_normal((T, 4, 8))
    dq, dk, dv = oc.attention_backward(q, k, v, L["start"], L["depth"], dout)
    dk2, dv2 = np.zeros_like(dk), np.zeros_like(dv)
    for c0 in range(0, T, 17):
        rows = np.arange(c0, min(T, c0 + 17))
        a, b, c = oc.attention_backward(q, k, v, L["start"], L["depth"], dout[rows], rows)
        np.testing.assert_allclose(a, dq[rows], rtol=1e-13, atol=1e-14)
        dk2 += b
        dv2 += c
    np.testing.assert_allclose(dk2, dk, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv2, dv, rtol=1e-12, atol=1e-13)
