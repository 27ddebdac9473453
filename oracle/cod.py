"""COD (chain-of-drafts) layout, visibility and masked attention in fp64.

[RFC] "Motivation": COD sampling predicts the next token from every start
position, then the token after that for a kept fraction of those chains
(e.g. 70%), then the third token for the kept fraction of those, and so on;
the layout therefore holds N * sum_{n<D} p^n positions.  [RFC] "Random
Anchor Subsampling": every original position is a depth-0 query and key.  [RFC] "Proposed
Change": only loss-mask=1 positions start chains at depth >= 1.
[RFC] "Proposed Change" (max_anchors): chains start only from a random
subset of the loss-mask=1 positions and only those anchors' rows are
queries, against every original position plus the anchors' deeper rows.
[PD] "Training on long sequences": with N positions and K parallel groups
there are N*K positions (N=8192, K=8 gives 65,536 and an attention matrix of
more than 4e9 elements), which the sequence partition splits into contiguous
chunks while keeping every attention dependency across chunk boundaries.

Visibility (the parallel-draft mask): the query at chain start i and depth d
sees every original position j <= i (depth-0 rows) and its own chain rows
(i, e) for 1 <= e <= d.  This module evaluates that predicate on row labels
(start, depth); it never looks at row order or parent links.
"""
import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)


def cod_rows(loss_mask, U, keep, n_depths):
    """Row labels (start, depth) of a COD sample in depth-major order.

    Chain i reaches depth e >= 1 when loss_mask[i] holds and its first e
    keep draws U[i, 0..e-1] are all below ``keep``.  Written as plain loops.
    """
    N = len(loss_mask)
    rows = [(i, 0) for i in range(N)]
    for e in range(1, n_depths):
        for i in range(N):
            if not loss_mask[i]:
                continue
            ok = True
            for t in range(e):
                if not (U[i][t] < keep):
                    ok = False
                    break
            if ok:
                rows.append((i, e))
    return rows


def anchor_rows(loss_mask, anchors, U, keep, n_depths):
    """Row labels and query rows of a random-anchor COD sample.

    [RFC] "Proposed Change": at most max_anchors chain starts, drawn from the
    loss-mask=1 positions, instead of every position; the keys/values are the
    whole original sequence plus the anchors' deeper rows, the queries only
    the anchors' rows (anchors x sum_{n<D} p^n queries against
    N + anchors x sum_{1<=n<D} p^n keys).  Anchor a reaches depth e >= 1 when
    its first e keep draws U[a, 0..e-1] are all below ``keep``.

    Returns (rows, queries): rows = (start, depth) labels in depth-major
    order, every original position at depth 0 first (row index = position);
    queries = the row indices of the anchors' depth-0 rows and of every chain
    row, in row order.  Written as plain loops.
    """
    N = len(loss_mask)
    chosen = sorted(int(a) for a in anchors)
    for a in chosen:
        if not loss_mask[a]:
            raise ValueError("anchor %d is not a loss-mask position" % a)
    rows = [(i, 0) for i in range(N)]
    queries = list(chosen)
    for e in range(1, n_depths):
        for a in chosen:
            ok = True
            for t in range(e):
                if not (U[a][t] < keep):
                    ok = False
                    break
            if ok:
                queries.append(len(rows))
                rows.append((a, e))
    return rows, queries


def visible(start_q, depth_q, start_k, depth_k, sink=0, window=0):
    """The parallel-draft / COD mask predicate (vectorised over keys).

    With ``window`` > 0 (the StreamingLLM variant, [RFC] "Separate Ablation:
    StreamingLLM"), a depth-0 key j <= start_q stays visible only when it is
    one of the first ``sink`` positions or one of the ``window`` most recent
    (start_q - j < window); chain keys are unchanged.
    """
    start_k = np.asarray(start_k)
    depth_k = np.asarray(depth_k)
    prefix = (depth_k == 0) & (start_k <= start_q)
    if window > 0:
        prefix = prefix & ((start_k < sink) | (start_q - start_k < window))
    chain = (start_k == start_q) & (depth_k >= 1) & (depth_k <= depth_q)
    return prefix | chain


def attention(q, k, v, start, depth, queries=None, scale=None, q_by_query=False, sink=0, window=0):
    """o = softmax(q k^T * scale) v over the visible keys of each query, per head.

    q [T,Hq,Dh], k/v [T,Hkv,Dh] float64 (any row order); start/depth [T].
    Query head h reads kv head h // (Hq/Hkv).  Returns (out [nq,Hq,Dh],
    lse [nq,Hq]) for the rows listed in ``queries`` (all rows by default),
    lse being the natural-log log-sum-exp of the scaled scores.  With
    ``q_by_query`` q holds one row per listed query ([nq,Hq,Dh], the
    random-anchor case where only the sampled rows are queries).  ``sink``
    and ``window`` select the StreamingLLM predicate of visible().
    """
    _, Hq, Dh = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(Dh)
    if queries is None:
        queries = np.arange(len(start))
    out = np.zeros((len(queries), Hq, Dh))
    lse = np.zeros((len(queries), Hq))
    for n, t in enumerate(queries):
        keys = np.nonzero(visible(start[t], depth[t], start, depth, sink, window))[0]
        Ks = k[keys]
        Vs = v[keys]
        qh = (q[n] if q_by_query else q[t]).reshape(Hkv, G, Dh)
        s = np.einsum("hgd,khd->hgk", qh, Ks) * scale
        m = s.max(axis=-1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=-1, keepdims=True)
        out[n] = (np.einsum("hgk,khd->hgd", p, Vs) / l).reshape(Hq, Dh)
        lse[n] = (m + np.log(l)).reshape(Hq)
    return out, lse


def attention_backward(q, k, v, start, depth, dout, queries=None, scale=None):
    """Gradients of L = sum_t <out[t], dout[t]> for the queries listed (all rows
    by default), the attention of attention() with the same predicate.

    [PD] "Training on long sequences": the sequence partition keeps every
    attention dependency across chunk boundaries, so a chunk of queries
    contributes to the key and value gradients of rows in earlier chunks.
    Per query t and head, with p = softmax(s), s = scale q.k over its visible
    keys, o = sum p v:
      dP = dout . v;  dS = p * (dP - sum(p dP));
      dq = scale * sum dS k;  dk[j] += scale * dS_j q;  dv[j] += p_j dout.
    q [T,Hq,Dh], k/v [T,Hkv,Dh], dout [nq,Hq,Dh] in query order (float64).
    Returns (dq [nq,Hq,Dh], dk [T,Hkv,Dh], dv [T,Hkv,Dh]); dk and dv hold
    only the listed queries' contributions.
    """
    T, Hq, Dh = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(Dh)
    if queries is None:
        queries = np.arange(T)
    dq = np.zeros((len(queries), Hq, Dh))
    dk = np.zeros((T, Hkv, Dh))
    dv = np.zeros((T, Hkv, Dh))
    for n, t in enumerate(queries):
        keys = np.nonzero(visible(start[t], depth[t], start, depth))[0]
        for h in range(Hq):
            kh = h // G
            Ks = k[keys, kh]
            Vs = v[keys, kh]
            sc = (Ks @ q[t, h]) * scale
            p = np.exp(sc - sc.max())
            p /= p.sum()
            dp = Vs @ dout[n, h]
            ds = p * (dp - np.dot(p, dp))
            dq[n, h] = scale * (ds @ Ks)
            dk[keys, kh] += scale * np.outer(ds, q[t, h])
            dv[keys, kh] += np.outer(p, dout[n, h])
    return dq, dk, dv


def attention_chunked(q, k, v, start, depth, chunk_rows, scale=None):
    """The same attention, queries taken chunk by chunk of ``chunk_rows`` rows.

    Every chunk's queries still read their keys from the whole layout, which
    is what keeps the dependencies across chunk boundaries exact.
    """
    T = q.shape[0]
    outs, lses = [], []
    for c0 in range(0, T, chunk_rows):
        o, l = attention(q, k, v, start, depth, np.arange(c0, min(T, c0 + chunk_rows)), scale)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs), np.concatenate(lses)


def mix64(x):
    """SplitMix64 output for state x (Steele, Lea and Flood, OOPSLA 2014;
    constants as published by Vigna): z = x + gamma, then two xor-shift-
    multiply rounds and a final xor-shift.  Wraps mod 2^64."""
    z = np.asarray(x, dtype=np.uint64) + GOLDEN_GAMMA
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def index_stats(start, depth, queries=None, row_offset=0, sink=0, window=0):
    """Per query: number of visible keys, and the sum mod 2^64 of mix64(key row).

    ``row_offset`` is added to every key row before hashing (the kv row
    index the GPU sees when the layout sits at an offset in a larger buffer).
    """
    T = len(start)
    if queries is None:
        queries = np.arange(T)
    cnt = np.zeros(len(queries), np.int64)
    hsh = np.zeros(len(queries), np.uint64)
    with np.errstate(over="ignore"):
        for n, t in enumerate(queries):
            keys = np.nonzero(visible(start[t], depth[t], start, depth, sink, window))[0]
            cnt[n] = len(keys)
            hsh[n] = np.sum(mix64(keys.astype(np.uint64) + np.uint64(row_offset)), dtype=np.uint64)
    return cnt, hsh


def region_index_stats(seg_base, prefix_end):
    """Index stats of a query whose keys are the rows seg_base + 0..prefix_end
    (the decode case: a query at position P sees its region's rows 0..P)."""
    keys = np.arange(seg_base, seg_base + prefix_end + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return len(keys), np.sum(mix64(keys), dtype=np.uint64)
