"""Drafter forward in fp64: stream RMSNorm + fc fusion, one pre-norm decoder
layer over the per-request KV regions, final RMSNorm + LM head + argmax.

[AD] section 2: the EAGLE-3 drafter feeds the target's fused hidden states
through a fully-connected projection (fc) into a single pre-norm decoder
layer.  [AD] section 4.1 / Observation 2: an RMSNorm is applied to each
captured target stream (low, mid, high) before it enters fc; RMS is
||x||_2 / sqrt(d).  [PD] "Step 2: parallel drafting": all positions then go
through the decoder layer(s) and the LM head, which predicts t_1..t_K in one
pass.  [RFC] "Experiment Setup": the drafter has one layer.

Readings where the pages are silent (listed with reasons in the design
notes): the token embedding is added to the fc output; RMSNorm is
x * g / sqrt(mean(x^2) + eps); a final RMSNorm precedes the LM head; linears
are bias-free; attention has no positional encoding and scale 1/sqrt(Dh);
query head h reads kv head floor(h / (Hq/Hkv)); the MLP is
down(silu(gate x) * up x); the argmax takes the lowest index among equal
maxima.
"""
import numpy as np


def bf16_to_f64(bits):
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def to_f64(a, dtype):
    if dtype == "bf16":
        return bf16_to_f64(a)
    return np.asarray(a, dtype=np.float64)


def rmsnorm(x, g, eps):
    """x * g / sqrt(mean(x^2) + eps) over the last axis ([AD] section 4.1)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x * g / np.sqrt(ms + eps)


def silu(z):
    return z / (1.0 + np.exp(-z))


def fuse_hidden(draft_hidden, ids, stream_gain, w_fc, embed_rows, eps):
    """x0 = E[id] + W_fc [norm(h_low); norm(h_mid); norm(h_high)].

    draft_hidden [T,3,d] f64, stream_gain [3,d], w_fc [d,3d] f64,
    embed_rows [T,d] f64 (= E[ids], gathered by the caller).
    """
    T, S, d = draft_hidden.shape
    u = np.concatenate([rmsnorm(draft_hidden[:, s, :], stream_gain[s], eps) for s in range(S)], axis=1)
    return embed_rows + u @ w_fc.T


def decoder_layer(x0, batch, kv_base, k_cache, v_cache, W, n_q_heads, n_kv_heads, head_dim, eps):
    """One pre-norm decoder layer over every non-rejected row of the batch.

    x0 [T,d] f64.  k_cache/v_cache [rows, Hkv, Dh] f64 are updated in place:
    each non-rejected row writes its k/v at slot_mapping (rejected rows map
    to -1 and write nothing, [PD] "KV cache").  Row t of request r, at
    position P, attends the rows kv_base[r] + 0..P of its region, i.e. the
    cached context, the accepted window rows, and the earlier draft slots.
    Returns x2 [T,d] (NaN on rejected rows) and the attention output o.
    """
    T, d = x0.shape
    Hq, Hkv, Dh = n_q_heads, n_kv_heads, head_dim
    G = Hq // Hkv
    live = batch["rejected"] == 0
    rows = np.nonzero(live)[0]
    a = rmsnorm(x0[rows], W["attn_gain"], eps)
    qkv = a @ W["w_qkv"].T
    q = qkv[:, :Hq * Dh].reshape(-1, Hq, Dh)
    k = qkv[:, Hq * Dh:(Hq + Hkv) * Dh].reshape(-1, Hkv, Dh)
    v = qkv[:, (Hq + Hkv) * Dh:].reshape(-1, Hkv, Dh)
    slots = batch["slot_mapping"][rows]
    k_cache[slots] = k
    v_cache[slots] = v

    scale = 1.0 / np.sqrt(Dh)
    o = np.zeros((len(rows), Hq, Dh))
    for n, t in enumerate(rows):
        r = batch["req_of_row"][t]
        P = batch["draft_pos"][t]
        base = kv_base[r]
        Kr = k_cache[base:base + P + 1]            # [P+1, Hkv, Dh]
        Vr = v_cache[base:base + P + 1]
        qh = q[n].reshape(Hkv, G, Dh)
        s = np.einsum("hgd,khd->hgk", qh, Kr) * scale
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=-1, keepdims=True)
        o[n] = np.einsum("hgk,khd->hgd", p, Vr).reshape(Hq, Dh)

    x1 = x0[rows] + o.reshape(len(rows), Hq * Dh) @ W["w_o"].T
    b = rmsnorm(x1, W["mlp_gain"], eps)
    h = silu(b @ W["w_gate"].T) * (b @ W["w_up"].T)
    x2r = x1 + h @ W["w_down"].T
    x2 = np.full((T, d), np.nan)
    x2[rows] = x2r
    o_full = np.full((T, Hq, Dh), np.nan)
    o_full[rows] = o
    return x2, o_full


def lm_head_argmax(x, final_gain, w_lm, eps, dtype="f64", chunk=16384, keep_logits=True):
    """f = RMSNorm(x); z = W_lm f; token = lowest index of the maximum.

    ``w_lm`` may be in storage dtype ("bf16" bits or "f32"); it is upcast to
    float64 one vocabulary slice at a time.  Returns (tokens, gap, logits,
    rms) where gap is the difference between the largest and second-largest
    logit of each row (0 on ties), logits is None unless kept and rms is the
    root mean square of each row's logits (the scale a tolerance on them is
    stated in).
    """
    f = rmsnorm(np.asarray(x, dtype=np.float64), final_gain, eps)
    V = w_lm.shape[0]
    n = f.shape[0]
    logits = np.empty((n, V)) if keep_logits else None
    best = np.full(n, -np.inf)
    second = np.full(n, -np.inf)
    tok = np.zeros(n, np.int64)
    ss = np.zeros(n)
    for s in range(0, V, chunk):
        w = w_lm[s:s + chunk]
        w = bf16_to_f64(w) if dtype == "bf16" else np.asarray(w, dtype=np.float64)
        z = f @ w.T
        ss += np.sum(z * z, axis=1)
        if keep_logits:
            logits[:, s:s + chunk] = z
        # running top-2; the first maximum wins ties, so an equal maximum in a
        # later slice keeps the earlier index (and leaves a gap of 0)
        ar = np.arange(n)
        j = np.argmax(z, axis=1)
        m1 = z[ar, j]
        z[ar, j] = -np.inf
        m2 = z.max(axis=1) if z.shape[1] > 1 else np.full(n, -np.inf)
        better = m1 > best
        second = np.where(better, np.maximum(best, m2), np.maximum(second, m1))
        tok = np.where(better, s + j, tok)
        best = np.where(better, m1, best)
    return tok, best - second, logits, np.sqrt(ss / V)


def lm_head_loss(x, final_gain, w_lm, eps, targets, dtype="f64", chunk=16384):
    """Log-sum-exp and cross-entropy of the LM-head logits, row by row.

    f = RMSNorm(x); z = W_lm f; lse = log sum_v exp(z_v);
    loss = lse - z[target] (the negative log-probability of the target
    token), 0 where the target is outside [0, V) (an ignored row: no logit
    exists for it).  [RFC] "Separate Ablation:
    StreamingLLM & The 32K Wall": at long sequences the [T, V] logits tensor,
    not attention, exhausts memory, which a loss computed slice by slice
    avoids.  ``w_lm`` is upcast to float64 one vocabulary slice at a time;
    the log-sum-exp is accumulated over the slices with a running maximum.
    Returns (lse, loss) [n] float64.
    """
    f = rmsnorm(np.asarray(x, dtype=np.float64), final_gain, eps)
    V = w_lm.shape[0]
    n = f.shape[0]
    targets = np.asarray(targets, dtype=np.int64)
    m = np.full(n, -np.inf)
    ssum = np.zeros(n)
    zt = np.zeros(n)
    for s in range(0, V, chunk):
        w = w_lm[s:s + chunk]
        w = bf16_to_f64(w) if dtype == "bf16" else np.asarray(w, dtype=np.float64)
        z = f @ w.T
        mz = np.maximum(m, z.max(axis=1))
        ssum = ssum * np.exp(m - mz) + np.exp(z - mz[:, None]).sum(axis=1)
        m = mz
        inside = (targets >= s) & (targets < s + z.shape[1])
        rows = np.nonzero(inside)[0]
        zt[rows] = z[rows, targets[rows] - s]
    lse = m + np.log(ssum)
    loss = np.where((targets >= 0) & (targets < V), lse - zt, 0.0)
    return lse, loss


def lm_head_kl_topk(x, final_gain, w_lm, eps, target_ids, target_probs, dtype="f64", chunk=16384):
    """KL divergence from a target distribution given by its top-k entries to
    the drafter's LM-head distribution, row by row.

    [RFC] "Experiment Setup": the drafter is trained with a KL loss against
    the verifier's output distribution.  The target arrives as k (token id,
    probability) pairs per row (the verifier's top-k, zero mass elsewhere):
        q = softmax(z),  z = W_lm RMSNorm(x),
        KL(p || q) = sum_j p_j (log p_j - log q_j)
                   = sum_j p_j (log p_j - z[id_j] + lse).
    A pair whose id lies outside [0, V) or whose probability is not positive
    adds nothing (p log p -> 0 as p -> 0; no logit exists outside the
    vocabulary).  The probabilities are used as given (no renormalisation).
    Returns (lse, kl) [n] float64; lse as in lm_head_loss.
    """
    ids = np.asarray(target_ids, dtype=np.int64)
    p = np.asarray(target_probs, dtype=np.float64)
    n = ids.shape[0]
    V = w_lm.shape[0]
    lse, _ = lm_head_loss(x, final_gain, w_lm, eps, np.full(n, -1), dtype=dtype, chunk=chunk)
    f = rmsnorm(np.asarray(x, dtype=np.float64), final_gain, eps)
    kl = np.zeros(n)
    for i in range(n):
        use = (ids[i] >= 0) & (ids[i] < V) & (p[i] > 0)
        t = ids[i][use]
        w = w_lm[t]
        w = bf16_to_f64(w) if dtype == "bf16" else np.asarray(w, dtype=np.float64)
        z = w @ f[i]
        kl[i] = np.sum(p[i][use] * (np.log(p[i][use]) - z + lse[i]))
    return lse, kl


def drafter_forward(dims, weights, batch, kv_base, k_cache, v_cache, keep_logits=True):
    """Stages 2-4 of the drafter on a built batch (stage 1 is oracle.batch).

    ``weights`` holds storage arrays as drawn (bf16 bits or float32), gains
    float32; ``k_cache``/``v_cache`` are storage arrays and are not modified
    (float64 copies are updated and returned).  Returns a dict with x0, the
    written caches, x2 of the query rows, tokens, gaps, logits and the rms of
    each query row's logits.
    """
    dt = dims.dtype
    T = batch["T"]
    hid = to_f64(batch["draft_hidden"], dt)
    ids = batch["draft_ids"]
    emb = to_f64(weights["embed"][ids], dt)
    x0 = fuse_hidden(hid, ids, np.asarray(weights["stream_gain"], np.float64),
                     to_f64(weights["w_fc"], dt), emb, dims.eps)
    x0[batch["rejected"] == 1] = np.nan
    W = {k: to_f64(weights[k], dt) for k in ("w_qkv", "w_o", "w_gate", "w_up", "w_down")}
    W["attn_gain"] = np.asarray(weights["attn_gain"], np.float64)
    W["mlp_gain"] = np.asarray(weights["mlp_gain"], np.float64)
    kc = to_f64(k_cache.view(np.uint16) if dt == "bf16" else k_cache, dt)
    vc = to_f64(v_cache.view(np.uint16) if dt == "bf16" else v_cache, dt)
    x2, o = decoder_layer(x0, batch, kv_base, kc, vc, W, dims.n_q_heads, dims.n_kv_heads,
                          dims.head_dim, dims.eps)
    xq = x2[batch["query_rows"]]
    tok, gap, logits, rms = lm_head_argmax(xq, np.asarray(weights["final_gain"], np.float64),
                                           weights["w_lm"], dims.eps, dtype=dt, keep_logits=keep_logits)
    return dict(x0=x0, k_cache=kc, v_cache=vc, x_query=xq, attn_out=o, tokens=tok,
                gap=gap, logits=logits, logit_rms=rms)
