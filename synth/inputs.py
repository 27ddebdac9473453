"""Seeded synthetic inputs for the parallel-drafting hot path.

Every tensor is drawn from ``numpy.random.default_rng([seed, tag])`` so that
each one can be regenerated on its own.  Floating-point draws are float32;
bf16 storage is the round-to-nearest-even of that float32 and is carried in
numpy as ``uint16`` bit patterns.  Nothing here normalises, projects, attends
or takes an argmax: this module only draws numbers and lays them out in the
shapes the drafter consumes.

Shapes follow the P-EAGLE pages: a drafter fed by three captured target
hidden streams (low/mid/high), K draft slots per request (one next-token slot
plus K-1 MASK slots that carry the shared hidden placeholder), a KV cache in
one contiguous region per request, and, for training-shaped attention, the
COD layout in which every start position spawns a chain that survives from
depth d to depth d+1 with the keep probability.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "SENTINEL_BF16", "SENTINEL_F32", "DrafterDims", "TINY_DIMS", "GPTOSS_DIMS",
    "rng", "f32_to_bf16_bits", "bf16_bits_to_f32", "to_storage", "storage_to_f64",
    "sentinel_bits", "drafter_weights", "decode_case", "decode_config",
    "cod_case", "cod_config", "COD_HEADS", "CONFIG_NAMES",
]

# Bit patterns a KV-cache row holds until something writes it.  Both are
# quiet NaNs, so a kernel that reads an unwritten row poisons its output.
SENTINEL_BF16 = 0x7FE5
SENTINEL_F32 = 0x7FE5A5A5

# Weight tensor tags (the second element of the rng key).
_W_TAGS = {
    "embed": 1, "w_fc": 2, "w_qkv": 3, "w_o": 4, "w_gate": 5, "w_up": 6,
    "w_down": 7, "w_lm": 8, "h_shared": 9,
}
_GAIN_TAGS = {"stream_gain": 10, "attn_gain": 11, "mlp_gain": 12, "final_gain": 13}

CONFIG_NAMES = {
    0: "tiny drafter fwd fp32, N=128, K=4",
    1: "decode c=1 bf16, 2048-position cache, K=7, d=2880, V=201088",
    2: "decode c=64 bf16, ragged contexts U[512,4096], K=7",
    3: "COD masked attention fwd bf16, N=4096, 5 depths, keep 0.7, loss mask 0.5",
    4: "parallel-group attention fwd bf16, N=8192, K=8, keep 1.0, 8 query chunks",
}


@dataclasses.dataclass(frozen=True)
class DrafterDims:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    dtype: str            # storage dtype of weights, hidden streams and KV: "f32" | "bf16"
    eps: float = 1e-6

    @property
    def mask_token_id(self) -> int:
        # The MASK id is the last id of the draft vocabulary.
        return self.vocab - 1

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


# One-layer drafter of the tiny fp32 case and the GPT-OSS-20B-class drafter.
TINY_DIMS = DrafterDims(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                        ffn=512, vocab=4096, dtype="f32")
GPTOSS_DIMS = DrafterDims(hidden=2880, n_q_heads=64, n_kv_heads=8, head_dim=64,
                          ffn=8192, vocab=201088, dtype="bf16")
# Training-shaped attention heads: 32 query heads, 8 kv heads, head dim 128.
COD_HEADS = (32, 8, 128)


def rng(seed: int, tag: int) -> np.random.Generator:
    return np.random.default_rng([seed, tag])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    # Process in slabs to bound temporary memory on the 1e9-element tensors.
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        v = flat_u[s:s + step]
        r = (v + np.uint32(0x7FFF) + ((v >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        flat_o[s:s + step] = r.astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of a storage array to float64."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    raise ValueError(dtype)


def sentinel_bits(dtype: str):
    return (np.uint16(SENTINEL_BF16), np.uint16) if dtype == "bf16" else (np.uint32(SENTINEL_F32), np.uint32)


def _normal(seed: int, tag: int, shape, std: float) -> np.ndarray:
    x = rng(seed, tag).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def drafter_weights(dims: DrafterDims, seed: int, random_gains: bool = False,
                    skip: Sequence[str] = ()) -> dict:
    """All drafter parameters, N(0, 0.02) in storage dtype; gains are float32.

    Linear weights are row-major ``[out, in]``.  ``w_qkv`` stacks the q rows
    (Hq*Dh), then k rows (Hkv*Dh), then v rows.  Gains are 1.0 unless
    ``random_gains`` (U[0.5, 1.5]) is asked for.  Names in ``skip`` are not drawn.
    """
    d, F, V = dims.hidden, dims.ffn, dims.vocab
    shapes = {
        "embed": (V, d), "w_fc": (d, 3 * d), "w_qkv": (dims.qkv_rows, d),
        "w_o": (d, dims.n_q_heads * dims.head_dim), "w_gate": (F, d), "w_up": (F, d),
        "w_down": (d, F), "w_lm": (V, d), "h_shared": (3, d),
    }
    out = {}
    for name, shape in shapes.items():
        if name in skip:
            continue
        out[name] = to_storage(_normal(seed, _W_TAGS[name], shape, 0.02), dims.dtype)
    gshapes = {"stream_gain": (3, d), "attn_gain": (d,), "mlp_gain": (d,), "final_gain": (d,)}
    for name, shape in gshapes.items():
        if random_gains:
            out[name] = rng(seed, _GAIN_TAGS[name]).uniform(0.5, 1.5, shape).astype(np.float32)
        else:
            out[name] = np.ones(shape, dtype=np.float32)
    return out


def decode_case(dims: DrafterDims, seed: int, R: int, K: int, W: Sequence[int],
                kv_len: Sequence[int], n_rej: Sequence[int],
                stream_rms=(0.5, 0.6, 0.8), extra_hidden_rows: int = 0,
                window_pos_from_kv: bool = True) -> dict:
    """One decode step's batch-build inputs plus the per-request KV regions.

    Request r owns ``W[r]`` window rows (the previous verify pass: the first
    ``W[r]-n_rej[r]`` accepted, the rest rejected), then one next-token slot
    and K-1 MASK slots.  Its KV region holds ``kv_len[r] + W[r] + K`` rows:
    rows below ``kv_len[r]`` are N(0,1) cache contents, the rest hold the
    NaN sentinel until the drafter writes them.  Window row j of request r
    sits at position ``kv_len[r] + j``.  Captured target hidden rows of
    request r are ``W[r]`` window rows followed by its h_context row, each
    of the three streams N(0,1) scaled to the stated RMS.
    """
    W = np.asarray(W, dtype=np.int64)
    kv_len = np.asarray(kv_len, dtype=np.int64)
    n_rej = np.asarray(n_rej, dtype=np.int64)
    assert W.shape == (R,) and kv_len.shape == (R,) and n_rej.shape == (R,)
    assert np.all(n_rej >= 0) and np.all(n_rej <= W)
    d, V = dims.hidden, dims.vocab
    cu_window = np.zeros(R + 1, dtype=np.int32)
    cu_window[1:] = np.cumsum(W)
    total_w = int(cu_window[-1])
    cap = kv_len + W + K
    kv_base = np.zeros(R, dtype=np.int64)
    kv_base[1:] = np.cumsum(cap)[:-1]
    kv_rows = int(cap.sum())

    window_ids = rng(seed, 20).integers(0, V, total_w).astype(np.int32)
    new_token = rng(seed, 21).integers(0, V, R).astype(np.int32)
    hrow_base = np.zeros(R, dtype=np.int64)
    hrow_base[1:] = np.cumsum(W + 1)[:-1]
    n_hidden = int((W + 1).sum()) + extra_hidden_rows
    streams = _normal(seed, 22, (n_hidden, 3, d), 1.0)
    streams *= np.asarray(stream_rms, dtype=np.float32)[None, :, None]
    target_hidden = to_storage(streams, dims.dtype)

    window_pos = np.zeros(total_w, dtype=np.int32)
    window_hrow = np.zeros(total_w, dtype=np.int32)
    for r in range(R):
        j = np.arange(W[r])
        s = cu_window[r]
        window_pos[s:s + W[r]] = (kv_len[r] if window_pos_from_kv else 0) + j
        window_hrow[s:s + W[r]] = hrow_base[r] + j
    ctx_hrow = (hrow_base + W).astype(np.int32)

    Hkv, Dh = dims.n_kv_heads, dims.head_dim
    sval, sdt = sentinel_bits(dims.dtype)
    k_cache = np.full((kv_rows, Hkv, Dh), sval, dtype=sdt)
    v_cache = np.full((kv_rows, Hkv, Dh), sval, dtype=sdt)
    n_exist = int(kv_len.sum())
    if n_exist:
        kd = to_storage(_normal(seed, 23, (n_exist, Hkv, Dh), 1.0), dims.dtype)
        vd = to_storage(_normal(seed, 24, (n_exist, Hkv, Dh), 1.0), dims.dtype)
        o = 0
        for r in range(R):
            n = int(kv_len[r])
            b = int(kv_base[r])
            k_cache[b:b + n] = kd[o:o + n].view(sdt)
            v_cache[b:b + n] = vd[o:o + n].view(sdt)
            o += n
    if dims.dtype == "f32":
        k_cache = k_cache.view(np.float32)
        v_cache = v_cache.view(np.float32)
    return dict(
        R=R, K=K, cu_window=cu_window, n_rej=n_rej.astype(np.int32),
        kv_len=kv_len.astype(np.int32), kv_base=kv_base.astype(np.int32),
        window_ids=window_ids, window_pos=window_pos, window_hrow=window_hrow,
        new_token=new_token, ctx_hrow=ctx_hrow, target_hidden=target_hidden,
        k_cache=k_cache, v_cache=v_cache, kv_rows=kv_rows,
    )


def decode_config(cfg: int, with_weights: bool = True) -> tuple:
    """(dims, weights, case) of the decode workloads: 0 the tiny fp32 step
    (N=128 window rows, K=4), 1 the single-request step (c=1, K=7, 2,048
    cached positions), 2 the 64-request step (c=64, K=7, ragged caches of
    512-4,096 positions)."""
    if cfg == 0:
        dims = TINY_DIMS
        case = decode_case(dims, 0, R=1, K=4, W=[128], kv_len=[0], n_rej=[0],
                           extra_hidden_rows=3)
        wseed = 0
    elif cfg == 1:
        dims = GPTOSS_DIMS
        case = decode_case(dims, 1, R=1, K=7, W=[0], kv_len=[2048], n_rej=[0])
        wseed = 1
    elif cfg == 2:
        dims = GPTOSS_DIMS
        R = 64
        kv_len = rng(2, 25).integers(512, 4097, R)
        n_rej = rng(2, 26).integers(0, 7, R)
        case = decode_case(dims, 2, R=R, K=7, W=[7] * R, kv_len=kv_len, n_rej=n_rej)
        wseed = 1  # the same drafter as the c=1 decode step
    else:
        raise ValueError(cfg)
    weights = drafter_weights(dims, wseed) if with_weights else None
    return dims, weights, case


def _depth_major(N: int, starters: np.ndarray, U: np.ndarray, keep: float, n_depths: int) -> dict:
    """Depth-major layout: group 0 = positions 0..N-1, group e = the starters
    whose first e draws U[i, 0..e-1] are below ``keep``, sorted by start;
    ``parent`` links each row of depth >= 2 to its (start, depth-1) row."""
    starts = [np.arange(N, dtype=np.int64)]
    alive = starters.copy()
    for e in range(1, n_depths):
        alive = alive & (U[:, e - 1] < keep)
        starts.append(np.nonzero(alive)[0].astype(np.int64))
    group_off = np.zeros(n_depths + 1, dtype=np.int64)
    group_off[1:] = np.cumsum([len(s) for s in starts])
    T = int(group_off[-1])
    start = np.concatenate(starts).astype(np.int32)
    depth = np.concatenate([np.full(len(s), e, dtype=np.int32) for e, s in enumerate(starts)])
    parent = np.full(T, -1, dtype=np.int32)
    for e in range(2, n_depths):
        pos = np.searchsorted(starts[e - 1], starts[e])
        parent[group_off[e]:group_off[e + 1]] = (group_off[e - 1] + pos).astype(np.int32)
    return dict(start=start, depth=depth, parent=parent, group_off=group_off.astype(np.int32), T=T)


def cod_case(N: int, n_depths: int, keep: float, loss_rate: float, seed: int,
             heads=COD_HEADS, dtype: str = "bf16", draw_qkv: bool = True) -> dict:
    """Training-shaped COD attention input in depth-major layout.

    Draws: ``loss_mask = U[0,1) < loss_rate`` (tag 30) and keep draws
    ``U`` of shape [N, n_depths-1] (tag 31).  Chain i reaches depth e >= 1
    when its loss mask is set and ``U[i, 0..e-1] < keep`` all hold; every
    original position is a depth-0 row.  Rows are grouped by depth and sorted
    by start inside a group.  ``parent[row]`` is the row of (start, depth-1)
    for depth >= 2 and -1 otherwise.  Q is [T, Hq, Dh], K/V are [T, Hkv, Dh],
    all N(0,1) (tags 32-34).
    """
    Hq, Hkv, Dh = heads
    loss_mask = rng(seed, 30).random(N) < loss_rate
    U = rng(seed, 31).random((N, max(n_depths - 1, 0)))
    out = dict(N=N, n_depths=n_depths, keep=keep, loss_mask=loss_mask, U=U, heads=heads, dtype=dtype)
    out.update(_depth_major(N, loss_mask, U, keep, n_depths))
    T = out["T"]
    if draw_qkv:
        out["q"] = to_storage(_normal(seed, 32, (T, Hq, Dh), 1.0), dtype)
        out["k"] = to_storage(_normal(seed, 33, (T, Hkv, Dh), 1.0), dtype)
        out["v"] = to_storage(_normal(seed, 34, (T, Hkv, Dh), 1.0), dtype)
    return out


def anchor_case(N: int, n_depths: int, keep: float, loss_rate: float, max_anchors: int, seed: int,
                heads=COD_HEADS, dtype: str = "bf16", draw_qkv: bool = True) -> dict:
    """Random-anchor COD attention input (the max_anchors variant).

    Draws: ``loss_mask = U[0,1) < loss_rate`` (tag 40); min(max_anchors,
    #loss-mask positions) anchors chosen uniformly without replacement among
    the loss-mask positions (tag 41); keep draws ``U`` [N, n_depths-1] (tag
    42).  Only anchors start chains.  Keys/values: the depth-major layout of
    all N positions plus the anchors' chain rows ([T, Hkv, Dh], tags 44-45);
    queries: the anchors' depth-0 rows, then every chain row, in row order
    (``q_rows``), with Q [num_q, Hq, Dh] in that order (tag 43).  All values
    N(0,1).
    """
    Hq, Hkv, Dh = heads
    loss_mask = rng(seed, 40).random(N) < loss_rate
    elig = np.nonzero(loss_mask)[0]
    na = min(max_anchors, len(elig))
    anchors = np.sort(rng(seed, 41).choice(elig, size=na, replace=False)).astype(np.int64)
    U = rng(seed, 42).random((N, max(n_depths - 1, 0)))
    starters = np.zeros(N, dtype=bool)
    starters[anchors] = True
    out = dict(N=N, n_depths=n_depths, keep=keep, loss_mask=loss_mask, U=U, anchors=anchors,
               heads=heads, dtype=dtype)
    out.update(_depth_major(N, starters, U, keep, n_depths))
    T = out["T"]
    q_rows = np.concatenate([anchors, np.arange(N, T)]).astype(np.int32)
    out["q_rows"] = q_rows
    out["num_q"] = len(q_rows)
    if draw_qkv:
        out["q"] = to_storage(_normal(seed, 43, (len(q_rows), Hq, Dh), 1.0), dtype)
        out["k"] = to_storage(_normal(seed, 44, (T, Hkv, Dh), 1.0), dtype)
        out["v"] = to_storage(_normal(seed, 45, (T, Hkv, Dh), 1.0), dtype)
    return out


# The pages' long-context setting for random anchors: 8K positions, 1024
# anchors, keep (down-sample ratio) 0.5, 8 depths; loss-mask rate 0.5 as in
# the N=4096 COD case.
ANCHOR_8K = dict(N=8192, n_depths=8, keep=0.5, loss_rate=0.5, max_anchors=1024, seed=5)


def anchor_config(draw_qkv: bool = True) -> dict:
    return anchor_case(draw_qkv=draw_qkv, **ANCHOR_8K)


def cod_config(cfg: int, draw_qkv: bool = True) -> dict:
    """Training-shaped attention layouts: 3 the COD layout at N=4096 (5
    depths, keep 0.7, loss mask rate 0.5), 4 the parallel groups at N=8192
    (8 depths, keep 1.0, every position a chain start)."""
    if cfg == 3:
        return cod_case(4096, 5, 0.7, 0.5, 3, draw_qkv=draw_qkv)
    if cfg == 4:
        # keep 1.0 and an all-ones loss mask: U[0,1) < 1.0 always holds.
        return cod_case(8192, 8, 1.0, 1.0, 4, draw_qkv=draw_qkv)
    raise ValueError(cfg)


def kl_targets(n: int, vocab: int, k: int, seed: int, tag: int = 51) -> tuple:
    """A stand-in for a verifier's top-k distribution per row: k distinct
    token ids drawn uniformly from the vocabulary and probabilities
    proportional to exp(2 N(0,1)), summing to 1 (float32).  Returns
    (ids [n, k] int32, probs [n, k] float32)."""
    g = rng(seed, tag)
    ids = np.empty((n, k), np.int32)
    for i in range(n):
        ids[i] = g.choice(vocab, k, replace=False)
    a = g.standard_normal((n, k)) * 2.0
    p = np.exp(a - a.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return ids, p.astype(np.float32)
