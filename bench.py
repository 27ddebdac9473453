"""Benchmark of the parallel-drafting hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]

A step is one drafter forward predicting all K=7 draft tokens of the decode
step with c=1 (2,048-position KV cache, d=2880, 64 q / 8 kv heads x 64,
SwiGLU 8192, vocab 201,088, bf16): pe_build_draft_batch -> pe_fuse_hidden ->
pe_draft_layer -> pe_lm_head_argmax, inputs resident in HBM.  The headline
value is draft positions per second (7 per step).  The JSON line also
carries the roofline of the dominant kernel (the LM-head weight stream),
the fp64 oracle's CPU rate on the same workload, and secondary measurements:
the c=64 decode step and the training-shaped COD / parallel-group attention.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

# HBM bytes per launch of the LM-head stage measured with rocprofv3 FETCH_SIZE /
# WRITE_SIZE, scaled by a 1 GiB copy (profiles/decode_c1_lm_head_hbm_counters.md),
# valid only for the kernel sources they were taken on.
LM_STAGE_TRAFFIC = {"fingerprint": "a48aa4c916559de9", "bytes": 1159581390}
LM_SOURCES = ("gemm.hip", "norm.hip", "common.h", "kernels.h", "epilogue.h")
# The same for one whole c=64 decode step (every kernel of the step), from
# profiles/decode_c64_step_counters.md.
DECODE64_TRAFFIC = {"fingerprint": "6997a73f08fa2498", "bytes": 2791270918}
ALL_SOURCES = ("api.hip", "attention.hip", "batch.hip", "common.h", "epilogue.h", "gemm.hip", "gemm_big.hip",
               "kernels.h", "norm.hip")


def source_fingerprint(files=LM_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "drafter_pe_build_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baselines")
    ap.add_argument("--cpu-workloads", default="0,1,2,3,4",
                    help="workloads whose oracle CPU baseline is timed, comma-separated: 0 tiny fp32 decode "
                         "(N=128, K=4), 1 decode c=1, 2 decode c=64, 3 COD attention N=4096, 4 parallel-group "
                         "attention N=8192")
    ap.add_argument("--no-extra", action="store_true", help="skip the c=64 decode and attention measurements")
    ap.add_argument("--attention-only", type=int, choices=(3, 4, 5, 6), default=0,
                    help="time only the COD (3), parallel-group (4), random-anchor (5) or windowed "
                         "parallel-group (6) attention workload and print its line")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the COD attention backward (N=4096 layout) and print its line")
    ap.add_argument("--loss-only", action="store_true",
                    help="time only the fused LM-head loss on a training-sized batch and print its line")
    ap.add_argument("--decode64-only", action="store_true",
                    help="time only the c=64 decode step and print its line")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also copy 1 GiB device-to-device 3 times (reference for HBM byte counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class CacheFlush:
    """Evicts the 256 MB Infinity Cache (and the L2s) between timed passes by
    reading a 512 MB buffer: a read-only pass leaves no dirty lines whose
    write-back would land in the next timed pass."""

    def __init__(self, nbytes=512 << 20):
        import torch
        self.buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")

    def __call__(self):
        return self.buf.sum()


_FLUSH = None


def flush_cache():
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = CacheFlush()
    _FLUSH()


def time_loop(fn, steps, warmup, stream):
    """W untimed passes, then exactly `steps` timed passes, each preceded by a
    cache flush outside its timed region and bracketed by HIP events on the
    stream the library launches on (torch's current stream); the whole timed
    loop sits between two device synchronisations.  Returns the median pass
    time in ms (the mean, min and max go to time_loop.last)."""
    import numpy as np
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        flush_cache()
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    d = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    time_loop.last = {"median_ms": float(np.median(d)), "mean_ms": float(d.mean()), "min_ms": float(d.min()),
                      "max_ms": float(d.max()), "passes": int(steps), "cache": "flushed before every pass"}
    return float(np.median(d))


time_loop.last = {}


def time_sustained(fn, min_steps, stream, warm_s=0.03, timed_s=0.05):
    """Time fn once its clocks have settled: one pass sizes the loops, then
    at least warm_s seconds of untimed passes and at least timed_s seconds
    (and min_steps passes) of timed ones, each timed pass after a cache
    flush; the median pass.  Short compute-bound kernels run well below their
    sustained clock during the first tens of milliseconds."""
    import math
    import torch
    fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    fn()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = max(e0.elapsed_time(e1) * 1e-3, 1e-6)
    return time_loop(fn, max(min_steps, math.ceil(timed_s / t1)), max(2, math.ceil(warm_s / t1)), stream)


def decode_bytes(dims, case, T, RK):
    """Algorithmic HBM bytes of one decode step: every weight once, the KV
    rows the queries read, the K/V rows written, the hidden rows read and
    copied, the embedding rows, and the activations in and out."""
    import numpy as np
    e = 2 if dims.dtype == "bf16" else 4
    d, F, V = dims.hidden, dims.ffn, dims.vocab
    qc = dims.n_q_heads * dims.head_dim
    kvc = dims.n_kv_heads * dims.head_dim
    weights = (d * 3 * d + dims.qkv_rows * d + d * qc + 2 * F * d + d * F + V * d) * e
    W = np.diff(case["cu_window"])
    n_acc = W - case["n_rej"]
    keys = int(np.sum(case["kv_len"].astype(np.int64) + n_acc + case["K"]))   # rows read per kv head
    live = int(np.sum(n_acc)) + RK
    kv = keys * 2 * kvc * e + live * 2 * kvc * e
    hidden = T * 3 * d * e * 3                     # target rows read, draft rows written, read by fc
    emb = T * d * e
    act = T * d * 4 + RK * d * 4 + RK * 4
    return weights + kv + hidden + emb + act, weights


ATTN_NAMES = {3: "cod_attention_n4096", 4: "group_attention_n8192_chunked", 5: "anchor_attention_n8192",
              6: "window_attention_n8192_chunked"}
# StreamingLLM setting of the pages' 8K ablation: sink 256, window 2048
WINDOW_SINK, WINDOW_LEN = 256, 2048


def measure_attention(cfg, steps, stream):
    """COD attention N=4096 (one launch) or parallel-group attention N=8192
    (8 query chunks of 8192; workload 6: with the StreamingLLM window): time
    per pass over all queries and rate."""
    import numpy as np
    import torch
    from drafter_pe_build_amd import _lib as L
    from drafter_pe_build_amd.step import to_device
    from synth import inputs as si
    log(ATTN_NAMES[cfg])
    Lay = si.cod_config(4 if cfg == 6 else cfg)
    sink, window = (WINDOW_SINK, WINDOW_LEN) if cfg == 6 else (0, 0)
    T = Lay["T"]
    Hq, Hkv, Dh = Lay["heads"]
    q, k, v = (to_device(Lay[n], "cuda") for n in ("q", "k", "v"))
    start = to_device(Lay["start"].astype(np.int32), "cuda")
    depth = to_device(Lay["depth"].astype(np.int32), "cuda")
    parent = to_device(Lay["parent"].astype(np.int32), "cuda")
    selfr = to_device(np.arange(T, dtype=np.int32), "cuda")
    base = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.empty((T, Hq, Dh), dtype=torch.bfloat16, device="cuda")
    chunks = [(0, T)] if cfg == 3 else [(8192 * c, 8192 * (c + 1)) for c in range(8)]
    arglist = [L.attn_args(num_q=c1 - c0, num_seg=1, q_per_seg=c1 - c0, num_kv_rows=T, n_q_heads=Hq,
                           n_kv_heads=Hkv, head_dim=Dh, scale=1.0 / np.sqrt(Dh), dtype=L.PE_BF16,
                           q=q[c0:c1], q_row_stride=Hq * Dh, k=k, v=v, seg_kv_base=base,
                           q_start=start[c0:c1], q_depth=depth[c0:c1], q_self_row=selfr[c0:c1],
                           kv_parent=parent, max_prefix=Lay["N"], out=out[c0:c1], window_sink=sink,
                           window_len=window, max_depth=max(1, int(Lay["depth"].max()))) for c0, c1 in chunks]
    wsb = max(L.pe_draft_attention_workspace(a) for a in arglist)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device="cuda")

    def run_attn():
        for a in arglist:
            L.pe_draft_attention(a, "cuda", workspace=ws)

    msa = time_sustained(run_attn, steps, stream)
    i = Lay["start"].astype(np.int64)
    if window:   # visible depth-0 keys: the sink plus the window, per query
        pairs = int(np.sum(np.minimum(sink, i + 1) + np.maximum(0, i - np.maximum(sink, i - window + 1) + 1)
                           + Lay["depth"]))
    else:
        pairs = int(np.sum(i + 1 + Lay["depth"]))
    fl = pairs * Hq * 4 * Dh
    log("  %.1f us, %.0f TFLOP/s" % (msa * 1e3, fl / (msa * 1e-3) / 1e12))
    del q, k, v, out
    torch.cuda.empty_cache()
    return {"T": T, "ms": msa, "positions_per_s": T / (msa * 1e-3), "visible_pairs": pairs,
            "tflops": fl / (msa * 1e-3) / 1e12, "mfma_frac": fl / (msa * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "launches": len(chunks)}


def measure_anchor(steps, stream):
    """Random-anchor (max_anchors) attention at 8K: 1024 anchors' rows query
    every original position plus the anchors' chain rows; one launch."""
    import numpy as np
    import torch
    from drafter_pe_build_amd import _lib as L
    from drafter_pe_build_amd.step import to_device
    from synth import inputs as si
    log("random-anchor attention N=8192")
    A = si.anchor_config()
    qr = A["q_rows"]
    nq, T = A["num_q"], A["T"]
    Hq, Hkv, Dh = A["heads"]
    q, k, v = (to_device(A[n], "cuda") for n in ("q", "k", "v"))
    q_start = to_device(A["start"][qr].astype(np.int32), "cuda")
    q_depth = to_device(A["depth"][qr].astype(np.int32), "cuda")
    q_self = to_device(qr.astype(np.int32), "cuda")
    parent = to_device(A["parent"].astype(np.int32), "cuda")
    base = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.empty((nq, Hq, Dh), dtype=torch.bfloat16, device="cuda")
    a = L.attn_args(num_q=nq, num_seg=1, q_per_seg=nq, num_kv_rows=T, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=Dh,
                    scale=1.0 / np.sqrt(Dh), dtype=L.PE_BF16, q=q, q_row_stride=Hq * Dh, k=k, v=v,
                    seg_kv_base=base, q_start=q_start, q_depth=q_depth, q_self_row=q_self, kv_parent=parent,
                    max_prefix=A["N"], out=out, max_depth=max(1, int(A["depth"].max())))
    ws = torch.empty(max(L.pe_draft_attention_workspace(a), 256), dtype=torch.uint8, device="cuda")
    msa = time_sustained(lambda: L.pe_draft_attention(a, "cuda", workspace=ws), steps, stream)
    pairs = int(np.sum(A["start"][qr].astype(np.int64) + 1 + A["depth"][qr]))
    fl = pairs * Hq * 4 * Dh
    log("  %.1f us, %.0f TFLOP/s" % (msa * 1e3, fl / (msa * 1e-3) / 1e12))
    del q, k, v, out
    torch.cuda.empty_cache()
    return {"queries": nq, "key_rows": T, "anchors": int(len(A["anchors"])), "ms": msa,
            "queries_per_s": nq / (msa * 1e-3), "visible_pairs": pairs, "tflops": fl / (msa * 1e-3) / 1e12,
            "mfma_frac": fl / (msa * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, "launches": 1}


def measure_backward(steps, stream):
    """COD attention backward over the N=4096 training layout (one call over
    all queries): delta, dQ and dK/dV kernels.  Algorithmic work: 10 Hq Dh
    flops per visible pair (recomputed scores, dP, dV, dQ, dK)."""
    import numpy as np
    import torch
    from drafter_pe_build_amd import _lib as L
    from drafter_pe_build_amd.step import to_device
    from synth import inputs as si
    log("COD attention backward N=4096")
    Lay = si.cod_config(3)
    T = Lay["T"]
    Hq, Hkv, Dh = Lay["heads"]
    q, k, v = (to_device(Lay[n], "cuda") for n in ("q", "k", "v"))
    start = to_device(Lay["start"].astype(np.int32), "cuda")
    depth = to_device(Lay["depth"].astype(np.int32), "cuda")
    parent = to_device(Lay["parent"].astype(np.int32), "cuda")
    goff = to_device(Lay["group_off"].astype(np.int32), "cuda")
    selfr = to_device(np.arange(T, dtype=np.int32), "cuda")
    base = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.empty((T, Hq, Dh), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    fa = L.attn_args(num_q=T, num_seg=1, q_per_seg=T, num_kv_rows=T, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=Dh,
                     scale=1.0 / np.sqrt(Dh), dtype=L.PE_BF16, q=q, q_row_stride=Hq * Dh, k=k, v=v,
                     seg_kv_base=base, q_start=start, q_depth=depth, q_self_row=selfr, kv_parent=parent,
                     max_prefix=Lay["N"], out=out, lse=lse, max_depth=max(1, int(Lay["depth"].max())))
    L.pe_draft_attention(fa, "cuda")
    dout = torch.randn((T, Hq, Dh), dtype=torch.float32, device="cuda").to(torch.bfloat16)
    dq = torch.empty((T, Hq, Dh), dtype=torch.float32, device="cuda")
    dk = torch.zeros((T, Hkv, Dh), dtype=torch.float32, device="cuda")
    dv = torch.zeros((T, Hkv, Dh), dtype=torch.float32, device="cuda")
    ba = L.attn_bwd_args(num_rows=T, n_pos=Lay["N"], n_groups=len(Lay["group_off"]) - 1, n_q_heads=Hq,
                         n_kv_heads=Hkv, head_dim=Dh, scale=1.0 / np.sqrt(Dh), dtype=L.PE_BF16, group_off=goff,
                         start=start, depth=depth, q=q, k=k, v=v, out=out, dout=dout, lse=lse, q_begin=0,
                         q_end=T, dq=dq, dk=dk, dv=dv)
    ws = torch.empty(L.pe_draft_attention_backward_workspace(ba), dtype=torch.uint8, device="cuda")
    ms = time_sustained(lambda: L.pe_draft_attention_backward(ba, "cuda", workspace=ws), steps, stream)
    pairs = int(np.sum(Lay["start"].astype(np.int64) + 1 + Lay["depth"]))
    fl = pairs * Hq * 10 * Dh
    log("  %.1f us, %.0f TFLOP/s" % (ms * 1e3, fl / (ms * 1e-3) / 1e12))
    del q, k, v, out, dout, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return {"T": T, "ms": ms, "positions_per_s": T / (ms * 1e-3), "visible_pairs": pairs,
            "tflops": fl / (ms * 1e-3) / 1e12, "mfma_frac": fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "launches": 3}


def measure_loss(dims, steps, stream, W=None):
    """LM-head log-sum-exp + cross-entropy over a training-sized batch (the
    COD N=4096 layout's 7,794 rows) without materialising the logits."""
    import numpy as np
    import torch
    from drafter_pe_build_amd import _lib as L
    from drafter_pe_build_amd.step import to_device
    from synth import inputs as si
    n = si.cod_config(3, draw_qkv=False)["T"]
    log("fused LM-head loss, %d rows" % n)
    if W is None:
        W = si.drafter_weights(dims, 1, skip=("embed", "w_fc", "w_qkv", "w_o", "w_gate", "w_up", "w_down",
                                              "h_shared"))
    cd = L.dims_struct(dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.ffn, dims.vocab,
                       dims.mask_token_id, dims.eps, dims.dtype)
    cw = L.weights_struct({"w_lm": L.pe_pack_weight(to_device(W["w_lm"], "cuda")),
                           "final_gain": to_device(W["final_gain"], "cuda")})
    g = np.random.default_rng(7)
    x = torch.from_numpy(g.standard_normal((n, dims.hidden)).astype(np.float32)).cuda()
    t = torch.from_numpy(g.integers(0, dims.vocab, n).astype(np.int32)).cuda()
    lse = torch.empty(n, dtype=torch.float32, device="cuda")
    loss = torch.empty(n, dtype=torch.float32, device="cuda")
    ws = torch.empty(L.pe_lm_head_loss_workspace(cd, n), dtype=torch.uint8, device="cuda")
    ms = time_sustained(lambda: L.pe_lm_head_loss(cd, cw, n, x, t, lse, loss, workspace=ws), steps, stream)
    fl = 2.0 * n * dims.vocab * dims.hidden
    log("  %.1f us, %.0f TFLOP/s" % (ms * 1e3, fl / (ms * 1e-3) / 1e12))
    # the top-k KL variant on the same rows: k = 32 target pairs per row
    k = 32
    ids, pr = si.kl_targets(n, dims.vocab, k, 7)
    ids, pr = torch.from_numpy(ids).cuda(), torch.from_numpy(pr).cuda()
    kl = torch.empty(n, dtype=torch.float32, device="cuda")
    wsk = torch.empty(L.pe_lm_head_kl_workspace(cd, n), dtype=torch.uint8, device="cuda")
    kms = time_sustained(lambda: L.pe_lm_head_kl(cd, cw, n, x, k, ids, pr, kl, lse, workspace=wsk), steps, stream)
    log("  top-%d KL: %.1f us" % (k, kms * 1e3))
    # the same with the target rows read from the row-major LM head
    w_rows = to_device(W["w_lm"], "cuda")
    rms = time_sustained(lambda: L.pe_lm_head_kl(cd, cw, n, x, k, ids, pr, kl, lse, w_lm_rows=w_rows, workspace=wsk),
                         steps, stream)
    log("  top-%d KL, row-major target rows: %.1f us" % (k, rms * 1e3))
    del cw, x, t, lse, loss, ws, ids, pr, kl, wsk, w_rows
    torch.cuda.empty_cache()
    return {"rows": n, "ms": ms, "rows_per_s": n / (ms * 1e-3), "tflops": fl / (ms * 1e-3) / 1e12,
            "mfma_frac": fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "logits_bytes_avoided": n * dims.vocab * 4,
            "kl_topk": {"k": k, "ms": kms, "rows_per_s": n / (kms * 1e-3),
                        "tflops": fl / (kms * 1e-3) / 1e12, "mfma_frac": fl / (kms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                        "ms_row_major_targets": rms,
                        "note": "log-sum-exp pass plus one fp32 dot product per target pair (n * k rows of W_lm "
                                "gathered from the packed weight; ms_row_major_targets reads them from a row-major "
                                "copy)"}}


def measure_decode64(dims, W, steps, stream):
    """The c=64 decode step (64 requests x 7 slots, ragged caches), one graph
    replay per step: time, rate, HBM and matrix-core fractions."""
    import numpy as np
    import torch
    from drafter_pe_build_amd.step import DraftStep, GraphStep
    from synth import inputs as si
    log("c=64 decode step")
    _, _, case2 = si.decode_config(2, with_weights=False)
    st2 = DraftStep(dims, W, case2)
    RK2 = st2.R * st2.K
    gs2 = GraphStep(st2)
    ms2 = time_sustained(gs2.replay, steps, stream)
    st_stats = dict(time_loop.last)
    # the dominant kernel's stage alone: final RMSNorm, LM head with the fused
    # top-2, the fp32 re-score of the two leading tokens
    ms_lm = time_sustained(lambda: st2.lm_head(False), steps, stream)
    lm_stats = dict(time_loop.last)
    b2, _ = decode_bytes(dims, case2, st2.T, RK2)
    W_ = np.diff(case2["cu_window"])
    n_acc = W_ - case2["n_rej"]
    live2 = int(np.sum(n_acc)) + RK2
    # attention: a query at position P sees P + 1 rows; positions kv_len + n_acc + j, j < K
    keys = int(np.sum((case2["kv_len"].astype(np.int64) + n_acc)[:, None] + 1 + np.arange(case2["K"])[None, :]))
    fl_attn = 4.0 * dims.n_q_heads * dims.head_dim * keys
    fl2 = 2.0 * (live2 * (3 * dims.hidden * dims.hidden + dims.qkv_rows * dims.hidden)
                 + RK2 * (dims.hidden * dims.n_q_heads * dims.head_dim + 3 * dims.ffn * dims.hidden
                          + dims.vocab * dims.hidden)) + fl_attn
    fl_lm = 2.0 * RK2 * dims.vocab * dims.hidden
    log("  step %.1f us, LM stage %.1f us" % (ms2 * 1e3, ms_lm * 1e3))
    del gs2, st2
    torch.cuda.empty_cache()
    tf_lm = fl_lm / (ms_lm * 1e-3) / 1e12
    traffic = (DECODE64_TRAFFIC["bytes"] if source_fingerprint(ALL_SOURCES) == DECODE64_TRAFFIC["fingerprint"]
               else None)
    return {"ms_per_step": ms2, "draft_positions_per_s": RK2 / (ms2 * 1e-3),
            "timing": st_stats,
            "algorithmic_bytes": b2, "algorithmic_flops": fl2,
            "hbm_gbs": b2 / (ms2 * 1e-3) / 1e9, "hbm_frac": b2 / (ms2 * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "gemm_tflops": fl2 / (ms2 * 1e-3) / 1e12,
            "mfma_frac": fl2 / (ms2 * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "binding": "mfma (%.0f flop per algorithmic byte, above the %.0f ridge)"
                       % (fl2 / b2, BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)),
            "step_traffic_bytes": traffic,
            "roofline": {"bound": "mfma",
                         "kernel": "LM-head stage (448 x 201,088 x 2,880 on the matrix cores with the final "
                                   "RMSNorm, the fused top-2 and the fp32 re-score of the two leading tokens)",
                         "achieved": tf_lm, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf_lm / BF16_PEAK_TFLOPS, "traffic": None, "launch_us": ms_lm * 1e3,
                         "algorithmic_flops": fl_lm, "timing": lm_stats}}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def oracle_threads():
    """Threads the fp64 oracle's BLAS calls use (the host cores it may run on)."""
    n = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            n = max(blas)
    except Exception:
        pass
    return n


def cpu_oracle_decode(dims, W, case):
    """One full decode step of the fp64 oracle (batch build, fuse, layer, LM
    head + argmax); seconds."""
    from oracle import batch as ob
    from oracle import drafter as od
    t0 = time.time()
    b = ob.build_draft_batch(case["K"], dims.mask_token_id, case["cu_window"], case["n_rej"], case["kv_len"],
                             case["kv_base"], case["window_ids"], case["window_pos"], case["window_hrow"],
                             case["new_token"], case["ctx_hrow"], case["target_hidden"], W["h_shared"])
    od.drafter_forward(dims, W, b, case["kv_base"], case["k_cache"], case["v_cache"], keep_logits=False)
    return time.time() - t0


def cpu_oracle_attention(cfg):
    """The fp64 oracle's COD attention on a seeded, bounded query sample of the
    N=4096 (workload 3) or N=8192 x 8 (workload 4) layout; the time is extrapolated per
    query to the whole layout (input generation and the bf16 -> fp64
    conversion excluded)."""
    import numpy as np
    from oracle import cod as oc
    from oracle import drafter as od
    from synth import inputs as si
    Lay = si.cod_config(cfg)
    q, k, v = (od.to_f64(Lay[n], "bf16") for n in ("q", "k", "v"))
    T = Lay["T"]
    if cfg == 3:
        qs = np.arange(0, T, 32)
        desc = "every 32nd of the %d query rows (%d queries, all depths)" % (T, len(qs))
    else:
        qs = np.concatenate([np.r_[8192 * c:8192 * c + 16, 8192 * (c + 1) - 16:8192 * (c + 1)] for c in range(8)])
        desc = ("the first and last 16 rows of each of the 8 query chunks (one chunk per depth: %d queries, "
                "starts 0-15 and 8176-8191)" % len(qs))
    t0 = time.time()
    oc.attention(q, k, v, Lay["start"], Lay["depth"], qs)
    t = time.time() - t0
    pairs_s = int(np.sum(Lay["start"][qs].astype(np.int64) + 1 + Lay["depth"][qs]))
    pairs = int(np.sum(Lay["start"].astype(np.int64) + 1 + Lay["depth"]))
    return {"sample_seconds": t, "sample_queries": int(len(qs)), "sample_pairs": pairs_s, "T": T,
            "visible_pairs": pairs, "seconds": t * T / len(qs), "sample": desc}


def cpu_baselines(dims, W, case1, which):
    """The fp64 oracle timed on the host cores, one entry per config."""
    from synth import inputs as si
    out = {"cpu_model": cpu_model(), "cores": oracle_threads(), "kind": "oracle",
           "note": "the plain fp64 numpy oracle as written (not tuned); a reported baseline, not a target"}
    for cfg in which:
        log("oracle CPU baseline, workload %d" % cfg)
        if cfg == 0:
            d0, W0, c0 = si.decode_config(0)
            t = cpu_oracle_decode(d0, W0, c0)
            n = c0["R"] * c0["K"]
            out["tiny_fp32_n128_k4"] = {"seconds": t, "value": n / t, "unit": "draft positions/s",
                                        "sample": "one full step (%d draft positions)" % n}
        elif cfg == 1:
            t = cpu_oracle_decode(dims, W, case1)
            n = case1["R"] * case1["K"]
            out["decode_c1"] = {"seconds": t, "value": n / t, "unit": "draft positions/s",
                                "sample": "one full step (%d draft positions)" % n}
        elif cfg == 2:
            _, _, c2 = si.decode_config(2, with_weights=False)
            t = cpu_oracle_decode(dims, W, c2)
            n = c2["R"] * c2["K"]
            out["decode_c64"] = {"seconds": t, "value": n / t, "unit": "draft positions/s",
                                 "sample": "one full step (%d draft positions)" % n}
        else:
            r = cpu_oracle_attention(cfg)
            name = "cod_attention_n4096" if cfg == 3 else "group_attention_n8192"
            out[name] = {**r, "value": r["T"] / r["seconds"], "unit": "positions/s (extrapolated per query)"}
        log("  done")
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from drafter_pe_build_amd import _lib as L
    from drafter_pe_build_amd.step import DraftStep, GraphStep, to_device
    from synth import inputs as si

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    if args.copy_probe:  # three 1 GiB device copies: the scale of the HBM byte counters
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    if args.attention_only:
        if args.attention_only == 5:
            r = measure_anchor(args.steps, stream)
        else:
            r = measure_attention(args.attention_only, args.steps, stream)
        print(json.dumps({"metric": ATTN_NAMES[args.attention_only], "value": r["tflops"], "unit": "TFLOP/s",
                          "higher_is_better": True, "dtype": "bf16", "data": "synthetic", **r}), flush=True)
        return
    dims = si.GPTOSS_DIMS
    if args.backward_only:
        r = measure_backward(args.steps, stream)
        print(json.dumps({"metric": "cod_attention_backward_n4096", "value": r["tflops"], "unit": "TFLOP/s",
                          "higher_is_better": True, "dtype": "bf16", "data": "synthetic", **r}), flush=True)
        return
    if args.loss_only:
        r = measure_loss(dims, args.steps, stream)
        print(json.dumps({"metric": "lm_head_loss_rows_per_s", "value": r["rows_per_s"], "unit": "rows/s",
                          "higher_is_better": True, "dtype": "bf16", "data": "synthetic", **r}), flush=True)
        return
    if args.decode64_only:
        log("generating the drafter weights")
        r = measure_decode64(dims, si.drafter_weights(dims, 1), args.steps, stream)
        print(json.dumps({"metric": "decode_c64_draft_positions_per_s", "value": r["draft_positions_per_s"],
                          "unit": "draft positions/s", "higher_is_better": True, "dtype": "bf16",
                          "data": "synthetic", **r}), flush=True)
        return
    log("generating the c=1 decode inputs and the drafter weights")
    t0 = time.time()
    W = si.drafter_weights(dims, 1)
    _, _, case1 = si.decode_config(1, with_weights=False)
    log("  %.1f s" % (time.time() - t0))
    st = DraftStep(dims, W, case1)
    RK = st.R * st.K
    ms_eager = time_loop(st.run, args.steps, args.warmup, stream)
    stats_eager = dict(time_loop.last)
    log("c=1 step, eager launches: %.1f us (median)" % (ms_eager * 1e3))
    gs = GraphStep(st)
    ms = time_loop(gs.replay, args.steps, args.warmup, stream)
    stats_graph = dict(time_loop.last)
    step_bytes, weight_bytes = decode_bytes(dims, case1, st.T, RK)
    ms_graph = ms
    log("c=1 step, one graph replay: %.1f us" % (ms_graph * 1e3))
    launch_mode = "one HIP graph replay of the four stage calls"
    stats = stats_graph
    if ms_eager < ms_graph:
        ms = ms_eager
        stats = stats_eager
        launch_mode = "the four stage calls launched eagerly on one stream"

    # dominant kernel: the LM-head stage (the W_lm stream with the final
    # RMSNorm in its staging and the fused argmax, then the reduce of the
    # per-workgroup partials)
    lm_ms = time_loop(lambda: st.lm_head(False), args.steps, args.warmup, stream)
    lm_stats = dict(time_loop.last)
    # algorithmic bytes: W_lm once, the x rows (f32), the tokens
    lm_bytes = dims.vocab * dims.hidden * 2 + RK * dims.hidden * 4 + RK * 4
    lm_gbs = lm_bytes / (lm_ms * 1e-3) / 1e9
    log("LM head stage: %.1f us, %.0f GB/s" % (lm_ms * 1e3, lm_gbs))

    result = {
        "metric": "draft positions/sec per drafter fwd",
        "value": RK / (ms * 1e-3),
        "unit": "draft positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "eager_ms_per_step": ms_eager,
        "graph_ms_per_step": ms_graph,
        "launch": launch_mode + " (the faster of eager launches and graph replay)",
        "timing": {**stats, "statistic": "median of the timed steps, each after a 512 MB cache flush, "
                                         "by HIP events on the library's stream"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) cache, scaled hidden streams)",
        "config": {"workload": "decode step c=1, K=7 draft slots, 2048-position KV cache, d=2880, "
                               "64q/8kv x 64, SwiGLU 8192, vocab 201088",
                   "requests": 1, "draft_slots": 7, "cache_positions": 2048},
        "step_hbm_gbs": step_bytes / (ms * 1e-3) / 1e9,
        "step_hbm_frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "step_algorithmic_bytes": step_bytes,
        "roofline": {"bound": "hbm",
                     "kernel": "LM-head stage: W_lm stream with the final RMSNorm and the argmax fused, partial reduce",
                     "achieved": lm_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": lm_gbs / HBM_PEAK_GBS,
                     "traffic": (LM_STAGE_TRAFFIC["bytes"]
                                 if source_fingerprint() == LM_STAGE_TRAFFIC["fingerprint"] else None),
                     "launch_us": lm_ms * 1e3, "algorithmic_bytes": lm_bytes, "timing": lm_stats},
    }
    del gs, st
    torch.cuda.empty_cache()

    if not args.no_extra:
        extra = {}
        extra["decode_c64"] = measure_decode64(dims, W, max(5, args.steps // 5), stream)
        for cfg, name in ((3, "cod_attention_n4096"), (4, "group_attention_n8192_chunked")):
            extra[name] = measure_attention(cfg, max(5, args.steps // 5), stream)
        extra["anchor_attention_n8192"] = measure_anchor(max(5, args.steps // 5), stream)
        extra["window_attention_n8192_chunked"] = measure_attention(6, max(5, args.steps // 5), stream)
        extra["lm_head_loss_7794_rows"] = measure_loss(dims, max(5, args.steps // 5), stream, W)
        extra["cod_attention_backward_n4096"] = measure_backward(max(5, args.steps // 5), stream)
        result["secondary"] = extra

    if not args.no_cpu:
        which = sorted({int(c) for c in args.cpu_workloads.split(",") if c.strip()} | {1})
        cb = cpu_baselines(dims, W, case1, which)
        c1 = cb["decode_c1"]
        result["cpu_baseline"] = {"value": c1["value"], "unit": "draft positions/s", "cores": cb["cores"],
                                  "kind": "oracle", "cpu_model": cb["cpu_model"],
                                  "sample": "one full c=1 decode step (7 draft positions), fp64 numpy, %.2f s"
                                            % c1["seconds"]}
        result["cpu_baseline_by_config"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
