"""GPU parity of pe_draft_attention (COD layout and decode regions) against the oracle.

* Outputs and LSE within the tolerance of oracle.cod.attention.
* Visible-key counts and SplitMix64 hashes bit-exact against
  oracle.cod.index_stats (they come from the kernel's own masking loop).
* Chunked (query chunks) == unchunked, bit for bit, on small layouts and on
  the N=8192, K=8 long-sequence case.
* The training-shaped N=4096 COD case with every query's index stats, and
  values on a sample of queries (every depth's first and last rows).
* Decode-shaped segments with ragged lengths through the split-KV path,
  plus empty queries and num_q = 0.
* Random anchors (max_anchors): the sampled query subset against every key
  row, small layouts in full (unsplit and split) and the 8K setting on a
  sample of queries, index stats of every query.
* StreamingLLM window (sink + recent window over the depth-0 keys): small
  layouts in full with chunked == unchunked, and the pages' sink 256 /
  window 2048 on the N=8192, K=8 layout (per-query counts in closed form,
  values on a sample).
"""
import numpy as np
import pytest
import torch

from drafter_pe_build_amd import _lib as L
from drafter_pe_build_amd.step import to_device
from helpers import TOL, bits, dev_to_f64, say
from oracle import cod as oc
from oracle import drafter as od
from oracle import metrics as om
from synth import inputs as si

pytestmark = pytest.mark.gpu


class LazyRows:
    """fp64 view of selected rows of a storage array (the oracle indexes q[t])."""

    def __init__(self, arr, dtype):
        self.arr, self.dtype, self.shape = arr, dtype, arr.shape

    def __getitem__(self, t):
        return od.to_f64(self.arr[t], self.dtype)


def upload_layout(Lay):
    dt = Lay["dtype"]
    return dict(q=to_device(Lay["q"], "cuda"), k=to_device(Lay["k"], "cuda"), v=to_device(Lay["v"], "cuda"),
                start=to_device(Lay["start"].astype(np.int32), "cuda"),
                depth=to_device(Lay["depth"].astype(np.int32), "cuda"),
                parent=to_device(Lay["parent"].astype(np.int32), "cuda"),
                self_row=to_device(np.arange(Lay["T"], dtype=np.int32), "cuda"),
                base=torch.zeros(1, dtype=torch.int32, device="cuda"), dtype=dt)


def run_cod(D, Lay, c0=0, c1=None, out=None, lse=None, dbg=True, split_len=0, sink=0, window=0):
    T = Lay["T"]
    c1 = T if c1 is None else c1
    nq = c1 - c0
    Hq, Hkv, Dh = Lay["heads"]
    sdt = torch.bfloat16 if D["dtype"] == "bf16" else torch.float32
    if out is None:
        out = torch.empty((nq, Hq, Dh), dtype=sdt, device="cuda")
    if lse is None:
        lse = torch.empty((nq, Hq), dtype=torch.float32, device="cuda")
    cnt = torch.zeros((nq, Hkv), dtype=torch.int64, device="cuda") if dbg else None
    hsh = torch.zeros((nq, Hkv), dtype=torch.int64, device="cuda") if dbg else None
    a = L.attn_args(num_q=nq, num_seg=1, q_per_seg=nq, num_kv_rows=T, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=Dh,
                    scale=1.0 / np.sqrt(Dh), dtype=L.PE_BF16 if D["dtype"] == "bf16" else L.PE_F32,
                    q=D["q"][c0:c1], q_row_stride=Hq * Dh, k=D["k"], v=D["v"], seg_kv_base=D["base"],
                    q_start=D["start"][c0:c1], q_depth=D["depth"][c0:c1], q_self_row=D["self_row"][c0:c1],
                    kv_parent=D["parent"], max_prefix=Lay["N"], split_len=split_len, out=out, lse=lse,
                    dbg_count=cnt, dbg_hash=hsh, window_sink=sink, window_len=window,
                    max_depth=max(1, int(Lay["depth"].max())))
    L.pe_draft_attention(a, "cuda")
    return out, lse, cnt, hsh


def check_against_oracle(Lay, out, lse, cnt, hsh, queries, name, sink=0, window=0):
    dt = Lay["dtype"]
    tol = TOL[dt]
    q64 = LazyRows(Lay["q"], dt)
    k64 = od.to_f64(Lay["k"], dt)
    v64 = od.to_f64(Lay["v"], dt)
    ref_o, ref_l = oc.attention(q64, k64, v64, Lay["start"], Lay["depth"], queries, sink=sink, window=window)
    o = dev_to_f64(out)[queries]
    e = om.relerr(o, ref_o)
    el = om.relerr(lse.cpu().numpy()[queries], ref_l)
    say("  [%s] out relerr %.3g  lse relerr %.3g  (%d queries)" % (name, e, el, len(queries)))
    assert e <= tol and el <= tol
    if cnt is not None:
        rc, rh = oc.index_stats(Lay["start"], Lay["depth"], queries, sink=sink, window=window)
        gc = cnt.cpu().numpy()[queries]
        gh = hsh.cpu().numpy().view(np.uint64)[queries]
        for j in range(gc.shape[1]):
            np.testing.assert_array_equal(gc[:, j], rc)
            np.testing.assert_array_equal(gh[:, j], rh)


@pytest.mark.parametrize("dtype,heads,N,D,keep,loss", [
    ("bf16", (8, 2, 128), 150, 5, 0.7, 0.5),
    ("bf16", (16, 4, 64), 150, 4, 0.6, 1.0),
    ("f32", (8, 2, 128), 160, 5, 0.7, 0.5),
    ("f32", (4, 4, 64), 140, 3, 1.0, 1.0),
    ("bf16", (32, 8, 128), 257, 8, 1.0, 1.0),
    ("bf16", (64, 1, 128), 90, 4, 0.8, 1.0),
    ("bf16", (8, 8, 128), 120, 5, 0.9, 0.7),
])
def test_cod_small_layouts(dtype, heads, N, D, keep, loss):
    Lay = si.cod_case(N, D, keep, loss, 21, heads=heads, dtype=dtype)
    name = "COD %s N=%d D=%d heads=%s T=%d" % (dtype, N, D, heads, Lay["T"])
    say(name)
    Dv = upload_layout(Lay)
    out, lse, cnt, hsh = run_cod(Dv, Lay)
    torch.cuda.synchronize()
    check_against_oracle(Lay, out, lse, cnt, hsh, np.arange(Lay["T"]), name)
    # chunked == unchunked, bit for bit (chunks of 256 rows and a ragged tail), with a
    # fixed split of the prefix range so that several splits and the combine are active
    assert Lay["T"] > 256
    out1, lse1, _, _ = run_cod(Dv, Lay, dbg=False, split_len=64)
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    for c0 in range(0, Lay["T"], 256):
        c1 = min(Lay["T"], c0 + 256)
        run_cod(Dv, Lay, c0, c1, out=out2[c0:c1], lse=lse2[c0:c1], dbg=False, split_len=64)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out2), bits(out1)) and np.array_equal(bits(lse2), bits(lse1))
    check_against_oracle(Lay, out1, lse1, None, None, np.arange(Lay["T"]), name + " split 64")


def test_cod_training_shape_n4096():
    Lay = si.cod_config(3)
    say("COD N=4096 T=%d" % Lay["T"])
    Dv = upload_layout(Lay)
    out, lse, cnt, hsh = run_cod(Dv, Lay)
    torch.cuda.synchronize()
    go = Lay["group_off"]
    # values: every query of the last 256 rows of each depth group (the
    # largest starts, so every prefix tile), the first 8 of each group, and
    # 2 % of all rows at random
    sample = set()
    for e in range(len(go) - 1):
        sample.update(range(go[e], min(go[e] + 8, go[e + 1])))
        sample.update(range(max(go[e], go[e + 1] - 256), go[e + 1]))
    sample.update(np.random.default_rng(0).choice(Lay["T"], int(0.02 * Lay["T"]) + 1, replace=False).tolist())
    check_against_oracle(Lay, out, lse, None, None, np.array(sorted(sample)), "N=4096 values")
    # index stats of every query
    rc, rh = oc.index_stats(Lay["start"], Lay["depth"])
    gc = cnt.cpu().numpy()
    gh = hsh.cpu().numpy().view(np.uint64)
    for j in range(gc.shape[1]):
        np.testing.assert_array_equal(gc[:, j], rc)
        np.testing.assert_array_equal(gh[:, j], rh)
    assert int(rc.sum()) == int(np.sum(Lay["start"].astype(np.int64) + 1 + Lay["depth"]))


@pytest.mark.parametrize("dtype,heads,N,D,keep,sink,window", [
    ("bf16", (8, 2, 128), 400, 5, 0.7, 16, 100),     # windows inside and across tiles, sink < one tile
    ("bf16", (32, 8, 128), 300, 8, 1.0, 64, 64),     # sink = one tile, window = one tile
    ("f32", (8, 2, 64), 350, 4, 0.8, 0, 37),         # no sink
    ("bf16", (16, 4, 64), 260, 3, 0.9, 100, 1),      # the window is the query itself
    ("bf16", (8, 8, 128), 200, 5, 0.7, 8, 500),      # window wider than the sequence
])
def test_window_small_layouts(dtype, heads, N, D, keep, sink, window):
    Lay = si.cod_case(N, D, keep, 0.5, 25, heads=heads, dtype=dtype)
    name = "window %s N=%d D=%d heads=%s sink=%d window=%d T=%d" % (dtype, N, D, heads, sink, window, Lay["T"])
    say(name)
    Dv = upload_layout(Lay)
    out, lse, cnt, hsh = run_cod(Dv, Lay, sink=sink, window=window)
    torch.cuda.synchronize()
    check_against_oracle(Lay, out, lse, cnt, hsh, np.arange(Lay["T"]), name, sink=sink, window=window)
    # chunks of 256 queries (and a ragged tail) give the same bits
    out1, lse1, _, _ = run_cod(Dv, Lay, dbg=False, sink=sink, window=window)
    out2 = torch.empty_like(out1)
    lse2 = torch.empty_like(lse1)
    for c0 in range(0, Lay["T"], 256):
        c1 = min(Lay["T"], c0 + 256)
        run_cod(Dv, Lay, c0, c1, out=out2[c0:c1], lse=lse2[c0:c1], dbg=False, sink=sink, window=window)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out2), bits(out1)) and np.array_equal(bits(lse2), bits(lse1))


def test_window_long_sequence_n8192():
    # the pages' StreamingLLM setting (sink 256, window 2048) on the N=8192, K=8 layout
    Lay = si.cod_config(4)
    T = Lay["T"]
    say("window N=8192 K=8 sink=256 window=2048")
    Dv = upload_layout(Lay)
    out, lse, cnt, hsh = run_cod(Dv, Lay, sink=256, window=2048)
    torch.cuda.synchronize()
    i = Lay["start"].astype(np.int64)
    closed = np.minimum(256, i + 1) + np.maximum(0, i - np.maximum(256, i - 2047) + 1) + Lay["depth"]
    np.testing.assert_array_equal(cnt[:, 0].cpu().numpy(), closed)
    g = np.random.default_rng(3)
    sample = set()
    for c in range(8):
        sample.update([8192 * c, 8192 * c + 300, 8192 * c + 2300, 8192 * c + 8191])
    sample.update(g.choice(T, 24, replace=False).tolist())
    check_against_oracle(Lay, out, lse, cnt, hsh, np.array(sorted(sample)), "window N=8192 sampled",
                         sink=256, window=2048)


def upload_anchor(A):
    qr = A["q_rows"]
    return dict(q=to_device(A["q"], "cuda"), k=to_device(A["k"], "cuda"), v=to_device(A["v"], "cuda"),
                q_start=to_device(A["start"][qr].astype(np.int32), "cuda"),
                q_depth=to_device(A["depth"][qr].astype(np.int32), "cuda"),
                q_self=to_device(qr.astype(np.int32), "cuda"),
                parent=to_device(A["parent"].astype(np.int32), "cuda"),
                base=torch.zeros(1, dtype=torch.int32, device="cuda"), dtype=A["dtype"])


def run_anchor(D, A, dbg=True, split_len=0):
    """Random-anchor attention: the num_q sampled rows query all T key rows."""
    nq, T = A["num_q"], A["T"]
    Hq, Hkv, Dh = A["heads"]
    sdt = torch.bfloat16 if D["dtype"] == "bf16" else torch.float32
    out = torch.empty((nq, Hq, Dh), dtype=sdt, device="cuda")
    lse = torch.empty((nq, Hq), dtype=torch.float32, device="cuda")
    cnt = torch.zeros((nq, Hkv), dtype=torch.int64, device="cuda") if dbg else None
    hsh = torch.zeros((nq, Hkv), dtype=torch.int64, device="cuda") if dbg else None
    a = L.attn_args(num_q=nq, num_seg=1, q_per_seg=nq, num_kv_rows=T, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=Dh,
                    scale=1.0 / np.sqrt(Dh), dtype=L.PE_BF16 if D["dtype"] == "bf16" else L.PE_F32,
                    q=D["q"], q_row_stride=Hq * Dh, k=D["k"], v=D["v"], seg_kv_base=D["base"],
                    q_start=D["q_start"], q_depth=D["q_depth"], q_self_row=D["q_self"], kv_parent=D["parent"],
                    max_prefix=A["N"], split_len=split_len, out=out, lse=lse, dbg_count=cnt, dbg_hash=hsh,
                    max_depth=max(1, int(A["depth"].max())))
    L.pe_draft_attention(a, "cuda")
    return out, lse, cnt, hsh


def check_anchor(A, out, lse, cnt, hsh, sel, name):
    """sel: indices into the query list compared by value; index stats of every query."""
    dt = A["dtype"]
    tol = TOL[dt]
    qr = A["q_rows"]
    q64 = od.to_f64(A["q"][sel], dt)
    ref_o, ref_l = oc.attention(q64, od.to_f64(A["k"], dt), od.to_f64(A["v"], dt), A["start"], A["depth"],
                                qr[sel], q_by_query=True)
    e = om.relerr(dev_to_f64(out)[sel], ref_o)
    el = om.relerr(lse.cpu().numpy()[sel], ref_l)
    say("  [%s] out relerr %.3g  lse relerr %.3g  (%d of %d queries)" % (name, e, el, len(sel), len(qr)))
    assert e <= tol and el <= tol
    if cnt is not None:
        rc, rh = oc.index_stats(A["start"], A["depth"], qr)
        gc = cnt.cpu().numpy()
        gh = hsh.cpu().numpy().view(np.uint64)
        for j in range(gc.shape[1]):
            np.testing.assert_array_equal(gc[:, j], rc)
            np.testing.assert_array_equal(gh[:, j], rh)


@pytest.mark.parametrize("dtype,heads,N,D,keep,anchors", [
    ("bf16", (8, 2, 128), 300, 5, 0.7, 40),
    ("bf16", (32, 8, 128), 520, 8, 0.5, 130),
    ("f32", (8, 2, 64), 260, 4, 0.9, 60),
    ("bf16", (16, 4, 64), 200, 3, 1.0, 500),   # more anchors than loss-mask positions: all of them
])
def test_anchor_small_layouts(dtype, heads, N, D, keep, anchors):
    A = si.anchor_case(N, D, keep, 0.5, anchors, 23, heads=heads, dtype=dtype)
    name = "anchors %s N=%d D=%d heads=%s queries=%d keys=%d" % (dtype, N, D, heads, A["num_q"], A["T"])
    say(name)
    Dv = upload_anchor(A)
    out, lse, cnt, hsh = run_anchor(Dv, A)
    torch.cuda.synchronize()
    check_anchor(A, out, lse, cnt, hsh, np.arange(A["num_q"]), name)
    # a fixed split of the prefix range (several splits and the combine) agrees too
    out1, lse1, _, _ = run_anchor(Dv, A, dbg=False, split_len=64)
    torch.cuda.synchronize()
    check_anchor(A, out1, lse1, None, None, np.arange(A["num_q"]), name + " split 64")


def test_anchor_long_sequence_n8192():
    A = si.anchor_config()
    say("random anchors N=8192: %d anchors, %d queries, %d key rows" % (len(A["anchors"]), A["num_q"], A["T"]))
    Dv = upload_anchor(A)
    out, lse, cnt, hsh = run_anchor(Dv, A)
    torch.cuda.synchronize()
    # the query set's visible pairs through the kernel's own counters
    qr = A["q_rows"]
    pairs = int(np.sum(A["start"][qr].astype(np.int64) + 1 + A["depth"][qr]))
    assert int(cnt[:, 0].sum().item()) == pairs
    first = np.searchsorted(qr, A["group_off"][:-1])   # first query of each depth group
    sel = set()
    for i in first.tolist() + [A["num_q"] - 1]:
        sel.update(range(max(0, i - 2), min(A["num_q"], i + 3)))
    sel.update(np.random.default_rng(2).choice(A["num_q"], 24, replace=False).tolist())
    check_anchor(A, out, lse, cnt, hsh, np.array(sorted(sel)), "anchors N=8192 sampled")


def test_long_sequence_chunked_n8192():
    Lay = si.cod_config(4)
    T = Lay["T"]
    assert T == 65536
    Hq, Hkv, Dh = Lay["heads"]
    Dv = upload_layout(Lay)
    out = torch.empty((T, Hq, Dh), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    say("parallel groups N=8192 K=8 T=%d: unchunked" % T)
    run_cod(Dv, Lay, out=out, lse=lse, dbg=False)
    torch.cuda.synchronize()
    say("  8 chunks of 8192")
    for c in range(8):
        run_cod(Dv, Lay, 8192 * c, 8192 * (c + 1), out=out2[8192 * c:8192 * (c + 1)],
                lse=lse2[8192 * c:8192 * (c + 1)], dbg=False)
    torch.cuda.synchronize()
    # nothing near the size of a dense mask (T^2 = 4.3e9 elements) was allocated
    assert free0 - torch.cuda.mem_get_info()[0] < (64 << 20)
    assert np.array_equal(bits(out2), bits(out)) and np.array_equal(bits(lse2), bits(lse))
    say("  index statistics run")
    out3, lse3, cnt, hsh = run_cod(Dv, Lay, dbg=True)
    torch.cuda.synchronize()
    # visible-pair closed form through the kernel's own counters
    assert int(cnt[:, 0].sum().item()) == 268697600
    g = np.random.default_rng(1)
    # values: every query of the first and last 64 rows of each chunk (two
    # 32-query workgroup tiles at both chunk edges; one chunk per depth) and
    # 0.5 % of all rows at random
    sample = set()
    for c in range(8):
        sample.update(range(8192 * c, 8192 * c + 64))
        sample.update(range(8192 * (c + 1) - 64, 8192 * (c + 1)))
    sample.update(g.choice(T, int(0.005 * T) + 1, replace=False).tolist())
    check_against_oracle(Lay, out, lse, cnt, hsh, np.array(sorted(sample)), "N=8192 sampled")


def test_decode_segments_split_kv():
    """Ragged decode regions: query k of segment s sits at position len_s-K+k and
    sees region rows 0..its position; several splits plus a combine."""
    g = np.random.default_rng(5)
    Hq, Hkv, Dh, K = 16, 2, 64, 7
    lens = np.array([100, 900, 37, 2000, 71, 7])
    base = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    rows = int(lens.sum())
    for dtype in ("bf16", "f32"):
        q = si.to_storage(g.standard_normal((rows, Hq, Dh)).astype(np.float32), dtype)
        k = si.to_storage(g.standard_normal((rows, Hkv, Dh)).astype(np.float32), dtype)
        v = si.to_storage(g.standard_normal((rows, Hkv, Dh)).astype(np.float32), dtype)
        R = len(lens)
        pos = np.concatenate([np.arange(l - K, l) for l in lens]).astype(np.int32)
        pos[5] = -1                                      # a query that sees nothing
        qrows = np.concatenate([b + np.arange(l - K, l) for b, l in zip(base, lens)]).astype(np.int32)
        sdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        for split_len in (0, 64, 4096):
            out = torch.empty((R * K, Hq, Dh), dtype=sdt, device="cuda")
            lse = torch.empty((R * K, Hq), dtype=torch.float32, device="cuda")
            cnt = torch.zeros((R * K, Hkv), dtype=torch.int64, device="cuda")
            hsh = torch.zeros((R * K, Hkv), dtype=torch.int64, device="cuda")
            a = L.attn_args(num_q=R * K, num_seg=R, q_per_seg=K, num_kv_rows=rows, n_q_heads=Hq, n_kv_heads=Hkv,
                            head_dim=Dh, scale=0.125, dtype=L.PE_BF16 if dtype == "bf16" else L.PE_F32,
                            q=to_device(q, "cuda"), q_row_stride=Hq * Dh, q_rows=to_device(qrows, "cuda"),
                            k=to_device(k, "cuda"), v=to_device(v, "cuda"), seg_kv_base=to_device(base, "cuda"),
                            q_start=to_device(pos, "cuda"), max_prefix=int(lens.max()), split_len=split_len,
                            out=out, lse=lse, dbg_count=cnt, dbg_hash=hsh)
            say("decode segments %s split_len=%d" % (dtype, split_len))
            L.pe_draft_attention(a, "cuda")
            torch.cuda.synchronize()
            o = dev_to_f64(out)
            for s in range(R):
                b, l = int(base[s]), int(lens[s])
                lab = np.arange(l)
                for j in range(K):
                    i = s * K + j
                    if pos[i] < 0:
                        assert np.all(o[i] == 0) and np.all(np.isneginf(lse.cpu().numpy()[i]))
                        assert int(cnt[i, 0]) == 0
                        continue
                    qq = np.zeros((l, Hq, Dh))
                    qq[pos[i]] = od.to_f64(q[b + pos[i]], dtype)
                    ro, rl = oc.attention(qq, od.to_f64(k[b:b + l], dtype), od.to_f64(v[b:b + l], dtype), lab,
                                          np.zeros(l, int), [pos[i]], 0.125)
                    assert om.relerr(o[i], ro[0]) <= TOL[dtype]
                    assert om.relerr(lse.cpu().numpy()[i], rl[0]) <= TOL[dtype]
                    c, h = oc.region_index_stats(b, int(pos[i]))
                    assert int(cnt[i, 0]) == c and int(cnt[i, 1]) == c
                    assert np.uint64(hsh[i, 0].item() & 0xFFFFFFFFFFFFFFFF) == h


def test_empty_query_set_is_noop():
    out = torch.empty(0, device="cuda")
    a = L.attn_args(num_q=0, num_seg=0, q_per_seg=0, num_kv_rows=0, n_q_heads=8, n_kv_heads=2, head_dim=64,
                    scale=0.125, dtype=L.PE_BF16, q_row_stride=512, out=out)
    L.pe_draft_attention(a, "cuda")
    torch.cuda.synchronize()
