"""GPU parity of the decode-step stages against the fp64 oracle.

Each case runs the four stage calls through the C ABI (via DraftStep) and
checks, stage by stage: the draft batch bit for bit; x0; the layer output of
the query rows, the K/V rows written, and that rejected / unwritten cache
rows keep their sentinel bits; logits and greedy tokens.  Cases cover both
storage dtypes, the GEMM kernels (M <= 16 with rows staged in LDS and the
norm fused, or rows in global memory after a separate norm; M > 16 tiled),
ragged windows, fully rejected windows, K = 1, and full-size decode steps
with 1, 2 and 64 requests.
"""
import numpy as np
import pytest
import torch

from helpers import GAP, TOL, bits, dev_to_f64, gptoss_weights, kernel_top2_ok, say
from oracle import batch as ob
from oracle import drafter as od
from oracle import metrics as om
from synth import inputs as si

pytestmark = pytest.mark.gpu

BATCH_KEYS = ("draft_ids", "draft_pos", "slot_mapping", "hidden_src", "req_of_row", "rejected", "masked",
              "query_rows", "cu_draft")


def oracle_batch(dims, W, c):
    return ob.build_draft_batch(c["K"], dims.mask_token_id, c["cu_window"], c["n_rej"], c["kv_len"], c["kv_base"],
                                c["window_ids"], c["window_pos"], c["window_hrow"], c["new_token"], c["ctx_hrow"],
                                c["target_hidden"], W["h_shared"])


def check_case(name, dims, W, c, logits=True):
    from drafter_pe_build_amd.step import DraftStep
    tol = TOL[dims.dtype]
    say("[%s] upload" % name)
    st = DraftStep(dims, W, c)
    rb = oracle_batch(dims, W, c)

    say("[%s] pe_build_draft_batch" % name)
    st.build_batch()
    torch.cuda.synchronize()
    for k in BATCH_KEYS:
        np.testing.assert_array_equal(st.batch[k].cpu().numpy(), rb[k], err_msg=k)
    hid = bits(st.batch["draft_hidden"])
    np.testing.assert_array_equal(hid, rb["draft_hidden"].view(hid.dtype))

    say("[%s] oracle forward" % name)
    ref = od.drafter_forward(dims, W, rb, c["kv_base"], c["k_cache"], c["v_cache"], keep_logits=logits)
    live = rb["rejected"] == 0

    say("[%s] pe_fuse_hidden" % name)
    st.fuse()
    torch.cuda.synchronize()
    e = om.relerr(st.x0.cpu().numpy()[live], ref["x0"][live])
    say("  x0 relerr %.3g" % e)
    assert e <= tol

    say("[%s] pe_draft_layer" % name)
    k_before = bits(st.k_cache)
    st.layer()
    torch.cuda.synchronize()
    e = om.relerr(st.x_out.cpu().numpy(), ref["x_query"])
    say("  layer out relerr %.3g" % e)
    assert e <= tol
    slots = rb["slot_mapping"][live]
    for gpu, refc in ((st.k_cache, ref["k_cache"]), (st.v_cache, ref["v_cache"])):
        g = dev_to_f64(gpu)
        ek = om.relerr(g[slots], refc[slots])
        say("  written kv relerr %.3g" % ek)
        assert ek <= tol
    k_after = bits(st.k_cache)
    untouched = np.ones(c["kv_rows"], bool)
    untouched[slots] = False
    np.testing.assert_array_equal(k_after[untouched], k_before[untouched])   # cache + sentinel rows keep their bits
    n_sentinel = int(np.sum(c["n_rej"]))
    cached = np.zeros(c["kv_rows"], bool)
    for r in range(c["R"]):
        cached[c["kv_base"][r]:c["kv_base"][r] + c["kv_len"][r]] = True
    assert int(np.sum(untouched & ~cached)) == n_sentinel

    say("[%s] pe_lm_head_argmax" % name)
    st.lm_head(with_logits=logits)
    torch.cuda.synchronize()
    tok = st.tokens.cpu().numpy()
    gap_min = GAP[dims.dtype]
    ok, n = om.tokens_agree(tok, ref["tokens"], ref["gap"], gap_min)
    dec = ref["gap"] > gap_min
    say("  tokens compared %d of %d (oracle top-2 gap > %g; smallest compared gap %.4g), equal %s"
        % (n, len(tok), gap_min, ref["gap"][dec].min() if n else float("nan"), ok))
    if not ok and logits:
        lg = st.logits.cpu().numpy().astype(np.float64)
        for i in np.nonzero((tok != ref["tokens"]) & (ref["gap"] > gap_min))[0]:
            t0, t1 = int(ref["tokens"][i]), int(tok[i])
            say("  row %d: oracle token %d gap %.4g; kernel token %d; kernel logits %.5g / %.5g, oracle %.5g / %.5g, "
                "row rms %.4g" % (i, t0, ref["gap"][i], t1, lg[i, t0], lg[i, t1], ref["logits"][i, t0],
                                  ref["logits"][i, t1], np.sqrt(np.mean(ref["logits"][i] ** 2))))
    assert ok and n > 0
    if logits:
        lg32 = st.logits.cpu().numpy()
        e = om.relerr(lg32, ref["logits"])
        say("  logits relerr %.3g" % e)
        assert e <= tol
        # the token is one of the two largest of the kernel's own logits (the
        # LM head scores those two again in fp32 and keeps the larger)
        assert kernel_top2_ok(tok, lg32)

    say("[%s] full step again (stage outputs must repeat bit for bit)" % name)
    t1 = st.tokens.clone()
    x1 = st.x_out.clone()
    st.run(with_logits=False)
    torch.cuda.synchronize()
    assert torch.equal(t1, st.tokens) and torch.equal(x1, st.x_out)
    return st


def small_dims(dtype, head_dim=64, hq=8, hkv=2):
    return si.DrafterDims(hidden=128, n_q_heads=hq, n_kv_heads=hkv, head_dim=head_dim, ffn=256, vocab=1000,
                          dtype=dtype)


def test_tiny_config_fp32():
    dims, W, c = si.decode_config(0)
    check_case("tiny fp32 N=128 K=4", dims, W, c)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_ragged_stream_and_tiled(dtype):
    # R*K = 15 query rows (weight-streaming GEMMs); T > 16 rows (tiled fc / qkv)
    dims = small_dims(dtype)
    W = si.drafter_weights(dims, 11, random_gains=True)
    c = si.decode_case(dims, 11, R=3, K=5, W=[6, 0, 9], kv_len=[40, 3, 130], n_rej=[2, 0, 9])
    check_case("small %s ragged R=3 K=5" % dtype, dims, W, c)


@pytest.mark.parametrize("dtype,head_dim", [("bf16", 64), ("bf16", 128), ("f32", 128)])
def test_small_many_queries(dtype, head_dim):
    dims = small_dims(dtype, head_dim=head_dim, hq=4, hkv=4)
    W = si.drafter_weights(dims, 12, random_gains=True)
    g = np.random.default_rng(12)
    R = 9
    Wn = g.integers(0, 8, R)
    n_rej = np.array([g.integers(0, w + 1) for w in Wn])
    c = si.decode_case(dims, 12, R=R, K=7, W=Wn, kv_len=g.integers(0, 300, R), n_rej=n_rej)
    check_case("small %s Dh=%d R=9 K=7" % (dtype, head_dim), dims, W, c)


def test_many_requests_large_tile_lm_head():
    # R*K = 140 query rows: the LM head runs on one 224-row LDS tile (a partial
    # row tile and a partial feature tile), hidden 96 gives three 32-wide
    # k-steps, as many as the copy ring has stages
    dims = si.DrafterDims(hidden=96, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=160, vocab=1000, dtype="bf16")
    W = si.drafter_weights(dims, 15, random_gains=True)
    g = np.random.default_rng(15)
    R = 20
    Wn = g.integers(0, 4, R)
    n_rej = np.array([g.integers(0, w + 1) for w in Wn])
    c = si.decode_case(dims, 15, R=R, K=7, W=Wn, kv_len=g.integers(0, 100, R), n_rej=n_rej)
    check_case("LM 256-row tiles R=20 K=7 d=96", dims, W, c)


def test_many_requests_two_row_tiles():
    # R*K = 301 query rows: the LM head reads its normalised rows in the 1 KB
    # operand layout over two 224-row tiles; the second tile ends inside a
    # 16-row group (zero padding rows) and clamps the groups past it
    dims = small_dims("bf16")
    W = si.drafter_weights(dims, 19, random_gains=True)
    g = np.random.default_rng(19)
    R = 43
    Wn = g.integers(0, 4, R)
    n_rej = np.array([g.integers(0, w + 1) for w in Wn])
    c = si.decode_case(dims, 19, R=R, K=7, W=Wn, kv_len=g.integers(0, 150, R), n_rej=n_rej)
    check_case("LM two row tiles R=43 K=7", dims, W, c)


def test_many_requests_split_k():
    # hidden 1024 with ~170 draft rows: fc, QKV, gate/up and down split K over
    # several workgroups (partial products reduced in a second kernel)
    dims = si.DrafterDims(hidden=1024, n_q_heads=8, n_kv_heads=2, head_dim=64, ffn=1024, vocab=1000, dtype="bf16")
    W = si.drafter_weights(dims, 16, random_gains=True)
    g = np.random.default_rng(16)
    R = 20
    Wn = g.integers(0, 4, R)
    n_rej = np.array([g.integers(0, w + 1) for w in Wn])
    c = si.decode_case(dims, 16, R=R, K=7, W=Wn, kv_len=g.integers(0, 200, R), n_rej=n_rej)
    check_case("split K R=20 K=7 d=1024", dims, W, c)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sixteen_rows_streaming(dtype):
    # T = R*K = 16: every contraction on the weight-streaming kernels with a
    # full 16-row operand (no padding rows), norms folded into them
    dims = small_dims(dtype)
    W = si.drafter_weights(dims, 17, random_gains=True)
    c = si.decode_case(dims, 17, R=2, K=8, W=[0, 0], kv_len=[50, 130], n_rej=[0, 0])
    check_case("16 rows %s" % dtype, dims, W, c)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_few_rows_with_rejections(dtype):
    # T = 13 rows, two rejected: the fused stream norms + fc (rows staged in
    # LDS) in both storage types, rejected rows skipped
    dims = small_dims(dtype)
    W = si.drafter_weights(dims, 18, random_gains=True)
    c = si.decode_case(dims, 18, R=2, K=5, W=[2, 1], kv_len=[20, 75], n_rej=[1, 1])
    check_case("13 rows %s" % dtype, dims, W, c)


@pytest.mark.parametrize("dtype,hidden", [("bf16", 32), ("f32", 16)])
def test_hidden_of_one_k_step(dtype, hidden):
    # hidden = one 32-wide (bf16) or 16-wide (f32) k-step: the LM head's K
    # split gives some waves no step at all (their padding loads must stay
    # inside the weight block)
    dims = si.DrafterDims(hidden=hidden, n_q_heads=2, n_kv_heads=1, head_dim=64, ffn=64, vocab=500, dtype=dtype)
    W = si.drafter_weights(dims, 24, random_gains=True)
    c = si.decode_case(dims, 24, R=2, K=4, W=[3, 1], kv_len=[30, 8], n_rej=[1, 0])
    check_case("hidden %d %s" % (hidden, dtype), dims, W, c)


def test_batch_build_many_requests():
    # 300 requests, some with empty windows: the row's request is found in
    # several rounds of 64 probes (up to 64 requests take one); the batch is
    # compared bit for bit, the later stages are covered by the other cases
    from drafter_pe_build_amd.step import DraftStep
    dims = small_dims("bf16")
    W = si.drafter_weights(dims, 25)
    g = np.random.default_rng(25)
    R = 300
    Wn = g.integers(0, 5, R)
    n_rej = np.array([g.integers(0, w + 1) for w in Wn])
    c = si.decode_case(dims, 25, R=R, K=3, W=Wn, kv_len=g.integers(0, 20, R), n_rej=n_rej)
    say("[batch R=300 K=3] pe_build_draft_batch")
    st = DraftStep(dims, W, c)
    rb = oracle_batch(dims, W, c)
    st.build_batch()
    torch.cuda.synchronize()
    for k in BATCH_KEYS:
        np.testing.assert_array_equal(st.batch[k].cpu().numpy(), rb[k], err_msg=k)
    hid = bits(st.batch["draft_hidden"])
    np.testing.assert_array_equal(hid, rb["draft_hidden"].view(hid.dtype))


def test_single_draft_slot():
    dims = small_dims("bf16", hq=16, hkv=2)
    W = si.drafter_weights(dims, 13)
    c = si.decode_case(dims, 13, R=4, K=1, W=[3, 1, 0, 5], kv_len=[10, 0, 70, 1], n_rej=[1, 1, 0, 0])
    check_case("K=1", dims, W, c)


def test_decode_c1_full_size():
    dims = si.GPTOSS_DIMS
    _, _, c = si.decode_config(1, with_weights=False)
    check_case("decode c=1 d=2880 V=201088", dims, gptoss_weights(), c)


def test_decode_two_requests_full_size():
    # T = 15 rows with one rejected window row: the fc and down-projection rows
    # exceed LDS (separate norm, then the weight stream over rows in global
    # memory); the other contractions stage their rows in LDS, norm fused
    dims = si.GPTOSS_DIMS
    c = si.decode_case(dims, 14, R=2, K=7, W=[1, 0], kv_len=[700, 1500], n_rej=[1, 0])
    check_case("decode R=2 K=7 d=2880 V=201088", dims, gptoss_weights(), c)


def test_decode_c64_full_size():
    dims = si.GPTOSS_DIMS
    _, _, c = si.decode_config(2, with_weights=False)
    check_case("decode c=64 d=2880 V=201088", dims, gptoss_weights(), c)
