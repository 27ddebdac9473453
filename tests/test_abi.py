"""Host-only checks of libpe.so: it loads, exports every function include/pe.h
declares, and rejects bad arguments before launching anything (no GPU needed:
every call below fails validation, so no HIP call is made)."""
import ctypes
import os
import re

import pytest

from drafter_pe_build_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libpe.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pe_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"pe_build_draft_batch", "pe_fuse_hidden", "pe_draft_attention", "pe_draft_layer",
            "pe_lm_head_argmax"} <= set(names)
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) <= set(L.EXPORTS)


def test_version_and_status_strings():
    lib = L.lib()
    assert lib.pe_version().decode().startswith("pe ")
    assert lib.pe_status_string(1) == b"PE_ERR_INVALID_ARG"
    assert lib.pe_status_string(2) == b"PE_ERR_UNSUPPORTED"


def _dims(**kw):
    base = dict(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=512, vocab=4096, mask_token_id=4095,
                eps=1e-6, dtype="f32")
    base.update(kw)
    return L.dims_struct(**base)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def test_dims_validation_codes():
    lib = L.lib()
    n = ctypes.c_size_t()
    ok = _dims()
    assert lib.pe_fuse_hidden_workspace(ctypes.byref(ok), 10, ctypes.byref(n)) == 0
    assert n.value >= 10 * 3 * 256 * 4
    cases = [(dict(head_dim=96), 2), (dict(n_kv_heads=3), 1), (dict(hidden=200), 2),
             (dict(mask_token_id=4096), 1), (dict(eps=-1.0), 1), (dict(vocab=0), 1),
             (dict(n_q_heads=128, n_kv_heads=1), 2), (dict(hidden=272, dtype="bf16"), 2)]
    for kw, code in cases:
        d = _dims(**kw)
        assert lib.pe_fuse_hidden_workspace(ctypes.byref(d), 10, ctypes.byref(n)) == code, kw
    assert lib.pe_fuse_hidden_workspace(ctypes.byref(ok), -1, ctypes.byref(n)) == 1


def test_entry_points_reject_before_launch():
    lib = L.lib()
    d = _dims()
    w = L.PeWeights()
    b = L.PeBatchOut()
    # batch build: R = 0, then a NULL output buffer
    args = [ctypes.byref(d), 0, 4, 0, 1] + [FAKE] * 11 + [ctypes.byref(b), None]
    assert lib.pe_build_draft_batch(*args) == 1
    args = [ctypes.byref(d), 1, 4, 0, 1] + [FAKE] * 11 + [ctypes.byref(b), None]
    assert lib.pe_build_draft_batch(*args) == 1
    # misaligned hidden pointer
    b2 = L.PeBatchOut(*([FAKE] * 9 + [ctypes.c_void_p(0x1004)]))
    args = [ctypes.byref(d), 1, 4, 0, 1] + [FAKE] * 11 + [ctypes.byref(b2), None]
    assert lib.pe_build_draft_batch(*args) == 1
    # fuse: missing weights, then workspace too small
    assert lib.pe_fuse_hidden(ctypes.byref(d), ctypes.byref(w), 8, FAKE, None, FAKE, FAKE, FAKE, 1 << 20, None) == 1
    w2 = L.PeWeights(*([FAKE] * 12))
    assert lib.pe_fuse_hidden(ctypes.byref(d), ctypes.byref(w2), 8, FAKE, None, FAKE, FAKE, FAKE, 16, None) == 1
    # layer: more queries than rows
    assert lib.pe_draft_layer(ctypes.byref(d), ctypes.byref(w2), 3, 1, 4, FAKE, ctypes.byref(b2), FAKE, FAKE, FAKE,
                              10, 10, FAKE, FAKE, 1 << 30, None) == 1
    # lm head: workspace too small
    assert lib.pe_lm_head_argmax(ctypes.byref(d), ctypes.byref(w2), 4, FAKE, FAKE, None, FAKE, 16, None) == 1
    # empty inputs are valid no-ops
    assert lib.pe_fuse_hidden(ctypes.byref(d), ctypes.byref(w), 0, None, None, None, None, None, 0, None) == 0
    assert lib.pe_lm_head_argmax(ctypes.byref(d), ctypes.byref(w), 0, None, None, None, None, 0, None) == 0
    # lm head loss: neither output, a loss without targets, workspace too small; empty is a no-op
    big = 1 << 40
    assert lib.pe_lm_head_loss(ctypes.byref(d), ctypes.byref(w2), 4, FAKE, FAKE, None, None, FAKE, big, None) == 1
    assert lib.pe_lm_head_loss(ctypes.byref(d), ctypes.byref(w2), 4, FAKE, None, None, FAKE, FAKE, big, None) == 1
    assert lib.pe_lm_head_loss(ctypes.byref(d), ctypes.byref(w2), 4, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == 1
    assert lib.pe_lm_head_loss(ctypes.byref(d), ctypes.byref(w), 0, None, None, None, None, None, 0, None) == 0
    n = ctypes.c_size_t()
    assert lib.pe_lm_head_loss_workspace(ctypes.byref(d), 7, ctypes.byref(n)) == 0 and n.value > 0
    # top-k KL loss: k < 1, missing ids / probabilities / output, n * k past int32, workspace too small,
    # a misaligned row-major weight;
    # empty is a no-op; its workspace holds the loss's plus the rows' log-sum-exp
    kl = lib.pe_lm_head_kl
    assert kl(ctypes.byref(d), ctypes.byref(w2), 4, FAKE, 0, FAKE, FAKE, None, None, FAKE, FAKE, big, None) == 1
    assert kl(ctypes.byref(d), ctypes.byref(w2), 4, FAKE, 3, None, FAKE, None, None, FAKE, FAKE, big, None) == 1
    assert kl(ctypes.byref(d), ctypes.byref(w2), 4, FAKE, 3, FAKE, None, None, None, FAKE, FAKE, big, None) == 1
    assert kl(ctypes.byref(d), ctypes.byref(w2), 4, FAKE, 3, FAKE, FAKE, None, FAKE, None, FAKE, big, None) == 1
    assert kl(ctypes.byref(d), ctypes.byref(w2), 1 << 16, FAKE, 1 << 15, FAKE, FAKE, None, None, FAKE, FAKE, big, None) == 1
    assert kl(ctypes.byref(d), ctypes.byref(w2), 4, FAKE, 3, FAKE, FAKE, None, None, FAKE, FAKE, 16, None) == 1
    assert kl(ctypes.byref(d), ctypes.byref(w2), 4, FAKE, 3, FAKE, FAKE, ctypes.c_void_p(0x1002), None, FAKE, FAKE, big, None) == 1
    assert kl(ctypes.byref(d), ctypes.byref(w), 0, None, 3, None, None, None, None, None, None, 0, None) == 0
    m = ctypes.c_size_t()
    assert lib.pe_lm_head_kl_workspace(ctypes.byref(d), 7, ctypes.byref(m)) == 0 and m.value >= n.value + 7 * 4


def test_attention_validation_and_workspace():
    lib = L.lib()
    n = ctypes.c_size_t()
    a = L.attn_args(num_q=7, num_seg=1, q_per_seg=7, num_kv_rows=2055, n_q_heads=64, n_kv_heads=8, head_dim=64,
                    scale=0.125, dtype=L.PE_BF16, q=FAKE, q_row_stride=4096, k=FAKE, v=FAKE, seg_kv_base=FAKE,
                    q_start=FAKE, out=FAKE, max_prefix=2055)
    assert lib.pe_draft_attention_workspace(ctypes.byref(a), ctypes.byref(n)) == 0
    assert n.value > 7 * 64 * 64 * 4            # decode shape is split over the cache
    bad = [dict(num_q=8), dict(head_dim=80), dict(n_kv_heads=7), dict(q_row_stride=100), dict(scale=0.0),
           dict(q=ctypes.c_void_p(0x1002)), dict(q_depth=FAKE)]
    for kw in bad:
        a2 = L.attn_args(**{**dict(num_q=7, num_seg=1, q_per_seg=7, num_kv_rows=2055, n_q_heads=64, n_kv_heads=8,
                                    head_dim=64, scale=0.125, dtype=L.PE_BF16, q=FAKE, q_row_stride=4096, k=FAKE,
                                    v=FAKE, seg_kv_base=FAKE, q_start=FAKE, out=FAKE, max_prefix=2055), **kw})
        assert lib.pe_draft_attention(ctypes.byref(a2), None, 0, None) in (1, 2), kw
    # split path without workspace is refused
    assert lib.pe_draft_attention(ctypes.byref(a), None, 0, None) == 1
    # StreamingLLM window: negative sizes are invalid, a requested split is unsupported,
    # and a window is never split (no workspace needed)
    base = dict(num_q=7, num_seg=1, q_per_seg=7, num_kv_rows=2055, n_q_heads=64, n_kv_heads=8, head_dim=64,
                scale=0.125, dtype=L.PE_BF16, q=FAKE, q_row_stride=4096, k=FAKE, v=FAKE, seg_kv_base=FAKE,
                q_start=FAKE, out=FAKE, max_prefix=2055)
    for kw, code in ((dict(window_len=-1), 1), (dict(window_sink=-3, window_len=8), 1),
                     (dict(window_sink=4, window_len=64, split_len=128), 2)):
        a3 = L.attn_args(**{**base, **kw})
        assert lib.pe_draft_attention(ctypes.byref(a3), None, 0, None) == code, kw
    # backward: bad chunk bounds, f32, missing gradient buffers, too many groups
    bw = dict(num_rows=100, n_pos=60, n_groups=3, n_q_heads=8, n_kv_heads=2, head_dim=128, scale=0.088,
              dtype=L.PE_BF16, group_off=FAKE, start=FAKE, depth=FAKE, q=FAKE, k=FAKE, v=FAKE, out=FAKE,
              dout=FAKE, lse=FAKE, q_begin=0, q_end=100, dq=FAKE, dk=FAKE, dv=FAKE)
    for kw, code in ((dict(q_end=101), 1), (dict(q_begin=5, q_end=4), 1), (dict(dtype=L.PE_F32), 2),
                     (dict(dk=None), 1), (dict(n_groups=17), 2), (dict(q=None), 1), (dict(head_dim=96), 2)):
        b3 = L.attn_bwd_args(**{**bw, **kw})
        assert lib.pe_draft_attention_backward(ctypes.byref(b3), FAKE, 1 << 20, None) == code, kw
    assert lib.pe_draft_attention_backward(ctypes.byref(L.attn_bwd_args(**{**bw, "q_begin": 7, "q_end": 7})),
                                           None, 0, None) == 0
    # chain depth: a host bound is required with q_depth and must fit the kernel's
    # chain list (16 rows, 8 when every query head has its own kv head)
    chain = dict(q_depth=FAKE, q_self_row=FAKE, kv_parent=FAKE)
    for kw, code in ((dict(max_depth=0), 1), (dict(max_depth=-2), 1), (dict(max_depth=17), 2),
                     (dict(max_depth=16), 0), (dict(max_depth=1), 0),
                     (dict(max_depth=9, n_q_heads=8, n_kv_heads=8, q_row_stride=512), 2),
                     (dict(max_depth=8, n_q_heads=8, n_kv_heads=8, q_row_stride=512), 0),
                     (dict(max_depth=16, n_q_heads=16, n_kv_heads=8, q_row_stride=1024), 0)):
        a5 = L.attn_args(**{**base, **chain, **kw})
        assert lib.pe_draft_attention_workspace(ctypes.byref(a5), ctypes.byref(n)) == code, kw
        if code:
            assert lib.pe_draft_attention(ctypes.byref(a5), FAKE, 1 << 30, None) == code, kw
    a4 = L.attn_args(**{**base, "window_sink": 256, "window_len": 2048})
    assert lib.pe_draft_attention_workspace(ctypes.byref(a4), ctypes.byref(n)) == 0
    assert n.value == 16
    # launch sizes and their work split: 2,048 queries of G = 4 at head_dim 128 are
    # 64 tiles x 8 kv heads = 512 workgroups (a planned launch with cut tiles: plan
    # arrays and partials), 4,096 queries 1,024 (the fixed grid, no workspace), and
    # an explicit split length keeps the fixed split
    train = dict(num_seg=1, num_kv_rows=8192, n_q_heads=32, n_kv_heads=8, head_dim=128, scale=0.088,
                 dtype=L.PE_BF16, q=FAKE, q_row_stride=4096, k=FAKE, v=FAKE, seg_kv_base=FAKE, q_start=FAKE,
                 out=FAKE, max_prefix=8192)
    sizes = {}
    for nq, extra in ((2048, {}), (4096, {}), (2048, {"split_len": 4096})):
        a6 = L.attn_args(**{**train, "num_q": nq, "q_per_seg": nq, **extra})
        assert lib.pe_draft_attention_workspace(ctypes.byref(a6), ctypes.byref(n)) == 0
        sizes[(nq, bool(extra))] = n.value
        if n.value > 16:  # a launch that needs workspace refuses to run without it
            assert lib.pe_draft_attention(ctypes.byref(a6), None, 0, None) == 1
    nqh = 2048 * 32
    assert sizes[(2048, False)] >= 3 * nqh * (128 + 2) * 4 + 64 * 3 * 8  # three pieces' partials + the plan
    assert sizes[(4096, False)] == 16
    assert sizes[(2048, True)] >= 2 * nqh * (128 + 2) * 4             # two fixed 4,096-key splits


def test_noalloc_lm_head_refuses_oversized_batches_before_any_device_call():
    # 598 rows of a 201,088 x 2,880 bf16 head need more workspace than the
    # fixed array holds: PE_ERR_UNSUPPORTED, decided on the host; 597 fit
    lib = L.lib()
    d = L.dims_struct(2880, 64, 8, 64, 8192, 201088, 201087, 1e-6, "bf16")
    n = ctypes.c_size_t()
    assert lib.pe_lm_head_argmax_workspace(ctypes.byref(d), 597, ctypes.byref(n)) == 0
    assert n.value <= (32 << 20)
    assert lib.pe_lm_head_argmax_workspace(ctypes.byref(d), 598, ctypes.byref(n)) == 0
    assert n.value > (32 << 20)
    w = L.PeWeights()
    w.w_lm = FAKE
    w.final_gain = FAKE
    assert lib.pe_lm_head_argmax_noalloc(ctypes.byref(d), ctypes.byref(w), 598, FAKE, FAKE, None, None) == 2
    # the usual argument checks come first
    assert lib.pe_lm_head_argmax_noalloc(ctypes.byref(d), ctypes.byref(w), 7, None, FAKE, None, None) == 1
    assert lib.pe_lm_head_argmax_noalloc(ctypes.byref(d), ctypes.byref(w), -1, FAKE, FAKE, None, None) == 1
    assert lib.pe_lm_head_argmax_noalloc(ctypes.byref(d), ctypes.byref(w), 0, None, None, None, None) == 0
