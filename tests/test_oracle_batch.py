"""Pins of the oracle's draft-batch construction.

Hand-worked example (tests/golden/batch_build_example.json) plus the
invariants the pages fix: the batch grows by K rows per request, rejected
rows and only they carry PADDING_SLOT_ID, MASK rows carry h_shared, slots
are distinct, positions increase within a request.
"""
import json
import os

import numpy as np
import pytest

from oracle import batch as ob
from synth import inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "batch_build_example.json")


def _golden_inputs():
    g = json.load(open(GOLDEN))
    i = g["inputs"]
    th = np.zeros((8, 3, 2), np.float32)
    for r in range(8):
        for s in range(3):
            for c in range(2):
                th[r, s, c] = 10 * r + s + 0.25 * c
    args = dict(K=i["K"], mask_token_id=i["mask_token_id"],
                cu_window=np.array(i["cu_window"]), n_rej=np.array(i["n_rej"]),
                kv_len=np.array(i["kv_len"]), kv_base=np.array(i["kv_base"]),
                window_ids=np.array(i["window_ids"]), window_pos=np.array(i["window_pos"]),
                window_hrow=np.array(i["window_hrow"]), new_token=np.array(i["new_token"]),
                ctx_hrow=np.array(i["ctx_hrow"]), target_hidden=th,
                h_shared=np.array(i["h_shared"], np.float32))
    return g, args


def test_golden_example():
    g, args = _golden_inputs()
    out = ob.build_draft_batch(**args)
    e = g["expected"]
    assert out["T"] == e["T"]
    for name in ("cu_draft", "draft_ids", "draft_pos", "slot_mapping", "hidden_src",
                 "req_of_row", "rejected", "masked", "query_rows"):
        np.testing.assert_array_equal(out[name], np.array(e[name]), err_msg=name)
    for row in (0, 3, 4, 7):
        np.testing.assert_array_equal(out["draft_hidden"][row], np.array(e["draft_hidden_row%d" % row]))


def check_invariants(out, K, R, cu_window, n_rej, kv_len, kv_base, target_hidden, h_shared, mask_id):
    T = out["T"]
    assert T == int(cu_window[-1]) + R * K            # the batch grows by K per request
    assert int(out["masked"].sum()) == R * (K - 1)
    rej = out["rejected"].astype(bool)
    assert int(rej.sum()) == int(np.sum(n_rej))
    assert np.all((out["slot_mapping"] == -1) == rej)
    live_slots = out["slot_mapping"][~rej]
    assert len(np.unique(live_slots)) == len(live_slots)
    for r in range(R):
        rows = np.nonzero((out["req_of_row"] == r) & ~rej)[0]
        p = out["draft_pos"][rows]
        assert np.all(np.diff(p) > 0)
        np.testing.assert_array_equal(out["slot_mapping"][rows], kv_base[r] + p)
        qr = out["query_rows"][r * K:(r + 1) * K]
        np.testing.assert_array_equal(out["draft_pos"][qr], kv_len[r] + (cu_window[r + 1] - cu_window[r] - n_rej[r]) + np.arange(K))
        assert np.all(out["draft_ids"][qr[1:]] == mask_id)
        assert np.all(out["masked"][qr[1:]] == 1) and out["masked"][qr[0]] == 0
    m = out["masked"].astype(bool)
    assert np.all(out["draft_hidden"][m] == h_shared[None])
    assert np.all(out["hidden_src"][m] == -1)
    nm = ~m
    np.testing.assert_array_equal(out["draft_hidden"][nm], target_hidden[out["hidden_src"][nm]])


@pytest.mark.parametrize("seed,R,K", [(5, 3, 4), (6, 8, 7), (7, 1, 1)])
def test_invariants_random(seed, R, K):
    dims = si.DrafterDims(64, 4, 2, 32, 128, 512, "bf16")
    g = np.random.default_rng(seed)
    W = g.integers(0, 9, R)
    n_rej = np.array([g.integers(0, w + 1) for w in W])
    kv_len = g.integers(0, 50, R)
    c = si.decode_case(dims, seed, R, K, W, kv_len, n_rej)
    hs = si.to_storage(np.full((3, 64), 0.5, np.float32), "bf16")
    out = ob.build_draft_batch(K, dims.mask_token_id, c["cu_window"], c["n_rej"], c["kv_len"],
                               c["kv_base"], c["window_ids"], c["window_pos"], c["window_hrow"],
                               c["new_token"], c["ctx_hrow"], c["target_hidden"], hs)
    check_invariants(out, K, R, c["cu_window"], c["n_rej"], c["kv_len"], c["kv_base"],
                     c["target_hidden"], hs, dims.mask_token_id)


def test_planted_mistake_is_caught():
    """A next-token row placed one position late breaks the golden example."""
    g, args = _golden_inputs()
    args["kv_len"] = args["kv_len"] + 1
    out = ob.build_draft_batch(**args)
    assert not np.array_equal(out["draft_pos"], np.array(g["expected"]["draft_pos"]))
