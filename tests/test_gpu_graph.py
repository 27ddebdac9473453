"""The whole drafter forward captured into a HIP graph: every replay, with
eager work and synchronisation between replays, must equal the eager result
bit for bit (tokens, layer output, written KV rows).  Cases: the tiny f32
config, a small bf16 case with split KV ranges, and a 24-request bf16 case
whose contractions take the large-M kernels (K splits and their reduces)."""
import numpy as np
import pytest
import torch

from drafter_pe_build_amd.step import DraftStep, GraphStep
from helpers import bits, say
from synth import inputs as si

pytestmark = pytest.mark.gpu


def _case(name):
    if name == "tiny":
        return si.decode_config(0)
    if name == "many_requests_large_m":
        # 168 query rows and 336 draft rows: the LDS-tiled large-M kernel for
        # the LM head, K-split fc / QKV / O / down with their reduces, and
        # normalised rows in the operand layout
        dims = si.DrafterDims(hidden=1024, n_q_heads=16, n_kv_heads=4, head_dim=64, ffn=2048, vocab=8192,
                              dtype="bf16")
        W = si.drafter_weights(dims, 33)
        g = np.random.default_rng(33)
        R = 24
        c = si.decode_case(dims, 33, R=R, K=7, W=[7] * R, kv_len=[int(x) for x in g.integers(100, 600, R)],
                           n_rej=[int(x) for x in g.integers(0, 7, R)])
        return dims, W, c
    dims = si.DrafterDims(hidden=128, n_q_heads=8, n_kv_heads=2, head_dim=64, ffn=256, vocab=1000, dtype="bf16")
    W = si.drafter_weights(dims, 31)
    c = si.decode_case(dims, 31, R=2, K=7, W=[3, 0], kv_len=[300, 1200], n_rej=[1, 0])
    return dims, W, c


@pytest.mark.parametrize("name", ["tiny", "small_bf16_split_kv", "many_requests_large_m"])
def test_graph_replay_equals_eager(name):
    say("graph %s" % name)
    dims, W, c = _case(name)
    st = DraftStep(dims, W, c)
    st.run()
    torch.cuda.synchronize()
    tok, xo, kc = st.tokens.clone(), st.x_out.clone(), st.k_cache.clone()
    gs = GraphStep(st)
    for i in range(3):
        st.x_out.zero_()
        st.tokens.fill_(-7)
        gs.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.tokens, tok), i
        assert np.array_equal(bits(st.x_out), bits(xo)), i
        assert np.array_equal(bits(st.k_cache), bits(kc)), i
        st.run()                       # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(st.tokens, tok)
